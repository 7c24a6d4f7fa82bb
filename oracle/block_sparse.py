"""Block-sparse top-k variant of jagged self-attention, in fp64.

Test infrastructure only (see the package docstring).

The pages describe the variant in one paragraph ("Jagged Flash Attention on TLX",
aixai.ru, the closing section on variants): a cheap first stage averages blocks of Q
and of K and picks, for every block of queries, the top-k most relevant blocks of
keys; the attention kernel then attends only over those blocks.  Readings where the
paragraph is silent (each one a parameter here):

* blocks: query blocks of ``q_block`` = 256 consecutive rows of one sequence and head
  (the forward kernel's query tile), key blocks of ``k_block`` = 64 keys; the last
  block of a sequence holds the remaining rows;
* pooling: the arithmetic mean of the block's rows;
* relevance: the dot product of the pooled query block and the pooled key block;
* k: ``max(1, ceil(ratio * nkb))`` blocks per query block, nkb = ceil(L / k_block),
  with ``ratio`` taken as the given float32 value and the product formed in float64;
* ties: between equal relevance the lower block index wins;
* attention: exact softmax of each query row over the keys of its query block's kept
  key blocks (the order of the blocks does not change the result).

Grouped-query attention: k, v may carry Hkv heads (query head h reads key/value head
h // (H // Hkv)), as in ``attention.attention_forward``.  Self attention only.

Backward: the paragraph names the variant's speed-up for the forward only.  Read
plainly, the backward of the variant is the gradient of sum(O * dO) with the selection
held fixed (the pooling and top-k choose which keys take part; that discrete choice
carries no gradient), i.e. for every (sequence, head, query block) the exact-attention
gradient over the kept keys, the key and value gradients summed over the query blocks
that kept them.  One query/key-value head per key-value head (H == Hkv), as for the
dense backward.
"""

import math

import numpy as np

from .attention import sequence_backward, sequence_forward
from .offsets import validate_offsets

Q_BLOCK = 256
K_BLOCK = 64


def keep_count(length, ratio, k_block=K_BLOCK):
    """Key blocks kept per query block of a sequence of ``length`` tokens."""
    if length <= 0:
        return 0
    nkb = -(-int(length) // k_block)
    return max(1, math.ceil(float(np.float32(ratio)) * nkb))


def pooled_blocks(x, s, e, block):
    """Means of consecutive ``block``-row groups of x[s:e] (rows, heads, dim) -> [n, heads, dim]."""
    x = np.asarray(x, dtype=np.float64)
    out = []
    for r in range(s, e, block):
        out.append(x[r:min(r + block, e)].mean(axis=0))
    return np.array(out).reshape(len(out), x.shape[1], x.shape[2])


def block_scores(q, k, offsets, q_block=Q_BLOCK, k_block=K_BLOCK):
    """Relevance of every key block for every query block.

    Returns a list over sequences of arrays [H, nqb, nkb] (empty sequences: shape
    [H, 0, 0])."""
    off = validate_offsets(offsets, k.shape[0])
    h, hkv = q.shape[1], k.shape[1]
    group = h // hkv
    out = []
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        if e == s:
            out.append(np.zeros((h, 0, 0)))
            continue
        qb = pooled_blocks(q, s, e, q_block)   # [nqb, H, D]
        kb = pooled_blocks(k, s, e, k_block)   # [nkb, Hkv, D]
        sc = np.zeros((h, qb.shape[0], kb.shape[0]))
        for hh in range(h):
            sc[hh] = qb[:, hh] @ kb[:, hh // group].T
        out.append(sc)
    return out


def top_k_blocks(scores, kk):
    """Indices (ascending) of the kk largest entries of a 1-D score vector; between
    equal scores the lower index wins."""
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    return sorted(order[:kk])


def select_blocks(q, k, offsets, ratio, q_block=Q_BLOCK, k_block=K_BLOCK):
    """Kept key blocks per (sequence, head, query block): a list over sequences of
    lists [H][nqb] of ascending index lists."""
    off = validate_offsets(offsets, k.shape[0])
    sel = []
    for b, sc in enumerate(block_scores(q, k, offsets, q_block, k_block)):
        kk = keep_count(off[b + 1] - off[b], ratio, k_block)
        sel.append([[top_k_blocks(sc[hh, i], kk) for i in range(sc.shape[1])] for hh in range(sc.shape[0])])
    return sel


def block_sparse_forward(q, k, v, offsets, selection, scale=None, q_block=Q_BLOCK, k_block=K_BLOCK):
    """Self attention where the rows of query block i of (sequence b, head h) attend
    to the keys of the blocks selection[b][h][i] only.  Returns (o [T, H, D], lse
    [H, T]) like ``attention.attention_forward``."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    t, hkv, d = k.shape
    h = q.shape[1]
    group = h // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    off = validate_offsets(offsets, t)
    o = np.zeros((t, h, d))
    lse = np.zeros((h, t))
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        for hh in range(h):
            hk = hh // group
            for i, r0 in enumerate(range(s, e, q_block)):
                r1 = min(r0 + q_block, e)
                keys = np.concatenate([np.arange(s + j * k_block, min(s + (j + 1) * k_block, e))
                                       for j in selection[b][hh][i]]).astype(np.int64)
                ob, lb, _ = sequence_forward(q[r0:r1, hh], k[keys, hk], v[keys, hk], scale)
                o[r0:r1, hh] = ob
                lse[hh, r0:r1] = lb
    return o, lse


def block_sparse_backward(q, k, v, do, offsets, selection, scale=None, q_block=Q_BLOCK, k_block=K_BLOCK,
                          o_given=None):
    """Gradient of sum(O * dO) of ``block_sparse_forward`` for a fixed selection.
    Returns (dq, dk, dv), each [T, H, D].  o_given [T, H, D]: the forward output Di is
    formed from (default: the exact O; see attention.py)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    og = None if o_given is None else np.asarray(o_given, dtype=np.float64)
    t, h, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or do.shape != q.shape:
        raise ValueError("the block-sparse backward takes q, k, v, do all [T, H, D] (no grouped heads)")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    off = validate_offsets(offsets, t)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        for hh in range(h):
            for i, r0 in enumerate(range(s, e, q_block)):
                r1 = min(r0 + q_block, e)
                keys = np.concatenate([np.arange(s + j * k_block, min(s + (j + 1) * k_block, e))
                                       for j in selection[b][hh][i]]).astype(np.int64)
                g_q, g_k, g_v = sequence_backward(q[r0:r1, hh], k[keys, hh], v[keys, hh], do[r0:r1, hh], scale,
                                                  None if og is None else og[r0:r1, hh])
                dq[r0:r1, hh] = g_q
                dk[keys, hh] += g_k
                dv[keys, hh] += g_v
    return dq, dk, dv
