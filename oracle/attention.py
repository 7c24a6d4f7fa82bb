"""Exact softmax attention over jagged (packed, variable-length) inputs, in fp64.

Test infrastructure only (see the package docstring).

This is the plain definition the fast path reaches up to rounding order: for every
sequence b and head h, S = scale * Q_b K_b^T, P = softmax(S) along keys, O_b = P V_b,
and the per-row log-sum-exp L = m + ln(l) with m = rowmax(S), l = rowsum(exp(S - m))
(bittide page, section 2.1, Listing 1 and the sentence after it: L is what the
backward needs to rebuild P).  The backward is the analytic gradient of
sum(O * dO): dV = P^T dO, dP = dO V^T, Di = rowsum(dO * O), dS = P * (dP - Di),
dQ = scale * dS K, dK = scale * dS^T Q (bittide page, section 4, for the five products
and the inline Di = rowsum(dO * O)).

Modes (aixai.ru page, "What is Jagged Flash Attention"; yuxiaoba page, "why unequal
lengths change the problem"; bittide page, section 1):

* MODE_SELF (0): every packed sequence attends to itself; q, k, v are [T, H, D].
* MODE_BROADCAST_Q (1): one dense Q [Mq, H, D] attends to each sequence's own K/V
  [T, H, D]; outputs are per sequence, o [B, Mq, H, D], lse [B, H, Mq]; dQ is the sum
  over all sequences of the per-sequence dQ.
* MODE_BLOCK_DIAG (2): each sequence is cut into fixed 64-token groups that attend
  only within themselves; shapes as in MODE_SELF.

Grouped-query attention (aixai.ru page, list of supported features: GQA in the
forward, the backward only with one query group): k and v may carry Hkv heads with
H % Hkv == 0; query head h then attends with key/value head h // (H // Hkv).  The
forward takes this form; the backward requires Hkv == H.

Readings where the pages are silent:

* lse is in natural-log units of the scaled scores, fp32 on the device, laid out
  [H, T] for MODE_SELF / MODE_BLOCK_DIAG and [B, H, Mq] for MODE_BROADCAST_Q.
* A broadcast-Q sequence of length 0 gives O[b] = 0 and lse[b] = -inf and adds
  nothing to any gradient; in the other modes an empty sequence has no rows at all.
* Attention is non-causal and unwindowed.

All inputs are promoted to float64 before any arithmetic; bf16 inputs therefore
enter with their exact values.

The backward takes the forward's output O as one of its inputs (bittide page, section
4: Di = rowsum(dO * O) is formed from the O the forward wrote).  By default the oracle
uses its own exact O, which gives the analytic gradient; with ``o_given`` it forms Di
from the O passed in (for instance the bf16 O of the library's forward), which is the
same backward formula evaluated on the inputs the library's backward receives.  The
two differ only through Di: dV is unchanged, and dQ, dK move by the first-order terms
of dS = P * (dP - Di) in Di.
"""

import numpy as np

from .offsets import validate_offsets, block_offsets

MODE_SELF = 0
MODE_BROADCAST_Q = 1
MODE_BLOCK_DIAG = 2


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def sequence_forward(q, k, v, scale):
    """One head of one sequence.  q [Lq, D], k [Lk, D], v [Lk, D] -> (o [Lq, D],
    lse [Lq], p [Lq, Lk]).

    S = scale * q k^T; m = rowmax S; E = exp(S - m); l = rowsum E; P = E / l;
    O = P v; lse = m + ln l.  With Lk = 0 the softmax has no terms: O = 0 and
    lse = -inf (reading for the empty broadcast-Q sequence)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, lk = q.shape[0], k.shape[0]
    if lk == 0:
        return (np.zeros((lq, v.shape[1])), np.full(lq, -np.inf), np.zeros((lq, 0)))
    s = scale * (q @ k.T)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    o = p @ v
    lse = m + np.log(l)
    return o, lse, p


def sequence_backward(q, k, v, do, scale, o_given=None):
    """Gradient of sum(O * dO) for one head of one sequence, P recomputed from
    (q, k, v) in fp64.  Returns (dq [Lq, D], dk [Lk, D], dv [Lk, D]).  o_given [Lq, D]:
    the forward output Di is formed from (default: the exact O)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if k.shape[0] == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    o, _, p = sequence_forward(q, k, v, scale)
    if o_given is not None:
        o = _f64(o_given)
    dv = p.T @ do
    dp = do @ v.T
    di = (do * o).sum(axis=1)
    ds = p * (dp - di[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def _segments(offsets, mode, block):
    off = validate_offsets(offsets)
    if mode == MODE_BLOCK_DIAG:
        off = [int(x) for x in block_offsets(off, block)]
    return off


def attention_forward(q, k, v, offsets, mode=MODE_SELF, scale=None, block=64):
    """Forward over the whole jagged batch.

    Returns (o, lse) in the library's layouts: MODE_SELF / MODE_BLOCK_DIAG:
    o [T, H, D], lse [H, T]; MODE_BROADCAST_Q: o [B, Mq, H, D], lse [B, H, Mq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    t, hkv, d = k.shape
    h = q.shape[1]
    if v.shape != k.shape or q.shape[2] != d or h % hkv:
        raise ValueError("q [., H, D], k and v [T, Hkv, D] with H a multiple of Hkv")
    group = h // hkv  # query heads per key/value head
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if mode == MODE_BROADCAST_Q:
        off = validate_offsets(offsets, t)
        nb, mq = len(off) - 1, q.shape[0]
        o = np.zeros((nb, mq, h, d))
        lse = np.zeros((nb, h, mq))
        for b in range(nb):
            s, e = off[b], off[b + 1]
            for hh in range(h):
                hk = hh // group
                ob, lb, _ = sequence_forward(q[:, hh], k[s:e, hk], v[s:e, hk], scale)
                o[b, :, hh] = ob
                lse[b, hh] = lb
        return o, lse
    if q.shape[0] != t:
        raise ValueError("self / block-diagonal attention needs q and k of one length")
    validate_offsets(offsets, t)
    seg = _segments(offsets, mode, block)
    o = np.zeros((t, h, d))
    lse = np.zeros((h, t))
    for b in range(len(seg) - 1):
        s, e = seg[b], seg[b + 1]
        if e == s:
            continue
        for hh in range(h):
            hk = hh // group
            ob, lb, _ = sequence_forward(q[s:e, hh], k[s:e, hk], v[s:e, hk], scale)
            o[s:e, hh] = ob
            lse[hh, s:e] = lb
    return o, lse


def attention_backward(q, k, v, do, offsets, mode=MODE_SELF, scale=None, block=64, o_given=None):
    """Backward over the whole jagged batch; returns (dq, dk, dv) with the shapes of
    (q, k, v).  In MODE_BROADCAST_Q dq sums the per-sequence contributions and do is
    [B, Mq, H, D].  o_given (the layout of the forward's o): the forward output Di is
    formed from (default: the exact O)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    og = None if o_given is None else _f64(o_given)
    t, h, d = k.shape
    if q.shape[1] != h:
        raise ValueError("the backward needs one query head per key/value head")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if mode == MODE_BROADCAST_Q:
        off = validate_offsets(offsets, t)
        for b in range(len(off) - 1):
            s, e = off[b], off[b + 1]
            for hh in range(h):
                g_q, g_k, g_v = sequence_backward(q[:, hh], k[s:e, hh], v[s:e, hh], do[b, :, hh], scale,
                                                  None if og is None else og[b, :, hh])
                dq[:, hh] += g_q
                dk[s:e, hh] = g_k
                dv[s:e, hh] = g_v
        return dq, dk, dv
    validate_offsets(offsets, t)
    seg = _segments(offsets, mode, block)
    for b in range(len(seg) - 1):
        s, e = seg[b], seg[b + 1]
        if e == s:
            continue
        for hh in range(h):
            g_q, g_k, g_v = sequence_backward(q[s:e, hh], k[s:e, hh], v[s:e, hh], do[s:e, hh], scale,
                                              None if og is None else og[s:e, hh])
            dq[s:e, hh] = g_q
            dk[s:e, hh] = g_k
            dv[s:e, hh] = g_v
    return dq, dk, dv
