"""Work and traffic accounting over valid tokens only (no padding counted).

Valid query-key pairs: self-attention sum_b L_b^2; broadcast-Q Mq * sum_b L_b;
64-token block-diagonal sum over blocks of len^2.  Forward FLOPs = 4 * H * D * pairs
(two products, 2 FLOPs per multiply-add); backward FLOPs = 2.5 x forward (five
products).  Algorithmic bytes are each input read once and each output written once
(bf16 tensors, fp32 lse).
"""

import numpy as np

MODE_SELF = 0
MODE_BROADCAST_Q = 1
MODE_BLOCK_DIAG = 2


def valid_pairs(lengths, mode, num_q=0, block=64):
    lengths = np.asarray(lengths, dtype=np.int64)
    if mode == MODE_SELF:
        return int((lengths * lengths).sum())
    if mode == MODE_BROADCAST_Q:
        return int(num_q) * int(lengths.sum())
    if mode == MODE_BLOCK_DIAG:
        full = lengths // block
        rem = lengths % block
        return int((full * block * block + rem * rem).sum())
    raise ValueError("unknown mode")


def padded_pairs(lengths):
    lengths = np.asarray(lengths, dtype=np.int64)
    return int(len(lengths) * int(lengths.max(initial=0)) ** 2)


def fwd_flops(lengths, mode, num_heads, head_dim, num_q=0):
    return 4 * num_heads * head_dim * valid_pairs(lengths, mode, num_q)


def bwd_flops(lengths, mode, num_heads, head_dim, num_q=0):
    return 10 * num_heads * head_dim * valid_pairs(lengths, mode, num_q)


def fwd_bytes(lengths, mode, num_heads, head_dim, num_q=0, num_kv_heads=None):
    """Q (or the shared Q) and K, V in, O and lse out; K, V carry num_kv_heads heads
    (grouped-query attention), the rest num_heads."""
    t = int(np.asarray(lengths, dtype=np.int64).sum())
    h, d = num_heads, head_dim
    hkv = h if num_kv_heads is None else num_kv_heads
    if mode == MODE_BROADCAST_Q:
        b = len(lengths)
        return 2 * num_q * h * d + 4 * t * hkv * d + 2 * b * num_q * h * d + 4 * b * h * num_q
    return 4 * t * h * d + 4 * t * hkv * d + 4 * t * h


def bwd_bytes(lengths, mode, num_heads, head_dim, num_q=0):
    t = int(np.asarray(lengths, dtype=np.int64).sum())
    h, d = num_heads, head_dim
    if mode == MODE_BROADCAST_Q:
        b = len(lengths)
        return 4 * num_q * h * d + 8 * t * h * d + 4 * b * num_q * h * d + 4 * b * h * num_q
    return 16 * t * h * d + 4 * t * h


def block_sparse_pairs(lengths, num_heads, keep, selection, q_block=256, k_block=64):
    """Query-key pairs the block-sparse forward attends: for every (sequence, head,
    query block) the block's rows times the keys of its kept key blocks.  ``keep`` is
    the kept count per sequence and ``selection`` the flat int32 kept-block lists in
    the layout jfa_fwd_block_sparse writes (sequence, then head, then query block)."""
    sel = np.asarray(selection, dtype=np.int64)
    pairs, at = 0, 0
    for n, kk in zip(np.asarray(lengths, dtype=np.int64).tolist(), keep):
        if n == 0:
            continue
        nqb = -(-n // q_block)
        rows = np.minimum(q_block, n - q_block * np.arange(nqb))
        blocks = sel[at:at + num_heads * nqb * kk].reshape(num_heads, nqb, kk)
        at += num_heads * nqb * kk
        keys = np.minimum(k_block, n - k_block * blocks).sum(axis=2)  # [H, nqb]
        pairs += int((keys * rows[None, :]).sum())
    return pairs


def block_sparse_tile_pairs(lengths, num_heads, keep, selection, q_block=256, k_block=64, tile_keys=128):
    """Query-key pairs the block-sparse dK/dV kernel executes: it works on tiles of
    ``tile_keys`` keys (two key blocks), so a query block that kept either block of a
    tile costs the block's rows times all of the tile's keys (the other block's share is
    masked to zero)."""
    sel = np.asarray(selection, dtype=np.int64)
    pairs, at = 0, 0
    per_tile = tile_keys // k_block
    for n, kk in zip(np.asarray(lengths, dtype=np.int64).tolist(), keep):
        if n == 0:
            continue
        nqb = -(-n // q_block)
        rows = np.minimum(q_block, n - q_block * np.arange(nqb))
        blocks = sel[at:at + num_heads * nqb * kk].reshape(num_heads, nqb, kk)
        at += num_heads * nqb * kk
        for hh in range(num_heads):
            for i in range(nqb):
                tiles = np.unique(blocks[hh, i] // per_tile)
                pairs += int(rows[i] * np.minimum(tile_keys, n - tile_keys * tiles).sum())
    return pairs
