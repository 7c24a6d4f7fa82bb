"""Block-diagonal attention with a rotary position embedding fused in, in fp64.

Test infrastructure only (see the package docstring).

The pages mention the fusion in one sentence ("TLX Block Attention", bittide page,
opening summary: with the rotary embedding fused into the attention's
post-processing, the attention plus rotary backward runs about 3.5x faster than the
unfused baseline) and give neither the rotation's layout nor its formula.  Readings
(each a parameter or a plain choice here):

* the operation is block-diagonal attention (64-token blocks) over rope(q), rope(k)
  and v, with rope the rotary position embedding of RoFormer (Su et al.): pair
  (x_i, x_{i + D/2}), i < D/2 ("rotate half" pairing), is turned by the angle
  p * theta_i with theta_i = base^(-2i/D), base = 10000;
* the position p of a token is its index inside its own sequence (it restarts at 0 for
  every sequence of the jagged batch);
* the backward returns the gradients with respect to the un-rotated q and k (the
  rotation's backward, R^T, is the attention backward's post-processing).

The cos / sin values enter as a table [P, D/2, 2] (cos, sin of p * theta_i), the form
the library takes them in; ``rope_table`` builds it from the definition.
"""

import numpy as np

from .attention import MODE_BLOCK_DIAG, attention_backward, attention_forward
from .offsets import validate_offsets


def rope_table(max_pos, head_dim, base=10000.0):
    """cos and sin of p * base^(-2i/D) for p < max_pos, i < D/2: [max_pos, D/2, 2] fp64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1)


def positions(offsets, total):
    """Index of every token inside its own sequence: [T] int64."""
    off = validate_offsets(offsets, total)
    pos = np.zeros(total, dtype=np.int64)
    for b in range(len(off) - 1):
        pos[off[b]:off[b + 1]] = np.arange(off[b + 1] - off[b])
    return pos


def rotate(x, offsets, table, inverse=False):
    """rope(x) for x [T, H, D] (R^T x with inverse=True), angles from ``table``."""
    x = np.asarray(x, dtype=np.float64)
    t, _, d = x.shape
    h2 = d // 2
    tab = np.asarray(table, dtype=np.float64)
    pos = positions(offsets, t)
    if t and pos.max() >= tab.shape[0]:
        raise ValueError("the table holds fewer positions than the longest sequence")
    cos = tab[pos, :, 0][:, None, :]   # [T, 1, D/2]
    sin = tab[pos, :, 1][:, None, :]
    if inverse:
        sin = -sin
    x1, x2 = x[..., :h2], x[..., h2:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def rotary_block_forward(q, k, v, offsets, table, scale=None, block=64):
    """Block-diagonal attention of rope(q), rope(k), v.  Returns (o [T, H, D], lse [H, T])."""
    return attention_forward(rotate(q, offsets, table), rotate(k, offsets, table), v, offsets, MODE_BLOCK_DIAG,
                             scale, block)


def rotary_block_backward(q, k, v, do, offsets, table, scale=None, block=64, o_given=None):
    """Gradients of sum(O * dO) with respect to q, k (un-rotated) and v.  o_given: the
    forward output Di is formed from (default: the exact O; see attention.py)."""
    gq, gk, gv = attention_backward(rotate(q, offsets, table), rotate(k, offsets, table), v, do, offsets,
                                    MODE_BLOCK_DIAG, scale, block, o_given)
    return rotate(gq, offsets, table, inverse=True), rotate(gk, offsets, table, inverse=True), gv
