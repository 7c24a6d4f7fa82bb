"""MXFP8 variant of jagged self-attention, in fp64.

Test infrastructure only (see the package docstring).

The pages name the variant in one line ("Jagged Flash Attention on TLX", aixai.ru,
closing section on variants: MXFP8 data, block scales, P quantised on the fly, the same
pipeline).  MXFP8 is the OCP Microscaling format: blocks of 32 elements share one
E8M0 scale 2^X (X in [-127, 127]) and each element is an FP8 E4M3 value (4 exponent
bits, bias 7, 3 mantissa bits, largest finite 448, no infinities).  Readings:

* quantisation of a block (OCP MX rule): X = floor(log2(max |x|)) - 8 (8 = the largest
  E4M3 exponent), each element x / 2^X rounded to nearest E4M3 (ties to even) and
  clamped to +-448; an all-zero block takes X = 0;
* Q and K are blocked along the head dimension (the contraction of Q K^T); V along the
  keys of each sequence (the contraction of P V), 32 keys per block from the
  sequence's start, the last block partial;
* S, the softmax and its statistics are exact functions of the dequantised Q, K (fp32
  in the kernel); P enters the P V product quantised per 32 keys of a query row with
  the smallest power-of-two scale that keeps the block's largest value at most 448 (no
  saturation) -- the kernel quantises the running, not the final, P, so this oracle
  keeps P exact and ``p_quantisation_bound`` bounds what quantising it can change.
"""

import numpy as np

from .attention import MODE_SELF, attention_backward, attention_forward
from .offsets import validate_offsets

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_round(x):
    """Nearest E4M3 value of every element (ties to even), clamped to +-448.  fp64 in, fp64 out."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.exp2(np.maximum(e, -6.0) - 3.0)       # spacing: 2^(e-3) for normals, 2^-9 below 2^-6
    q = np.round(a / step) * step                     # np.round: ties to even
    return np.sign(x) * np.minimum(q, E4M3_MAX)


def e4m3_codes(v):
    """E4M3 byte codes of values that are already E4M3 (sign bit, exponent, mantissa)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e + 7, 0).astype(np.int64)
    mant = np.where(normal, a / np.exp2(e) - 1.0, a / 2.0 ** -6) * 8
    code = (exp_field << 3) | np.rint(mant).astype(np.int64)
    return (code | np.where(np.signbit(v) & (a > 0), 0x80, 0)).astype(np.uint8)


def e4m3_decode(codes):
    c = np.asarray(codes, dtype=np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(s == 1, -v, v)


def block_scale_exponents(blocks):
    """OCP MX shared exponent of each block (last axis = the 32 elements)."""
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        x = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8
    return np.clip(np.where(amax > 0, x, 0), -127, 127).astype(np.int64)


def quantise_blocks(blocks):
    """(E4M3 values, shared exponents X) of blocks [..., 32]; x ~= value * 2^X."""
    blocks = np.asarray(blocks, dtype=np.float64)
    x = block_scale_exponents(blocks)
    return e4m3_round(blocks / np.exp2(x)[..., None]), x


def quantise_qk(t):
    """Q or K [T, H, D] blocked along D: (values [T, H, D], X [T, H, D/32])."""
    t = np.asarray(t, dtype=np.float64)
    n, h, d = t.shape
    vals, x = quantise_blocks(t.reshape(n, h, d // BLOCK, BLOCK))
    return vals.reshape(n, h, d), x


def quantise_v(v, offsets):
    """V [T, H, D] blocked along the keys of each sequence (32 from its start, the last
    block partial, i.e. zero-padded): (values [T, H, D], X as a list over sequences of
    [nblocks, H, D])."""
    v = np.asarray(v, dtype=np.float64)
    off = validate_offsets(offsets, v.shape[0])
    vals = np.zeros_like(v)
    xs = []
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        nb = -(-(e - s) // BLOCK)
        pad = np.zeros((nb * BLOCK,) + v.shape[1:])
        pad[:e - s] = v[s:e]
        blk = pad.reshape(nb, BLOCK, v.shape[1], v.shape[2]).transpose(0, 2, 3, 1)   # [nb, H, D, 32]
        qv, x = quantise_blocks(blk)
        vals[s:e] = qv.transpose(0, 3, 1, 2).reshape(nb * BLOCK, v.shape[1], v.shape[2])[:e - s]
        xs.append(x)
    return vals, xs


def dequantise_qk(vals, x):
    n, h, d = vals.shape
    return (vals.reshape(n, h, d // BLOCK, BLOCK) * np.exp2(x)[..., None]).reshape(n, h, d)


def dequantise_v(vals, xs, offsets):
    off = validate_offsets(offsets, vals.shape[0])
    out = np.zeros_like(vals, dtype=np.float64)
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        keys = np.arange(e - s)
        out[s:e] = vals[s:e] * np.exp2(xs[b][keys // BLOCK])
    return out


def mxfp8_forward(q, k, v, offsets, scale=None):
    """Self attention of the dequantised inputs (fp64, exact P).  Returns (o, lse)."""
    return attention_forward(q, k, v, offsets, MODE_SELF, scale)


def mxfp8_backward(q, k, v, do, offsets, scale=None, o_given=None):
    """Gradient (dq, dk, dv) of self attention with respect to the dequantised inputs
    (fp64).  Reading: the pages report an MXFP8 backward without saying which of its
    products run in FP8; this one decodes the inputs and differentiates attention at the
    decoded point, P and dS unquantised, and lets gradients pass the quantisation
    straight through.  o_given: the forward output Di is formed from (the MXFP8
    forward's O, whose P was quantised; default: the exact O)."""
    return attention_backward(q, k, v, do, offsets, MODE_SELF, scale, o_given=o_given)


def p_quantisation_bound(q, k, v, offsets, scale=None):
    """Per (row, head) bound [T, H] on what quantising P per 32 keys can change in O:
    every element of P is rounded with relative error <= 2^-4 (no saturation, by the
    choice of scale), or, below the E4M3 normal range, with absolute error <= 2^-10 of a
    block scale that is at most 2/448 of the block's largest value (<= 1 after the
    softmax's final rescaling), so
        |dO| <= (2^-4 sum_j P_j |V_j| + 2^-9 / 448 sum_j |V_j|) / l."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    t, h, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    off = validate_offsets(offsets, t)
    out = np.zeros((t, h))
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        if e == s:
            continue
        for hh in range(h):
            sc = scale * q[s:e, hh] @ k[s:e, hh].T
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            l = p.sum(axis=1)
            av = np.abs(v[s:e, hh])
            out[s:e, hh] = ((2.0 ** -4) * (p @ av) + (2.0 ** -9 / E4M3_MAX) * av.sum(axis=0)[None, :]).max(axis=1) / l
    return out
