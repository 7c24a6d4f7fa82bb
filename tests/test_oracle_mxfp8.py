"""Pins of the MXFP8 oracle (oracle/mxfp8.py) against the E4M3 and MX definitions:
every finite E4M3 value is a fixed point of the rounding, midpoints go to the even
neighbour, the named constants of the format, the OCP shared-exponent rule including
saturation, the partial last V block, and the P-quantisation bound against an explicit
quantisation of P."""

import numpy as np
import pytest

import oracle
from oracle import mxfp8 as M

RNG = np.random.default_rng(31)


def _finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_format_constants():
    assert M.e4m3_decode(0x7E) == 448.0            # largest finite
    assert M.e4m3_decode(0x01) == 2.0 ** -9        # smallest subnormal
    assert M.e4m3_decode(0x08) == 2.0 ** -6        # smallest normal
    assert M.e4m3_decode(0x38) == 1.0
    assert M.e4m3_decode(0xC6) == -3.5


def test_every_finite_value_is_a_fixed_point_and_round_trips_its_code():
    codes = np.array([c for c in _finite_codes() if c != 0x80])
    vals = M.e4m3_decode(codes)
    np.testing.assert_array_equal(M.e4m3_round(vals), vals)
    np.testing.assert_array_equal(M.e4m3_codes(vals), codes)


def test_midpoints_round_to_even_mantissa_and_large_values_saturate():
    pos = np.sort(M.e4m3_decode(np.arange(0, 0x7F)))   # 0 .. 448
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        got = M.e4m3_round(mid)
        even = lo if (int(M.e4m3_codes(lo)) & 1) == 0 else hi
        assert got == even, (lo, hi, got)
        assert M.e4m3_round(np.nextafter(mid, 0)) == lo and M.e4m3_round(np.nextafter(mid, 1e9)) == hi
    assert M.e4m3_round(480.0) == 448.0 and M.e4m3_round(-1e6) == -448.0


def test_shared_exponent_rule():
    def blk(amax):
        b = np.zeros(32)
        b[5] = amax
        return b
    np.testing.assert_array_equal(M.block_scale_exponents(np.stack([blk(448.0), blk(1.0), blk(0.0), blk(500.0),
                                                                   blk(2.0 ** -140)])), [0, -8, 0, 0, -127])
    vals, x = M.quantise_blocks(blk(500.0))
    assert x == 0 and vals[5] == 448.0                  # OCP rule saturates: 500 / 2^0 > 448
    vals, x = M.quantise_blocks(blk(3.0) + np.arange(32) * 0.01)
    assert x == -7                                      # floor(log2 3.31) - 8


def test_quantisation_error_within_half_ulp_of_each_element():
    x = RNG.standard_normal((50, 2, 64))
    vals, xs = M.quantise_qk(x)
    deq = M.dequantise_qk(vals, xs)
    blocks = np.abs(x).reshape(50, 2, 2, 32)
    scale = np.exp2(xs)[..., None]
    # relative 2^-4 in the normal range, absolute 2^-10 * 2^X below it, and the OCP
    # rule's saturation: an element above 448 * 2^X becomes 448 * 2^X
    ax = np.abs(x).reshape(blocks.shape)
    bound = np.maximum(np.maximum(2.0 ** -4 * ax, 2.0 ** -10 * scale), ax - 448.0 * scale)
    assert (ax > 448.0 * scale).any()          # the sample does exercise saturation
    assert (np.abs(deq - x).reshape(blocks.shape) <= bound + 1e-15).all()


def test_v_blocks_restart_per_sequence_and_the_last_is_partial():
    lengths = [40, 3]
    off = oracle.offsets_from_lengths(lengths)
    v = np.ones((43, 1, 32))
    v[32:40] = 100.0                                   # second block of sequence 0 only
    vals, xs = M.quantise_v(v, off)
    assert [x.shape for x in xs] == [(2, 1, 32), (1, 1, 32)]
    assert (xs[0][0] == -8).all() and (xs[0][1] == np.floor(np.log2(100.0)) - 8).all() and (xs[1] == -8).all()
    np.testing.assert_allclose(M.dequantise_v(vals, xs, off), v, rtol=2.0 ** -4)


def _quantise_p(p):
    """P [rows, keys] quantised per 32 keys with the smallest power-of-two scale that
    keeps the block maximum at most 448."""
    out = np.zeros_like(p)
    for j in range(0, p.shape[1], 32):
        blk = p[:, j:j + 32]
        amax = blk.max(axis=1, keepdims=True)
        x = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0))
        out[:, j:j + 32] = M.e4m3_round(blk / np.exp2(x)) * np.exp2(x)
    return out


def test_p_quantisation_bound_holds_for_quantised_p():
    lengths = [70, 1, 200]
    off = oracle.offsets_from_lengths(lengths)
    q, k, v = (RNG.standard_normal((271, 2, 64)) for _ in range(3))
    bound = M.p_quantisation_bound(q, k, v, off, 0.125)
    o, _ = M.mxfp8_forward(q, k, v, off, 0.125)
    changed = False
    for b in range(3):
        s, e = int(off[b]), int(off[b + 1])
        for h in range(2):
            sc = 0.125 * q[s:e, h] @ k[s:e, h].T
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            oq = _quantise_p(p) @ v[s:e, h] / p.sum(axis=1, keepdims=True)
            err = np.abs(oq - o[s:e, h]).max(axis=1)
            assert (err <= bound[s:e, h] + 1e-12).all()
            changed = changed or bool((err > 0).any())
    assert changed                                      # quantising P does change O


def test_mxfp8_backward_matches_finite_differences_at_the_decoded_point():
    """Brute force: central differences of L = sum(O * dO) with respect to single
    elements of the dequantised q, k, v of two sequences."""
    lengths = [5, 3]
    off = oracle.offsets_from_lengths(lengths)
    rng = np.random.default_rng(11)
    raw = [rng.standard_normal((8, 1, 32)) for _ in range(3)]
    qv, qx = M.quantise_qk(raw[0])
    kv, kx = M.quantise_qk(raw[1])
    vv, vx = M.quantise_v(raw[2], off)
    q, k = M.dequantise_qk(qv, qx), M.dequantise_qk(kv, kx)
    v = M.dequantise_v(vv, vx, off)
    do = rng.standard_normal((8, 1, 32))
    grads = M.mxfp8_backward(q, k, v, do, off, 0.2)
    eps = 1e-6

    def loss(qq, kk, vv_):
        o, _ = M.mxfp8_forward(qq, kk, vv_, off, 0.2)
        return float((o * do).sum())

    for which in range(3):
        for (t, d) in ((0, 0), (4, 17), (6, 31)):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][t, 0, d] += eps
            up = loss(*args)
            args[which][t, 0, d] -= 2 * eps
            down = loss(*args)
            fd = (up - down) / (2 * eps)
            assert abs(fd - grads[which][t, 0, d]) <= 1e-6 * max(1.0, abs(fd)), (which, t, d)
