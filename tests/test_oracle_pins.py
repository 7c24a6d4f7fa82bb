"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each pin is a value printed on the
pages (tests/golden), an independent library routine (torch's fp64 CPU
scaled_dot_product_attention and autograd, scipy's logsumexp), a closed form, an
invariant, or central finite differences.  ``test_planted_mistakes_are_caught``
plants plausible mistakes in copies of the oracle and checks that the pins fail.
"""

import json
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


# ----------------------------------------------------------------------------- offsets

def test_worked_offsets_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_offsets.json")))
    off = oracle.offsets_from_lengths(g["lengths"])
    assert off.tolist() == g["offsets"]
    assert int(off[-1]) == g["total_tokens"]
    assert oracle.lengths_from_offsets(g["offsets"]).tolist() == g["lengths"]
    padded = len(g["lengths"]) * max(g["lengths"])
    assert padded == g["padded_tokens"]
    waste = 1 - g["total_tokens"] / padded
    assert 0.55 < waste <= g["padding_waste_up_to"]


@pytest.mark.parametrize("bad,msg", [([1, 2, 3], "offsets\\[0\\]"), ([0, 5, 3], "decrease")])
def test_offsets_validation_rejects(bad, msg):
    with pytest.raises(ValueError, match=msg):
        oracle.validate_offsets(bad)
    with pytest.raises(ValueError, match="packed token count"):
        oracle.validate_offsets([0, 2, 4], total_tokens=5)


def test_block_offsets_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "blockdiag_example.json")))
    assert oracle.block_offsets(g["offsets"], g["block"]).tolist() == g["refined_offsets"]


# ------------------------------------------------------------------ independent refs

def _padded_sdpa(q, k, v, offsets, scale, block=None, requires_grad=False):
    """Brute force: pad to [B, H, Lmax, D], mask invalid keys (and, for the block-
    diagonal case, keys of other blocks), run torch's fp64 math attention, return
    per-sequence outputs plus the torch tensors for autograd."""
    off = [int(x) for x in offsets]
    nb = len(off) - 1
    lmax = max(1, max(off[b + 1] - off[b] for b in range(nb)))
    h, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    qp = torch.zeros(nb, h, lmax, d, dtype=torch.float64)
    kp = torch.zeros(nb, hkv, lmax, d, dtype=torch.float64)
    vp = torch.zeros_like(kp)
    mask = torch.zeros(nb, 1, lmax, lmax, dtype=torch.bool)
    for b in range(nb):
        s, e = off[b], off[b + 1]
        n = e - s
        qp[b, :, :n] = torch.from_numpy(q[s:e]).permute(1, 0, 2)
        kp[b, :, :n] = torch.from_numpy(k[s:e]).permute(1, 0, 2)
        vp[b, :, :n] = torch.from_numpy(v[s:e]).permute(1, 0, 2)
        for i in range(lmax):
            for j in range(n):
                if block is None or (i < n and i // block == j // block):
                    mask[b, 0, i, j] = True
            if i >= n:
                mask[b, 0, i, 0] = True  # padded query rows: any finite output, dropped later
    if requires_grad:
        qp.requires_grad_(True)
        kp.requires_grad_(True)
        vp.requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask, scale=scale,
                                                         enable_gqa=hkv != h)
    return o, (qp, kp, vp), off


def _check_forward(fwd, q, k, v, offsets, scale, mode=A.MODE_SELF, block=64):
    o, lse = fwd(q, k, v, offsets, mode, scale, block)
    ot, _, off = _padded_sdpa(q, k, v, offsets, scale, block=block if mode == A.MODE_BLOCK_DIAG else None)
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        ref = ot[b, :, : e - s].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(o[s:e], ref, rtol=1e-11, atol=1e-12)
        group = q.shape[1] // k.shape[1]
        for hh in range(q.shape[1]):
            for i in range(e - s):
                lo, hi = (s, e)
                if mode == A.MODE_BLOCK_DIAG:
                    lo = s + (i // block) * block
                    hi = min(lo + block, e)
                scores = scale * (k[lo:hi, hh // group] @ q[s + i, hh])
                np.testing.assert_allclose(lse[hh, s + i], logsumexp(scores), rtol=1e-12, atol=1e-12)


def _check_backward(bwd, q, k, v, do, offsets, scale, mode=A.MODE_SELF, block=64):
    dq, dk, dv = bwd(q, k, v, do, offsets, mode, scale, block)
    o, (qp, kp, vp), off = _padded_sdpa(q, k, v, offsets, scale,
                                        block=block if mode == A.MODE_BLOCK_DIAG else None,
                                        requires_grad=True)
    dop = torch.zeros_like(o)
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        dop[b, :, : e - s] = torch.from_numpy(do[s:e]).permute(1, 0, 2)
    (o * dop).sum().backward()
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        for got, ref in ((dq, qp.grad), (dk, kp.grad), (dv, vp.grad)):
            np.testing.assert_allclose(got[s:e], ref[b, :, : e - s].permute(1, 0, 2).numpy(),
                                       rtol=1e-10, atol=1e-11)


JAGGED = dict(lengths=[5, 1, 7, 0, 3], h=2, d=8)


def _jagged_inputs(lengths, h, d):
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    return _rand(t, h, d), _rand(t, h, d), _rand(t, h, d), _rand(t, h, d), off


def test_forward_equals_padded_masked_brute_force():
    q, k, v, _, off = _jagged_inputs(**JAGGED)
    _check_forward(A.attention_forward, q, k, v, off, 0.37)


@pytest.mark.parametrize("hkv", [1, 2])
@pytest.mark.parametrize("mode", [A.MODE_SELF, A.MODE_BLOCK_DIAG])
def test_grouped_query_forward_equals_library_gqa_attention(hkv, mode):
    # torch's own grouped-query attention (enable_gqa) on the padded, masked batch
    lengths = [5, 1, 7, 0, 3] if mode == A.MODE_SELF else [70, 3, 129]
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v = _rand(t, 4, 8), _rand(t, hkv, 8), _rand(t, hkv, 8)
    _check_forward(A.attention_forward, q, k, v, off, 0.41, mode=mode)


def test_grouped_query_heads_see_only_their_key_value_head():
    off = oracle.offsets_from_lengths([6, 4])
    q, k, v = _rand(10, 6, 8), _rand(10, 3, 8), _rand(10, 3, 8)
    o, lse = A.attention_forward(q, k, v, off, A.MODE_SELF, 0.3)
    k2, v2 = k.copy(), v.copy()
    k2[:, 1] += 1.0
    v2[:, 1] -= 2.0
    o2, lse2 = A.attention_forward(q, k2, v2, off, A.MODE_SELF, 0.3)
    changed = [not np.allclose(o[:, hh], o2[:, hh]) for hh in range(6)]
    assert changed == [False, False, True, True, False, False]  # heads 2, 3 read key/value head 1
    # identical queries in one group give identical rows within the group
    q3 = q.copy()
    q3[:, 1] = q3[:, 0]
    o3, _ = A.attention_forward(q3, k, v, off, A.MODE_SELF, 0.3)
    np.testing.assert_array_equal(o3[:, 0], o3[:, 1])


def test_grouped_query_broadcast_q_equals_per_head_cross_attention():
    off = oracle.offsets_from_lengths([4, 0, 6])
    q, k, v = _rand(5, 4, 8), _rand(10, 2, 8), _rand(10, 2, 8)
    o, lse = A.attention_forward(q, k, v, off, A.MODE_BROADCAST_Q, 0.5)
    for b, (s, e) in enumerate([(0, 4), (4, 4), (4, 10)]):
        for hh in range(4):
            if e == s:
                assert np.all(o[b, :, hh] == 0) and np.all(np.isneginf(lse[b, hh]))
                continue
            scores = 0.5 * q[:, hh] @ k[s:e, hh // 2].T
            p = np.exp(scores - logsumexp(scores, axis=1, keepdims=True))
            np.testing.assert_allclose(o[b, :, hh], p @ v[s:e, hh // 2], rtol=1e-12, atol=1e-13)


def test_grouped_query_backward_is_refused():
    off = oracle.offsets_from_lengths([3])
    with pytest.raises(ValueError):
        A.attention_backward(_rand(3, 4, 8), _rand(3, 2, 8), _rand(3, 2, 8), _rand(3, 4, 8), off)


def test_backward_equals_torch_autograd():
    q, k, v, do, off = _jagged_inputs(**JAGGED)
    _check_backward(A.attention_backward, q, k, v, do, off, 0.37)


def test_block_diag_equals_block_masked_attention():
    # block 3 keeps the brute force tiny; lengths include a trailing partial block
    q, k, v, do, off = _jagged_inputs([7, 3, 2, 0, 6], 2, 4)
    _check_forward(A.attention_forward, q, k, v, off, 0.5, A.MODE_BLOCK_DIAG, block=3)
    _check_backward(A.attention_backward, q, k, v, do, off, 0.5, A.MODE_BLOCK_DIAG, block=3)


def test_block_diag_64_token_blocks():
    q, k, v, do, off = _jagged_inputs([130, 64, 5], 1, 4)
    _check_forward(A.attention_forward, q, k, v, off, 0.5, A.MODE_BLOCK_DIAG, block=64)


# ------------------------------------------------------------ closed forms, invariants

def test_softmax_rows_sum_to_one():
    _, _, p = A.sequence_forward(_rand(6, 5), _rand(9, 5), _rand(9, 5), 0.3)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (p > 0).all()


def test_length_one_gives_o_equal_v_exactly():
    v = _rand(1, 8)
    o, lse, _ = A.sequence_forward(_rand(1, 8), _rand(1, 8), v, 0.25)
    assert np.array_equal(o, v)


def test_zero_query_gives_mean_of_v_and_log_length():
    v = _rand(11, 4)
    o, lse, _ = A.sequence_forward(np.zeros((3, 4)), _rand(11, 4), v, 0.8)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), (3, 4)), rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(11.0), rtol=1e-14)


def test_constant_v_gives_constant_o():
    o, _, _ = A.sequence_forward(_rand(4, 6), _rand(5, 6), np.ones((5, 6)), 1.3)
    np.testing.assert_allclose(o, 1.0, rtol=1e-14)


def test_finite_differences_of_sum_o_do():
    rng = np.random.default_rng(7)
    lengths, h, d, scale = [3, 1, 4], 2, 4, 0.7
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v, do = (rng.standard_normal((t, h, d)) for _ in range(4))

    def f(qq, kk, vv):
        o, _ = A.attention_forward(qq, kk, vv, off, A.MODE_SELF, scale)
        return float((o * do).sum())

    dq, dk, dv = A.attention_backward(q, k, v, do, off, A.MODE_SELF, scale)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, k, v]
        num = np.zeros_like(grad)
        for idx in np.ndindex(grad.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            num[idx] = (f(*plus) - f(*minus)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_di_identity():
    q, k, v, do = _rand(5, 4), _rand(7, 4), _rand(7, 4), _rand(5, 4)
    o, _, p = A.sequence_forward(q, k, v, 0.6)
    dp = do @ v.T
    np.testing.assert_allclose((do * o).sum(axis=1), (p * dp).sum(axis=1), rtol=1e-12, atol=1e-13)


def test_backward_on_a_given_forward_output():
    """o_given (the forward output the backward receives) enters only through
    Di = rowsum(dO * O): with O' = O + E and delta = rowsum(dO * E), dV is unchanged and
    dS = P (dP - Di) moves by -P delta, so dQ moves by -scale delta (P K) and dK by
    -scale (P * delta)^T Q.  Checked against torch autograd of the exact gradient and an
    independent softmax (scipy), for self and broadcast-Q batches."""
    from scipy.special import softmax
    lengths, h, d, scale = [3, 1, 6], 2, 4, 0.45
    off = np.concatenate([[0], np.cumsum(lengths)])
    t = int(off[-1])
    q, k, v, do = _rand(t, h, d), _rand(t, h, d), _rand(t, h, d), _rand(t, h, d)
    o, _ = oracle.attention_forward(q, k, v, off, 0, scale)
    e = 0.01 * _rand(t, h, d)
    g0 = oracle.attention_backward(q, k, v, do, off, 0, scale)
    g1 = oracle.attention_backward(q, k, v, do, off, 0, scale, o_given=o + e)
    ge = oracle.attention_backward(q, k, v, do, off, 0, scale, o_given=o)
    for a, b in zip(g0, ge):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(g1[2], g0[2])
    for b in range(len(lengths)):
        s0, s1 = off[b], off[b + 1]
        for hh in range(h):
            qq, kk = q[s0:s1, hh], k[s0:s1, hh]
            pt = torch.tensor(qq, requires_grad=True)
            kt = torch.tensor(kk, requires_grad=True)
            ot = torch.softmax(scale * pt @ kt.T, dim=-1) @ torch.tensor(v[s0:s1, hh])
            (ot * torch.tensor(do[s0:s1, hh])).sum().backward()
            P = softmax(scale * qq @ kk.T, axis=1)
            delta = (do[s0:s1, hh] * e[s0:s1, hh]).sum(axis=1)
            np.testing.assert_allclose(g1[0][s0:s1, hh], pt.grad.numpy() - scale * delta[:, None] * (P @ kk),
                                       rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(g1[1][s0:s1, hh], kt.grad.numpy() - scale * (P * delta[:, None]).T @ qq,
                                       rtol=1e-10, atol=1e-12)
    # broadcast-Q: o [B, Mq, H, D]; dq sums the sequences' shifted contributions
    mq = 3
    qb = _rand(mq, h, d)
    dob = _rand(len(lengths), mq, h, d)
    ob, _ = oracle.attention_forward(qb, k, v, off, 1, scale)
    eb = 0.01 * _rand(*ob.shape)
    b0 = oracle.attention_backward(qb, k, v, dob, off, 1, scale)
    b1 = oracle.attention_backward(qb, k, v, dob, off, 1, scale, o_given=ob + eb)
    np.testing.assert_array_equal(b1[2], b0[2])
    shift = np.zeros_like(qb)
    for b in range(len(lengths)):
        s0, s1 = off[b], off[b + 1]
        for hh in range(h):
            P = softmax(scale * qb[:, hh] @ k[s0:s1, hh].T, axis=1)
            delta = (dob[b, :, hh] * eb[b, :, hh]).sum(axis=1)
            shift[:, hh] -= scale * delta[:, None] * (P @ k[s0:s1, hh])
    np.testing.assert_allclose(b1[0], b0[0] + shift, rtol=1e-10, atol=1e-12)


def test_identical_keys_give_zero_dq():
    k = np.tile(_rand(1, 4), (6, 1))
    dq, _, _ = A.sequence_backward(_rand(3, 4), k, _rand(6, 4), _rand(3, 4), 0.9)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)


def test_identical_values_give_zero_dq_dk():
    v = np.tile(_rand(1, 4), (6, 1))
    dq, dk, _ = A.sequence_backward(_rand(6, 4), _rand(6, 4), v, _rand(6, 4), 0.9)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)


def test_length_one_gradients():
    do = _rand(1, 4)
    dq, dk, dv = A.sequence_backward(_rand(1, 4), _rand(1, 4), _rand(1, 4), do, 0.9)
    # dP - Di = dO.v - dO.o with o = v exactly: zero up to the rounding of two dot products
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_array_equal(dv, do)


# ------------------------------------------------------------------------ broadcast-Q

def _bq_inputs(lengths, mq, h, d):
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    return _rand(mq, h, d), _rand(t, h, d), _rand(t, h, d), _rand(len(lengths), mq, h, d), off


def test_broadcast_q_b1_equals_cross_attention():
    q, k, v, do, off = _bq_inputs([6], 4, 2, 8)
    o, lse = A.attention_forward(q, k, v, off, A.MODE_BROADCAST_Q, 0.4)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.4)
    np.testing.assert_allclose(o[0], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)
    for hh in range(2):
        np.testing.assert_allclose(lse[0, hh], logsumexp(0.4 * (q[:, hh] @ k[:, hh].T), axis=1), rtol=1e-13)


def test_broadcast_q_dq_is_sum_of_single_sequence_dq():
    lengths = [3, 5, 0, 2]
    q, k, v, do, off = _bq_inputs(lengths, 4, 2, 4)
    dq, dk, dv = A.attention_backward(q, k, v, do, off, A.MODE_BROADCAST_Q, 0.5)
    total = np.zeros_like(q)
    for b, n in enumerate(lengths):
        s = int(off[b])
        qq = torch.from_numpy(q).permute(1, 0, 2).clone().requires_grad_(True)
        kk = torch.from_numpy(k[s:s + n]).permute(1, 0, 2).clone().requires_grad_(True)
        vv = torch.from_numpy(v[s:s + n]).permute(1, 0, 2).clone().requires_grad_(True)
        if n == 0:
            continue
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.5)
        (o * torch.from_numpy(do[b]).permute(1, 0, 2)).sum().backward()
        total += qq.grad.permute(1, 0, 2).numpy()
        np.testing.assert_allclose(dk[s:s + n], kk.grad.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv[s:s + n], vv.grad.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq, total, rtol=1e-11, atol=1e-12)


def test_broadcast_q_with_own_queries_equals_self_mode():
    n, h, d = 5, 2, 4
    q, k, v, do = (_rand(n, h, d) for _ in range(4))
    off = [0, n]
    o_b, lse_b = A.attention_forward(q, k, v, off, A.MODE_BROADCAST_Q, 0.3)
    o_s, lse_s = A.attention_forward(q, k, v, off, A.MODE_SELF, 0.3)
    np.testing.assert_allclose(o_b[0], o_s, rtol=1e-13)
    np.testing.assert_allclose(lse_b[0], lse_s, rtol=1e-13)


def test_broadcast_q_empty_sequence():
    q, k, v, do, off = _bq_inputs([2, 0], 3, 1, 4)
    o, lse = A.attention_forward(q, k, v, off, A.MODE_BROADCAST_Q, 0.3)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    dq_full, _, _ = A.attention_backward(q, k, v, do, off, A.MODE_BROADCAST_Q, 0.3)
    dq_one, _, _ = A.attention_backward(q, k[:2], v[:2], do[:1], [0, 2], A.MODE_BROADCAST_Q, 0.3)
    np.testing.assert_array_equal(dq_full, dq_one)


# -------------------------------------------------------------- planted mistakes

def _mutant_backward(kind):
    def seq_bwd(q, k, v, do, scale, o_given=None):
        o, _, p = A.sequence_forward(q, k, v, scale)
        if o_given is not None:
            o = o_given
        dv = p.T @ do
        dp = do @ v.T
        di = (do * o).sum(axis=1)
        if kind == "no_di":
            di = 0 * di
        ds = p * (dp - di[:, None])
        if kind == "ds_sign":
            ds = -ds
        dq = scale * (ds @ k)
        if kind == "dq_no_scale":
            dq = ds @ k
        dk = scale * (ds.T @ q)
        if kind == "dk_transposed":
            dk = scale * (ds @ q)
        if kind == "dv_transposed":
            dv = p @ do
        return dq, dk, dv

    def bwd(q, k, v, do, offsets, mode, scale, block=64):
        orig = A.sequence_backward
        try:
            A.sequence_backward = seq_bwd
            return A.attention_backward(q, k, v, do, offsets, mode, scale, block)
        finally:
            A.sequence_backward = orig
    return bwd


def _mutant_forward(kind):
    def seq_fwd(q, k, v, scale):
        s = scale * (q @ k.T)
        if kind == "no_scale":
            s = q @ k.T
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        p = e / l[:, None]
        if kind == "p_transposed":
            p = p.T
        o = p @ v
        lse = m + np.log(l)
        if kind == "lse_drops_m":
            lse = np.log(l)
        return o, lse, p

    def fwd(q, k, v, offsets, mode, scale, block=64):
        orig = A.sequence_forward
        try:
            A.sequence_forward = seq_fwd
            return A.attention_forward(q, k, v, offsets, mode, scale, block)
        finally:
            A.sequence_forward = orig
    return fwd


@pytest.mark.parametrize("kind", ["no_scale", "p_transposed", "lse_drops_m"])
def test_planted_forward_mistakes_are_caught(kind):
    # square sequences so that a transposed operand still has a valid shape
    q, k, v, _, off = _jagged_inputs([4, 4], 2, 4)
    with pytest.raises(AssertionError):
        _check_forward(_mutant_forward(kind), q, k, v, off, 0.37)


@pytest.mark.parametrize("kind", ["no_di", "ds_sign", "dq_no_scale", "dk_transposed", "dv_transposed"])
def test_planted_backward_mistakes_are_caught(kind):
    q, k, v, do, off = _jagged_inputs([4, 4], 2, 4)
    with pytest.raises(AssertionError):
        _check_backward(_mutant_backward(kind), q, k, v, do, off, 0.37)
