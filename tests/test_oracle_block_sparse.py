"""Pins of the block-sparse top-k oracle (oracle/block_sparse.py) against closed
forms, a hand-built example, an independent top-k (numpy's stable argsort) and
torch's attention with an explicit key mask."""

import numpy as np
import pytest
import torch

import oracle
from oracle import block_sparse as S

RNG = np.random.default_rng(11)


def _rand(*shape):
    return RNG.standard_normal(shape)


@pytest.mark.parametrize("length,ratio,want", [(0, 0.5, 0), (1, 0.5, 1), (64, 0.5, 1), (65, 0.5, 1),
                                               (640, 0.5, 5), (641, 0.5, 6), (640, 1.0, 10), (192, 0.25, 1),
                                               (4000, 0.5, 32), (4000, 0.25, 16)])
def test_keep_count_closed_form(length, ratio, want):
    assert S.keep_count(length, ratio) == want


def test_pooled_blocks_hand_example():
    x = np.arange(10 * 1 * 2, dtype=np.float64).reshape(10, 1, 2)
    p = S.pooled_blocks(x, 2, 9, 3)   # rows 2-4, 5-7, 8
    np.testing.assert_array_equal(p[:, 0], [[6.0, 7.0], [12.0, 13.0], [16.0, 17.0]])


def _constructed(c):
    """One sequence of 64*len(c) tokens: key block j is c[j] * u in every row, all
    queries are u, so the relevance of block j is exactly c[j]."""
    n = len(c)
    u = np.zeros(8)
    u[3] = 1.0
    k = np.concatenate([np.tile(cj * u, (64, 1)) for cj in c])[:, None, :]
    q = np.tile(u, (64 * n, 1))[:, None, :]
    return q, k, [0, 64 * n]


@pytest.mark.parametrize("c,ratio,want", [([3, 1, 4, 1], 0.5, [0, 2]), ([2, 5, 5, 1], 0.5, [1, 2]),
                                          ([2, 5, 5, 1], 0.25, [1]), ([1, 1, 1, 1], 0.5, [0, 1]),
                                          ([0, -1, 7, 7, 7, 2], 0.5, [2, 3, 4])])
def test_selection_hand_examples(c, ratio, want):
    q, k, off = _constructed(c)
    sc = S.block_scores(q, k, off)[0]
    np.testing.assert_allclose(sc[0, 0], c)
    assert S.select_blocks(q, k, off, ratio)[0][0][0] == want


def test_top_k_equals_stable_argsort():
    for _ in range(200):
        n = int(RNG.integers(1, 40))
        sc = RNG.integers(-3, 4, size=n).astype(np.float64)  # many ties
        kk = int(RNG.integers(1, n + 1))
        want = sorted(np.argsort(-sc, kind="stable")[:kk].tolist())
        assert S.top_k_blocks(sc, kk) == want


def _masked_sdpa(q, k, v, offsets, selection, scale, q_block=S.Q_BLOCK, k_block=S.K_BLOCK):
    """Independent reference: per sequence, torch's fp64 attention with a boolean
    mask that lets row r of query block i see exactly the keys of its kept blocks."""
    off = [int(x) for x in offsets]
    h, hkv = q.shape[1], k.shape[1]
    o = np.zeros_like(q)
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        n = e - s
        if n == 0:
            continue
        mask = torch.zeros(h, n, n, dtype=torch.bool)
        for hh in range(h):
            for i, r0 in enumerate(range(0, n, q_block)):
                for j in selection[b][hh][i]:
                    mask[hh, r0:min(r0 + q_block, n), j * k_block:min((j + 1) * k_block, n)] = True
        qt = torch.from_numpy(q[s:e]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k[s:e]).permute(1, 0, 2)[None]
        vt = torch.from_numpy(v[s:e]).permute(1, 0, 2)[None]
        ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None], scale=scale,
                                                              enable_gqa=hkv != h)
        o[s:e] = ot[0].permute(1, 0, 2).numpy()
    return o


def _random_selection(lengths, h, ratio):
    sel = []
    for n in lengths:
        nqb, nkb = -(-n // S.Q_BLOCK), -(-n // S.K_BLOCK)
        kk = S.keep_count(n, ratio)
        sel.append([[sorted(RNG.choice(nkb, size=kk, replace=False).tolist()) for _ in range(nqb)]
                    for _ in range(h)])
    return sel


@pytest.mark.parametrize("hkv", [2, 1])
def test_sparse_forward_equals_masked_attention(hkv):
    lengths = [300, 1, 70, 0, 520]
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v = _rand(t, 2, 8), _rand(t, hkv, 8), _rand(t, hkv, 8)
    sel = _random_selection(lengths, 2, 0.5)
    o, lse = S.block_sparse_forward(q, k, v, off, sel, 0.4)
    np.testing.assert_allclose(o, _masked_sdpa(q, k, v, off, sel, 0.4), rtol=1e-11, atol=1e-12)
    # lse over exactly the kept keys, for one row of each sequence
    for b in (0, 4):
        s = int(off[b])
        keys = np.concatenate([np.arange(s + 64 * j, min(s + 64 * (j + 1), int(off[b + 1]))) for j in sel[b][1][0]])
        sc = 0.4 * k[keys, 1 // (2 // hkv)] @ q[s, 1]
        np.testing.assert_allclose(lse[1, s], np.log(np.exp(sc - sc.max()).sum()) + sc.max(), rtol=1e-12)


def test_ratio_one_equals_dense_attention():
    lengths = [300, 5, 129]
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v = _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8)
    sel = S.select_blocks(q, k, off, 1.0)
    assert all(lst == list(range(-(-n // 64))) for b, n in enumerate(lengths) for per_h in sel[b] for lst in per_h)
    o, lse = S.block_sparse_forward(q, k, v, off, sel, 0.3)
    o_d, lse_d = oracle.attention_forward(q, k, v, off, oracle.MODE_SELF, 0.3)
    np.testing.assert_allclose(o, o_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o, _masked_sdpa(q, k, v, off, sel, 0.3), rtol=1e-11, atol=1e-12)


def test_planted_selection_mistake_is_caught():
    lengths = [520]
    off = oracle.offsets_from_lengths(lengths)
    q, k, v = _rand(520, 1, 8), _rand(520, 1, 8), _rand(520, 1, 8)
    sel = _random_selection(lengths, 1, 0.5)
    shifted = [[[min(j + 1, 8) for j in lst] for lst in per_h] for per_h in sel[0]]
    o, _ = S.block_sparse_forward(q, k, v, off, [shifted], 0.4)
    assert not np.allclose(o, _masked_sdpa(q, k, v, off, sel, 0.4), rtol=1e-6, atol=1e-8)


def _masked_sdpa_grads(q, k, v, do, offsets, selection, scale):
    """Independent reference for the backward: torch autograd through fp64 attention
    with the same boolean key mask as _masked_sdpa."""
    off = [int(x) for x in offsets]
    grads = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        n = e - s
        if n == 0:
            continue
        h = q.shape[1]
        mask = torch.zeros(h, n, n, dtype=torch.bool)
        for hh in range(h):
            for i, r0 in enumerate(range(0, n, S.Q_BLOCK)):
                for j in selection[b][hh][i]:
                    mask[hh, r0:min(r0 + S.Q_BLOCK, n), j * S.K_BLOCK:min((j + 1) * S.K_BLOCK, n)] = True
        ts = [torch.from_numpy(np.ascontiguousarray(x[s:e].transpose(1, 0, 2)))[None].requires_grad_() for x in (q, k, v)]
        ot = torch.nn.functional.scaled_dot_product_attention(*ts, attn_mask=mask[None], scale=scale)
        ot.backward(torch.from_numpy(np.ascontiguousarray(do[s:e].transpose(1, 0, 2)))[None])
        for g, tt in zip(grads, ts):
            g[s:e] = tt.grad[0].permute(1, 0, 2).numpy()
    return grads


def test_sparse_backward_equals_autograd_of_masked_attention():
    lengths = [300, 1, 70, 0, 520, 64]
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v, do = _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8)
    sel = _random_selection(lengths, 2, 0.5)
    sel[4][0] = [[0, 1, 2, 3, 4], [0, 1, 2, 3, 5], [1, 2, 3, 4, 5]]   # key blocks 6-8 kept by no query block
    got = S.block_sparse_backward(q, k, v, do, off, sel, 0.4)
    want = _masked_sdpa_grads(q, k, v, do, off, sel, 0.4)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12)
    # a key block that no query block kept gets zero dK, dV
    for jb in (6, 7, 8):
        r = slice(int(off[4]) + 64 * jb, min(int(off[4]) + 64 * (jb + 1), int(off[5])))
        assert not got[1][r, 0].any() and not got[2][r, 0].any()


def test_sparse_backward_ratio_one_equals_dense_backward():
    lengths = [300, 5, 129]
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v, do = _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8)
    sel = S.select_blocks(q, k, off, 1.0)
    got = S.block_sparse_backward(q, k, v, do, off, sel, 0.3)
    want = oracle.attention_backward(q, k, v, do, off, oracle.MODE_SELF, 0.3)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-12, atol=1e-13)


def test_sparse_backward_finite_difference():
    """d/dx of sum(O * dO) by central differences at a few coordinates of q, k, v."""
    lengths = [300]
    off = oracle.offsets_from_lengths(lengths)
    q, k, v, do = _rand(300, 1, 4), _rand(300, 1, 4), _rand(300, 1, 4), _rand(300, 1, 4)
    sel = [[[[0, 3, 4], [1, 4]]]]
    grads = S.block_sparse_backward(q, k, v, do, off, sel, 0.5)
    f = lambda qq, kk, vv: float((S.block_sparse_forward(qq, kk, vv, off, sel, 0.5)[0] * do).sum())
    eps = 1e-6
    for which, (r, c) in [(0, (5, 1)), (0, (290, 3)), (1, (10, 0)), (1, (260, 2)), (2, (70, 1)), (2, (299, 0))]:
        args = [q, k, v]
        plus = [a.copy() for a in args]
        minus = [a.copy() for a in args]
        plus[which][r, 0, c] += eps
        minus[which][r, 0, c] -= eps
        fd = (f(*plus) - f(*minus)) / (2 * eps)
        assert abs(fd - grads[which][r, 0, c]) < 1e-6 * max(1.0, abs(fd)), (which, r, c)


def test_sparse_backward_refuses_grouped_heads():
    off = oracle.offsets_from_lengths([70])
    with pytest.raises(ValueError):
        S.block_sparse_backward(_rand(70, 2, 8), _rand(70, 1, 8), _rand(70, 1, 8), _rand(70, 2, 8), off,
                                [[[[0]], [[0]]]], 0.3)
