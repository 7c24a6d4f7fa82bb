"""Pins of the rotary block-attention oracle (oracle/rotary.py): hand examples of the
rotate-half pairing, closed-form table entries, the rotation-group property (attention
depends only on relative positions), torch autograd through an independent
complex-number form of the rotation, and central differences."""

import numpy as np
import pytest
import torch

import oracle
from oracle import rotary as R

RNG = np.random.default_rng(23)


def _rand(*shape):
    return RNG.standard_normal(shape)


def test_table_closed_form_entries():
    tab = R.rope_table(50, 8)
    np.testing.assert_array_equal(tab[0, :, 0], 1.0)
    np.testing.assert_array_equal(tab[0, :, 1], 0.0)
    np.testing.assert_allclose(tab[7, 0], [np.cos(7.0), np.sin(7.0)], rtol=0, atol=1e-15)   # theta_0 = 1
    np.testing.assert_allclose(tab[7, 2], [np.cos(0.07), np.sin(0.07)], rtol=0, atol=1e-15)  # 10000^(-1/2)
    np.testing.assert_allclose(tab[49, 1], [np.cos(4.9), np.sin(4.9)], rtol=0, atol=1e-14)   # 10000^(-1/4) = 0.1


def test_rotate_half_pairing_hand_example():
    """D = 4, one token at position 1: element 0 pairs with element 2 and turns by
    theta_0 = 1 rad, element 1 pairs with element 3 and turns by 0.01 rad."""
    tab = R.rope_table(2, 4)
    off = [0, 1, 2]   # second sequence's token is at position 0, the first's at 0 too
    off2 = [0, 2]     # one sequence: tokens at positions 0 and 1
    x = np.zeros((2, 1, 4))
    x[1, 0, 0] = 1.0
    np.testing.assert_allclose(R.rotate(x, off2, tab)[1, 0], [np.cos(1), 0, np.sin(1), 0], atol=1e-15)
    x[1, 0] = [0, 0, 1, 0]
    np.testing.assert_allclose(R.rotate(x, off2, tab)[1, 0], [-np.sin(1), 0, np.cos(1), 0], atol=1e-15)
    x[1, 0] = [0, 1, 0, 0]
    np.testing.assert_allclose(R.rotate(x, off2, tab)[1, 0], [0, np.cos(0.01), 0, np.sin(0.01)], atol=1e-15)
    np.testing.assert_array_equal(R.rotate(x, off, tab), x)  # both tokens at position 0: unchanged


def test_positions_restart_per_sequence():
    np.testing.assert_array_equal(R.positions([0, 3, 3, 5], 5), [0, 1, 2, 0, 1])


def test_rotation_is_orthogonal_and_inverse_undoes_it():
    off = oracle.offsets_from_lengths([70, 1, 200])
    x = _rand(271, 2, 16)
    tab = R.rope_table(256, 16)
    y = R.rotate(x, off, tab)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(R.rotate(y, off, tab, inverse=True), x, rtol=1e-12, atol=1e-13)


def test_attention_depends_only_on_relative_positions():
    """Shifting every position by s (a table starting at angle s * theta) leaves the
    block attention unchanged: q.k after rotation depends on p_q - p_k only."""
    lengths = [130, 64, 5]
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v = _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8)
    o0, l0 = R.rotary_block_forward(q, k, v, off, R.rope_table(200, 8), 0.3)
    o1, l1 = R.rotary_block_forward(q, k, v, off, R.rope_table(237, 8)[37:], 0.3)
    np.testing.assert_allclose(o1, o0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=1e-12, atol=1e-12)
    # ... and the rotation does change the result
    o2, _ = oracle.attention_forward(q, k, v, off, oracle.MODE_BLOCK_DIAG, 0.3)
    assert not np.allclose(o0, o2, atol=1e-3)


def test_zero_angles_reduce_to_block_attention():
    lengths = [100, 64]
    off = oracle.offsets_from_lengths(lengths)
    q, k, v, do = _rand(164, 1, 8), _rand(164, 1, 8), _rand(164, 1, 8), _rand(164, 1, 8)
    tab = np.zeros((100, 4, 2))
    tab[..., 0] = 1.0
    o, lse = R.rotary_block_forward(q, k, v, off, tab, 0.4)
    o_ref, lse_ref = oracle.attention_forward(q, k, v, off, oracle.MODE_BLOCK_DIAG, 0.4)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)
    for g, r in zip(R.rotary_block_backward(q, k, v, do, off, tab, 0.4),
                    oracle.attention_backward(q, k, v, do, off, oracle.MODE_BLOCK_DIAG, 0.4)):
        np.testing.assert_array_equal(g, r)


def _torch_reference(q, k, v, do, lengths, base, scale):
    """Independent form: rotation as multiplication of (x_i + 1j x_{i+D/2}) by
    exp(1j p theta_i) (torch.polar), attention by torch SDPA with a block mask, and
    the gradients from torch autograd."""
    d = q.shape[-1]
    ts = [torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v)]
    pos = torch.cat([torch.arange(n, dtype=torch.float64) for n in lengths])
    theta = torch.exp(-torch.arange(d // 2, dtype=torch.float64) * (2.0 / d) * np.log(base))
    rot = torch.polar(torch.ones(len(pos), d // 2, dtype=torch.float64), pos[:, None] * theta[None, :])[:, None, :]

    def rope(x):
        z = torch.complex(x[..., :d // 2], x[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    qr, kr = rope(ts[0]), rope(ts[1])
    t = len(pos)
    blk = torch.cat([torch.full((n,), i, dtype=torch.int64) for i, n in enumerate(lengths)]) * 1000 + \
        torch.cat([torch.arange(n) // 64 for n in lengths])
    mask = blk[:, None] == blk[None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qr.permute(1, 0, 2)[None], kr.permute(1, 0, 2)[None],
                                                         ts[2].permute(1, 0, 2)[None], attn_mask=mask[None, None],
                                                         scale=scale)[0].permute(1, 0, 2)
    o.backward(torch.from_numpy(do.copy()))
    assert o.shape[0] == t
    return o.detach().numpy(), [x.grad.numpy() for x in ts]


def test_forward_and_backward_equal_torch_autograd_of_complex_rotation():
    lengths = [130, 1, 64, 70]
    off = oracle.offsets_from_lengths(lengths)
    t = int(off[-1])
    q, k, v, do = _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8), _rand(t, 2, 8)
    tab = R.rope_table(256, 8)
    o, _ = R.rotary_block_forward(q, k, v, off, tab, 0.35)
    grads = R.rotary_block_backward(q, k, v, do, off, tab, 0.35)
    o_ref, refs = _torch_reference(q, k, v, do, lengths, 10000.0, 0.35)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    for g, r in zip(grads, refs):
        np.testing.assert_allclose(g, r, rtol=1e-9, atol=1e-11)
    # planted mistake: rotating the gradients forward instead of back is caught
    gq_bad = R.rotate(oracle.attention_backward(R.rotate(q, off, tab), R.rotate(k, off, tab), v, do, off,
                                                oracle.MODE_BLOCK_DIAG, 0.35)[0], off, tab)
    assert not np.allclose(gq_bad, refs[0], atol=1e-6)


def test_backward_central_differences():
    off = oracle.offsets_from_lengths([90])
    q, k, v, do = _rand(90, 1, 4), _rand(90, 1, 4), _rand(90, 1, 4), _rand(90, 1, 4)
    tab = R.rope_table(90, 4)
    grads = R.rotary_block_backward(q, k, v, do, off, tab, 0.5)
    f = lambda qq, kk, vv: float((R.rotary_block_forward(qq, kk, vv, off, tab, 0.5)[0] * do).sum())
    eps = 1e-6
    for which, (r, c) in [(0, (3, 0)), (0, (70, 3)), (1, (10, 1)), (1, (89, 2)), (2, (65, 0))]:
        plus = [a.copy() for a in (q, k, v)]
        minus = [a.copy() for a in (q, k, v)]
        plus[which][r, 0, c] += eps
        minus[which][r, 0, c] -= eps
        fd = (f(*plus) - f(*minus)) / (2 * eps)
        assert abs(fd - grads[which][r, 0, c]) < 1e-6 * max(1.0, abs(fd)), (which, r, c)


def test_table_too_short_is_refused():
    with pytest.raises(ValueError):
        R.rotate(_rand(10, 1, 4), [0, 10], R.rope_table(9, 4))
