"""GPU parity of the block-diagonal attention with the fused rotary embedding
(jfa_fwd_rotary / jfa_bwd_rotary) against the fp64 oracle (oracle/rotary.py).

The library builds its cos/sin table on the device (jfa_rope_table, fp32); the oracle
builds its own in fp64 from the definition, so the table's rounding is inside the
tolerance, and the device table equals the oracle's rounded to fp32 within one unit in
the last place.
A table of zero angles must reproduce the plain block-diagonal kernels bit for bit.

Tolerance of lse.  The rotated q and k enter the bf16 matrix product rounded to bf16
(relative error <= 2^-9 each), which the exact oracle does not do; S then differs by at
most scale * 2^-8 * sum_i |q_i| |k_i| (first order), and lse, 1-Lipschitz in S, by
at most the row's largest such bound.  So every row must lie within 1e-3 plus its
bound, and the mean lse error over all rows within 1e-3.  O keeps the common 2e-2
max-abs bound, the gradients the common 1e-2 relative L2."""

import numpy as np
import pytest
import torch

from oracle import rotary as R
from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu


def _check_fwd(o, lse, o_ref, lse_ref, q, k, offsets, tab, scale, label):
    """O against the common bound; lse per row within 1e-3 + the bf16 rounding bound of
    the rotated operands (see the module docstring), and on average within 1e-3."""
    o_np, lse_np = G.f64(o), G.f64(lse)
    assert np.isfinite(o_np).all(), f"{label}: non-finite O"
    err = float(np.abs(o_np - o_ref).max(initial=0.0))
    assert err <= G.O_TOL, f"{label}: O max-abs {err:.3e} > {G.O_TOL}"
    qr, kr = R.rotate(q, offsets, tab), R.rotate(k, offsets, tab)
    group = qr.shape[1] // kr.shape[1]
    bound = np.zeros_like(lse_ref)
    off = [int(x) for x in offsets]
    for b in range(len(off) - 1):
        for s0 in range(off[b], off[b + 1], 64):
            s1 = min(s0 + 64, off[b + 1])
            for h in range(qr.shape[1]):
                m = np.abs(qr[s0:s1, h]) @ np.abs(kr[s0:s1, h // group]).T   # [rows, keys]
                bound[h, s0:s1] = scale * 2.0 ** -8 * m.max(axis=1)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_np), fin), f"{label}: lse finiteness differs"
    d = np.abs(lse_np - lse_ref)[fin]
    worst = float((d - bound[fin]).max(initial=-1.0))
    assert worst <= 1e-3, f"{label}: lse exceeds 1e-3 + bound by {worst:.3e}"
    assert float(d.mean()) <= 1e-3, f"{label}: mean lse error {d.mean():.3e} > 1e-3"
    print(f"{label}: lse max {d.max():.2e} mean {d.mean():.2e}, largest bound {bound.max():.2e}", flush=True)

LENGTHS = [64, 130, 5, 0, 256, 1, 63, 65, 700]


def _run(lengths, heads, head_dim, seed, num_kv_heads=None, bwd=True, label="", table_rows=None, opts=None):
    print(f"[case] rotary {label} lengths={lengths} H={heads} Hkv={num_kv_heads or heads} D={head_dim} "
          f"seed={seed} bwd={bwd}", flush=True)
    p = W.make_problem(lengths, heads, head_dim, W.MODE_BLOCK_DIAG, seed=seed, device="cpu", with_grad=bwd,
                       num_kv_heads=num_kv_heads)
    g = G.to_gpu(p)
    rows = table_rows or max(1, max(lengths))
    rope = B.rope_table(rows, head_dim, device="cuda")
    o, lse = B.fwd_rotary(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"], rope, g["scale"], opts,
                          *G.nan_outputs_fwd(g))
    torch.cuda.synchronize()
    tab = R.rope_table(rows, head_dim)
    o_ref, lse_ref = R.rotary_block_forward(G.f64(p["q"]), G.f64(p["k"]), G.f64(p["v"]), p["offsets_host"], tab,
                                            p["scale"])
    _check_fwd(o, lse, o_ref, lse_ref, G.f64(p["q"]), G.f64(p["k"]), p["offsets_host"], tab, p["scale"], label)
    grads = None
    if bwd:
        grads = B.bwd_rotary(g["q"], g["k"], g["v"], o, g["do"], lse, g["offsets"], g["offsets_host"], rope,
                             g["scale"], opts, G.nan_like(g["q"]), G.nan_like(g["k"]), G.nan_like(g["v"]))
        torch.cuda.synchronize()
        refs = R.rotary_block_backward(G.f64(p["q"]), G.f64(p["k"]), G.f64(p["v"]), G.f64(p["do"]),
                                       p["offsets_host"], tab, p["scale"])
        refs_o = R.rotary_block_backward(G.f64(p["q"]), G.f64(p["k"]), G.f64(p["v"]), G.f64(p["do"]),
                                         p["offsets_host"], tab, p["scale"], o_given=G.f64(o))
        G.check_bwd(grads, refs, label + " bwd", p, refs_o)
    return p, g, o, lse, grads


@pytest.mark.parametrize("head_dim", [64, 128])
def test_rotary_block_attention(head_dim):
    _run(LENGTHS, 3, head_dim, seed=61, label=f"D{head_dim}")


def test_rotary_long_positions_and_spare_table_rows():
    # positions up to 4031 (angles up to 4031 rad in the first pair), table longer than needed
    _run([4032, 17, 2000], 2, 64, seed=62, label="long", table_rows=4100)


def test_rotary_grouped_query_forward():
    _run(LENGTHS, 4, 128, seed=63, num_kv_heads=2, bwd=False, label="gqa")


def test_rotary_zero_angles_equal_plain_block_attention_bit_exactly():
    for d in (64, 128):
        p = W.make_problem(LENGTHS, 2, d, W.MODE_BLOCK_DIAG, seed=64, device="cpu", with_grad=True)
        g = G.to_gpu(p)
        rope = torch.zeros((700, d // 2, 2), dtype=torch.float32, device="cuda")
        rope[..., 0] = 1.0
        o, lse = B.fwd_rotary(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"], rope, g["scale"], None,
                          *G.nan_outputs_fwd(g))
        o_p, lse_p = G.gpu_fwd(g)
        grads = B.bwd_rotary(g["q"], g["k"], g["v"], o, g["do"], lse, g["offsets"], g["offsets_host"], rope,
                             g["scale"], None, G.nan_like(g["q"]), G.nan_like(g["k"]), G.nan_like(g["v"]))
        plain = G.gpu_bwd(g, o_p, lse_p)
        torch.cuda.synchronize()
        assert torch.equal(o, o_p) and torch.equal(lse, lse_p)
        for name, a, b in zip(("dq", "dk", "dv"), grads, plain):
            assert torch.equal(a, b), name


def test_rotary_full_workload_sampled():
    """Workload 8 at full size in the launch configuration bench.py times; sampled
    sequences against the oracle (each sequence depends on itself only)."""
    print("[case] rotary full-size workload 8", flush=True)
    p = W.make_workload(8, seed=0, device="cuda")
    lengths = p["lengths"]
    rows = int(max(lengths))
    rope = B.rope_table(rows, p["head_dim"], device="cuda")
    o, lse = B.fwd_rotary(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], rope, p["scale"], None,
                          *G.nan_outputs_fwd(p))
    dq, dk, dv = B.bwd_rotary(p["q"], p["k"], p["v"], o, p["do"], lse, p["offsets"], p["offsets_host"], rope,
                              p["scale"], None, G.nan_like(p["q"]), G.nan_like(p["k"]), G.nan_like(p["v"]))
    torch.cuda.synchronize()
    tab = R.rope_table(rows, p["head_dim"])
    off = p["offsets_host"].astype(np.int64)
    order = np.argsort(lengths, kind="stable")
    for b in sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), 9, 900}):
        s, e = int(off[b]), int(off[b + 1])
        sub = lambda t: G.f64(t[s:e])
        o_ref, lse_ref = R.rotary_block_forward(sub(p["q"]), sub(p["k"]), sub(p["v"]), [0, e - s], tab, p["scale"])
        _check_fwd(o[s:e], lse[:, s:e], o_ref, lse_ref, sub(p["q"]), sub(p["k"]), [0, e - s], tab, p["scale"],
                   f"workload 8 seq {b} (L={e - s})")
        refs = R.rotary_block_backward(sub(p["q"]), sub(p["k"]), sub(p["v"]), sub(p["do"]), [0, e - s], tab,
                                       p["scale"])
        refs_o = R.rotary_block_backward(sub(p["q"]), sub(p["k"]), sub(p["v"]), sub(p["do"]), [0, e - s], tab,
                                         p["scale"], o_given=sub(o))
        G.check_bwd((dq[s:e], dk[s:e], dv[s:e]), refs, f"workload 8 seq {b} (L={e - s})",
                    {"offsets_host": [0, e - s], "mode": p["mode"]}, refs_o)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_library_rope_table_equals_oracle_table_rounded(head_dim):
    rows = 4100
    got = B.rope_table(rows, head_dim, device="cuda").cpu().numpy()
    want = R.rope_table(rows, head_dim)
    assert got.shape == want.shape and got.dtype == np.float32
    # at most one fp32 unit in the last place from the fp64 values, and exactly the
    # rounded value almost everywhere
    ulp = np.spacing(np.abs(want).astype(np.float32))
    assert np.all(np.abs(got.astype(np.float64) - want) <= ulp)
    assert np.mean(got == want.astype(np.float32)) > 0.999
