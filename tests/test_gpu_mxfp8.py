"""GPU parity of the MXFP8 variant (jfa_mxfp8_quantize_qk / _v, jfa_fwd_mxfp8,
jfa_bwd_mxfp8) against the fp64 oracle (oracle/mxfp8.py).

Quantisation is integer work once the block maximum is known: the GPU's E8M0 bytes and
the values of its E4M3 bytes must equal the oracle's exactly (zero's sign aside).  The
forward is checked against fp64 attention of the dequantised GPU codes: lse within
1e-3 (S and the softmax statistics are exact functions of the quantised inputs up to
fp32 rounding), O within the common 2e-2 plus the oracle's bound on what quantising P
per 32 keys can change (the kernel quantises the running P of each key step, which the
bound covers).  The backward is checked against the oracle's gradient at the decoded
inputs (decoded from the GPU's own codes) with Di formed from the MXFP8 forward's O,
to the common gradient tolerances (whole batch and every sequence and head)."""

import numpy as np
import pytest
import torch

from oracle import mxfp8 as M
from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu

LENGTHS = [64, 130, 5, 0, 256, 1, 63, 65, 700, 33]


def _vbase(lengths):
    return np.concatenate([[0], np.cumsum([-(-int(n) // 64) * 64 for n in lengths])]).astype(np.int64)


def _gpu_v_to_tokens(codes, scales, lengths):
    """GPU V layout ([H, D, Tp] codes, [H, D, Tp/32] scales) -> values [T, H, D] and per
    sequence exponents [nb, H, D] (the oracle's layout); also checks the padding."""
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    vb = _vbase(lengths)
    vals, xs = [], []
    for b, n in enumerate(lengths):
        n = int(n)
        seg = codes[:, :, vb[b]:vb[b + 1]]
        assert (seg[:, :, n:] == 0).all(), "padding keys must be zero codes"
        vals.append(M.e4m3_decode(seg[:, :, :n]).transpose(2, 0, 1))
        sx = scales[:, :, vb[b] // 32:vb[b + 1] // 32].astype(np.int64) - 127
        nb = -(-n // 32)
        assert (sx[:, :, nb:] == 0).all(), "all-padding blocks take X = 0"
        xs.append(sx[:, :, :nb].transpose(2, 0, 1))
    return np.concatenate(vals) if vals else np.zeros((0,) + codes.shape[:2]), xs


def _same_values(a, b, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, f"{what}: {bad.size} values differ, first at {bad[0]}: {a.ravel()[bad[0]]} vs {b.ravel()[bad[0]]}"


def _run(lengths, heads, head_dim, seed, label="", opts=None):
    print(f"[case] mxfp8 {label} lengths={list(lengths)[:12]} H={heads} D={head_dim} seed={seed}", flush=True)
    p = W.make_problem(lengths, heads, head_dim, seed=seed, device="cpu", with_grad=False)
    g = G.to_gpu(p)
    q8, qs = B.mxfp8_quantize_qk(g["q"])
    k8, ks = B.mxfp8_quantize_qk(g["k"])
    v8, vs, tp = B.mxfp8_quantize_v(g["v"], g["offsets"], g["offsets_host"])
    o, lse = B.fwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, g["offsets"], g["offsets_host"], g["scale"], opts)
    torch.cuda.synchronize()
    # quantisers: bit-exact against the oracle
    qv_ref, qx_ref = M.quantise_qk(G.f64(p["q"]))
    kv_ref, kx_ref = M.quantise_qk(G.f64(p["k"]))
    vv_ref, vx_ref = M.quantise_v(G.f64(p["v"]), p["offsets_host"])
    _same_values(qs.cpu().numpy().astype(np.int64) - 127, qx_ref, "Q exponents")
    _same_values(M.e4m3_decode(q8.cpu().numpy()), qv_ref, "Q values")
    _same_values(ks.cpu().numpy().astype(np.int64) - 127, kx_ref, "K exponents")
    _same_values(M.e4m3_decode(k8.cpu().numpy()), kv_ref, "K values")
    vvals, vxs = _gpu_v_to_tokens(v8, vs, p["lengths"])
    _same_values(vvals, vv_ref, "V values")
    for b in range(len(vxs)):
        _same_values(vxs[b], vx_ref[b], f"V exponents of sequence {b}")
    # forward: attention of the dequantised inputs, O bound widened by the P quantisation
    qd = M.dequantise_qk(qv_ref, qx_ref)
    kd = M.dequantise_qk(kv_ref, kx_ref)
    vd = M.dequantise_v(vv_ref, vx_ref, p["offsets_host"])
    o_ref, lse_ref = M.mxfp8_forward(qd, kd, vd, p["offsets_host"], p["scale"])
    bound = M.p_quantisation_bound(qd, kd, vd, p["offsets_host"], p["scale"])
    o_np, lse_np = G.f64(o), G.f64(lse)
    assert np.isfinite(o_np).all()
    err = np.abs(o_np - o_ref).max(axis=2)                       # [T, H]
    excess = float((err - G.O_TOL - bound).max(initial=-1.0))
    assert excess <= 0, f"{label}: O exceeds 2e-2 + P bound by {excess:.3e}"
    fin = np.isfinite(lse_ref)
    lerr = float(np.abs(lse_np[fin] - lse_ref[fin]).max(initial=0.0))
    assert lerr <= G.LSE_TOL, f"{label}: lse max-abs {lerr:.3e}"
    print(f"{label}: O max err {err.max(initial=0):.3e} (mean {err.mean() if err.size else 0:.2e}), "
          f"largest P bound {bound.max(initial=0):.2e}, lse err {lerr:.2e}", flush=True)
    return p, o, lse


@pytest.mark.parametrize("head_dim", [64, 128])
def test_mxfp8_forward(head_dim):
    _run(LENGTHS, 2, head_dim, seed=71, label=f"D{head_dim}")


@pytest.mark.parametrize("nprog", [1, 3, 7])
def test_mxfp8_forward_many_tiles_per_program(nprog):
    """Few programs, so that each walks many tiles (at head_dim 128 every tile loads the
    next tile's first stages and Q rows while it finishes): against the oracle, and bit
    for bit against the default launch (a tile's result does not depend on the program
    that runs it or on the tile before it).  The MXFP8 forward deals its tiles statically."""
    lengths = LENGTHS + [1000, 2, 129]
    p, o, lse = _run(lengths, 3, 128, seed=74, label=f"{nprog} programs",
                     opts=B.make_opts(num_programs=nprog))
    g = G.to_gpu(p)
    q8, qs = B.mxfp8_quantize_qk(g["q"])
    k8, ks = B.mxfp8_quantize_qk(g["k"])
    v8, vs, tp = B.mxfp8_quantize_v(g["v"], g["offsets"], g["offsets_host"])
    o0, l0 = B.fwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, g["offsets"], g["offsets_host"], g["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o0.view(torch.int16)), "O differs from the default launch"
    fin = torch.isfinite(l0)
    assert torch.equal(fin, torch.isfinite(lse)) and torch.equal(lse[fin], l0[fin]), "lse differs"


@pytest.mark.parametrize("nprog", [0, 3])
def test_mxfp8_forward_generic_kernel_at_head_dim_128(monkeypatch, nprog):
    """The one-group kernel that serves head_dim 128 past the ping-pong kernel's 32-bit
    copy offsets (D * Tp >= 2^32, too large to check against the oracle), forced at a
    small size: against the oracle, and close to the ping-pong kernel's output."""
    lengths = LENGTHS + [1000]
    monkeypatch.setenv("JFA_MX_GENERIC", "1")
    opts = B.make_opts(num_programs=nprog)
    p, o, lse = _run(lengths, 2, 128, seed=75, label=f"generic kernel, programs {nprog}", opts=opts)
    monkeypatch.delenv("JFA_MX_GENERIC")
    _, o2, l2 = _run(lengths, 2, 128, seed=75, label=f"ping-pong kernel, programs {nprog}", opts=opts)
    d = float((o.float() - o2.float()).abs().max())
    fin = torch.isfinite(l2)
    assert torch.equal(fin, torch.isfinite(lse))
    dl = float((lse[fin] - l2[fin]).abs().max())
    print(f"generic vs ping-pong: O max diff {d:.3e}, lse max diff {dl:.3e}")
    # same arithmetic in another order of the fp32 sums (measured: 9.8e-4, one bf16
    # step of O, and 1.4e-6)
    assert d <= 4e-3 and dl <= 1e-4


def test_mxfp8_large_and_small_magnitudes():
    """Inputs spread over many binades: exercises the shared exponents and subnormal
    elements of every block."""
    lengths = [300, 97]
    p = W.make_problem(lengths, 2, 128, seed=72, device="cpu", with_grad=False)
    scale_rows = torch.exp2(torch.linspace(-12, 12, p["q"].shape[0]))[:, None, None]
    for name in ("q", "k", "v"):
        p[name] = (p[name].float() * scale_rows).to(torch.bfloat16)
    g = G.to_gpu(p)
    q8, qs = B.mxfp8_quantize_qk(g["q"])
    v8, vs, tp = B.mxfp8_quantize_v(g["v"], g["offsets"], g["offsets_host"])
    torch.cuda.synchronize()
    qv_ref, qx_ref = M.quantise_qk(G.f64(p["q"]))
    vv_ref, vx_ref = M.quantise_v(G.f64(p["v"]), p["offsets_host"])
    _same_values(qs.cpu().numpy().astype(np.int64) - 127, qx_ref, "Q exponents")
    _same_values(M.e4m3_decode(q8.cpu().numpy()), qv_ref, "Q values")
    vvals, vxs = _gpu_v_to_tokens(v8, vs, lengths)
    _same_values(vvals, vv_ref, "V values")
    for b in range(2):
        _same_values(vxs[b], vx_ref[b], f"V exponents {b}")


def test_mxfp8_production_lengths_reduced():
    _run(W.workload_lengths(3, 0, 40).tolist(), 2, 128, seed=73, label="production lengths, 40 sequences")


def test_mxfp8_full_workload_sampled():
    """Workload 9 at full size in the launch configuration bench.py times; sampled
    sequences against the oracle (each depends on itself only)."""
    print("[case] mxfp8 full-size workload 9", flush=True)
    p = W.make_workload(9, seed=0, device="cuda")
    q8, qs = B.mxfp8_quantize_qk(p["q"])
    k8, ks = B.mxfp8_quantize_qk(p["k"])
    v8, vs, tp = B.mxfp8_quantize_v(p["v"], p["offsets"], p["offsets_host"])
    o, lse = B.fwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, p["offsets"], p["offsets_host"], p["scale"])
    torch.cuda.synchronize()
    off = p["offsets_host"].astype(np.int64)
    order = np.argsort(p["lengths"], kind="stable")
    vb = _vbase(p["lengths"])
    for b in sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), 13, 700}):
        s, e = int(off[b]), int(off[b + 1])
        n = e - s
        qd = M.e4m3_decode(q8[s:e].cpu().numpy()).reshape(n, -1, 4, 32) * \
            np.exp2(qs[s:e].cpu().numpy().astype(np.float64) - 127)[..., None]
        kd = M.e4m3_decode(k8[s:e].cpu().numpy()).reshape(n, -1, 4, 32) * \
            np.exp2(ks[s:e].cpu().numpy().astype(np.float64) - 127)[..., None]
        vcodes = v8[:, :, vb[b]:vb[b] + n].cpu().numpy()
        vx = vs[:, :, vb[b] // 32:vb[b] // 32 + -(-n // 32)].cpu().numpy().astype(np.float64) - 127
        vd = (M.e4m3_decode(vcodes) * np.exp2(np.repeat(vx, 32, axis=2)[:, :, :n])).transpose(2, 0, 1)
        qd, kd = qd.reshape(n, -1, 128), kd.reshape(n, -1, 128)
        o_ref, lse_ref = M.mxfp8_forward(qd, kd, vd, [0, n], p["scale"])
        bound = M.p_quantisation_bound(qd, kd, vd, [0, n], p["scale"])
        err = np.abs(G.f64(o[s:e]) - o_ref).max(axis=2)
        assert float((err - G.O_TOL - bound).max()) <= 0, f"workload 9 seq {b} (L={n})"
        assert float(np.abs(G.f64(lse[:, s:e]) - lse_ref).max()) <= G.LSE_TOL, f"workload 9 seq {b} lse"


def _decoded(q8, qs, k8, ks, v8, vs, lengths, offsets_host):
    """fp64 q, k, v decoded from the GPU's codes (the oracle's decoder)."""
    qd = M.dequantise_qk(M.e4m3_decode(q8.cpu().numpy()), qs.cpu().numpy().astype(np.int64) - 127)
    kd = M.dequantise_qk(M.e4m3_decode(k8.cpu().numpy()), ks.cpu().numpy().astype(np.int64) - 127)
    vvals, vxs = _gpu_v_to_tokens(v8, vs, lengths)
    return qd, kd, M.dequantise_v(vvals, vxs, offsets_host)


def _run_bwd(lengths, heads, head_dim, seed, opts=None, label=""):
    print(f"[case] mxfp8 backward {label} lengths={list(lengths)[:12]} H={heads} D={head_dim} seed={seed}",
          flush=True)
    p = W.make_problem(lengths, heads, head_dim, seed=seed, device="cpu", with_grad=True)
    g = G.to_gpu(p)
    q8, qs = B.mxfp8_quantize_qk(g["q"])
    k8, ks = B.mxfp8_quantize_qk(g["k"])
    v8, vs, tp = B.mxfp8_quantize_v(g["v"], g["offsets"], g["offsets_host"])
    o, lse = B.fwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, g["offsets"], g["offsets_host"], g["scale"])
    grads = B.bwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, o, g["do"], lse, g["offsets"], g["offsets_host"], g["scale"],
                        opts, G.nan_like(g["q"]), G.nan_like(g["k"]), G.nan_like(g["v"]))
    torch.cuda.synchronize()
    qd, kd, vd = _decoded(q8, qs, k8, ks, v8, vs, p["lengths"], p["offsets_host"])
    refs = M.mxfp8_backward(qd, kd, vd, G.f64(p["do"]), p["offsets_host"], p["scale"], o_given=G.f64(o))
    errs = G.check_bwd(grads, refs, label, p, refs)
    print(f"{label}: rel-L2 dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}", flush=True)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_mxfp8_backward(head_dim):
    _run_bwd(LENGTHS, 2, head_dim, seed=74, label=f"D{head_dim}")


def test_mxfp8_backward_stored_ds_path_and_production_lengths():
    lengths = W.workload_lengths(3, 0, 24).tolist()
    shape = B.make_shape(len(lengths), 2, 128, int(sum(lengths)))
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    opts = B.make_opts(sched=1, ds_budget_mib=B.ds_budget_mib(shape, off))
    _run_bwd(lengths, 2, 128, seed=75, opts=opts, label="stored dS, production lengths, 24 sequences")


def test_mxfp8_backward_full_workload_sampled():
    """Workload 9's backward at full size in the launch configuration bench.py times
    (run-time schedule, stored-dS path); sampled sequences against the oracle's gradient
    at the decoded inputs (each sequence's gradient depends on that sequence only)."""
    print("[case] mxfp8 backward full-size workload 9", flush=True)
    p = W.make_workload(9, seed=0, device="cuda")
    shape = B.make_shape(p["num_seqs"], p["num_heads"], p["head_dim"], p["total_tokens"])
    opts = B.bench_opts(W.MODE_SELF, shape, p["offsets_host"])
    q8, qs = B.mxfp8_quantize_qk(p["q"])
    k8, ks = B.mxfp8_quantize_qk(p["k"])
    v8, vs, tp = B.mxfp8_quantize_v(p["v"], p["offsets"], p["offsets_host"])
    o, lse = B.fwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, p["offsets"], p["offsets_host"], p["scale"], opts)
    dq, dk, dv = B.bwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, o, p["do"], lse, p["offsets"], p["offsets_host"],
                             p["scale"], opts, G.nan_like(p["q"]), G.nan_like(p["k"]), G.nan_like(p["v"]))
    torch.cuda.synchronize()
    off = p["offsets_host"].astype(np.int64)
    order = np.argsort(p["lengths"], kind="stable")
    vb = _vbase(p["lengths"])
    d = p["head_dim"]
    for b in sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), 29, 900}):
        s, e = int(off[b]), int(off[b + 1])
        n = e - s
        qd = M.dequantise_qk(M.e4m3_decode(q8[s:e].cpu().numpy()), qs[s:e].cpu().numpy().astype(np.int64) - 127)
        kd = M.dequantise_qk(M.e4m3_decode(k8[s:e].cpu().numpy()), ks[s:e].cpu().numpy().astype(np.int64) - 127)
        vcodes = v8[:, :, vb[b]:vb[b] + n].cpu().numpy()
        vx = vs[:, :, vb[b] // 32:vb[b] // 32 + -(-n // 32)].cpu().numpy().astype(np.float64) - 127
        vd = (M.e4m3_decode(vcodes) * np.exp2(np.repeat(vx, 32, axis=2)[:, :, :n])).transpose(2, 0, 1)
        refs = M.mxfp8_backward(qd, kd, vd, G.f64(p["do"][s:e]), [0, n], p["scale"], o_given=G.f64(o[s:e]))
        G.check_bwd((dq[s:e], dk[s:e], dv[s:e]), refs, f"workload 9 bwd seq {b} (L={n})",
                    {"offsets_host": [0, n], "mode": W.MODE_SELF}, refs)
    assert d == 128
