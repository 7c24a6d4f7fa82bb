"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same seeded inputs and compare them.

Tolerances (bf16 inputs, fp32 accumulation, against the fp64 oracle): O max-abs
<= 2e-2; lse max-abs <= 1e-3; dQ, dK, dV relative L2 <= 1e-2, where
rel_l2(x, ref) = ||x - ref|| / max(||ref||, 1e-12), falling back to max-abs <= 1e-3
when ||ref|| = 0.  The gradient bound holds over the whole batch against the exact
gradient, and also for every (sequence, head) slice on its own (a long sequence cannot
hide a wrong short one).  The slices are compared with the same backward formula
evaluated by the oracle on the forward output O the library's backward received
(Di = rowsum(dO * O) from that O; bittide page, section 4): on short rows where
dP - Di nearly cancels, the bf16 rounding of O alone moves a slice by ~1e-2 of its
norm (a 2-token sequence: 1.2e-2 in a CPU emulation of the rounding), which says
nothing about the kernels.  A slice whose reference is too small for a relative bound
(e.g. dQ = dK = 0 of a one-token sequence, which fp64 rounding leaves at ~1e-16)
passes on max-abs <= 1e-3.

Outputs are pre-filled with NaN before every call, so a row that no tile writes
(a tile the schedule skipped) fails the finiteness checks."""

import numpy as np
import torch

import oracle
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

O_TOL = 2e-2
LSE_TOL = 1e-3
GRAD_TOL = 1e-2


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-12))


def to_gpu(p):
    g = dict(p)
    for k in ("q", "k", "v", "do", "offsets"):
        if p.get(k) is not None:
            g[k] = p[k].cuda()
    return g


def nan_like(t):
    return torch.full_like(t, float("nan"))


def nan_outputs_fwd(g):
    """NaN-filled o, lse of the forward's output shapes for g."""
    nb, h, d = len(g["offsets_host"]) - 1, g["q"].shape[1], g["q"].shape[2]
    t = int(g["offsets_host"][-1])
    if g["mode"] == W.MODE_BROADCAST_Q:
        mq = g["q"].shape[0]
        o_shape, l_shape = (nb, mq, h, d), (nb, h, mq)
    else:
        o_shape, l_shape = (t, h, d), (h, t)
    return (torch.full(o_shape, float("nan"), dtype=torch.bfloat16, device=g["q"].device),
            torch.full(l_shape, float("nan"), dtype=torch.float32, device=g["q"].device))


def gpu_fwd(g, opts=None, host_offsets=True):
    o, lse = nan_outputs_fwd(g)
    return B.fwd(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"] if host_offsets else None,
                 g["mode"], g["scale"], opts, o, lse)


def gpu_bwd(g, o, lse, opts=None, host_offsets=True):
    return B.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, g["offsets"],
                 g["offsets_host"] if host_offsets else None, g["mode"], g["scale"], opts,
                 nan_like(g["q"]), nan_like(g["k"]), nan_like(g["v"]))


def oracle_fwd(p):
    return oracle.attention_forward(f64(p["q"]), f64(p["k"]), f64(p["v"]), p["offsets_host"], p["mode"], p["scale"])


def oracle_bwd(p, o_given=None):
    """The oracle's gradient: exact, or with Di formed from o_given (a torch tensor or
    array in the forward's o layout, e.g. the library's bf16 forward output)."""
    og = None if o_given is None else (f64(o_given) if isinstance(o_given, torch.Tensor) else o_given)
    return oracle.attention_backward(f64(p["q"]), f64(p["k"]), f64(p["v"]), f64(p["do"]), p["offsets_host"],
                                     p["mode"], p["scale"], o_given=og)


def check_fwd(o, lse, o_ref, lse_ref, label=""):
    o_np, lse_np = f64(o), f64(lse)
    assert np.isfinite(o_np).all(), f"{label}: non-finite O"
    err = float(np.abs(o_np - o_ref).max(initial=0.0))
    assert err <= O_TOL, f"{label}: O max-abs {err:.3e} > {O_TOL}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_np), fin), f"{label}: lse finiteness differs"
    assert np.array_equal(lse_np[~fin], lse_ref[~fin]), f"{label}: lse of empty rows is not -inf"
    lerr = float(np.abs(lse_np[fin] - lse_ref[fin]).max(initial=0.0))
    assert lerr <= LSE_TOL, f"{label}: lse max-abs {lerr:.3e} > {LSE_TOL}"
    return err, lerr


def check_slice(x, ref, what):
    """One (sequence, head) slice: rel-L2 <= GRAD_TOL, or max-abs <= 1e-3 where the
    reference is too small for a relative bound to mean anything."""
    e = rel_l2(x, ref)
    if e <= GRAD_TOL:
        return e
    a = float(np.abs(x - ref).max(initial=0.0))
    assert a <= 1e-3, f"{what}: rel-L2 {e:.3e} > {GRAD_TOL} and max-abs {a:.3e} > 1e-3 (|ref| {np.linalg.norm(ref):.3e})"
    return e


def check_bwd_slices(grads, refs, offsets_host, mode, label=""):
    """Per (sequence, head) gradient checks: dk, dv of each sequence's own key rows and
    (self / block-diagonal) dq of its query rows; broadcast-Q dq per head (summed over
    the sequences)."""
    off = np.asarray(offsets_host, dtype=np.int64)
    names = ("dq", "dk", "dv")
    gs = [f64(g) for g in grads]
    worst = 0.0
    heads = gs[1].shape[1]
    for h in range(heads):
        if mode == W.MODE_BROADCAST_Q:
            worst = max(worst, check_slice(gs[0][:, h], refs[0][:, h], f"{label}: dq head {h}"))
        for b in range(len(off) - 1):
            s, e = int(off[b]), int(off[b + 1])
            if e == s:
                continue
            for i, name in enumerate(names):
                if i == 0 and mode == W.MODE_BROADCAST_Q:
                    continue
                worst = max(worst, check_slice(gs[i][s:e, h], refs[i][s:e, h],
                                               f"{label}: {name} seq {b} (L={e - s}) head {h}"))
    return worst


def check_bwd(grads, refs, label="", p=None, slice_refs=None):
    """Whole-batch gradient checks against refs; with the problem p (or a dict with its
    offsets_host and mode) also every (sequence, head) slice, against slice_refs (the
    oracle's gradient with Di from the library's O; default refs)."""
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        gn = f64(g)
        assert np.isfinite(gn).all(), f"{label}: non-finite {name}"
        if np.linalg.norm(r) == 0:
            e = float(np.abs(gn).max(initial=0.0))
            assert e <= 1e-3, f"{label}: {name} max-abs {e:.3e} > 1e-3 (zero reference)"
        else:
            e = rel_l2(gn, r)
            assert e <= GRAD_TOL, f"{label}: {name} rel-L2 {e:.3e} > {GRAD_TOL}"
        errs.append(e)
    if p is not None:
        check_bwd_slices(grads, refs if slice_refs is None else slice_refs, p["offsets_host"], p["mode"], label)
    return errs


def run_case(lengths, num_heads, head_dim, mode=W.MODE_SELF, num_q=0, seed=0, opts=None, bwd=True,
             host_offsets=True, label="", num_kv_heads=None):
    print(f"[case] {label} lengths={list(lengths)[:12]}{'...' if len(lengths) > 12 else ''} H={num_heads} "
          f"Hkv={num_kv_heads or num_heads} D={head_dim} mode={mode} Mq={num_q} seed={seed}", flush=True)
    p = W.make_problem(lengths, num_heads, head_dim, mode, num_q, seed, device="cpu", with_grad=bwd,
                       num_kv_heads=num_kv_heads)
    g = to_gpu(p)
    o, lse = gpu_fwd(g, opts, host_offsets)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(p)
    check_fwd(o, lse, o_ref, lse_ref, label)
    if not bwd:
        return p, g, (o, lse), None
    grads = gpu_bwd(g, o, lse, opts, host_offsets)
    torch.cuda.synchronize()
    check_bwd(grads, oracle_bwd(p), label, p, oracle_bwd(p, o))
    return p, g, (o, lse), grads
