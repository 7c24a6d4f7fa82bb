"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same seeded inputs and compare them.

Tolerances (bf16 inputs, fp32 accumulation, against the fp64 oracle): O max-abs
<= 2e-2; lse max-abs <= 1e-3; dQ, dK, dV relative L2 <= 1e-2, where
rel_l2(x, ref) = ||x - ref|| / max(||ref||, 1e-12), falling back to max-abs <= 1e-3
when ||ref|| = 0."""

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


def gpu_fwd(g, opts=None, host_offsets=True):
    return B.fwd(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"] if host_offsets else None,
                 g["mode"], g["scale"], opts)


def gpu_bwd(g, o, lse, opts=None, host_offsets=True):
    return B.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, g["offsets"],
                 g["offsets_host"] if host_offsets else None, g["mode"], g["scale"], opts)


def oracle_fwd(p):
    return oracle.attention_forward(f64(p["q"]), f64(p["k"]), f64(p["v"]), p["offsets_host"], p["mode"], p["scale"])


def oracle_bwd(p):
    return oracle.attention_backward(f64(p["q"]), f64(p["k"]), f64(p["v"]), f64(p["do"]), p["offsets_host"],
                                     p["mode"], p["scale"])


def check_fwd(o, lse, o_ref, lse_ref, label=""):
    o_np, lse_np = f64(o), f64(lse)
    assert np.isfinite(o_np).all(), f"{label}: non-finite O"
    err = float(np.abs(o_np - o_ref).max(initial=0.0))
    assert err <= O_TOL, f"{label}: O max-abs {err:.3e} > {O_TOL}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_np), fin), f"{label}: lse finiteness differs"
    lerr = float(np.abs(lse_np[fin] - lse_ref[fin]).max(initial=0.0))
    assert lerr <= LSE_TOL, f"{label}: lse max-abs {lerr:.3e} > {LSE_TOL}"
    return err, lerr


def check_bwd(grads, refs, label=""):
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
    check_bwd(grads, oracle_bwd(p), label)
    return p, g, (o, lse), grads
