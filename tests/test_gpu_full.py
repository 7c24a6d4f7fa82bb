"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each workload is generated at full size on the GPU and run through jfa_fwd / jfa_bwd
with the options bench.py uses by default (per-XCD run-time tile counters; the stored-dS
self-attention backward at head_dim 128, the recompute one at 64; the three broadcast-Q dQ
paths), and workload 3 also with the recompute backward.
The oracle then checks sampled sequences one by one -- the longest, the shortest, the
median and a few seeded picks -- since in self and block-diagonal attention every
sequence's outputs and gradients depend on that sequence alone.  Broadcast-Q (whose
dQ sums over all sequences) is small enough to check whole."""

import numpy as np
import pytest
import torch

import oracle
from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu


def _sample_sequences(lengths, k, seed):
    order = np.argsort(lengths, kind="stable")
    picks = {int(order[-1]), int(order[0]), int(order[len(order) // 2])}
    rng = np.random.default_rng(seed)
    while len(picks) < min(k, len(lengths)):
        picks.add(int(rng.integers(0, len(lengths))))
    return sorted(picks)


def _shape(p):
    hkv = p["num_kv_heads"]
    return B.make_shape(p["num_seqs"], p["num_heads"], p["head_dim"], p["total_tokens"], p["num_q"],
                        hkv if hkv != p["num_heads"] else 0)


def _run(workload, opts=None, bench=False, self_bwd="auto"):
    p = W.make_workload(workload, seed=0, device="cuda")
    if bench:
        opts = B.bench_opts(p["mode"], _shape(p), p["offsets_host"], self_bwd=self_bwd)
    if p["do"] is None:
        print("[case] forward only (grouped-query attention)", flush=True)
    print(f"[case] full-size workload {workload} opts=({opts.sched if opts else 0}, "
          f"{opts.dq_path if opts else 0}, {opts.num_programs if opts else 0}, "
          f"{opts.ds_budget_mib if opts else 0})", flush=True)
    # outputs pre-filled with NaN: a row no tile writes fails the finiteness checks
    o, lse = B.fwd(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], p["mode"], p["scale"], opts,
                   *G.nan_outputs_fwd(p))
    grads = None
    if p["do"] is not None:
        grads = B.bwd(p["q"], p["k"], p["v"], o, p["do"], lse, p["offsets"], p["offsets_host"], p["mode"],
                      p["scale"], opts, G.nan_like(p["q"]), G.nan_like(p["k"]), G.nan_like(p["v"]))
    torch.cuda.synchronize()
    return p, o, lse, grads


@pytest.mark.parametrize("workload,samples,self_bwd", [(1, 4, "auto"), (3, 6, "auto"), (4, 1, "auto"), (5, 6, "auto"),
                                                      (3, 4, "recompute"), (6, 4, "auto")])
def test_full_size_sampled_sequences(workload, samples, self_bwd):
    p, o, lse, grads = _run(workload, bench=True, self_bwd=self_bwd)
    off = p["offsets_host"].astype(np.int64)
    mode = p["mode"]
    for b in _sample_sequences(p["lengths"], samples, workload):
        s, e = int(off[b]), int(off[b + 1])
        sub = lambda t: G.f64(t[s:e])
        q, k, v = sub(p["q"]), sub(p["k"]), sub(p["v"])
        do = sub(p["do"]) if grads is not None else None
        sub_off = [0, e - s]
        o_ref, lse_ref = oracle.attention_forward(q, k, v, sub_off, mode, p["scale"])
        G.check_fwd(o[s:e], lse[:, s:e], o_ref, lse_ref, f"workload {workload} seq {b} (L={e - s})")
        if grads is None:
            continue
        dq, dk, dv = grads
        refs = oracle.attention_backward(q, k, v, do, sub_off, mode, p["scale"])
        refs_o = oracle.attention_backward(q, k, v, do, sub_off, mode, p["scale"], o_given=G.f64(o[s:e]))
        G.check_bwd((dq[s:e], dk[s:e], dv[s:e]), refs, f"workload {workload} seq {b} (L={e - s})",
                    {"offsets_host": sub_off, "mode": mode}, refs_o)


@pytest.mark.parametrize("dq_path", [0, 1, 2])
def test_full_size_broadcast_q(dq_path):
    p, o, lse, grads = _run(2, B.make_opts(dq_path=dq_path))
    o_ref, lse_ref = G.oracle_fwd(p)
    G.check_fwd(o, lse, o_ref, lse_ref, "workload 2 full")
    G.check_bwd(grads, G.oracle_bwd(p), "workload 2 full", p, G.oracle_bwd(p, o))


@pytest.mark.parametrize("self_bwd", ["auto", "recompute"])
def test_tensors_beyond_2_31_elements(self_bwd):
    # 4200 sequences of 512 tokens, H = 8, D = 128: every [T, H, D] tensor holds 2.2e9
    # elements, so the last sequences start past element 2^31 of q, k, v, o, dO, dQ, dK,
    # dV (64-bit offsets everywhere); checked on the first, the last and seeded picks.
    lengths = [512] * 4200
    print(f"[case] 4200 x 512 tokens, H=8, D=128, self_bwd={self_bwd}", flush=True)
    p = W.make_problem(lengths, 8, 128, W.MODE_SELF, seed=91, device="cuda")
    assert p["total_tokens"] * 8 * 128 > 2 ** 31
    opts = B.bench_opts(p["mode"], _shape(p), p["offsets_host"], self_bwd=self_bwd)
    o, lse = B.fwd(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], p["mode"], p["scale"], opts)
    dq, dk, dv = B.bwd(p["q"], p["k"], p["v"], o, p["do"], lse, p["offsets"], p["offsets_host"], p["mode"],
                       p["scale"], opts)
    torch.cuda.synchronize()
    off = p["offsets_host"].astype(np.int64)
    rng = np.random.default_rng(91)
    picks = sorted({0, 4199, 4198, 2097} | {int(x) for x in rng.integers(0, 4200, size=2)})
    for b in picks:
        s, e = int(off[b]), int(off[b + 1])
        sub = lambda t: G.f64(t[s:e])
        q, k, v, do = sub(p["q"]), sub(p["k"]), sub(p["v"]), sub(p["do"])
        o_ref, lse_ref = oracle.attention_forward(q, k, v, [0, e - s], p["mode"], p["scale"])
        G.check_fwd(o[s:e], lse[:, s:e], o_ref, lse_ref, f"beyond 2^31 seq {b}")
        refs = oracle.attention_backward(q, k, v, do, [0, e - s], p["mode"], p["scale"])
        refs_o = oracle.attention_backward(q, k, v, do, [0, e - s], p["mode"], p["scale"], o_given=G.f64(o[s:e]))
        G.check_bwd((dq[s:e], dk[s:e], dv[s:e]), refs, f"beyond 2^31 seq {b}",
                    {"offsets_host": [0, e - s], "mode": p["mode"]}, refs_o)
