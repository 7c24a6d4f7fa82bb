"""GPU parity of the block-sparse top-k forward (jfa_fwd_block_sparse) against the
fp64 oracle (oracle/block_sparse.py).

The kept key blocks are decided from fp32 block means on the GPU; where two blocks'
relevance differ by less than fp32 rounding either choice is correct.  So the
selection is checked for validity against the oracle's fp64 relevance (right count,
ascending, no duplicates, and no dropped block beats a kept one by more than a bound
on the fp32 error), and the attention is checked element by element against the
oracle run on the GPU's own selection.  With ratio 1 every block is kept and the
result must equal the dense forward bit for bit.

The backward (jfa_bwd_block_sparse) is checked against the oracle's backward for the
same (GPU) selection; at ratio 1 it walks every query and key step in the dense
recompute backward's order.  Its dQ then equals jfa_bwd's (no dS budget) bit for bit,
and so do dK, dV at head_dim 64, where both run the same one-wave-per-32-keys kernel.
At head_dim 128 the dense dK/dV kernel splits every 64-row query step over two wave
groups and adds the groups' fp32 partials at the tile end, while the block-sparse one
(64-key tiles) sums all rows in one wave: the two sum the same products in another
order and agree to within one bf16 rounding."""

import numpy as np
import pytest
import torch

from oracle import block_sparse as S
from oracle import schedule as spec
from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu

LENGTHS = [1, 63, 64, 65, 300, 520, 777, 1030, 0, 2049]


def _split_selection(sel, lengths, heads, ratio):
    """GPU selection array -> list over sequences of [H][nqb] lists."""
    sel = sel.cpu().numpy()
    out, at = [], 0
    for n in lengths:
        nqb, kk = -(-n // S.Q_BLOCK), S.keep_count(n, ratio)
        per_h = []
        for _ in range(heads):
            rows = []
            for _ in range(nqb):
                rows.append(sel[at:at + kk].tolist())
                at += kk
            per_h.append(rows)
        out.append(per_h)
    return out, at


def _check_selection(p, gpu_sel, ratio):
    q, k = G.f64(p["q"]), G.f64(p["k"])
    scores = S.block_scores(q, k, p["offsets_host"])
    ref = S.select_blocks(q, k, p["offsets_host"], ratio)
    exact = total = 0
    for b, n in enumerate(p["lengths"]):
        if n == 0:
            continue
        nkb, kk = -(-int(n) // S.K_BLOCK), S.keep_count(int(n), ratio)
        qb = S.pooled_blocks(q, int(p["offsets_host"][b]), int(p["offsets_host"][b + 1]), S.Q_BLOCK)
        kb = S.pooled_blocks(k, int(p["offsets_host"][b]), int(p["offsets_host"][b + 1]), S.K_BLOCK)
        group = q.shape[1] // k.shape[1]
        for hh in range(q.shape[1]):
            for i in range(scores[b].shape[1]):
                got = gpu_sel[b][hh][i]
                assert len(got) == kk and got == sorted(set(got)) and all(0 <= j < nkb for j in got), (b, hh, i, got)
                s = scores[b][hh, i]
                dropped = [j for j in range(nkb) if j not in got]
                tol = 1e-4 * np.linalg.norm(qb[i, hh]) * max(np.linalg.norm(kb[j, hh // group]) for j in range(nkb))
                if dropped:
                    assert min(s[got]) >= max(s[dropped]) - tol - 1e-9, (b, hh, i)
                exact += got == ref[b][hh][i]
                total += 1
    print(f"selection identical to the oracle's on {exact}/{total} query blocks", flush=True)


def _run(lengths, heads, head_dim, ratio, seed, num_kv_heads=None, opts=None, label="", bwd=False):
    print(f"[case] block sparse {label} lengths={lengths} H={heads} Hkv={num_kv_heads or heads} D={head_dim} "
          f"ratio={ratio} seed={seed} bwd={bwd}", flush=True)
    p = W.make_problem(lengths, heads, head_dim, seed=seed, device="cpu", with_grad=bwd, num_kv_heads=num_kv_heads)
    g = G.to_gpu(p)
    o, lse, sel = B.fwd_block_sparse(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"], ratio, g["scale"],
                                     opts, *G.nan_outputs_fwd(g))
    torch.cuda.synchronize()
    gpu_sel, used = _split_selection(sel, p["lengths"], heads, ratio)
    assert used == B.block_sparse_entries(B.make_shape(len(lengths), heads, head_dim, p["total_tokens"], 0,
                                                       num_kv_heads or 0), p["offsets_host"], ratio)
    _check_selection(p, gpu_sel, ratio)
    o_ref, lse_ref = S.block_sparse_forward(G.f64(p["q"]), G.f64(p["k"]), G.f64(p["v"]), p["offsets_host"],
                                            gpu_sel, p["scale"])
    G.check_fwd(o, lse, o_ref, lse_ref, label)
    if bwd:
        grads = B.bwd_block_sparse(g["q"], g["k"], g["v"], o, g["do"], lse, g["offsets"], g["offsets_host"], ratio,
                                   sel, g["scale"], opts, G.nan_like(g["q"]), G.nan_like(g["k"]), G.nan_like(g["v"]))
        torch.cuda.synchronize()
        refs = S.block_sparse_backward(G.f64(p["q"]), G.f64(p["k"]), G.f64(p["v"]), G.f64(p["do"]),
                                       p["offsets_host"], gpu_sel, p["scale"])
        refs_o = S.block_sparse_backward(G.f64(p["q"]), G.f64(p["k"]), G.f64(p["v"]), G.f64(p["do"]),
                                         p["offsets_host"], gpu_sel, p["scale"], o_given=G.f64(o))
        G.check_bwd(grads, refs, label + " bwd", p, refs_o)
        return p, g, o, lse, sel, grads
    return p, g, o, lse


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("ratio", [0.5, 0.25])
def test_block_sparse_forward(head_dim, ratio):
    _run(LENGTHS, 2, head_dim, ratio, seed=41, label=f"D{head_dim} r{ratio}")


def test_block_sparse_grouped_query_and_dynamic_schedule():
    _run(LENGTHS, 4, 128, 0.5, seed=42, num_kv_heads=2, label="gqa")
    _run(LENGTHS, 2, 128, 0.5, seed=43, opts=B.make_opts(sched=1, num_programs=7), label="dynamic")


def test_block_sparse_ratio_one_equals_dense_forward_bit_exactly():
    p, g, o, lse = _run(LENGTHS, 2, 128, 1.0, seed=44, label="ratio 1")
    # the dense forward with 16 programs, whose share leaves every sequence whole (with
    # more programs it would cut the longest sequences' keys into chunks)
    assert not spec.self_chunks_cut(LENGTHS, 2, 256, 16)
    o_d, lse_d = G.gpu_fwd(g, B.make_opts(num_programs=16))
    torch.cuda.synchronize()
    assert torch.equal(o, o_d)
    assert torch.equal(lse, lse_d)


def test_block_sparse_production_lengths_reduced():
    lengths = W.workload_lengths(3, 0, 48).tolist()
    _run(lengths, 4, 128, 0.5, seed=45, label="production lengths, 48 sequences")


def test_block_sparse_full_production_workload_sampled():
    """Workload 7 at full size, in the launch configuration bench.py times; the oracle
    checks sampled sequences (every sequence's selection and output depend on that
    sequence alone)."""
    print("[case] block sparse full-size workload 7", flush=True)
    p = W.make_workload(7, seed=0, device="cuda")
    ratio = W.WORKLOADS[7]["sparse_ratio"]
    o, lse, sel = B.fwd_block_sparse(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], ratio, p["scale"])
    torch.cuda.synchronize()
    gpu_sel, _ = _split_selection(sel, p["lengths"], p["num_heads"], ratio)
    off = p["offsets_host"].astype(np.int64)
    order = np.argsort(p["lengths"], kind="stable")
    picks = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), 7, 500})
    for b in picks:
        s, e = int(off[b]), int(off[b + 1])
        sub = {"q": p["q"][s:e].cpu(), "k": p["k"][s:e].cpu(), "v": p["v"][s:e].cpu(), "lengths": [e - s],
               "offsets_host": np.array([0, e - s])}
        _check_selection(sub, [gpu_sel[b]], ratio)
        o_ref, lse_ref = S.block_sparse_forward(G.f64(sub["q"]), G.f64(sub["k"]), G.f64(sub["v"]), [0, e - s],
                                                [gpu_sel[b]], p["scale"])
        G.check_fwd(o[s:e], lse[:, s:e], o_ref, lse_ref, f"workload 7 seq {b} (L={e - s})")


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("ratio", [0.5, 0.25])
def test_block_sparse_backward(head_dim, ratio):
    _run(LENGTHS, 2, head_dim, ratio, seed=51, label=f"D{head_dim} r{ratio}", bwd=True)


def test_block_sparse_backward_dynamic_schedule_and_few_programs():
    _run(LENGTHS, 3, 128, 0.5, seed=52, opts=B.make_opts(sched=1, num_programs=5), label="dynamic", bwd=True)
    _run(LENGTHS, 2, 64, 0.3, seed=53, opts=B.make_opts(num_programs=3), label="3 programs", bwd=True)


def test_block_sparse_backward_ratio_one_equals_dense_backward():
    for d in (64, 128):
        p, g, o, lse, sel, grads = _run(LENGTHS, 2, d, 1.0, seed=54, label=f"ratio 1 D{d}", bwd=True)
        dense = G.gpu_bwd(g, o, lse)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), grads, dense):
            if name == "dq" or d == 64:
                assert torch.equal(a, b), f"D{d} {name}"
                continue
            # same products summed in another order, each side rounded once to bf16:
            # one bf16 step (2^-7 relative) apart, plus cancellation near zero
            a64, b64 = G.f64(a), G.f64(b)
            amax = float(np.abs(b64).max())
            bound = 2.0 ** -7 * np.maximum(np.abs(a64), np.abs(b64)) + 2.0 ** -12 * amax
            bad = np.abs(a64 - b64) > bound
            assert not bad.any(), f"D{d} {name}: {int(bad.sum())} elements beyond one rounding step"


def test_block_sparse_backward_long_sequences():
    # 8448 keys: 33 query blocks, so the tiles' bitmaps take two words
    _run([8448, 3, 2500], 1, 128, 0.25, seed=55, label="long", bwd=True)


def test_block_sparse_backward_production_lengths_reduced():
    lengths = W.workload_lengths(3, 0, 48).tolist()
    _run(lengths, 4, 128, 0.5, seed=57, label="production lengths, 48 sequences", bwd=True)


def test_block_sparse_backward_full_production_workload_sampled():
    """Workload 7 (forward + backward) at full size in the launch configuration bench.py
    times; sampled sequences checked against the oracle."""
    print("[case] block sparse backward full-size workload 7", flush=True)
    p = W.make_workload(7, seed=0, device="cuda")
    ratio = W.WORKLOADS[7]["sparse_ratio"]
    o, lse, sel = B.fwd_block_sparse(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], ratio, p["scale"],
                                     None, *G.nan_outputs_fwd(p))
    dq, dk, dv = B.bwd_block_sparse(p["q"], p["k"], p["v"], o, p["do"], lse, p["offsets"], p["offsets_host"], ratio,
                                    sel, p["scale"], None, G.nan_like(p["q"]), G.nan_like(p["k"]), G.nan_like(p["v"]))
    torch.cuda.synchronize()
    gpu_sel, _ = _split_selection(sel, p["lengths"], p["num_heads"], ratio)
    off = p["offsets_host"].astype(np.int64)
    order = np.argsort(p["lengths"], kind="stable")
    for b in sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), 11, 600}):
        s, e = int(off[b]), int(off[b + 1])
        sub = lambda t: G.f64(t[s:e])
        refs = S.block_sparse_backward(sub(p["q"]), sub(p["k"]), sub(p["v"]), sub(p["do"]), [0, e - s],
                                       [gpu_sel[b]], p["scale"])
        refs_o = S.block_sparse_backward(sub(p["q"]), sub(p["k"]), sub(p["v"]), sub(p["do"]), [0, e - s],
                                         [gpu_sel[b]], p["scale"], o_given=sub(o))
        G.check_bwd((dq[s:e], dk[s:e], dv[s:e]), refs, f"workload 7 bwd seq {b} (L={e - s})",
                    {"offsets_host": [0, e - s], "mode": p["mode"]}, refs_o)


def test_block_sparse_largest_sequence():
    """One sequence of 2048 key blocks (131072 tokens), the most the variant takes: at
    ratio 1 forward and backward equal the dense kernels bit for bit; at ratio 0.5 the
    selections of sampled query blocks are valid against fp64 relevance computed for
    those blocks only."""
    n = 64 * 2048
    print(f"[case] block sparse largest sequence L={n} H=1 D=64", flush=True)
    p = W.make_problem([n], 1, 64, seed=58, device="cuda", with_grad=True)
    o1, l1, sel1 = B.fwd_block_sparse(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], 1.0, p["scale"])
    od, ld = B.fwd(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], W.MODE_SELF, p["scale"])
    gs = B.bwd_block_sparse(p["q"], p["k"], p["v"], o1, p["do"], l1, p["offsets"], p["offsets_host"], 1.0, sel1,
                            p["scale"])
    gd = B.bwd(p["q"], p["k"], p["v"], od, p["do"], ld, p["offsets"], p["offsets_host"], W.MODE_SELF, p["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1, od) and torch.equal(l1, ld)
    for name, a, b in zip(("dq", "dk", "dv"), gs, gd):
        assert torch.equal(a, b), name
    _, _, sel = B.fwd_block_sparse(p["q"], p["k"], p["v"], p["offsets"], p["offsets_host"], 0.5, p["scale"])
    torch.cuda.synchronize()
    kk = S.keep_count(n, 0.5)
    sel = sel.cpu().numpy()
    q, k = G.f64(p["q"]), G.f64(p["k"])
    kb = S.pooled_blocks(k, 0, n, S.K_BLOCK)[:, 0]          # [2048, D]
    for i in (0, 1, 255, 511):
        got = sel[i * kk:(i + 1) * kk].tolist()
        assert len(got) == kk and got == sorted(set(got)) and all(0 <= j < 2048 for j in got)
        qb = q[i * S.Q_BLOCK:(i + 1) * S.Q_BLOCK, 0].mean(axis=0)
        s = kb @ qb
        dropped = np.setdiff1d(np.arange(2048), got)
        tol = 1e-4 * np.linalg.norm(qb) * np.linalg.norm(kb, axis=1).max()
        assert s[got].min() >= s[dropped].max() - tol - 1e-9, i
