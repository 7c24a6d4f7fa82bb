#!/usr/bin/env python3
"""Benchmark of the jagged flash attention hot path on one MI355X.

A step is one forward plus one backward (jfa_fwd + jfa_bwd through the C ABI: offsets
intake, host schedule, schedule upload, attention kernels; the self-attention backward
at head_dim 128 takes the stored-dS path, whose workspace the bench grants) over one
batch of the production-shaped jagged self-attention workload: B=1152
sequences with log-normal lengths (median ~600, clipped to [1, 4000]), H=4, D=128,
bf16 N(0,1) inputs drawn with seed 0, already resident in HBM.  The reported value is
valid-token TFLOPS (forward 4*H*D*sum L^2 plus backward 2.5x that) per step.

Prints one JSON line.  ``--workload N`` benchmarks another numbered workload (see
variable_length_flash_jagged_amd/workloads.py) instead.
"""

import argparse
import math
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "valid-token TFLOPS fwd+bwd (bf16, D=128 jagged) and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--sched", type=int, default=1,
                    help="0 static host schedule, 1 (default) the same tiles with one run-time counter per XCD")
    ap.add_argument("--dq-path", type=int, default=2,
                    help="broadcast-Q backward: 0 fused kernel + fp32 atomics, 1 fused kernel + per-program slabs, "
                         "2 dQ and dK/dV kernels + key-chunk slabs")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--self-bwd", choices=("auto", "stored", "recompute"), default="auto",
                    help="self-attention backward: stored-dS (the bench grants the dS workspace), recompute, "
                         "or auto (stored-dS at head_dim 128, recompute at 64)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (scales HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench with "
                         "--calibrate-copy-mib into profiles/traffic_<workload>.json and exit")
    return ap.parse_args()


def _code_only(text):
    """C/C++ source with comments removed and whitespace runs collapsed (string and
    character literals kept as they are), so that an edit to a comment leaves the
    digest of the code unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


FLUSH_MIB = 512
FLUSH_WORKLOADS = ("broadcast_q", "block_diag")
SDPA_WORKLOADS = ("dense_equivalent",)


def padded_sdpa(q, k, v, do, lengths, h, d, scale, args):
    """Context for the dense-equivalent workload: the same batch as padded dense tensors
    [B, H, L, D] (every length equal, so no padding is added) through PyTorch's fused
    scaled_dot_product_attention, forward + backward, timed like the jagged step.  Only
    the fused flash / memory-efficient kernels are allowed (never the unfused math
    path); if neither is available the field is null.  Not part of the library."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    nb, n = len(lengths), int(lengths[0])
    if any(int(x) != n for x in lengths):
        return None
    dense = lambda t: t.view(nb, n, h, d).transpose(1, 2).contiguous()
    qd, kd, vd, dod = dense(q).requires_grad_(), dense(k).requires_grad_(), dense(v).requires_grad_(), dense(do)
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            def run():
                out = F.scaled_dot_product_attention(qd, kd, vd, scale=scale)
                out.backward(dod)
                return out
            for _ in range(args.warmup):
                run()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            e[0].record()
            for _ in range(args.steps):
                run()
            e[1].record()
            torch.cuda.synchronize()
    except RuntimeError as exc:
        return {"error": str(exc).splitlines()[0][:200]}
    ms = e[0].elapsed_time(e[1]) / args.steps
    flops = 3.5 * 4 * h * d * nb * n * n
    return {"shape": [nb, h, n, d], "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "backends": "flash or memory-efficient (PyTorch)"}


def kernel_source_digest():
    """Digest of the kernel sources' code (comments excluded); traffic counters are only
    reported for the code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "variable_length_flash_jagged_amd", "csrc")
    for f in sorted(sum((glob.glob(os.path.join(csrc, "*" + ext)) for ext in (".hip", ".cpp", ".h")), [])):
        with open(f, encoding="utf-8", errors="replace") as fh:
            h.update(os.path.basename(f).encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


KERNEL_NAMES = {"fwd_kernel": "fwd_kernel<", "dq_kernel": "dq_kernel<", "dkdv_kernel": "dkdv_kernel<",
                "dkdv2_kernel": "dkdv2_kernel<",
                "dq_ds_kernel": "dq_ds_kernel<", "prep_kernel": "prep_kernel<", "mark_kernel": "mark_kernel",
                "mx_fwd_kernel": "mx_fwd_kernel<", "mx2_fwd_kernel": "mx2_fwd_kernel(",
                "bwd_kernel": "bwd_kernel<", "bd_fwd_kernel": "bd_fwd_kernel<", "bd_bwd_kernel": "bd_bwd_kernel<"}


def summarize_pmc(fetch_dir, write_dir, workload, copy_mib):
    """Per-kernel average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) and the scale factors
    that map the counters onto the bytes of the calibration copy."""
    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return rows
    out = {"workload": workload, "src_digest": kernel_source_digest(), "calibration_copy_mib": copy_mib}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = load(d, counter)
        copies = [v for n, v in rows if "copyBuffer" in n]
        out[f"{counter}_scale"] = (copy_mib * 1024.0) / max(copies) if copies and max(copies) > 0 else None
        for short, key in KERNEL_NAMES.items():
            vals = [v for n, v in rows if key in n]
            if vals:
                out.setdefault("kernels", {}).setdefault(short, {})[counter + "_kib"] = sum(vals) / len(vals)
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(path)


def traffic_bytes(workload, kernel):
    """Calibrated HBM bytes per launch of `kernel` from profiles/, or None when absent or
    taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    k = t.get("kernels", {}).get(kernel)
    if t.get("src_digest") != kernel_source_digest() or not k or not t.get("FETCH_SIZE_scale") \
            or not t.get("WRITE_SIZE_scale"):
        return None
    return int(1024 * (k["FETCH_SIZE_kib"] * t["FETCH_SIZE_scale"] + k["WRITE_SIZE_kib"] * t["WRITE_SIZE_scale"]))


def cpu_baseline(p_cpu_fn, lengths, mode, num_heads, head_dim, num_q, target_s, fwd_only=False, sparse_ratio=None,
                 rotary=False, mxfp8=False):
    """Time the fp64 oracle on the first sequences of the same batch (bounded sample)."""
    import numpy as np
    import oracle
    from variable_length_flash_jagged_amd import metrics as M
    # The oracle's matrix products run in the BLAS thread pool; its size comes from the
    # environment (OMP_NUM_THREADS / OPENBLAS_NUM_THREADS, which a GPU host may set to
    # the process's share of its cores) and is recorded with the machine's core count.
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in blas] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    done, flops, spent, b = 0, 0, 0.0, 0
    chunk = 8
    while b < len(lengths) and spent < target_s:
        e = min(len(lengths), b + chunk)
        q, k, v, do, off = p_cpu_fn(b, e)
        t0 = time.perf_counter()
        if sparse_ratio is not None:
            from oracle import block_sparse as S
            sel = S.select_blocks(q, k, off, sparse_ratio)
            S.block_sparse_forward(q, k, v, off, sel, 1.0 / np.sqrt(head_dim))
            if not fwd_only:
                S.block_sparse_backward(q, k, v, do, off, sel, 1.0 / np.sqrt(head_dim))
            spent += time.perf_counter() - t0
            sub = lengths[b:e]
            keep = [S.keep_count(n, sparse_ratio) for n in sub]
            flat = [j for per_b in sel for per_h in per_b for lst in per_h for j in lst]
            pairs = M.block_sparse_pairs(sub, num_heads, keep, flat)  # pairs over heads
            flops += (4 if fwd_only else 14) * head_dim * pairs
            done, b = e, e
            continue
        if mxfp8:
            from oracle import mxfp8 as MX
            qv, qx = MX.quantise_qk(q)
            kv, kx = MX.quantise_qk(k)
            vv, vx = MX.quantise_v(v, off)
            qd, kd, vd = MX.dequantise_qk(qv, qx), MX.dequantise_qk(kv, kx), MX.dequantise_v(vv, vx, off)
            o_mx, _ = MX.mxfp8_forward(qd, kd, vd, off, 1.0 / np.sqrt(head_dim))
            if not fwd_only:
                MX.mxfp8_backward(qd, kd, vd, do, off, 1.0 / np.sqrt(head_dim), o_given=o_mx)
        elif rotary:
            from oracle import rotary as R
            tab = R.rope_table(max(1, int(max(lengths[b:e]))), head_dim)
            R.rotary_block_forward(q, k, v, off, tab, 1.0 / np.sqrt(head_dim))
            R.rotary_block_backward(q, k, v, do, off, tab, 1.0 / np.sqrt(head_dim))
        else:
            oracle.attention_forward(q, k, v, off, mode, 1.0 / np.sqrt(head_dim))
            if not fwd_only:
                oracle.attention_backward(q, k, v, do, off, mode, 1.0 / np.sqrt(head_dim))
        spent += time.perf_counter() - t0
        sub = lengths[b:e]
        flops += M.fwd_flops(sub, mode, num_heads, head_dim, num_q)
        if not fwd_only:
            flops += M.bwd_flops(sub, mode, num_heads, head_dim, num_q)
        done, b = e, e
    return {
        "value": round(flops / spent / 1e12, 6),
        "unit": "TFLOPS",
        "cores": int(threads),
        "os_cpu_count": os.cpu_count(),
        "thread_env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")},
        "kind": "oracle",
        "sample": f"first {done} of {len(lengths)} sequences of the same batch (sum L = {int(sum(lengths[:done]))}), "
                  f"one fp64 {'block-sparse ' if sparse_ratio else 'rotary ' if rotary else 'MXFP8 ' if mxfp8 else ''}"
                  f"{'forward' if fwd_only else 'forward + backward'}"
                  f" each, {spent:.1f} s",
    }


def main():
    args = parse()
    if args.summarize_pmc:
        from variable_length_flash_jagged_amd import workloads as W
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], W.WORKLOADS[args.workload]["name"],
                      args.calibrate_copy_mib or 1024)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from variable_length_flash_jagged_amd import binding as B
    from variable_length_flash_jagged_amd import metrics as M
    from variable_length_flash_jagged_amd import workloads as W

    torch.cuda.init()
    w = W.WORKLOADS[args.workload]
    p = W.make_workload(args.workload, seed=args.seed, device="cuda")
    mode, h, d, mq = p["mode"], p["num_heads"], p["head_dim"], p["num_q"]
    hkv = p["num_kv_heads"]
    fwd_only = bool(w.get("fwd_only", False))  # grouped-query attention: forward only
    ratio = w.get("sparse_ratio")
    rotary = bool(w.get("rotary", False))
    mxfp8 = bool(w.get("mxfp8", False))
    lengths = p["lengths"]
    rope = B.rope_table(int(max(lengths)), d, device="cuda") if rotary else None
    shape = B.make_shape(p["num_seqs"], h, d, p["total_tokens"], mq, hkv if hkv != h else 0)
    opts = B.bench_opts(mode, shape, p["offsets_host"], args.sched, args.dq_path, self_bwd=args.self_bwd)
    q, k, v, do, off, off_h = p["q"], p["k"], p["v"], p["do"], p["offsets"], p["offsets_host"]
    if mode == W.MODE_BROADCAST_Q:
        o = torch.empty((p["num_seqs"], mq, h, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((p["num_seqs"], h, mq), dtype=torch.float32, device="cuda")
    else:
        o = torch.empty_like(q)
        lse = torch.empty((h, p["total_tokens"]), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_f = B.alloc_workspace(shape, mode, B.PASS_FWD_SPARSE if ratio else B.PASS_FWD, opts, "cuda")
    sel = None
    if ratio:
        sel = torch.empty(max(1, B.block_sparse_entries(shape, p["offsets_host"], ratio)), dtype=torch.int32,
                          device="cuda")
    if fwd_only:
        ws_b = None
    elif mxfp8:
        ws_b = B.alloc_workspace(shape, mode, B.PASS_BWD_MXFP8, opts, "cuda")
    elif ratio:
        ws_b = torch.empty(B.bwd_block_sparse_workspace_size(shape, p["offsets_host"], opts), dtype=torch.uint8,
                           device="cuda")
    else:
        ws_b = B.alloc_workspace(shape, mode, B.PASS_BWD, opts, "cuda")
    scale = p["scale"]
    mx = None
    if mxfp8:
        # inputs are resident in MXFP8: quantised before the timed region (the quantisers
        # are timed on a second, warm call, for context)
        for rep in range(2):
            B.kernel_timing(rep == 1)
            q8, qs = B.mxfp8_quantize_qk(q)
            k8, ks = B.mxfp8_quantize_qk(k)
            v8, vs, tp = B.mxfp8_quantize_v(v, off, off_h)
            torch.cuda.synchronize()
        nq, tq = B.kernel_times(B.KERNEL_MX_QUANT)
        B.kernel_timing(False)
        ws_f = B.alloc_workspace(shape, mode, B.PASS_FWD_MXFP8, opts, "cuda")
        mx = dict(q8=q8, qs=qs, k8=k8, ks=ks, v8=v8, vs=vs, tp=tp, quant_ms=tq, quant_launches=nq)

    ev = {n: [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)] for n in ("f0", "f1", "b1")}

    def step(i=None):
        if i is not None:
            ev["f0"][i].record()
        if ratio:
            B.fwd_block_sparse(q, k, v, off, off_h, ratio, scale, opts, o, lse, sel, ws_f)
        elif rotary:
            B.fwd_rotary(q, k, v, off, off_h, rope, scale, opts, o, lse, ws_f)
        elif mxfp8:
            B.fwd_mxfp8(mx["q8"], mx["qs"], mx["k8"], mx["ks"], mx["v8"], mx["vs"], mx["tp"], off, off_h, scale, opts,
                        o, lse, ws_f)
        else:
            B.fwd(q, k, v, off, off_h, mode, scale, opts, o, lse, ws_f)
        if i is not None:
            ev["f1"][i].record()
        if ratio:
            B.bwd_block_sparse(q, k, v, o, do, lse, off, off_h, ratio, sel, scale, opts, dq, dk, dv, ws_b)
        elif rotary:
            B.bwd_rotary(q, k, v, o, do, lse, off, off_h, rope, scale, opts, dq, dk, dv, ws_b)
        elif mxfp8 and not fwd_only:
            B.bwd_mxfp8(mx["q8"], mx["qs"], mx["k8"], mx["ks"], mx["v8"], mx["vs"], mx["tp"], o, do, lse, off, off_h,
                        scale, opts, dq, dk, dv, ws_b)
        elif not fwd_only:
            B.bwd(q, k, v, o, do, lse, off, off_h, mode, scale, opts, dq, dk, dv, ws_b)
        if i is not None:
            ev["b1"][i].record()

    if args.calibrate_copy_mib > 0:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # Workloads whose working set fits the 256 MB last-level cache (MALL) and the ones
    # the measurement plan names (broadcast-Q, block-diagonal) write a 512 MiB buffer
    # between steps, outside the per-step events, so that no step reads the previous
    # step's data from cache; the step time is then the sum of the per-step intervals.
    flush = torch.empty(FLUSH_MIB << 20, dtype=torch.uint8, device="cuda") if w["name"] in FLUSH_WORKLOADS else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    B.kernel_timing(True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    if flush is not None:
        total_ms = sum(ev["f0"][i].elapsed_time(ev["b1"][i]) for i in range(args.steps))
        del flush
    ms_step = total_ms / args.steps
    fwd_ms = sum(ev["f0"][i].elapsed_time(ev["f1"][i]) for i in range(args.steps)) / args.steps
    bwd_ms = sum(ev["f1"][i].elapsed_time(ev["b1"][i]) for i in range(args.steps)) / args.steps
    kt = {name: B.kernel_times(kid) for name, kid in
          (("fwd", B.KERNEL_FWD), ("bwd", B.KERNEL_BWD), ("bwd_dq", B.KERNEL_BWD_DQ), ("bwd_prep", B.KERNEL_BWD_PREP),
           ("select", B.KERNEL_SPARSE_SELECT), ("mx_decode", B.KERNEL_MX_QUANT))}
    B.kernel_timing(False)

    ff = M.fwd_flops(lengths, mode, h, d, mq)
    fb = 0 if fwd_only else M.bwd_flops(lengths, mode, h, d, mq)
    dense = None
    plain = None
    if mxfp8:
        # the bf16 forward of the same batch, for context: alternated with the MXFP8
        # forward in one loop of forwards, so that both run at the same clock (the timed
        # steps above interleave backward passes, which heat the chip)
        ws_d = B.alloc_workspace(shape, mode, B.PASS_FWD, opts, "cuda")
        o2 = torch.empty_like(o)
        lse2 = torch.empty_like(lse)
        for _ in range(args.warmup):
            B.fwd(q, k, v, off, off_h, mode, scale, opts, o2, lse2, ws_d)
        ee = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ee[i][0].record()
            B.fwd(q, k, v, off, off_h, mode, scale, opts, o2, lse2, ws_d)
            ee[i][1].record()
            B.fwd_mxfp8(mx["q8"], mx["qs"], mx["k8"], mx["ks"], mx["v8"], mx["vs"], mx["tp"], off, off_h, scale, opts,
                        o, lse, ws_f)
            ee[i][2].record()
        torch.cuda.synchronize()
        plain = [sum(e[0].elapsed_time(e[1]) for e in ee) / args.steps, 0.0,
                 sum(e[1].elapsed_time(e[2]) for e in ee) / args.steps]
    if rotary:
        # the same batch through the plain block-diagonal kernels, for the rotary's cost
        evp = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(args.warmup):
            B.fwd(q, k, v, off, off_h, mode, scale, opts, o, lse, ws_f)
            B.bwd(q, k, v, o, do, lse, off, off_h, mode, scale, opts, dq, dk, dv, ws_b)
        plain = [0.0, 0.0]
        for _ in range(args.steps):
            evp[0].record()
            B.fwd(q, k, v, off, off_h, mode, scale, opts, o, lse, ws_f)
            evp[1].record()
            B.bwd(q, k, v, o, do, lse, off, off_h, mode, scale, opts, dq, dk, dv, ws_b)
            evp[2].record()
            torch.cuda.synchronize()
            plain[0] += evp[0].elapsed_time(evp[1]) / args.steps
            plain[1] += evp[1].elapsed_time(evp[2]) / args.steps
    if ratio:
        # attended pairs only; the dense forward and backward of the same batch (the
        # bench's dense options) are timed for context
        keep = [max(1, math.ceil(float(np.float32(ratio)) * -(-int(n) // 64))) if n else 0 for n in lengths]
        sel_h = sel.cpu().numpy()
        sp_pairs = M.block_sparse_pairs(lengths, h, keep, sel_h)  # pairs summed over heads
        ff, fb = 4 * d * sp_pairs, 10 * d * sp_pairs
        # the dK/dV kernel runs 64-key tiles at head_dim 128, 128-key tiles otherwise
        tile_pairs = M.block_sparse_tile_pairs(lengths, h, keep, sel_h, tile_keys=64 if d == 128 else 128)
        ws_d = B.alloc_workspace(shape, mode, B.PASS_FWD, opts, "cuda")
        ws_db = B.alloc_workspace(shape, mode, B.PASS_BWD, opts, "cuda")
        evd = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(args.warmup):
            B.fwd(q, k, v, off, off_h, mode, scale, opts, o, lse, ws_d)
            B.bwd(q, k, v, o, do, lse, off, off_h, mode, scale, opts, dq, dk, dv, ws_db)
        dense = [0.0, 0.0]
        for _ in range(args.steps):
            evd[0].record()
            B.fwd(q, k, v, off, off_h, mode, scale, opts, o, lse, ws_d)
            evd[1].record()
            B.bwd(q, k, v, o, do, lse, off, off_h, mode, scale, opts, dq, dk, dv, ws_db)
            evd[2].record()
            torch.cuda.synchronize()
            dense[0] += evd[0].elapsed_time(evd[1]) / args.steps
            dense[1] += evd[1].elapsed_time(evd[2]) / args.steps
        del ws_db
    bytes_f = M.fwd_bytes(lengths, mode, h, d, mq, hkv)
    bytes_b = 0 if fwd_only else M.bwd_bytes(lengths, mode, h, d, mq)
    value = (ff + fb) / (ms_step * 1e-3) / 1e12
    # Per attention kernel: average launch time and the algorithmic work of one launch.
    work = {"fwd": (ff, bytes_f)}
    bwd_path = B.last_bwd_path()
    stored_ds = not ratio and bwd_path == B.BWD_PATH_STORED_DS
    if ratio:
        # Block-sparse backward: mark kernel (selection in, bitmaps out), dQ kernel over
        # the kept blocks (S, dP, dQ on attended pairs), dK/dV kernel (S, dP, dV, dK on
        # attended pairs; it executes whole 128-key tiles, see block_sparse.tile_pairs).
        t = int(p["total_tokens"])
        work["bwd_prep"] = (0, 4 * int(sel.numel()))
        work["bwd_dq"] = (6 * d * sp_pairs, 12 * t * h * d + 20 * t * h)
        work["bwd"] = (8 * d * sp_pairs, 12 * t * h * d + 16 * t * h)
    elif mode == W.MODE_SELF and stored_ds:
        # Stored-dS backward: row-term kernel (O, dO in, lse in, 16-byte term out per
        # row and head), dK/dV kernel (S, dP, dV, dK; Q, K, V, dO in, dK, dV out, the
        # row term in, dS out as bf16 per valid pair) and dQ = dS K (dS and K in, dQ out).
        pairs = M.valid_pairs(lengths, mode)
        t = int(p["total_tokens"])
        work["bwd_prep"] = (2 * t * h * d, 4 * t * h * d + 20 * t * h)
        work["bwd"] = (8 * h * d * pairs, 12 * t * h * d + 16 * t * h + 2 * h * pairs)
        work["bwd_dq"] = (2 * h * d * pairs, 4 * t * h * d + 2 * h * pairs)
    elif mode == W.MODE_SELF and not fwd_only:
        # Recompute backward: a dQ kernel (S, dP, dQ: 3 of the 5 products plus the 2 it
        # recomputes; Q, K, V, O, dO in, dQ out, lse in and the 16-byte row term out per
        # row and head) and a dK/dV kernel (S, dP, dV, dK; Q, K, V, dO in, dK, dV out,
        # the row term in).
        # With few tiles the row terms come from the row-term kernel and the dQ kernel
        # runs beside the dK/dV kernel (it then reads lse and writes no row term).
        pairs = M.valid_pairs(lengths, mode)
        t = int(p["total_tokens"])
        side = bwd_path == B.BWD_PATH_RECOMPUTE_SIDE
        if side:
            work["bwd_prep"] = (2 * t * h * d, 4 * t * h * d + 20 * t * h)
        work["bwd_dq"] = (6 * h * d * pairs, 12 * t * h * d + (4 if side else 20) * t * h)
        work["bwd"] = (8 * h * d * pairs, 12 * t * h * d + 16 * t * h)
    elif mode == W.MODE_BROADCAST_Q and not fwd_only and kt["bwd_dq"][0] > 0:
        # Broadcast-Q through the dQ and dK/dV kernels (dq_path 2): a dQ kernel (S, dP,
        # dQ; Q, K, V, O, dO in, lse in, dQ out, the 16-byte row term out per row) and a
        # dK/dV kernel (S, dP, dV, dK; Q, K, V, dO in, the row term in, dK, dV out).
        sl = int(sum(lengths))
        nb = len(lengths)
        work["bwd_dq"] = (6 * h * d * mq * sl, 4 * mq * h * d + 4 * sl * h * d + 4 * nb * mq * h * d + 20 * nb * h * mq)
        work["bwd"] = (8 * h * d * mq * sl, 2 * mq * h * d + 8 * sl * h * d + 2 * nb * mq * h * d + 16 * nb * h * mq)
    elif not fwd_only:
        work["bwd"] = (fb, bytes_b)
    if ratio:
        # stage 1 reads Q and K once (the block means and lists are small)
        work["select"] = (0, 2 * int(p["total_tokens"]) * (h + hkv) * d)
    kernels = {}
    for name, (fl, by) in work.items():
        n, tot = kt[name]
        if n == 0:
            continue
        ms = tot / (args.steps if name == "select" else n)  # stage 1 of the sparse forward: 3 launches a step
        kernels[name] = {"launches_per_step": n // args.steps, "ms": round(ms, 4), "flops": fl, "bytes": by,
                         "tflops": round(fl / (ms * 1e-3) / 1e12, 1), "gbs": round(by / (ms * 1e-3) / 1e9, 1)}
    hbm_bound = mode == W.MODE_BLOCK_DIAG
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    if hbm_bound:
        achieved = kd["bytes"] / (kd["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        achieved = kd["flops"] / (kd["ms"] * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if (mxfp8 and dom == "fwd") else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    roof["kernel"] = {"fwd": "fwd_kernel", "bwd": "dkdv_kernel" if mode == W.MODE_SELF or "bwd_dq" in work else
                      ("bd_bwd_kernel" if mode == W.MODE_BLOCK_DIAG else "bwd_kernel"),
                      "bwd_dq": "dq_ds_kernel" if stored_ds else "dq_kernel",
                      "bwd_prep": "mark_kernel" if ratio else "prep_kernel",
                      "select": "select_kernel"}[dom]
    if mode == W.MODE_BLOCK_DIAG and dom == "fwd":
        roof["kernel"] = "bd_fwd_kernel"
    if mxfp8 and dom == "fwd":
        # head_dim 128 runs the two-group ping-pong kernel
        roof["kernel"] = "mx2_fwd_kernel" if d == 128 else "mx_fwd_kernel"
    if dom == "bwd" and mode == W.MODE_SELF and d == 128 and not ratio:
        roof["kernel"] = "dkdv2_kernel"  # the two-waves-per-SIMD dK/dV kernel of self attention
    roof["kernel_ms"] = kd["ms"]
    roof["traffic"] = traffic_bytes(w["name"], roof["kernel"])

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3, e8m0 scales), fp32 accumulate" if mxfp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": w["name"],
            "mode": ["self", "broadcast_q", "block_diag"][mode],
            "num_seqs": int(p["num_seqs"]), "num_heads": h, "num_kv_heads": hkv, "head_dim": d, "num_q": mq,
            "passes": "fwd" if fwd_only else "fwd+bwd",
            "total_tokens": int(p["total_tokens"]), "max_len": int(max(lengths)),
            "sched": ["static", "dynamic"][args.sched], "dq_path": args.dq_path, "seed": args.seed,
            "self_bwd": B.BWD_PATH_NAMES[bwd_path] if mode == W.MODE_SELF and not fwd_only else None,
            "ds_budget_mib": int(opts.ds_budget_mib),
        },
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 1),
                "pct_of_peak": round(100 * ff / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                "flops": ff, "bytes": bytes_f},
        "bwd": None if fwd_only else {
            "ms": round(bwd_ms, 4), "tflops": round(fb / (bwd_ms * 1e-3) / 1e12, 1),
            "pct_of_peak": round(100 * fb / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "flops": fb, "bytes": bytes_b},
        "kernels": kernels,
        "roofline": roof,
        "wall_s_timed": round(wall, 3),
        "block_sparse": None if not ratio else {
            "ratio": ratio, "attended_pairs_fraction": round(ff / M.fwd_flops(lengths, mode, h, d, mq), 4),
            "dkdv_executed_pairs_fraction": round(tile_pairs / M.valid_pairs(lengths, mode) / h, 4),
            "dense_fwd_ms": round(dense[0], 4), "speedup_vs_dense_fwd": round(dense[0] / fwd_ms, 3),
            "dense_bwd_ms": round(dense[1], 4), "speedup_vs_dense_bwd": round(dense[1] / bwd_ms, 3),
            "speedup_vs_dense_step": round((dense[0] + dense[1]) / ms_step, 3)},
        "mxfp8": None if not mxfp8 else {
            "v_tokens": int(mx["tp"]), "quantise_ms": round(mx["quant_ms"], 4),
            "quantise_launches": int(mx["quant_launches"]), "bf16_fwd_ms": round(plain[0], 4),
            "mxfp8_fwd_ms_alternating": round(plain[2], 4),
            "speedup_vs_bf16_fwd": round(plain[0] / plain[2], 3),
            # the backward decodes its MXFP8 inputs to bf16 (3 launches a step) before the
            # bf16 backward kernels
            "bwd_decode_ms": None if fwd_only else round(kt["mx_decode"][1] / max(1, args.steps), 4),
            "bwd_decode_launches_per_step": None if fwd_only else kt["mx_decode"][0] // max(1, args.steps)},
        "cache_flush_mib_between_steps": FLUSH_MIB if w["name"] in FLUSH_WORKLOADS else 0,
        "padding": None if mode != W.MODE_SELF else {
            # the work a padded batch would do (every sequence padded to the longest)
            "valid_pairs": int(M.valid_pairs(lengths, mode)),
            "padded_pairs": int(len(lengths)) * int(max(lengths)) ** 2,
            "valid_fraction": round(M.valid_pairs(lengths, mode) / (len(lengths) * float(max(lengths)) ** 2), 4)},
        "padded_sdpa": padded_sdpa(q, k, v, do, lengths, h, d, scale, args) if w["name"] in SDPA_WORKLOADS else None,
        "rotary": None if not rotary else {
            "table_rows": int(rope.shape[0]), "plain_fwd_ms": round(plain[0], 4), "plain_bwd_ms": round(plain[1], 4),
            "fwd_cost_vs_plain": round(fwd_ms / plain[0], 3), "bwd_cost_vs_plain": round(bwd_ms / plain[1], 3)},
    }
    if not args.no_cpu_baseline:
        offs = np.asarray(off_h, dtype=np.int64)

        def sub_problem(b0, b1):
            s, e = int(offs[b0]), int(offs[b1])
            f = lambda t: t[s:e].float().cpu().numpy().astype(np.float64)
            sub_off = offs[b0:b1 + 1] - s
            if mode == W.MODE_BROADCAST_Q:
                return (q.float().cpu().numpy().astype(np.float64), f(k), f(v),
                        do[b0:b1].float().cpu().numpy().astype(np.float64), sub_off)
            return f(q), f(k), f(v), (None if do is None else f(do)), sub_off

        out["cpu_baseline"] = cpu_baseline(sub_problem, [int(x) for x in lengths], mode, h, d, mq, args.cpu_seconds,
                                           fwd_only, ratio, rotary, mxfp8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
