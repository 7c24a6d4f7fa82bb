"""Seeded synthetic inputs shaped like the jagged-attention workloads on the pages.

This module holds none of the attention arithmetic: it only draws sequence lengths
and N(0, 1) tensors rounded to bf16 (round to nearest even), and packs the lengths
into an offsets array.  Both the library's tests/bench and the CPU oracle are fed
from it.

Workloads (the pages' production length traces are not public; these seeded
generators stand in for them):

1. ``self_4seq_d64``: self-attention, lengths [128, 4096, 512, 2048] (the worked
   offsets example), H=1, D=64.
2. ``broadcast_q``: one shared Q of Mq=256 rows, H=4, D=128, B=64 K/V sequences with
   log-uniform lengths L = clip(floor(exp(U[0, ln 4097))), 1, 4096).
3. ``production_jagged``: self-attention, B=1152, L = clip(rint(exp(N(ln 600, 1))),
   1, 4000) (median ~600), H=4, D=128.
4. ``dense_equivalent``: self-attention, B=16 sequences of 4096, H=8, D=128.
5. ``block_diag``: 64-token block-diagonal attention, B=1152, L = 64 * n with
   n ~ U{1..63}, H=4, D=64.
6. ``production_jagged_gqa``: the lengths of workload 3 with H=4 query heads sharing
   one key/value head (grouped-query attention, forward only).
7. ``production_jagged_sparse``: workload 3 through the block-sparse top-k forward and
   backward at ratio 0.5.
8. ``block_diag_rotary``: workload 5 with the rotary position embedding fused into the
   block-diagonal attention (cos/sin table of the longest sequence's positions).
9. ``production_jagged_mxfp8``: the lengths and shape of workload 3 through the MXFP8
   forward (inputs quantised to OCP MXFP8 before the timed region).

Draw order: lengths (numpy ``default_rng(seed)``), then q, k, v, dO from one
``torch.Generator`` seeded with ``seed`` on the target device, each drawn in fp32 and
rounded to bf16.
"""

import math

import numpy as np

MODE_SELF = 0
MODE_BROADCAST_Q = 1
MODE_BLOCK_DIAG = 2

WORKLOADS = {
    1: dict(name="self_4seq_d64", mode=MODE_SELF, num_heads=1, head_dim=64, num_q=0),
    2: dict(name="broadcast_q", mode=MODE_BROADCAST_Q, num_heads=4, head_dim=128, num_q=256),
    3: dict(name="production_jagged", mode=MODE_SELF, num_heads=4, head_dim=128, num_q=0),
    4: dict(name="dense_equivalent", mode=MODE_SELF, num_heads=8, head_dim=128, num_q=0),
    5: dict(name="block_diag", mode=MODE_BLOCK_DIAG, num_heads=4, head_dim=64, num_q=0),
    6: dict(name="production_jagged_gqa", mode=MODE_SELF, num_heads=4, num_kv_heads=1, head_dim=128, num_q=0,
            fwd_only=True),
    7: dict(name="production_jagged_sparse", mode=MODE_SELF, num_heads=4, head_dim=128, num_q=0,
            sparse_ratio=0.5),
    8: dict(name="block_diag_rotary", mode=MODE_BLOCK_DIAG, num_heads=4, head_dim=64, num_q=0, rotary=True),
    9: dict(name="production_jagged_mxfp8", mode=MODE_SELF, num_heads=4, head_dim=128, num_q=0, mxfp8=True),
}


def workload_lengths(workload, seed=0, num_seqs=None):
    """Sequence lengths of a numbered workload (int64 numpy array).  ``num_seqs``
    draws a shorter batch from the same distribution (parity-test sizes)."""
    rng = np.random.default_rng(seed)
    if workload == 1:
        lengths = np.array([128, 4096, 512, 2048], dtype=np.int64)
        return lengths if num_seqs is None else lengths[:num_seqs]
    if workload == 2:
        n = 64 if num_seqs is None else num_seqs
        u = rng.uniform(0.0, math.log(4097.0), size=n)
        return np.clip(np.floor(np.exp(u)), 1, 4096).astype(np.int64)
    if workload in (3, 6, 7, 9):
        n = 1152 if num_seqs is None else num_seqs
        x = rng.normal(math.log(600.0), 1.0, size=n)
        return np.clip(np.rint(np.exp(x)), 1, 4000).astype(np.int64)
    if workload == 4:
        n = 16 if num_seqs is None else num_seqs
        return np.full(n, 4096, dtype=np.int64)
    if workload in (5, 8):
        n = 1152 if num_seqs is None else num_seqs
        return (64 * rng.integers(1, 64, size=n)).astype(np.int64)
    raise ValueError(f"unknown workload {workload}")


def pack_offsets(lengths):
    """Offsets input array [B+1] (int64 numpy) for the given lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([np.zeros(1, dtype=np.int64), np.cumsum(lengths)])


def make_problem(lengths, num_heads, head_dim, mode=MODE_SELF, num_q=0, seed=0,
                 device="cpu", with_grad=True, num_kv_heads=None):
    """Draw q, k, v (and dO) for the given lengths.

    Returns a dict with torch bf16 tensors ``q`` ([T,H,D], or [Mq,H,D] in broadcast-Q
    mode), ``k``, ``v`` ([T,Hkv,D], Hkv = ``num_kv_heads`` or H), ``do`` (shape of o:
    [T,H,D] or [B,Mq,H,D]),
    ``offsets`` (int32 tensor on ``device``), ``offsets_host`` (int32 numpy),
    ``lengths``, and the problem sizes.  ``scale`` is 1/sqrt(D)."""
    import torch

    lengths = np.asarray(lengths, dtype=np.int64)
    offsets = pack_offsets(lengths)
    total = int(offsets[-1])
    nb = len(lengths)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))

    def draw(*shape):
        x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
        return x.to(torch.bfloat16)

    if mode == MODE_BROADCAST_Q:
        q = draw(num_q, num_heads, head_dim)
    else:
        q = draw(total, num_heads, head_dim)
    hkv = num_heads if num_kv_heads is None else int(num_kv_heads)
    k = draw(total, hkv, head_dim)
    v = draw(total, hkv, head_dim)
    do = None
    if with_grad:
        if mode == MODE_BROADCAST_Q:
            do = draw(nb, num_q, num_heads, head_dim)
        else:
            do = draw(total, num_heads, head_dim)
    return dict(
        q=q, k=k, v=v, do=do,
        offsets=torch.as_tensor(offsets.astype(np.int32), device=device),
        offsets_host=offsets.astype(np.int32),
        lengths=lengths, mode=mode, num_heads=num_heads, num_kv_heads=hkv, head_dim=head_dim,
        num_q=num_q, num_seqs=nb, total_tokens=total, scale=1.0 / math.sqrt(head_dim),
    )


def make_workload(workload, seed=0, device="cpu", num_seqs=None, with_grad=True):
    """Problem for a numbered workload (see the module docstring)."""
    w = WORKLOADS[workload]
    lengths = workload_lengths(workload, seed, num_seqs)
    p = make_problem(lengths, w["num_heads"], w["head_dim"], w["mode"], w["num_q"], seed,
                     device, with_grad and not w.get("fwd_only", False), w.get("num_kv_heads"))
    p["workload"] = workload
    p["workload_name"] = w["name"]
    return p
