"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on seeded
inputs, at sizes the oracle finishes in seconds: several tiles, ragged tails, empty
and length-1 sequences, both head dims, all three modes, both schedules and both
broadcast-Q dQ paths.  Tolerances are in tests/gpu_helpers.py."""

import numpy as np
import pytest
import torch

from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu

RAGGED = [1, 5, 63, 64, 65, 127, 128, 129, 200, 257]


@pytest.mark.parametrize("head_dim", [64, 128])
def test_self_ragged(head_dim):
    G.run_case(RAGGED, 2, head_dim, label=f"self ragged D{head_dim}")


@pytest.mark.parametrize("head_dim", [64, 128])
def test_self_with_empty_sequences(head_dim):
    G.run_case([0, 33, 0, 70, 0, 300, 0], 3, head_dim, seed=3, label="self empties")


def test_self_dynamic_schedule():
    G.run_case(RAGGED + [511, 2], 2, 128, opts=B.make_opts(sched=1), seed=4, label="self dynamic")


@pytest.mark.parametrize("nprog", [16, 24])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_self_dynamic_per_xcd_counter_groups(nprog, head_dim):
    # nprog a multiple of 8: eight counter groups (one per XCD) of nprog / 8 programs,
    # each serving the tiles the static deal gives its programs, several per program
    lengths = RAGGED + [700, 33, 1, 400]
    G.run_case(lengths, 2, head_dim, opts=B.make_opts(sched=1, num_programs=nprog), seed=61,
               label=f"self xcd groups P{nprog} D{head_dim}")
    G.run_case(lengths, 2, head_dim, opts=_ds_opts(lengths, 2, head_dim, sched=1, num_programs=nprog), seed=62,
               label=f"stored dS xcd groups P{nprog} D{head_dim}")


def test_self_few_programs():
    # many tiles per persistent workgroup
    G.run_case(RAGGED, 2, 128, opts=B.make_opts(num_programs=3), seed=5, label="self 3 programs")


@pytest.mark.parametrize("head_dim", [64, 128])
def test_self_recompute_side_by_side_and_sequential(head_dim):
    """Recompute backward (no dS budget): with few tiles the dQ kernel runs on the
    library's side stream beside the dK/dV kernel, the row terms from the row-term
    kernel; with more tiles than CUs the two kernels run one after the other.  Both
    against the oracle."""
    G.run_case(RAGGED, 2, head_dim, seed=24, label=f"recompute side by side D{head_dim}")
    assert B.last_bwd_path() == B.BWD_PATH_RECOMPUTE_SIDE
    many = [128] * 300 + [5, 0, 77]  # 302 dQ and 302 dK/dV tiles: more than the CUs
    G.run_case(many, 1, head_dim, seed=25, label=f"recompute sequential D{head_dim}")
    assert B.last_bwd_path() == B.BWD_PATH_RECOMPUTE


def _ds_opts(lengths, heads, head_dim, **kw):
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), heads, head_dim, int(off[-1]))
    return B.make_opts(ds_budget_mib=B.ds_budget_mib(shape, off), **kw)


def _ran_stored_ds(fn):
    """Run fn(); True when its last backward call took the stored-dS path."""
    fn()
    return B.last_bwd_path() == B.BWD_PATH_STORED_DS


@pytest.mark.parametrize("head_dim", [64, 128])
def test_self_stored_ds_ragged(head_dim):
    opts = _ds_opts(RAGGED, 2, head_dim)
    assert _ran_stored_ds(lambda: G.run_case(RAGGED, 2, head_dim, opts=opts, seed=21,
                                             label=f"self stored dS D{head_dim}"))


@pytest.mark.parametrize("head_dim", [64, 128])
def test_self_stored_ds_empties_and_long(head_dim):
    lengths = [0, 33, 0, 70, 1, 0, 700, 2, 383, 0]
    G.run_case(lengths, 3, head_dim, opts=_ds_opts(lengths, 3, head_dim), seed=22, label="self stored dS empties")


def test_self_stored_ds_dynamic_and_few_programs():
    lengths = RAGGED + [511, 2]
    G.run_case(lengths, 2, 128, opts=_ds_opts(lengths, 2, 128, sched=1), seed=23, label="stored dS dynamic")
    G.run_case(lengths, 2, 128, opts=_ds_opts(lengths, 2, 128, num_programs=3), seed=24, label="stored dS 3 progs")


def test_self_stored_ds_budget_too_small_falls_back():
    lengths = [2000, 700]
    opts = B.make_opts(ds_budget_mib=1)  # needs 2 * 2048 * 2048 * 2 + ... bytes > 1 MiB
    assert not _ran_stored_ds(lambda: G.run_case(lengths, 2, 128, opts=opts, seed=25, label="budget too small"))


def test_self_stored_ds_and_recompute_paths_on_one_forward():
    """Both backward paths on the same forward outputs.  dV comes from the same dK/dV
    arithmetic on both (bit-identical); dK differs only in the summation order of Di;
    dQ is formed from a bf16 dS on both paths, rounded from P computed in two different
    kernels, so the two dQ agree only to bf16 rounding -- each is checked against the
    oracle."""
    lengths = [130, 1, 640, 64, 257]
    p = W.make_problem(lengths, 2, 128, seed=26, device="cpu")
    g = G.to_gpu(p)
    o, lse = G.gpu_fwd(g)
    a = G.gpu_bwd(g, o, lse)
    b = G.gpu_bwd(g, o, lse, _ds_opts(lengths, 2, 128))
    torch.cuda.synchronize()
    assert torch.equal(a[2], b[2])
    assert G.rel_l2(G.f64(b[1]), G.f64(a[1])) < 1e-3
    refs = G.oracle_bwd(p)
    ea = G.check_bwd(a, refs, "recompute path", p, G.oracle_bwd(p, o))
    eb = G.check_bwd(b, refs, "stored-dS path", p, G.oracle_bwd(p, o))
    print(f"rel-L2 vs oracle: recompute {ea}, stored dS {eb}", flush=True)


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("num_kv_heads", [1, 2])
def test_grouped_query_forward(head_dim, num_kv_heads):
    G.run_case(RAGGED + [511], 4, head_dim, bwd=False, seed=31, num_kv_heads=num_kv_heads,
               label=f"gqa self D{head_dim} Hkv{num_kv_heads}")


def test_grouped_query_forward_broadcast_q_and_block_diag():
    G.run_case([1, 0, 64, 129, 300, 7], 4, 128, W.MODE_BROADCAST_Q, 100, bwd=False, seed=32, num_kv_heads=2,
               label="gqa broadcast-q")
    G.run_case([64, 130, 5, 0, 256, 1, 63], 4, 64, W.MODE_BLOCK_DIAG, bwd=False, seed=33, num_kv_heads=1,
               label="gqa block-diag")
    G.run_case(RAGGED, 6, 128, bwd=False, seed=34, num_kv_heads=3, opts=B.make_opts(sched=1, num_programs=5),
               label="gqa dynamic schedule")


def test_grouped_query_backward_is_refused():
    p = W.make_problem([5, 9], 4, 64, seed=35, device="cpu", num_kv_heads=2)
    g = G.to_gpu(p)
    o, lse = G.gpu_fwd(g)
    with pytest.raises(B.JfaError) as e:
        G.gpu_bwd(g, o, lse)
    assert e.value.code == -2


def test_self_device_offsets_slow_path():
    G.run_case([17, 130, 64], 1, 64, host_offsets=False, seed=6, label="self slow path")


def test_length_one_gives_o_equal_v_bit_exact():
    p = W.make_problem([1, 1, 1], 2, 128, seed=7, device="cpu", with_grad=False)
    g = G.to_gpu(p)
    o, lse = G.gpu_fwd(g)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), p["v"])
    dots = (p["q"].float() * p["k"].float()).sum(-1).T * p["scale"]  # [H, T]
    assert torch.allclose(lse.cpu(), dots, atol=1e-5)


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("num_q", [1, 100, 256])
@pytest.mark.parametrize("dq_path", [0, 1, 2])
def test_broadcast_q(head_dim, num_q, dq_path):
    lengths = [1, 0, 64, 129, 300, 7, 0, 256]
    G.run_case(lengths, 2, head_dim, W.MODE_BROADCAST_Q, num_q, seed=8,
               opts=B.make_opts(dq_path=dq_path), label=f"bq D{head_dim} Mq{num_q} path{dq_path}")


@pytest.mark.parametrize("sched", [0, 1])
@pytest.mark.parametrize("dq_path", [1, 2])
def test_broadcast_q_schedules_and_program_counts(sched, dq_path):
    lengths = [40, 300, 1, 129, 128]
    for nprog in (2, 5, 64):
        G.run_case(lengths, 3, 128, W.MODE_BROADCAST_Q, 70, seed=9,
                   opts=B.make_opts(sched=sched, dq_path=dq_path, num_programs=nprog),
                   label=f"bq sched{sched} path{dq_path} P{nprog}")


@pytest.mark.parametrize("sched", [0, 1])
def test_broadcast_q_split_path_key_chunks(sched):
    # the dQ kernel cuts long sequences into key chunks (one fp32 slab each): a long
    # sequence among short ones, a ragged query tail, chunks with and without a tail
    for nprog in (0, 7):
        G.run_case([2500, 3, 0, 900, 64], 2, 128, W.MODE_BROADCAST_Q, 300, seed=18,
                   opts=B.make_opts(sched=sched, dq_path=2, num_programs=nprog),
                   label=f"bq path2 chunks sched{sched} P{nprog}")


def test_broadcast_q_split_path_many_heads_dynamic():
    # more head groups than the old 64-counter region held (one counter per head group)
    G.run_case([33, 0, 200], 70, 64, W.MODE_BROADCAST_Q, 40, seed=19,
               opts=B.make_opts(sched=1, dq_path=2, num_programs=140), label="bq path2 H70 dynamic")


@pytest.mark.parametrize("dq_path", [1, 2])
def test_broadcast_q_partials_are_run_to_run_identical(dq_path):
    p = W.make_problem([90, 300, 17], 2, 128, W.MODE_BROADCAST_Q, 128, seed=10, device="cpu")
    g = G.to_gpu(p)
    opts = B.make_opts(dq_path=dq_path)
    o, lse = G.gpu_fwd(g, opts)
    a = G.gpu_bwd(g, o, lse, opts)
    b = G.gpu_bwd(g, o, lse, opts)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_block_diag(head_dim):
    G.run_case([64, 130, 5, 0, 256, 1, 63], 3, head_dim, W.MODE_BLOCK_DIAG, seed=11, label=f"bd D{head_dim}")


def test_block_diag_few_programs():
    G.run_case([64 * 5, 64 * 3, 64], 4, 64, W.MODE_BLOCK_DIAG, seed=12, opts=B.make_opts(num_programs=2),
               label="bd 2 programs")


def test_bwd_from_oracle_forward():
    """Feed the backward the oracle's O (rounded to bf16) and lse, isolating its error."""
    p = W.make_problem(RAGGED, 2, 128, seed=13, device="cpu")
    g = G.to_gpu(p)
    o_ref, lse_ref = G.oracle_fwd(p)
    o = torch.from_numpy(o_ref).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(lse_ref).float().cuda()
    grads = G.gpu_bwd(g, o, lse)
    torch.cuda.synchronize()
    G.check_bwd(grads, G.oracle_bwd(p), "bwd from oracle fwd", p, G.oracle_bwd(p, o))


def test_outputs_leave_guard_canaries_untouched():
    p = W.make_problem([70, 5, 200], 2, 64, seed=14, device="cpu")
    g = G.to_gpu(p)
    t, h, d = p["k"].shape
    pad = 4096
    sentinel = -12345.0
    ob = torch.full((t * h * d + 2 * pad,), sentinel, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((t * h + 2 * pad,), sentinel, dtype=torch.float32, device="cuda")
    o = ob[pad:pad + t * h * d].view(t, h, d)
    lse = lb[pad:pad + t * h].view(h, t)
    B.fwd(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"], 0, g["scale"], None, o, lse)
    bufs = [torch.full((t * h * d + 2 * pad,), sentinel, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    views = [b[pad:pad + t * h * d].view(t, h, d) for b in bufs]
    B.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, g["offsets"], g["offsets_host"], 0, g["scale"], None, *views)
    torch.cuda.synchronize()
    for buf in [ob, lb] + bufs:
        assert torch.all(buf[:pad] == sentinel) and torch.all(buf[-pad:] == sentinel)
    G.check_fwd(o, lse, *G.oracle_fwd(p), "canary")


@pytest.mark.parametrize("workload,num_seqs", [(1, None), (2, 16), (3, 24), (4, 2), (5, 24)])
def test_workloads_reduced(workload, num_seqs):
    w = W.WORKLOADS[workload]
    lengths = W.workload_lengths(workload, 0, num_seqs)
    G.run_case(lengths, w["num_heads"], w["head_dim"], w["mode"], w["num_q"], seed=workload,
               label=f"workload {workload} ({w['name']}) reduced")


@pytest.mark.parametrize("seed", range(8))
def test_random_configurations(seed):
    """Seeded random sweep over modes, head dims, head counts, grouped key/value heads,
    schedules, program counts and length mixes (including empty and 1-token sequences
    and lengths around tile edges)."""
    rng = np.random.default_rng(1000 + seed)
    mode = int(rng.integers(0, 3))
    d = int(rng.choice([64, 128]))
    h = int(rng.choice([1, 2, 3, 4]))
    nb = int(rng.integers(1, 9))
    edges = [1, 63, 64, 65, 127, 128, 129, 255, 256, 257]
    lengths = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(0, 700)) for _ in range(nb)]
    if mode == W.MODE_BLOCK_DIAG and rng.random() < 0.5:
        lengths = [64 * int(rng.integers(0, 9)) for _ in range(nb)]
    opts = B.make_opts(sched=int(rng.integers(0, 2)), num_programs=int(rng.choice([0, 1, 3, 17])),
                       dq_path=int(rng.integers(0, 3)))
    num_q = int(rng.integers(1, 300)) if mode == W.MODE_BROADCAST_Q else 0
    hkv = int(rng.choice([x for x in range(1, h + 1) if h % x == 0]))
    gqa = hkv != h and rng.random() < 0.5
    G.run_case(lengths, h, d, mode, num_q, seed=2000 + seed, opts=opts, bwd=not gqa,
               num_kv_heads=hkv if gqa else None,
               label=f"random mode{mode} D{d} H{h} Hkv{hkv if gqa else h} opts=({opts.sched},{opts.num_programs},"
                     f"{opts.dq_path})")
