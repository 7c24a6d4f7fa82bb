"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every
symbol include/jfa.h declares, rejects bad arguments before any device work, and its
tile schedules equal the specification in oracle/schedule.py bit for bit."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import schedule as spec
from variable_length_flash_jagged_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# Tests that pass fabricated (never dereferenced) device addresses rely on a host-side
# check failing before any launch; they run only where no GPU is visible, so that a
# check moved behind a launch can never send a kernel to a bogus address.
def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fabricated device addresses: host-only test")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "jfa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(jfa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"jfa_fwd", "jfa_bwd", "jfa_workspace_size", "jfa_schedule", "jfa_error_string",
            "jfa_last_error_detail", "jfa_version"} <= set(names)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.jfa_version() == 160


def test_error_strings():
    lib = B.lib()
    for code in range(0, -12, -1):
        assert lib.jfa_error_string(code)
    assert b"unknown" in lib.jfa_error_string(-99)


@pytest.mark.parametrize("kw,mode,code", [
    (dict(num_seqs=-1), 0, -2),
    (dict(num_heads=0), 0, -2),
    (dict(head_dim=96), 0, -3),
    (dict(), 7, -4),
    (dict(num_q=0), 1, -2),
    (dict(total_tokens=1 << 31), 0, -9),
])
def test_workspace_size_rejects_bad_shapes(kw, mode, code):
    args = dict(num_seqs=2, num_heads=2, head_dim=64, total_tokens=10, num_q=4)
    args.update(kw)
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(B.make_shape(**args), mode, 0)
    assert e.value.code == code


@pytest.mark.parametrize("hkv,code", [(0, 0), (1, 0), (2, 0), (4, 0), (3, -2), (5, -2), (-1, -2)])
def test_kv_heads_must_divide_query_heads(hkv, code):
    shape = B.make_shape(2, 4, 64, 10, num_kv_heads=hkv)
    if code == 0:
        assert B.workspace_size(shape, 0, 0) > 0
    else:
        with pytest.raises(B.JfaError) as e:
            B.workspace_size(shape, 0, 0)
        assert e.value.code == code
    bad = B.make_shape(2, 4, 64, 10)
    bad.reserved = 1
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(bad, 0, 0)
    assert e.value.code == -2


@no_gpu_only
def test_backward_refuses_grouped_query_heads_before_device_work():
    lib = B.lib()
    shape = B.make_shape(1, 4, 64, 4, num_kv_heads=2)
    off = np.array([0, 4], dtype=np.int32)
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the check fails first
    lse = ctypes.c_void_p(1 << 20)
    rc = lib.jfa_bwd(ctypes.byref(shape), 0, 0.125, fake, fake, fake, fake, fake, lse, fake, off.ctypes.data,
                     fake, fake, fake, fake, 1 << 30, None, None)
    assert rc == -2
    assert b"num_kv_heads" in lib.jfa_last_error_detail()
    # a call refused before choosing a backward path reports none
    assert B.last_bwd_path() == B.BWD_PATH_OTHER


@pytest.mark.parametrize("lengths", [[0], [1], [300, 0, 65], [4000, 600, 64]])
@pytest.mark.parametrize("ratio", [1.0, 0.5, 0.25, 0.3])
def test_block_sparse_entries_formula(lengths, ratio):
    import math
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), 3, 128, int(off[-1]))
    want = 0
    for n in lengths:
        if n:
            nkb = -(-n // 64)
            want += 3 * (-(-n // 256)) * max(1, math.ceil(float(np.float32(ratio)) * nkb))
    assert B.block_sparse_entries(shape, off, ratio) == want


def test_block_sparse_argument_errors():
    off = np.array([0, 300], dtype=np.int32)
    shape = B.make_shape(1, 2, 64, 300)
    for bad in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(B.JfaError) as e:
            B.block_sparse_entries(shape, off, bad)
        assert e.value.code == -8
    big = np.array([0, 64 * 2048 + 1], dtype=np.int32)  # 2049 key blocks
    with pytest.raises(B.JfaError) as e:
        B.block_sparse_entries(B.make_shape(1, 1, 64, int(big[-1])), big, 0.5)
    assert e.value.code == -9
    assert B.block_sparse_entries(B.make_shape(1, 1, 64, 64 * 2048), np.array([0, 64 * 2048], np.int32), 0.5) > 0
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(shape, 2, B.PASS_FWD_SPARSE)  # self mode only
    assert e.value.code == -4
    # the sparse forward's workspace holds at least the block means of q and k
    assert B.workspace_size(shape, 0, B.PASS_FWD_SPARSE) >= 2 * (300 // 64 + 2) * 2 * 64 * 4


def test_bad_options_and_pass():
    shape = B.make_shape(2, 2, 64, 10)
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(shape, 0, 0, B.make_opts(sched=3))
    assert e.value.code == -8
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(shape, 0, 5)   # passes 0 .. 4
    assert e.value.code == -4


@pytest.mark.parametrize("off,code", [([1, 4, 10], -5), ([0, 6, 4], -5), ([0, 4, 9], -5)])
def test_schedule_rejects_bad_offsets(off, code):
    with pytest.raises(B.JfaError) as e:
        B.schedule(B.make_shape(2, 1, 64, 10), 0, 0, off)
    assert e.value.code == code


def test_fwd_rejects_null_pointers_before_any_device_work():
    lib = B.lib()
    shape = B.make_shape(1, 1, 64, 4)
    off = np.array([0, 4], dtype=np.int32)
    rc = lib.jfa_fwd(ctypes.byref(shape), 0, 0.125, None, None, None, None, off.ctypes.data, None, None, None, 0,
                     None, None)
    assert rc == -1
    assert b"non-NULL" in lib.jfa_last_error_detail()


def test_ds_budget_option_range():
    shape = B.make_shape(2, 2, 64, 10)
    for bad in (-1, (1 << 20) + 1):
        with pytest.raises(B.JfaError) as e:
            B.workspace_size(shape, 0, 1, B.make_opts(ds_budget_mib=bad))
        assert e.value.code == -8
    # the budget is added to the self-mode backward's workspace only
    base = B.workspace_size(shape, 0, 1)
    assert B.workspace_size(shape, 0, 1, B.make_opts(ds_budget_mib=3)) >= base + 3 * (1 << 20)
    assert B.workspace_size(shape, 0, 0, B.make_opts(ds_budget_mib=3)) == B.workspace_size(shape, 0, 0)
    assert B.workspace_size(shape, 2, 1, B.make_opts(ds_budget_mib=3)) == B.workspace_size(shape, 2, 1)


@pytest.mark.parametrize("lengths", [[0], [1], [64, 65, 128, 129], [600, 4000, 1, 0, 257]])
@pytest.mark.parametrize("heads", [1, 4])
def test_ds_bytes_formula(lengths, heads):
    # dS of every (query, key) pair per head in bf16, keys padded to 128, queries to 64
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), heads, 128, int(off[-1]))
    want = sum(heads * (-(-n // 128) * 128) * (-(-n // 64) * 64) * 2 for n in lengths)
    assert B.ds_bytes(shape, off) == want
    assert B.ds_budget_mib(shape, off) == max(1, -(-want // (1 << 20)))
    with pytest.raises(B.JfaError) as e:
        B.ds_bytes(shape, off + 1)
    assert e.value.code == -5


def test_workspace_sizes():
    # a function of (B, H, D, Mq, T) and the options only, never of B * max L
    s = B.make_shape(3, 4, 128, 100000)
    self_ws = B.workspace_size(s, 0, 1, B.make_opts(num_programs=64))
    assert self_ws < 100000 * 4 * 128  # self backward keeps no dQ accumulator
    bq = B.make_shape(3, 4, 128, 100000, num_q=256)
    assert B.workspace_size(bq, 1, 1, B.make_opts(num_programs=64)) >= 256 * 4 * 128 * 4
    assert B.workspace_size(bq, 1, 1, B.make_opts(dq_path=1, num_programs=64)) >= 64 * 256 * 128 * 4
    # split path: per-sequence fp32 dQ slabs [B, Mq, H, D] and row terms [B, H, Mq, 8] bf16
    assert B.workspace_size(bq, 1, 1, B.make_opts(dq_path=2, num_programs=64)) >= 3 * 256 * 4 * 128 * 4 + 3 * 4 * 256 * 16
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(bq, 1, 1, B.make_opts(dq_path=3))
    assert "dq_path" in str(e.value)


def _lengths(rng, n, hi):
    x = rng.integers(0, hi, size=n)
    x[rng.random(n) < 0.15] = 0
    x[rng.random(n) < 0.15] = 1
    return x


def _to_lists(tiles, seg):
    return [tuple(int(v) for v in t) for t in tiles], [int(v) for v in seg]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("pass_", [0, 1])
@pytest.mark.parametrize("sched", [0, 1])
def test_schedule_matches_spec_bit_exactly(seed, mode, pass_, sched):
    rng = np.random.default_rng(seed * 7 + mode)
    lengths = _lengths(rng, int(rng.integers(1, 60)), 700)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    h, mq = int(rng.integers(1, 5)), int(rng.integers(1, 300))
    nprog = int(rng.integers(1, 90))
    shape = B.make_shape(len(lengths), h, 128, int(off[-1]), mq)
    opts = B.make_opts(sched=sched, num_programs=nprog)
    tiles, seg, progs, rows = B.schedule(shape, mode, pass_, off, opts)
    got_t, got_s = _to_lists(tiles, seg)
    lens = lengths.tolist()
    if mode == 2:
        want = spec.blockdiag_schedule(lens, h, nprog, 64, min_tiles=4)  # workgroups of four waves
        assert rows == 64
    elif pass_ == 0:
        want = spec.fwd_schedule(lens, h, mode, mq, rows, nprog, dynamic=bool(sched))
    else:
        want = spec.bwd_schedule(lens, h, mode, rows, nprog, dynamic=bool(sched))
    assert got_t == [tuple(t) for t in want[0]]
    assert got_s == list(want[1])
    assert progs == want[2]


def test_schedule_tile_rows():
    off = np.array([0, 300], dtype=np.int32)
    shape = B.make_shape(1, 1, 128, 300)
    assert B.schedule(shape, 0, 0, off)[3] == 256
    assert B.schedule(shape, 0, 1, off)[3] == 128
    assert B.schedule(shape, 2, 0, off)[3] == 64


def test_block_sparse_backward_workspace_size():
    lengths = [300, 0, 65, 4000]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), 3, 128, int(off[-1]))
    base = B.workspace_size(shape, 0, B.PASS_BWD)
    words = sum(3 * (-(-n // 128)) * 2 * (-(-(-(-n // 256)) // 32)) for n in lengths)
    got = B.bwd_block_sparse_workspace_size(shape, off)
    # + the per-sequence arrays and the dK/dV schedule (64-key tiles at head_dim 128:
    # 8 bytes per tile, at most H (T/64 + B + 1) tiles, and a segment array)
    tiles = 3 * (int(off[-1]) // 64 + len(lengths) + 1)
    assert base + 4 * words + 8 * tiles <= got <= base + 4 * words + 8 * tiles + 6 * 256 + 3 * 8 * (len(lengths) + 1) \
        + 4 * 4096
    # the dS budget does not enlarge it (the block-sparse backward recomputes dS)
    assert B.bwd_block_sparse_workspace_size(shape, off, B.make_opts(ds_budget_mib=64)) == got
    with pytest.raises(B.JfaError) as e:
        B.bwd_block_sparse_workspace_size(shape, np.array([0, 300, 300, 365, 4364], np.int32))
    assert e.value.code == -5


def _sparse_bwd_rc(shape, off, ratio=0.5, entries=1 << 20, ws_bytes=1 << 40, ptr=1 << 20):
    lib = B.lib()
    p = ctypes.c_void_p(ptr)
    return lib.jfa_bwd_block_sparse(ctypes.byref(shape), 0.125, ratio, p, p, p, p, p, p, p, off.ctypes.data, p,
                                    entries, p, p, p, p, ws_bytes, None, None)


@no_gpu_only
def test_block_sparse_backward_argument_errors_before_device_work():
    off = np.array([0, 300], dtype=np.int32)
    shape = B.make_shape(1, 2, 64, 300)
    assert _sparse_bwd_rc(B.make_shape(1, 4, 64, 300, num_kv_heads=2), off) == -2
    assert _sparse_bwd_rc(shape, off, ptr=0) == -1
    assert _sparse_bwd_rc(shape, off, ptr=(1 << 20) + 2) == -6
    for bad in (0.0, 1.5, float("nan")):
        assert _sparse_bwd_rc(shape, off, ratio=bad) == -8
    need = B.block_sparse_entries(shape, off, 0.5)
    assert _sparse_bwd_rc(shape, off, entries=need - 1) == -11
    ws = B.bwd_block_sparse_workspace_size(shape, off)
    assert _sparse_bwd_rc(shape, off, ws_bytes=ws - 1) == -7
    assert _sparse_bwd_rc(shape, np.array([0, 299], np.int32)) == -5


def _rotary_rc(fn, shape, mode, off, rows, ptr=1 << 20):
    lib = B.lib()
    p = ctypes.c_void_p(ptr)
    if fn == "fwd":
        return lib.jfa_fwd_rotary(ctypes.byref(shape), mode, 0.125, p, p, p, p, rows, p, off.ctypes.data, p, p, p,
                                  1 << 40, None, None)
    return lib.jfa_bwd_rotary(ctypes.byref(shape), mode, 0.125, p, p, p, p, p, p, p, rows, p, off.ctypes.data, p, p,
                              p, p, 1 << 40, None, None)


@no_gpu_only
@pytest.mark.parametrize("fn", ["fwd", "bwd"])
def test_rotary_argument_errors_before_device_work(fn):
    off = np.array([0, 300, 364], dtype=np.int32)
    shape = B.make_shape(2, 2, 64, 364)
    assert _rotary_rc(fn, shape, 0, off, 300) == -4          # self mode: not built
    assert _rotary_rc(fn, shape, 2, off, 299) == -2          # table shorter than the longest sequence
    assert b"rope_positions" in B.lib().jfa_last_error_detail()
    assert _rotary_rc(fn, shape, 2, off, 300, ptr=0) == -1   # NULL table (and tensors)
    assert _rotary_rc(fn, shape, 2, off, 300, ptr=(1 << 20) + 4) == -6


def test_rope_table_argument_errors():
    lib = B.lib()
    assert lib.jfa_rope_table(None, 5, 64, 10000.0, None) == -1
    p = ctypes.c_void_p(1 << 20)  # rejected before use
    assert lib.jfa_rope_table(p, 5, 32, 10000.0, None) == -3
    assert lib.jfa_rope_table(p, -1, 64, 10000.0, None) == -2
    assert lib.jfa_rope_table(p, 5, 64, 1.0, None) == -8


@no_gpu_only
def test_mxfp8_v_tokens_and_argument_errors():
    lengths = [300, 0, 64, 65, 1]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), 2, 128, int(off[-1]))
    assert B.mxfp8_v_tokens(shape, off) == 320 + 0 + 64 + 128 + 64
    with pytest.raises(B.JfaError) as e:
        B.mxfp8_v_tokens(B.make_shape(len(lengths), 4, 128, int(off[-1]), num_kv_heads=2), off)
    assert e.value.code == -2
    assert B.workspace_size(shape, 0, B.PASS_FWD_MXFP8) > 0
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(shape, 2, B.PASS_FWD_MXFP8)   # self mode only
    assert e.value.code == -4
    lib = B.lib()
    p = ctypes.c_void_p(1 << 20)
    rc = lib.jfa_fwd_mxfp8(ctypes.byref(shape), 0.1, p, p, p, p, p, p, 575, p, off.ctypes.data, p, p, p, 1 << 40,
                           None, None)
    assert rc == -2 and b"v_tokens" in lib.jfa_last_error_detail()   # 575 != 576
    rc = lib.jfa_fwd_mxfp8(ctypes.byref(shape), 0.1, p, p, p, p, p, p, 576, p, off.ctypes.data, p, p, p, 16,
                           None, None)
    assert rc == -7                                                    # workspace too small


@pytest.mark.parametrize("sched", [0, 1])
def test_broadcast_q_forward_key_chunks_match_spec(sched):
    # long sequences among short ones with many programs: the forward cuts keys into chunks
    lengths = [4096, 10, 0, 700, 300, 2000]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), 4, 128, int(off[-1]), 256)
    tiles, seg, progs, rows = B.schedule(shape, 1, 0, off, B.make_opts(sched=sched, num_programs=256))
    chunks = spec.bq_key_chunks(lengths, 4, 256, rows, 256)
    assert len(chunks) > len(lengths)  # some sequence is cut
    want = spec.fwd_schedule(lengths, 4, 1, 256, rows, 256, dynamic=bool(sched))
    got_t, got_s = _to_lists(tiles, seg)
    assert got_t == [tuple(t) for t in want[0]] and got_s == list(want[1]) and progs == want[2]


@no_gpu_only
def test_mxfp8_backward_argument_errors_before_device_work():
    lengths = [300, 0, 64, 65, 1]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), 2, 128, int(off[-1]))
    t = int(off[-1])
    ws = B.workspace_size(shape, 0, B.PASS_BWD_MXFP8)
    # the three decoded tensors plus the self-attention backward's workspace
    assert ws >= 3 * t * 2 * 128 * 2 + B.workspace_size(shape, 0, B.PASS_BWD)
    with pytest.raises(B.JfaError) as e:
        B.workspace_size(shape, 2, B.PASS_BWD_MXFP8)   # self mode only
    assert e.value.code == -4
    lib = B.lib()
    p = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every check fails first
    args = lambda tokens, ws_bytes, dq=p: (ctypes.byref(shape), 0.1, p, p, p, p, p, p, tokens, p, p, p, p,
                                           off.ctypes.data, dq, p, p, p, ws_bytes, None, None)
    assert lib.jfa_bwd_mxfp8(*args(575, 1 << 40)) == -2 and b"v_tokens" in lib.jfa_last_error_detail()
    assert lib.jfa_bwd_mxfp8(*args(576, 16)) == -7                    # workspace too small
    assert lib.jfa_bwd_mxfp8(*args(576, 1 << 40, None)) == -1         # dq is NULL


@pytest.mark.parametrize("sched", [0, 1])
@pytest.mark.parametrize("heads", [1, 3])
def test_self_forward_key_chunks_match_spec(sched, heads):
    # few long sequences and many programs: the self-attention forward cuts keys
    lengths = [128, 4096, 512, 2048, 0]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), heads, 64, int(off[-1]))
    tiles, seg, progs, rows = B.schedule(shape, 0, 0, off, B.make_opts(sched=sched, num_programs=256))
    assert spec.self_chunks_cut(lengths, heads, rows, 256)
    want = spec.fwd_schedule(lengths, heads, 0, 0, rows, 256, dynamic=bool(sched))
    got_t, got_s = _to_lists(tiles, seg)
    assert got_t == [tuple(t) for t in want[0]] and got_s == list(want[1]) and progs == want[2]


def test_self_forward_workspace_holds_key_chunk_partials():
    # 2 * 256 rows * P row-heads of fp32 partial O (D floats) and lse
    s = B.make_shape(4, 1, 64, 6784)
    ws = B.workspace_size(s, 0, 0, B.make_opts(num_programs=256))
    assert ws >= 2 * 256 * 256 * (64 + 1) * 4


@no_gpu_only
def test_tile_visit_counts_capacity_checked_before_device_work():
    lib = B.lib()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the capacity check fails first
    lengths = [300, 65, 1]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), 2, 128, int(off[-1]))
    assert lib.jfa_debug_tile_visits(fake, 0) == -8
    assert lib.jfa_debug_tile_visits(fake, 1) == 0
    try:
        rc = lib.jfa_fwd(ctypes.byref(shape), 0, 0.1, fake, fake, fake, fake, off.ctypes.data, fake, fake, fake,
                         1 << 30, None, None)
        assert rc == -11 and b"tile-visit" in lib.jfa_last_error_detail()
        n = ctypes.c_int64(-1)
        assert lib.jfa_debug_tile_list_size(0, ctypes.byref(n)) == 0 and n.value == 2 * 4  # 2 heads x (2 + 1 + 1) 256-row tiles
        assert lib.jfa_debug_tile_list_size(1, ctypes.byref(n)) == 0 and n.value == 0
    finally:
        assert lib.jfa_debug_tile_visits(None, 0) == 0
    assert lib.jfa_debug_tile_list_size(3, ctypes.byref(ctypes.c_int64())) == -4


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("dq_path", [0, 1, 2])
def test_broadcast_q_backward_schedule_default_programs_match_the_call(head_dim, dq_path):
    # num_programs = 0: jfa_schedule sizes the broadcast-Q backward schedule with the
    # workgroups per CU of the kernel jfa_bwd runs for this dq_path and head dim
    lengths = [700, 5, 0, 300, 64]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = B.make_shape(len(lengths), 2, head_dim, int(off[-1]), 100)
    _, _, progs, _ = B.schedule(shape, 1, 1, off, B.make_opts(dq_path=dq_path))
    cus = 256  # the host-only fallback when no device is visible
    per_cu = (2 if head_dim == 64 else 1) if dq_path == 2 else 1
    want = spec.bwd_schedule(lengths, 2, 1, 128, cus * per_cu)[2]
    if not _gpu_visible():
        assert progs == want
