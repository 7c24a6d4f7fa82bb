"""ctypes binding over libjfa.so (argument marshalling only).

Every function here forwards torch tensors' device pointers and the current HIP stream
to the C ABI declared in include/jfa.h; all of the attention work runs in the
library's kernels.  A missing library raises immediately: there is no fallback.
"""

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# JFA_LIBRARY names another build of the same library (e.g. the host-sanitizer build the
# CPU tests make); by default the in-tree libjfa.so.
LIB_PATH = os.environ.get("JFA_LIBRARY") or os.path.join(PKG, "libjfa.so")

MODE_SELF = 0
MODE_BROADCAST_Q = 1
MODE_BLOCK_DIAG = 2
PASS_FWD = 0
PASS_BWD = 1
PASS_FWD_SPARSE = 2
PASS_FWD_MXFP8 = 3
PASS_BWD_MXFP8 = 4
KERNEL_FWD = 0
KERNEL_BWD = 1
KERNEL_BWD_DQ = 2
KERNEL_BWD_PREP = 3
KERNEL_SPARSE_SELECT = 4
KERNEL_MX_QUANT = 5
BWD_PATH_OTHER = 0
BWD_PATH_RECOMPUTE = 1
BWD_PATH_RECOMPUTE_SIDE = 2
BWD_PATH_STORED_DS = 3
BWD_PATH_NAMES = {BWD_PATH_OTHER: "other", BWD_PATH_RECOMPUTE: "recompute", BWD_PATH_RECOMPUTE_SIDE: "recompute, dQ beside dK/dV",
                  BWD_PATH_STORED_DS: "stored dS"}


class JfaError(RuntimeError):
    def __init__(self, code, func, detail):
        super().__init__(f"{func} failed with {code}: {detail}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_q", ctypes.c_int32), ("total_tokens", ctypes.c_int64), ("num_kv_heads", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Opts(ctypes.Structure):
    _fields_ = [("sched", ctypes.c_int32), ("dq_path", ctypes.c_int32), ("num_programs", ctypes.c_int32),
                ("ds_budget_mib", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m variable_length_flash_jagged_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sp, op = ctypes.POINTER(Shape), ctypes.POINTER(Opts)
        i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        L.jfa_version.restype = ctypes.c_int
        L.jfa_error_string.restype = ctypes.c_char_p
        L.jfa_error_string.argtypes = [ctypes.c_int]
        L.jfa_last_error_detail.restype = ctypes.c_char_p
        L.jfa_workspace_size.restype = ctypes.c_int
        L.jfa_workspace_size.argtypes = [sp, ctypes.c_int, ctypes.c_int, op, ctypes.POINTER(ctypes.c_size_t)]
        L.jfa_fwd.restype = ctypes.c_int
        L.jfa_fwd.argtypes = [sp, ctypes.c_int, f32, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, op, vp]
        L.jfa_fwd_noalloc.restype = ctypes.c_int
        L.jfa_fwd_noalloc.argtypes = [sp, ctypes.c_int, f32, vp, vp, vp, vp, vp, vp, vp, op, vp]
        L.jfa_bwd.restype = ctypes.c_int
        L.jfa_bwd.argtypes = [sp, ctypes.c_int, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                              ctypes.c_size_t, op, vp]
        L.jfa_kernel_timing.restype = ctypes.c_int
        L.jfa_kernel_timing.argtypes = [ctypes.c_int]
        L.jfa_kernel_times.restype = ctypes.c_int
        L.jfa_kernel_times.argtypes = [ctypes.c_int, i64p, ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        L.jfa_debug_tile_visits.restype = ctypes.c_int
        L.jfa_debug_tile_visits.argtypes = [vp, i64]
        L.jfa_debug_tile_list_size.restype = ctypes.c_int
        L.jfa_debug_tile_list_size.argtypes = [ctypes.c_int, i64p]
        L.jfa_block_sparse_entries.restype = ctypes.c_int
        L.jfa_block_sparse_entries.argtypes = [sp, vp, f32, i64p]
        L.jfa_fwd_block_sparse.restype = ctypes.c_int
        L.jfa_fwd_block_sparse.argtypes = [sp, f32, f32, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, ctypes.c_size_t,
                                           op, vp]
        L.jfa_bwd_block_sparse_workspace_size.restype = ctypes.c_int
        L.jfa_bwd_block_sparse_workspace_size.argtypes = [sp, vp, op, ctypes.POINTER(ctypes.c_size_t)]
        L.jfa_bwd_block_sparse.restype = ctypes.c_int
        L.jfa_bwd_block_sparse.argtypes = [sp, f32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp,
                                           ctypes.c_size_t, op, vp]
        L.jfa_fwd_rotary.restype = ctypes.c_int
        L.jfa_fwd_rotary.argtypes = [sp, ctypes.c_int, f32, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, op, vp]
        L.jfa_bwd_rotary.restype = ctypes.c_int
        L.jfa_bwd_rotary.argtypes = [sp, ctypes.c_int, f32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp,
                                     vp, vp, vp, ctypes.c_size_t, op, vp]
        L.jfa_rope_table.restype = ctypes.c_int
        L.jfa_rope_table.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, f32, vp]
        L.jfa_mxfp8_v_tokens.restype = ctypes.c_int
        L.jfa_mxfp8_v_tokens.argtypes = [sp, vp, i64p]
        L.jfa_mxfp8_quantize_qk.restype = ctypes.c_int
        L.jfa_mxfp8_quantize_qk.argtypes = [sp, vp, vp, vp, vp]
        L.jfa_mxfp8_quantize_v.restype = ctypes.c_int
        L.jfa_mxfp8_quantize_v.argtypes = [sp, vp, vp, vp, vp, vp, i64, vp, ctypes.c_size_t, vp]
        L.jfa_fwd_mxfp8.restype = ctypes.c_int
        L.jfa_fwd_mxfp8.argtypes = [sp, f32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, ctypes.c_size_t, op, vp]
        L.jfa_bwd_mxfp8.restype = ctypes.c_int
        L.jfa_bwd_mxfp8.argtypes = [sp, f32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, ctypes.c_size_t, op, vp]
        L.jfa_ds_bytes.restype = ctypes.c_int
        L.jfa_ds_bytes.argtypes = [sp, vp, ctypes.POINTER(ctypes.c_size_t)]
        L.jfa_schedule.restype = ctypes.c_int
        L.jfa_schedule.argtypes = [sp, ctypes.c_int, ctypes.c_int, vp, op, vp, i64, vp, i64, i64p, i32p, i32p, i32p]
        _lib = L
    return _lib


def _check(rc, func):
    if rc != 0:
        L = lib()
        detail = L.jfa_last_error_detail().decode() or L.jfa_error_string(rc).decode()
        raise JfaError(rc, func, detail)


def make_shape(num_seqs, num_heads, head_dim, total_tokens, num_q=0, num_kv_heads=0):
    return Shape(int(num_seqs), int(num_heads), int(head_dim), int(num_q), int(total_tokens), int(num_kv_heads), 0)


def make_opts(sched=0, dq_path=0, num_programs=0, ds_budget_mib=0):
    return Opts(int(sched), int(dq_path), int(num_programs), int(ds_budget_mib))


def workspace_size(shape, mode, pass_, opts=None):
    n = ctypes.c_size_t(0)
    _check(lib().jfa_workspace_size(ctypes.byref(shape), mode, pass_, ctypes.byref(opts) if opts else None,
                                    ctypes.byref(n)), "jfa_workspace_size")
    return int(n.value)


def ds_bytes(shape, offsets_host):
    """Bytes of dS storage the stored-dS self-attention backward needs (jfa_ds_bytes)."""
    off = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    n = ctypes.c_size_t(0)
    _check(lib().jfa_ds_bytes(ctypes.byref(shape), off.ctypes.data, ctypes.byref(n)), "jfa_ds_bytes")
    return int(n.value)


def ds_budget_mib(shape, offsets_host):
    """Smallest ds_budget_mib that selects the stored-dS path for these lengths."""
    return max(1, -(-ds_bytes(shape, offsets_host) // (1 << 20)))


def bench_opts(mode, shape, offsets_host, sched=1, dq_path=2, self_bwd="auto"):
    """Options the benchmark runs with: the given schedule (default: one run-time tile
    counter per XCD, measured faster and with fewer HBM fetches than the static deal) and
    broadcast-Q dQ path (default 2, the fastest) and, for self attention, the backward
    path: "stored" grants
    the dS workspace (stored-dS backward), "recompute" does not, "auto" takes the
    stored-dS backward at head_dim 128 (measured faster there) and the recompute
    backward at 64."""
    if self_bwd not in ("auto", "stored", "recompute"):
        raise ValueError(f"self_bwd must be auto, stored or recompute, got {self_bwd!r}")
    stored = self_bwd == "stored" or (self_bwd == "auto" and shape.head_dim == 128)
    budget = ds_budget_mib(shape, offsets_host) if (stored and mode == MODE_SELF) else 0
    return make_opts(sched=sched, dq_path=dq_path, ds_budget_mib=budget)


def schedule(shape, mode, pass_, offsets_host, opts=None):
    """Host tile schedule: (tiles [N,3] int32, seg_ptr int32, programs, tile_rows)."""
    off = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    L = lib()
    n_tiles, n_segs = ctypes.c_int64(0), ctypes.c_int32(0)
    n_prog, rows = ctypes.c_int32(0), ctypes.c_int32(0)
    o = ctypes.byref(opts) if opts else None
    _check(L.jfa_schedule(ctypes.byref(shape), mode, pass_, off.ctypes.data, o, None, 0, None, 0,
                          ctypes.byref(n_tiles), ctypes.byref(n_segs), ctypes.byref(n_prog), ctypes.byref(rows)),
           "jfa_schedule")
    tiles = np.zeros((max(1, n_tiles.value), 3), dtype=np.int32)
    seg = np.zeros(max(1, n_segs.value), dtype=np.int32)
    _check(L.jfa_schedule(ctypes.byref(shape), mode, pass_, off.ctypes.data, o, tiles.ctypes.data, tiles.shape[0],
                          seg.ctypes.data, seg.shape[0], ctypes.byref(n_tiles), ctypes.byref(n_segs),
                          ctypes.byref(n_prog), ctypes.byref(rows)), "jfa_schedule")
    return tiles[: n_tiles.value], seg[: n_segs.value], n_prog.value, rows.value


def kernel_timing(enable):
    """Turn the library's per-launch kernel event timing on or off (forgets old events)."""
    _check(lib().jfa_kernel_timing(1 if enable else 0), "jfa_kernel_timing")


def kernel_times(kernel, reset=False):
    """(launches, total_ms) of one attention kernel (KERNEL_*) since the last reset."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(lib().jfa_kernel_times(kernel, ctypes.byref(n), ctypes.byref(ms), 1 if reset else 0), "jfa_kernel_times")
    return int(n.value), float(ms.value)


def last_bwd_path():
    """The self-attention backward (BWD_PATH_*) this thread's last jfa_bwd call enqueued."""
    return int(lib().jfa_last_bwd_path())


def debug_tile_visits(counts, stride):
    """Count tile visits into the zeroed device int32 tensor `counts` (3 * stride
    entries; None turns counting off): see jfa_debug_tile_visits."""
    _check(lib().jfa_debug_tile_visits(_ptr(counts) if counts is not None else None, int(stride)),
           "jfa_debug_tile_visits")


def debug_tile_list_size(kernel):
    """Tile-list length of `kernel` (KERNEL_FWD / KERNEL_BWD / KERNEL_BWD_DQ) in the last call."""
    n = ctypes.c_int64(0)
    _check(lib().jfa_debug_tile_list_size(kernel, ctypes.byref(n)), "jfa_debug_tile_list_size")
    return int(n.value)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_tensor(name, t, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _sizes(q, k, v, offsets, mode):
    """(B, H, D, T, Mq, Hkv): query heads from q, key/value heads from k."""
    total, kv_heads, head_dim = k.shape
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v has shape {tuple(v.shape)}, k has {tuple(k.shape)}")
    if q.dim() != 3 or q.shape[2] != head_dim:
        raise ValueError(f"q has shape {tuple(q.shape)}; expected [rows, H, {head_dim}]")
    nb = offsets.numel() - 1
    mq = q.shape[0] if mode == MODE_BROADCAST_Q else 0
    return nb, q.shape[1], head_dim, total, mq, kv_heads


def alloc_workspace(shape, mode, pass_, opts, device):
    import torch
    n = workspace_size(shape, mode, pass_, opts)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def fwd(q, k, v, offsets, offsets_host=None, mode=MODE_SELF, scale=None, opts=None, o=None, lse=None,
        workspace=None, stream=None):
    """Forward.  Returns (o, lse) with the layouts of include/jfa.h."""
    import torch
    nb, h, d, t, mq, hkv = _sizes(q, k, v, offsets, mode)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, x, torch.bfloat16)
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t, mq, hkv if hkv != h else 0)
    if mode == MODE_BROADCAST_Q:
        o_shape, lse_shape = (nb, mq, h, d), (nb, h, mq)
    else:
        o_shape, lse_shape = (t, h, d), (h, t)
    if o is None:
        o = torch.empty(o_shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    _check_tensor("o", o, torch.bfloat16, o_shape)
    _check_tensor("lse", lse, torch.float32, lse_shape)
    if workspace is None:
        workspace = alloc_workspace(shape, mode, PASS_FWD, opts, q.device)
    host = None
    if offsets_host is not None:
        host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_fwd(ctypes.byref(shape), mode, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                         host.ctypes.data if host is not None else None, _ptr(o), _ptr(lse), _ptr(workspace),
                         workspace.numel(), ctypes.byref(opts) if opts else None, _stream(stream)), "jfa_fwd")
    return o, lse


def fwd_noalloc(q, k, v, offsets, offsets_host=None, mode=MODE_SELF, scale=None, opts=None, o=None, lse=None,
                stream=None):
    """Forward through jfa_fwd_noalloc (no workspace argument: the library's device
    scratch array).  Returns (o, lse); o and lse are allocated here when not given."""
    import torch
    nb, h, d, t, mq, hkv = _sizes(q, k, v, offsets, mode)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, x, torch.bfloat16)
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t, mq, hkv if hkv != h else 0)
    if mode == MODE_BROADCAST_Q:
        o_shape, lse_shape = (nb, mq, h, d), (nb, h, mq)
    else:
        o_shape, lse_shape = (t, h, d), (h, t)
    if o is None:
        o = torch.empty(o_shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    _check_tensor("o", o, torch.bfloat16, o_shape)
    _check_tensor("lse", lse, torch.float32, lse_shape)
    host = None
    if offsets_host is not None:
        host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_fwd_noalloc(ctypes.byref(shape), mode, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                                 host.ctypes.data if host is not None else None, _ptr(o), _ptr(lse),
                                 ctypes.byref(opts) if opts else None, _stream(stream)), "jfa_fwd_noalloc")
    return o, lse


def bwd(q, k, v, o, do, lse, offsets, offsets_host=None, mode=MODE_SELF, scale=None, opts=None, dq=None,
        dk=None, dv=None, workspace=None, stream=None):
    """Backward.  Returns (dq, dk, dv) with the shapes of (q, k, v)."""
    import torch
    nb, h, d, t, mq, hkv = _sizes(q, k, v, offsets, mode)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(name, x, torch.bfloat16)
    _check_tensor("lse", lse, torch.float32)
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t, mq, hkv if hkv != h else 0)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = alloc_workspace(shape, mode, PASS_BWD, opts, q.device)
    host = None
    if offsets_host is not None:
        host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_bwd(ctypes.byref(shape), mode, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                         _ptr(offsets), host.ctypes.data if host is not None else None, _ptr(dq), _ptr(dk), _ptr(dv),
                         _ptr(workspace), workspace.numel(), ctypes.byref(opts) if opts else None,
                         _stream(stream)), "jfa_bwd")
    return dq, dk, dv


def block_sparse_entries(shape, offsets_host, ratio):
    """Selection entries jfa_fwd_block_sparse writes for these lengths and ratio."""
    off = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    n = ctypes.c_int64(0)
    _check(lib().jfa_block_sparse_entries(ctypes.byref(shape), off.ctypes.data, float(ratio), ctypes.byref(n)),
           "jfa_block_sparse_entries")
    return int(n.value)


def fwd_block_sparse(q, k, v, offsets, offsets_host, ratio, scale=None, opts=None, o=None, lse=None, selection=None,
                     workspace=None, stream=None):
    """Block-sparse top-k self-attention forward.  Returns (o, lse, selection) with the
    layouts of include/jfa.h (selection: int32 kept key-block lists)."""
    import torch
    nb, h, d, t, _, hkv = _sizes(q, k, v, offsets, MODE_SELF)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, x, torch.bfloat16)
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t, 0, hkv if hkv != h else 0)
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    entries = block_sparse_entries(shape, host, ratio)
    if o is None:
        o = torch.empty((t, h, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((h, t), dtype=torch.float32, device=q.device)
    if selection is None:
        selection = torch.empty(max(entries, 1), dtype=torch.int32, device=q.device)
    _check_tensor("o", o, torch.bfloat16, (t, h, d))
    _check_tensor("lse", lse, torch.float32, (h, t))
    _check_tensor("selection", selection, torch.int32)
    if workspace is None:
        workspace = alloc_workspace(shape, MODE_SELF, PASS_FWD_SPARSE, opts, q.device)
    _check(lib().jfa_fwd_block_sparse(ctypes.byref(shape), scale, float(ratio), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(offsets), host.ctypes.data, _ptr(o), _ptr(lse), _ptr(selection),
                                      selection.numel(), _ptr(workspace), workspace.numel(),
                                      ctypes.byref(opts) if opts else None, _stream(stream)), "jfa_fwd_block_sparse")
    return o, lse, selection


def bwd_block_sparse_workspace_size(shape, offsets_host, opts=None):
    """Workspace bytes jfa_bwd_block_sparse needs for these offsets."""
    out = ctypes.c_size_t()
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_bwd_block_sparse_workspace_size(ctypes.byref(shape), host.ctypes.data,
                                                     ctypes.byref(opts) if opts else None, ctypes.byref(out)),
           "jfa_bwd_block_sparse_workspace_size")
    return out.value


def bwd_block_sparse(q, k, v, o, do, lse, offsets, offsets_host, ratio, selection, scale=None, opts=None, dq=None,
                     dk=None, dv=None, workspace=None, stream=None):
    """Backward of the block-sparse top-k forward for the selection it wrote.  Returns
    (dq, dk, dv) with the shapes of (q, k, v)."""
    import torch
    nb, h, d, t, _, hkv = _sizes(q, k, v, offsets, MODE_SELF)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(name, x, torch.bfloat16)
    _check_tensor("lse", lse, torch.float32, (h, t))
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    _check_tensor("selection", selection, torch.int32)
    shape = make_shape(nb, h, d, t, 0, hkv if hkv != h else 0)
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        n = bwd_block_sparse_workspace_size(shape, host, opts)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    _check(lib().jfa_bwd_block_sparse(ctypes.byref(shape), scale, float(ratio), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(do), _ptr(lse), _ptr(offsets), host.ctypes.data, _ptr(selection),
                                      selection.numel(), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                      workspace.numel(), ctypes.byref(opts) if opts else None, _stream(stream)),
           "jfa_bwd_block_sparse")
    return dq, dk, dv


def rope_table(max_positions, head_dim, base=10000.0, device="cuda", stream=None):
    """The cos / sin table jfa_fwd_rotary takes, built by the library (jfa_rope_table):
    [max_positions, D/2, 2] fp32 on the device."""
    import torch
    t = torch.empty((int(max_positions), head_dim // 2, 2), dtype=torch.float32, device=device)
    _check(lib().jfa_rope_table(_ptr(t), int(max_positions), int(head_dim), float(base), _stream(stream)),
           "jfa_rope_table")
    return t


def fwd_rotary(q, k, v, offsets, offsets_host, rope, scale=None, opts=None, o=None, lse=None, workspace=None,
               stream=None, mode=MODE_BLOCK_DIAG):
    """Block-diagonal forward of rope(q), rope(k), v; rope from rope_table().  Returns (o, lse)."""
    import torch
    nb, h, d, t, _, hkv = _sizes(q, k, v, offsets, mode)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, x, torch.bfloat16)
    _check_tensor("rope", rope, torch.float32)
    if rope.dim() != 3 or rope.shape[1:] != (d // 2, 2):
        raise ValueError(f"rope must be [P, {d // 2}, 2], got {tuple(rope.shape)}")
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t, 0, hkv if hkv != h else 0)
    o = torch.empty((t, h, d), dtype=torch.bfloat16, device=q.device) if o is None else o
    lse = torch.empty((h, t), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("o", o, torch.bfloat16, (t, h, d))
    _check_tensor("lse", lse, torch.float32, (h, t))
    if workspace is None:
        workspace = alloc_workspace(shape, mode, PASS_FWD, opts, q.device)
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_fwd_rotary(ctypes.byref(shape), mode, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(rope),
                                rope.shape[0], _ptr(offsets), host.ctypes.data, _ptr(o), _ptr(lse), _ptr(workspace),
                                workspace.numel(), ctypes.byref(opts) if opts else None, _stream(stream)),
           "jfa_fwd_rotary")
    return o, lse


def bwd_rotary(q, k, v, o, do, lse, offsets, offsets_host, rope, scale=None, opts=None, dq=None, dk=None, dv=None,
               workspace=None, stream=None, mode=MODE_BLOCK_DIAG):
    """Backward of fwd_rotary: gradients with respect to the un-rotated q, k and v."""
    import torch
    nb, h, d, t, _, hkv = _sizes(q, k, v, offsets, mode)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(name, x, torch.bfloat16)
    _check_tensor("lse", lse, torch.float32, (h, t))
    _check_tensor("rope", rope, torch.float32)
    if rope.dim() != 3 or rope.shape[1:] != (d // 2, 2):
        raise ValueError(f"rope must be [P, {d // 2}, 2], got {tuple(rope.shape)}")
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t, 0, hkv if hkv != h else 0)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = alloc_workspace(shape, mode, PASS_BWD, opts, q.device)
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_bwd_rotary(ctypes.byref(shape), mode, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                _ptr(lse), _ptr(rope), rope.shape[0], _ptr(offsets), host.ctypes.data, _ptr(dq),
                                _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                ctypes.byref(opts) if opts else None, _stream(stream)), "jfa_bwd_rotary")
    return dq, dk, dv


def mxfp8_v_tokens(shape, offsets_host):
    """Token count of the transposed MXFP8 V layout (sequences padded to 64 keys)."""
    out = ctypes.c_int64()
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_mxfp8_v_tokens(ctypes.byref(shape), host.ctypes.data, ctypes.byref(out)), "jfa_mxfp8_v_tokens")
    return out.value


def mxfp8_quantize_qk(x, stream=None):
    """q or k [T, H, D] bf16 -> (codes uint8 [T, H, D], scales uint8 [T, H, D/32])."""
    import torch
    _check_tensor("x", x, torch.bfloat16)
    t, h, d = x.shape
    shape = make_shape(1, h, d, t)
    codes = torch.empty((t, h, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((t, h, d // 32), dtype=torch.uint8, device=x.device)
    if t:
        _check(lib().jfa_mxfp8_quantize_qk(ctypes.byref(shape), _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)),
               "jfa_mxfp8_quantize_qk")
    return codes, scales


def mxfp8_quantize_v(v, offsets, offsets_host, workspace=None, stream=None):
    """v [T, H, D] bf16 -> (codes uint8 [H, D, Tp], scales uint8 [H, D, Tp/32], Tp)."""
    import torch
    _check_tensor("v", v, torch.bfloat16)
    t, h, d = v.shape
    nb = len(offsets_host) - 1
    shape = make_shape(nb, h, d, t)
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    tp = mxfp8_v_tokens(shape, host)
    codes = torch.empty((h, d, max(tp, 64)), dtype=torch.uint8, device=v.device)
    scales = torch.empty((h, d, max(tp, 64) // 32), dtype=torch.uint8, device=v.device)
    if workspace is None:
        workspace = alloc_workspace(shape, MODE_SELF, PASS_FWD_MXFP8, None, v.device)
    _check(lib().jfa_mxfp8_quantize_v(ctypes.byref(shape), _ptr(v), _ptr(offsets), host.ctypes.data, _ptr(codes),
                                      _ptr(scales), tp, _ptr(workspace), workspace.numel(), _stream(stream)),
           "jfa_mxfp8_quantize_v")
    return codes[:, :, :tp], scales[:, :, :tp // 32], tp


def fwd_mxfp8(q8, q_scales, k8, k_scales, v8t, v_scales, v_tokens, offsets, offsets_host, scale=None, opts=None,
              o=None, lse=None, workspace=None, stream=None):
    """MXFP8 self-attention forward over quantised inputs.  Returns (o bf16 [T, H, D], lse [H, T])."""
    import torch
    t, h, d = q8.shape
    nb = len(offsets_host) - 1
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q8", q8), ("q_scales", q_scales), ("k8", k8), ("k_scales", k_scales), ("v8t", v8t),
                    ("v_scales", v_scales)):
        _check_tensor(name, x, torch.uint8)
    if k8.shape != q8.shape or q_scales.shape != (t, h, d // 32) or k_scales.shape != (t, h, d // 32):
        raise ValueError("q8, k8 [T, H, D] and their scales [T, H, D/32]")
    if v8t.shape != (h, d, v_tokens) or v_scales.shape != (h, d, v_tokens // 32):
        raise ValueError("v8t [H, D, Tp] and v_scales [H, D, Tp/32]")
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t)
    o = torch.empty((t, h, d), dtype=torch.bfloat16, device=q8.device) if o is None else o
    lse = torch.empty((h, t), dtype=torch.float32, device=q8.device) if lse is None else lse
    _check_tensor("o", o, torch.bfloat16, (t, h, d))
    _check_tensor("lse", lse, torch.float32, (h, t))
    if workspace is None:
        workspace = alloc_workspace(shape, MODE_SELF, PASS_FWD_MXFP8, opts, q8.device)
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_fwd_mxfp8(ctypes.byref(shape), scale, _ptr(q8), _ptr(q_scales), _ptr(k8), _ptr(k_scales),
                               _ptr(v8t), _ptr(v_scales), v_tokens, _ptr(offsets), host.ctypes.data, _ptr(o), _ptr(lse),
                               _ptr(workspace), workspace.numel(), ctypes.byref(opts) if opts else None,
                               _stream(stream)), "jfa_fwd_mxfp8")
    return o, lse


def bwd_mxfp8(q8, q_scales, k8, k_scales, v8t, v_scales, v_tokens, o, do, lse, offsets, offsets_host, scale=None,
              opts=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward of the MXFP8 self-attention forward: gradients (dq, dk, dv bf16 [T, H, D])
    with respect to the decoded inputs."""
    import torch
    t, h, d = q8.shape
    nb = len(offsets_host) - 1
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    for name, x in (("q8", q8), ("q_scales", q_scales), ("k8", k8), ("k_scales", k_scales), ("v8t", v8t),
                    ("v_scales", v_scales)):
        _check_tensor(name, x, torch.uint8)
    if k8.shape != q8.shape or q_scales.shape != (t, h, d // 32) or k_scales.shape != (t, h, d // 32):
        raise ValueError("q8, k8 [T, H, D] and their scales [T, H, D/32]")
    if v8t.shape != (h, d, v_tokens) or v_scales.shape != (h, d, v_tokens // 32):
        raise ValueError("v8t [H, D, Tp] and v_scales [H, D, Tp/32]")
    for name, x in (("o", o), ("do", do)):
        _check_tensor(name, x, torch.bfloat16, (t, h, d))
    _check_tensor("lse", lse, torch.float32, (h, t))
    _check_tensor("offsets", offsets, torch.int32, (nb + 1,))
    shape = make_shape(nb, h, d, t)
    dq = torch.empty((t, h, d), dtype=torch.bfloat16, device=q8.device) if dq is None else dq
    dk = torch.empty((t, h, d), dtype=torch.bfloat16, device=q8.device) if dk is None else dk
    dv = torch.empty((t, h, d), dtype=torch.bfloat16, device=q8.device) if dv is None else dv
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, x, torch.bfloat16, (t, h, d))
    if workspace is None:
        workspace = alloc_workspace(shape, MODE_SELF, PASS_BWD_MXFP8, opts, q8.device)
    host = np.ascontiguousarray(np.asarray(offsets_host, dtype=np.int32))
    _check(lib().jfa_bwd_mxfp8(ctypes.byref(shape), scale, _ptr(q8), _ptr(q_scales), _ptr(k8), _ptr(k_scales),
                               _ptr(v8t), _ptr(v_scales), v_tokens, _ptr(o), _ptr(do), _ptr(lse), _ptr(offsets),
                               host.ctypes.data, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                               ctypes.byref(opts) if opts else None, _stream(stream)), "jfa_bwd_mxfp8")
    return dq, dk, dv
