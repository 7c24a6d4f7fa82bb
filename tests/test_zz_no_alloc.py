"""The allocation-free forward jfa_fwd_noalloc (workspace in the library's device
scratch array) against jfa_fwd (caller's workspace) through the C ABI: two calls in a
row, the second on a smaller input, each within the common tolerances of the fp64
oracle and bit-identical to jfa_fwd on the same inputs (same kernels, same schedule)
-- except where jfa_fwd cuts a self-attention sequence's keys into chunks (few long
sequences, oracle/schedule.py's self_chunks_cut), which jfa_fwd_noalloc never does:
then the two sum the same keys in another grouping and O agrees to one bf16 step.
The size limit is checked on the host before any device work."""

import numpy as np
import pytest
import torch

from oracle import schedule as spec
from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W


def _nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def _one_call(lengths, heads, head_dim, mode, seed, opts, num_q=0):
    print(f"[case] noalloc lengths={lengths[:8]} H={heads} D={head_dim} mode={mode} seed={seed}", flush=True)
    p = W.make_problem(lengths, heads, head_dim, mode, num_q, seed, device="cpu", with_grad=False)
    g = G.to_gpu(p)
    o_ref, lse_ref = G.gpu_fwd(g, opts)
    o_sh, l_sh = tuple(o_ref.shape), tuple(lse_ref.shape)
    o, lse = B.fwd_noalloc(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"], mode, g["scale"], opts,
                           _nan_like(o_sh, torch.bfloat16), _nan_like(l_sh, torch.float32))
    torch.cuda.synchronize()
    nprog = opts.num_programs if opts is not None and opts.num_programs > 0 else \
        torch.cuda.get_device_properties(0).multi_processor_count
    if mode == W.MODE_SELF and spec.self_chunks_cut(lengths, heads, 256, nprog):
        d = (o.float() - o_ref.float()).abs()
        assert float(d.max()) <= 2.0 ** -7 * float(o_ref.float().abs().max()), "O differs from jfa_fwd"
        fin = torch.isfinite(lse_ref)
        assert torch.equal(fin, torch.isfinite(lse))
        assert float((lse[fin] - lse_ref[fin]).abs().max()) <= 1e-5 * max(1.0, float(lse_ref[fin].abs().max()))
    else:
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from jfa_fwd"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), "lse differs from jfa_fwd"
    o64, l64 = G.oracle_fwd(p)
    G.check_fwd(o, lse, o64, l64, "noalloc")


@pytest.mark.gpu
@pytest.mark.parametrize("sched", [0, 1])
def test_noalloc_forward_matches_jfa_fwd_twice_smaller_second(sched):
    opts = B.make_opts(sched=sched, num_programs=24)
    big = [1, 5, 63, 64, 65, 127, 128, 129, 200, 257, 700, 33, 0, 1024]
    assert spec.self_chunks_cut(big, 2, 256, 24)  # jfa_fwd cuts the 1024-token sequence
    _one_call(big, 2, 128, W.MODE_SELF, 71, opts)
    _one_call([3, 300, 17], 2, 128, W.MODE_SELF, 72, opts)
    _one_call(big, 2, 128, W.MODE_SELF, 71, B.make_opts(sched=sched, num_programs=8))  # no cut: bit-identical


@pytest.mark.gpu
def test_noalloc_forward_block_diag_and_head_dim_64():
    _one_call([70, 0, 300, 64, 129], 3, 64, W.MODE_BLOCK_DIAG, 73, None)
    _one_call([5, 64], 3, 64, W.MODE_BLOCK_DIAG, 74, None)
    _one_call([70, 0, 300, 64, 129], 2, 64, W.MODE_SELF, 75, None)


@pytest.mark.gpu
def test_noalloc_forward_broadcast_q_small():
    _one_call([1, 0, 700, 64], 2, 128, W.MODE_BROADCAST_Q, 76, B.make_opts(num_programs=16), num_q=100)
    _one_call([9, 3], 2, 128, W.MODE_BROADCAST_Q, 77, B.make_opts(num_programs=16), num_q=40)


def test_noalloc_rejects_shapes_beyond_its_scratch_before_device_work():
    # one million 1-token sequences need more schedule space than the array holds
    n = 1 << 20
    shape = B.make_shape(n, 4, 128, n)
    need = B.workspace_size(shape, B.MODE_SELF, B.PASS_FWD)
    assert need > 4 << 20
    rc = B.lib().jfa_fwd_noalloc(B.ctypes.byref(shape), B.MODE_SELF, 0.1, None, None, None, None, None, None,
                                 None, None, None)
    assert rc == -9, rc  # JFA_ERR_TOO_LARGE, ahead of the NULL-pointer check
    assert b"scratch" in B.lib().jfa_last_error_detail()
