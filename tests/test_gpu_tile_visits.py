"""Every scheduled tile is computed exactly once: the library's debug hook counts, per
kernel, how often each tile of its list is taken (jfa_debug_tile_visits), under the
static deal and the run-time counters (one group, and one per XCD at 16 and 24
programs, where programs walk several tiles each), forward and both self-attention
backward paths, broadcast-Q (key chunks, all three dQ paths), block-diagonal,
block-sparse and MXFP8.  A tile taken twice would write identical bytes and pass the
parity tests; a tile never taken would leave NaN there (see gpu_helpers), but only
this count tells the two schedules' bookkeeping apart from luck."""

import numpy as np
import pytest
import torch

from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu

STRIDE = 1 << 16
LENGTHS = [1, 5, 63, 64, 65, 127, 128, 129, 200, 257, 700, 33, 0, 1500, 400, 2]
ROLES = ((B.KERNEL_FWD, "fwd"), (B.KERNEL_BWD, "bwd"), (B.KERNEL_BWD_DQ, "bwd_dq"))


class Visits:
    def __enter__(self):
        self.counts = torch.zeros(3 * STRIDE, dtype=torch.int32, device="cuda")
        B.debug_tile_visits(self.counts, STRIDE)
        return self

    def __exit__(self, *exc):
        B.debug_tile_visits(None, 0)

    def check(self, label, expect_roles):
        torch.cuda.synchronize()
        c = self.counts.cpu().numpy().reshape(3, STRIDE)
        for role, name in ROLES:
            n = B.debug_tile_list_size(role)
            if name in expect_roles:
                assert n > 0, f"{label}: {name} ran no tiles"
            got = c[role]
            bad = np.nonzero(got[:n] != 1)[0]
            assert bad.size == 0, f"{label}: {name} tiles visited != 1: {bad[:10]} -> {got[bad[:10]]} (of {n})"
            assert not got[n:].any(), f"{label}: {name} counted past its {n} tiles"
            print(f"{label}: {name} {n} tiles, each once", flush=True)
        self.counts.zero_()


def _problem(lengths, heads, head_dim, mode, num_q=0, seed=0, kv=None):
    p = W.make_problem(lengths, heads, head_dim, mode, num_q, seed, device="cpu", num_kv_heads=kv)
    return p, G.to_gpu(p)


@pytest.mark.parametrize("sched,nprog", [(0, 0), (1, 0), (0, 16), (1, 16), (1, 24), (1, 5)])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_self_forward_and_both_backward_paths(sched, nprog, head_dim):
    p, g = _problem(LENGTHS, 2, head_dim, W.MODE_SELF, seed=81)
    off = p["offsets_host"]
    shape = B.make_shape(len(LENGTHS), 2, head_dim, int(off[-1]))
    label = f"self D{head_dim} sched {sched} P{nprog}"
    with Visits() as v:
        opts = B.make_opts(sched=sched, num_programs=nprog)
        o, lse = G.gpu_fwd(g, opts)
        v.check(label + " fwd", ("fwd",))
        G.gpu_bwd(g, o, lse, opts)
        v.check(label + " recompute bwd", ("bwd", "bwd_dq"))
        ds = B.make_opts(sched=sched, num_programs=nprog, ds_budget_mib=B.ds_budget_mib(shape, off))
        G.gpu_bwd(g, o, lse, ds)
        v.check(label + " stored-dS bwd", ("bwd", "bwd_dq"))


@pytest.mark.parametrize("sched,nprog", [(0, 0), (1, 0), (1, 16), (0, 24)])
@pytest.mark.parametrize("dq_path", [0, 1, 2])
def test_broadcast_q(sched, nprog, dq_path):
    lengths = [4096, 10, 0, 700, 300, 2000, 1, 64]
    p, g = _problem(lengths, 4, 128, W.MODE_BROADCAST_Q, num_q=300, seed=82)
    label = f"broadcast-Q sched {sched} P{nprog} dq_path {dq_path}"
    with Visits() as v:
        opts = B.make_opts(sched=sched, dq_path=dq_path, num_programs=nprog)
        o, lse = G.gpu_fwd(g, opts)
        v.check(label + " fwd", ("fwd",))
        G.gpu_bwd(g, o, lse, opts)
        v.check(label + " bwd", ("bwd", "bwd_dq") if dq_path == 2 else ("bwd",))


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("nprog", [0, 7])
def test_block_diagonal(head_dim, nprog):
    p, g = _problem([64 * 5, 1, 0, 129, 64, 700], 3, head_dim, W.MODE_BLOCK_DIAG, seed=83)
    with Visits() as v:
        opts = B.make_opts(num_programs=nprog)
        o, lse = G.gpu_fwd(g, opts)
        v.check(f"block-diag D{head_dim} P{nprog} fwd", ("fwd",))
        G.gpu_bwd(g, o, lse, opts)
        v.check(f"block-diag D{head_dim} P{nprog} bwd", ("bwd",))


@pytest.mark.parametrize("sched", [0, 1])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_block_sparse_and_grouped_query(sched, head_dim):
    p, g = _problem(LENGTHS, 2, head_dim, W.MODE_SELF, seed=84)
    opts = B.make_opts(sched=sched, num_programs=16)
    with Visits() as v:
        o, lse, sel = B.fwd_block_sparse(g["q"], g["k"], g["v"], g["offsets"], g["offsets_host"], 0.5, g["scale"],
                                         opts)
        v.check(f"block-sparse D{head_dim} sched {sched} fwd", ("fwd",))
        B.bwd_block_sparse(g["q"], g["k"], g["v"], o, g["do"], lse, g["offsets"], g["offsets_host"], 0.5, sel,
                           g["scale"], opts)
        v.check(f"block-sparse D{head_dim} sched {sched} bwd", ("bwd", "bwd_dq"))
    pk, gk = _problem(LENGTHS, 4, head_dim, W.MODE_SELF, seed=85, kv=1)
    with Visits() as v:
        G.gpu_fwd(gk, opts)
        v.check(f"grouped-query D{head_dim} sched {sched} fwd", ("fwd",))


@pytest.mark.parametrize("head_dim", [64, 128])
def test_mxfp8_forward(head_dim):
    p, g = _problem(LENGTHS, 2, head_dim, W.MODE_SELF, seed=86)
    q8, qs = B.mxfp8_quantize_qk(g["q"])
    k8, ks = B.mxfp8_quantize_qk(g["k"])
    v8, vs, tp = B.mxfp8_quantize_v(g["v"], g["offsets"], g["offsets_host"])
    with Visits() as v:
        B.fwd_mxfp8(q8, qs, k8, ks, v8, vs, tp, g["offsets"], g["offsets_host"], g["scale"],
                    B.make_opts(num_programs=11))
        v.check(f"mxfp8 D{head_dim} fwd", ("fwd",))
