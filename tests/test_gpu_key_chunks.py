"""GPU parity of the self-attention forward when a batch of few long sequences has its
keys cut into chunks (each chunk a tile of its own, partial O and lse merged by their
log-sum-exp afterwards; the rule is oracle/schedule.py's self_key_chunks).

Each case checks the chunked forward element by element against the fp64 oracle, the
backward run on its merged O and lse, and the chunked forward against the same call
with one program (whose share is the whole batch, so nothing is cut): the two sum the
same keys in another grouping and agree to fp32 rounding before the bf16 store."""

import numpy as np
import pytest
import torch

from oracle import schedule as spec
from tests import gpu_helpers as G
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu

ROWS = 256  # forward query tile


def _programs(opts_programs):
    return opts_programs if opts_programs > 0 else torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("sched", [0, 1])
def test_few_long_sequences_cut_into_key_chunks(head_dim, sched):
    lengths = [3000, 5, 0, 700, 1, 1300]
    heads, nprog = 3, 64
    assert spec.self_chunks_cut(lengths, heads, ROWS, nprog)
    opts = B.make_opts(sched=sched, num_programs=nprog)
    p, g, (o, lse), _ = G.run_case(lengths, heads, head_dim, W.MODE_SELF, seed=91, opts=opts,
                                   label=f"key chunks D{head_dim} sched {sched}")
    # nothing cut with one program: same attention up to summation grouping
    o1, l1 = G.gpu_fwd(g, B.make_opts(sched=sched, num_programs=1))
    torch.cuda.synchronize()
    assert not spec.self_chunks_cut(lengths, heads, ROWS, 1)
    d = (o.float() - o1.float()).abs()
    assert float(d.max()) <= 2.0 ** -7 * float(o1.float().abs().max()), "chunked vs unchunked O"
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(lse))
    assert float((lse[fin] - l1[fin]).abs().max()) <= 1e-5 * max(1.0, float(l1[fin].abs().max()))


@pytest.mark.parametrize("host_offsets", [True, False])
def test_workload_one_lengths_default_programs(host_offsets):
    """The four-sequence D=64 batch at full size in bench.py's launch configuration
    (default programs, dynamic schedule): forward and backward against the oracle."""
    lengths = W.workload_lengths(1).tolist()
    nprog = _programs(0)
    assert spec.self_chunks_cut(lengths, 1, ROWS, nprog)
    G.run_case(lengths, 1, 64, W.MODE_SELF, seed=92, opts=B.make_opts(sched=1), host_offsets=host_offsets,
               label=f"workload 1 lengths, host offsets {host_offsets}")


def test_single_long_sequence_many_heads_one_program_per_chunk():
    # one 8191-token sequence, 2 heads, 256 programs: share = 2 * 32 * 128 / 256 = 32
    # steps, so chunks of 2048 keys, the last one ragged (2047), and a ragged last
    # query tile
    lengths = [8191]
    assert spec.self_chunks_cut(lengths, 2, ROWS, 256)
    ch = spec.self_key_chunks(lengths, 2, ROWS, 256)
    assert len(ch) > 1 and ch[-1][2] < ch[0][2]
    G.run_case(lengths, 2, 128, W.MODE_SELF, seed=93, opts=B.make_opts(sched=1, num_programs=256), bwd=False,
               label="one long sequence")
