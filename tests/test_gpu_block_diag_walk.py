"""GPU parity of the block-diagonal kernels where a wave's walk over its tiles (a
workgroup's four waves take every fourth (block, head) tile of the program's range,
head fastest, the block's sequence found from the previous tile's) crosses runs of empty
sequences, head counts below and above that step of four, and program ranges that
start and end inside a sequence.  Forward and backward against the fp64 oracle, plain
and with the fused rotary embedding ("TLX Block Attention", bittide page: attention
within each 64-token block of a sequence; rotary: the rotate-half pairing of jfa.h)."""

import pytest

from tests import gpu_helpers as G
from tests import test_gpu_rotary as RT
from variable_length_flash_jagged_amd import binding as B
from variable_length_flash_jagged_amd import workloads as W

pytestmark = pytest.mark.gpu

# empty runs before, between and after sequences of 1, 63, 64, 65, 128 and 200 tokens
WALK = [0, 0, 65, 0, 0, 0, 1, 128, 0, 64, 0, 0, 0, 0, 0, 0, 0, 0, 200, 0, 63, 0]


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("heads", [1, 3, 5])
@pytest.mark.parametrize("nprog", [1, 3, 0])
def test_walk_over_empty_sequences(head_dim, heads, nprog):
    G.run_case(WALK, heads, head_dim, W.MODE_BLOCK_DIAG, seed=71 + heads, opts=B.make_opts(num_programs=nprog),
               label=f"bd walk D{head_dim} H{heads} P{nprog}")


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("nprog", [1, 3])
def test_rotary_walk_over_empty_sequences(head_dim, nprog):
    RT._run(WALK, 3, head_dim, seed=81, label=f"walk P{nprog}", opts=B.make_opts(num_programs=nprog))


def test_single_block_per_wave_and_many_programs():
    # 7 one-block sequences x 2 heads = 14 tiles over up to 256 programs: most programs
    # get no tile, some one; every wave's walk ends after its first tile
    G.run_case([64, 1, 64, 30, 64, 64, 2], 2, 64, W.MODE_BLOCK_DIAG, seed=83, label="bd one tile per wave")
