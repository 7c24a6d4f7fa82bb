"""Seeded random sweeps over the variants -- block-sparse top-k forward and backward,
rotary block-diagonal attention, MXFP8 forward -- each case checked against the fp64
oracle by the same checks as the variant's own test module (random head dims, head
counts, length mixes with empty, 1-token and tile-edge lengths, ratios, schedules and
program counts)."""

import numpy as np
import pytest

from tests import test_gpu_block_sparse as TS
from tests import test_gpu_mxfp8 as TM
from tests import test_gpu_rotary as TR
from variable_length_flash_jagged_amd import binding as B

pytestmark = pytest.mark.gpu

EDGES = [0, 1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513]


def _lengths(rng, nb, hi=900):
    return [int(rng.choice(EDGES)) if rng.random() < 0.4 else int(rng.integers(0, hi)) for _ in range(nb)]


@pytest.mark.parametrize("seed", range(6))
def test_random_block_sparse(seed):
    rng = np.random.default_rng(3000 + seed)
    d = int(rng.choice([64, 128]))
    h = int(rng.choice([1, 2, 3]))
    lengths = _lengths(rng, int(rng.integers(1, 7)))
    if sum(lengths) == 0:
        lengths[0] = 300
    ratio = float(rng.choice([0.1, 0.25, 0.5, 0.75, 1.0]))
    opts = B.make_opts(sched=int(rng.integers(0, 2)), num_programs=int(rng.choice([0, 1, 3, 17])))
    TS._run(lengths, h, d, ratio, seed=4000 + seed, opts=opts, bwd=True,
            label=f"random D{d} H{h} r{ratio} opts=({opts.sched},{opts.num_programs})")


@pytest.mark.parametrize("seed", range(4))
def test_random_rotary(seed):
    rng = np.random.default_rng(5000 + seed)
    d = int(rng.choice([64, 128]))
    h = int(rng.choice([1, 2, 3]))
    lengths = _lengths(rng, int(rng.integers(1, 7)))
    if sum(lengths) == 0:
        lengths[0] = 130
    extra = int(rng.integers(0, 50))
    TR._run(lengths, h, d, seed=6000 + seed, label=f"random D{d} H{h}", table_rows=max(1, max(lengths)) + extra)


@pytest.mark.parametrize("seed", range(4))
def test_random_mxfp8(seed):
    rng = np.random.default_rng(7000 + seed)
    d = int(rng.choice([64, 128]))
    h = int(rng.choice([1, 2, 3]))
    lengths = _lengths(rng, int(rng.integers(1, 7)))
    if sum(lengths) == 0:
        lengths[0] = 200
    TM._run(lengths, h, d, seed=8000 + seed, label=f"random D{d} H{h}")
