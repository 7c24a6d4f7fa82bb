"""Valid-token accounting pinned to the worked example on the explore.n1n.ai page
(section on the performance defects of padded tensors) and to closed forms."""

import json
import os

from variable_length_flash_jagged_amd import metrics as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_pairs_and_padding_waste():
    g = json.load(open(os.path.join(GOLDEN, "worked_offsets.json")))
    lengths = g["lengths"]
    assert M.valid_pairs(lengths, M.MODE_SELF) == 128**2 + 4096**2 + 512**2 + 2048**2 == 21_250_048
    assert M.padded_pairs(lengths) == 4 * 4096**2 == 67_108_864
    # token waste of padding: 1 - 6784 / 16384 ~ 58.6 %, the page's "up to 60 %"
    assert abs((1 - g["total_tokens"] / g["padded_tokens"]) - 0.586) < 1e-3


def test_block_diag_pairs_closed_form():
    # full blocks give 64^2 each; a trailing block of r tokens gives r^2
    assert M.valid_pairs([64 * 3, 70, 5], M.MODE_BLOCK_DIAG) == 4 * 64 * 64 + 36 + 25


def test_flop_and_byte_counts():
    assert M.fwd_flops([4, 2], M.MODE_SELF, 2, 8) == 4 * 2 * 8 * 20
    assert M.bwd_flops([4, 2], M.MODE_SELF, 2, 8) == 10 * 2 * 8 * 20
    assert M.valid_pairs([3, 5], M.MODE_BROADCAST_Q, num_q=7) == 56
    assert M.fwd_bytes([4, 2], M.MODE_SELF, 2, 8) == 8 * 6 * 16 + 4 * 12
    assert M.bwd_bytes([4, 2], M.MODE_SELF, 2, 8) == 16 * 6 * 16 + 4 * 12


def test_block_sparse_pairs_full_selection_is_dense_and_half_is_counted_exactly():
    lengths = [300, 1, 64, 65, 0, 700]
    keep = [-(-n // 64) if n else 0 for n in lengths]
    full, half, want_half = [], [], 0
    for n, kk in zip(lengths, keep):
        if n == 0:
            continue
        nqb = -(-n // 256)
        for _ in range(2):
            for i in range(nqb):
                full += list(range(kk))
                half += [0]  # first key block only: 64 keys (or n if shorter)
                want_half += min(256, n - 256 * i) * min(64, n)
    assert M.block_sparse_pairs(lengths, 2, keep, full) == 2 * M.valid_pairs(lengths, M.MODE_SELF)
    assert M.block_sparse_pairs(lengths, 2, [1 if n else 0 for n in lengths], half) == want_half


def test_block_sparse_tile_pairs():
    """Full selection: every tile runs whole, so the executed pairs are the valid pairs.
    One kept block per query block: the whole 128-key tile that holds it runs."""
    lengths = [300, 1, 64, 65, 0, 700]
    keep = [-(-n // 64) if n else 0 for n in lengths]
    full, one, want_one = [], [], 0
    for n, kk in zip(lengths, keep):
        if n == 0:
            continue
        nqb = -(-n // 256)
        for _ in range(2):
            for i in range(nqb):
                full += list(range(kk))
                jb = min(3, kk - 1)       # key block 3 (or the last) -> tile 1 (or 0)
                one += [jb]
                t = jb // 2
                want_one += min(256, n - 256 * i) * min(128, n - 128 * t)
    assert M.block_sparse_tile_pairs(lengths, 2, keep, full) == 2 * M.valid_pairs(lengths, M.MODE_SELF)
    assert M.block_sparse_tile_pairs(lengths, 2, [1 if n else 0 for n in lengths], one) == want_one
