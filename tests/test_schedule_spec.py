"""Pins of the scheduler specification (oracle/schedule.py): hand-worked examples of
the pages' rules (tests/golden) and invariants that hold for any input."""

import json
import os

import numpy as np
import pytest

from oracle import schedule as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cdiv(a, b):
    return -(-a // b)


def test_zigzag_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "zigzag_example.json")))
    order = S.sorted_cost_tiles(g["lengths"], g["num_heads"], g["rows"], lambda b: g["lengths"][b])
    assert [list(t) for t in order] == g["sorted_order"]
    tiles, ptr, p = S.fwd_schedule(g["lengths"], g["num_heads"], S.MODE_SELF, 0, g["rows"], g["num_programs"])
    assert p == g["num_programs"]
    got = [[list(t) for t in tiles[ptr[i]:ptr[i + 1]]] for i in range(p)]
    assert got == g["program_tiles"]


def test_zigzag_program_rule():
    # even passes left to right, odd passes right to left
    assert [S.zigzag_program(n, 3) for n in range(9)] == [0, 1, 2, 2, 1, 0, 0, 1, 2]


def test_blockdiag_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "blockdiag_example.json")))
    off = g["offsets"]
    lengths = [off[i + 1] - off[i] for i in range(len(off) - 1)]
    tiles, ptr, p = S.blockdiag_schedule(lengths, g["num_heads"], g["num_programs"], g["block"])
    assert [list(t) for t in tiles] == g["tiles"]
    assert ptr == g["program_ptr"]


def _random_lengths(rng, n):
    x = rng.integers(0, 300, size=n)
    x[rng.random(n) < 0.1] = 0
    x[rng.random(n) < 0.1] = 1
    return x.tolist()


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("mode", [S.MODE_SELF, S.MODE_BROADCAST_Q])
def test_fwd_covers_every_tile_once_and_balances(seed, mode):
    rng = np.random.default_rng(seed)
    lengths = _random_lengths(rng, 37)
    h, rows, mq, nprog = 3, 64, 100, 13
    tiles, ptr, p = S.fwd_schedule(lengths, h, mode, mq, rows, nprog)
    lq = (lambda b: lengths[b]) if mode == S.MODE_SELF else (lambda b: mq)
    expect = {(b, hh, i) for b in range(len(lengths)) for hh in range(h) for i in range(_cdiv(lq(b), rows))}
    assert len(tiles) == len(expect) == h * sum(_cdiv(lq(b), rows) for b in range(len(lengths)))
    assert set(tiles) == expect
    assert p == min(nprog, len(expect)) and ptr[-1] == len(tiles)
    # within a program, tiles keep sorted order; program loads differ by at most one tile cost
    cost = {t: lengths[t[0]] for t in tiles}
    loads = [sum(cost[t] for t in tiles[ptr[i]:ptr[i + 1]]) for i in range(p)]
    assert max(loads) - min(loads) <= max(lengths)
    # dynamic mode (13 programs: one counter group): the same tiles in global sorted order
    dt, dptr, dp = S.fwd_schedule(lengths, h, mode, mq, rows, nprog, dynamic=True)
    assert sorted(dt) == sorted(tiles) and dptr == [0, len(dt)] and dp == p
    keys = [(-lengths[t[0]], t) for t in dt]
    assert keys == sorted(keys)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("nprog", [16, 24, 40, 7])
def test_dynamic_counter_groups_hold_one_xcds_static_tiles(seed, nprog):
    # Dynamic schedules keep one counter per XCD when the program count is a multiple
    # of 8: group g (programs g P/8 .. (g+1) P/8 - 1) serves exactly the tiles the
    # static zigzag deal gives those programs, in sorted order.
    rng = np.random.default_rng(700 + seed)
    lengths = _random_lengths(rng, 40)
    h, rows = 2, 64
    tiles, ptr, p = S.bwd_schedule(lengths, h, S.MODE_SELF, rows, nprog)
    dt, dptr, dp = S.bwd_schedule(lengths, h, S.MODE_SELF, rows, nprog, dynamic=True)
    assert dp == p
    g = 8 if p % 8 == 0 else 1
    assert len(dptr) == g + 1 and sorted(dt) == sorted(tiles)
    order = S.sorted_cost_tiles(lengths, h, rows, lambda b: lengths[b])
    rank = {t: n for n, t in enumerate(order)}
    gs = p // g
    for k in range(g):
        seg = dt[dptr[k]:dptr[k + 1]]
        static = [t for q in range(k * gs, (k + 1) * gs) for t in tiles[ptr[q]:ptr[q + 1]]]
        assert sorted(seg) == sorted(static)
        assert [rank[t] for t in seg] == sorted(rank[t] for t in seg)
        # the group's first tiles are those its programs start with under the static deal
        assert seg[:gs] == [tiles[ptr[q]] for q in range(k * gs, (k + 1) * gs)][:len(seg)]


@pytest.mark.parametrize("seed", range(5))
def test_bwd_broadcast_q_head_pinned_round_robin(seed):
    rng = np.random.default_rng(100 + seed)
    lengths = _random_lengths(rng, 23)
    h, rows, nprog = 4, 128, 30
    tiles, ptr, p = S.bwd_schedule(lengths, h, S.MODE_BROADCAST_Q, rows, nprog)
    n_head = sum(_cdiv(n, rows) for n in lengths)
    p_h = max(1, min(nprog // h, n_head))
    assert p == p_h * h
    for prog in range(p):
        mine = tiles[ptr[prog]:ptr[prog + 1]]
        assert all(t[1] == prog // p_h for t in mine)  # one head per program
    # round robin within the head group, in (b, blk) order
    for hh in range(h):
        order = [(b, hh, j) for b in range(len(lengths)) for j in range(_cdiv(lengths[b], rows))]
        for n, t in enumerate(order):
            prog = hh * p_h + n % p_h
            assert t in tiles[ptr[prog]:ptr[prog + 1]]
    dt, dptr, dp = S.bwd_schedule(lengths, h, S.MODE_BROADCAST_Q, rows, nprog, dynamic=True)
    assert dp == p and len(dptr) == h + 1 and sorted(dt) == sorted(tiles)


def test_bwd_self_uses_sorted_zigzag():
    lengths = [300, 5, 0, 129, 64]
    tiles, ptr, p = S.bwd_schedule(lengths, 2, S.MODE_SELF, 64, 4)
    ft, fptr, fp = S.fwd_schedule(lengths, 2, S.MODE_SELF, 0, 64, 4)
    assert (tiles, ptr, p) == (ft, fptr, fp)


@pytest.mark.parametrize("nprog", [1, 3, 7, 1000])
def test_blockdiag_ranges_are_contiguous_and_balanced(nprog):
    rng = np.random.default_rng(nprog)
    lengths = (rng.integers(0, 5, size=20) * 64 + rng.integers(0, 2, size=20) * 7).tolist()
    tiles, ptr, p = S.blockdiag_schedule(lengths, 3, nprog)
    n = sum(_cdiv(x, 64) for x in lengths) * 3
    assert len(tiles) == n and p == min(nprog, n)
    sizes = [ptr[i + 1] - ptr[i] for i in range(p)]
    assert max(sizes) - min(sizes) <= 1 and ptr[0] == 0 and ptr[-1] == n
    # head fastest
    assert [t[1] for t in tiles[:3]] == [0, 1, 2]


def test_empty_batch():
    assert S.fwd_schedule([0, 0], 2, S.MODE_SELF, 0, 64, 8) == ([], [0], 0)
    assert S.bwd_schedule([0], 2, S.MODE_BROADCAST_Q, 64, 8) == ([], [0], 0)
    assert S.blockdiag_schedule([], 2, 8) == ([], [0], 0)
    # broadcast-Q forward keeps tiles of empty sequences (they write O = 0)
    t, _, _ = S.fwd_schedule([0, 0], 1, S.MODE_BROADCAST_Q, 64, 64, 8)
    assert sorted(t) == [(0, 0, 0), (1, 0, 0)]


def test_bq_key_chunks_hand_example():
    # 16 + 1 key steps of 64; one 256-row query block, one head, 8 programs:
    # share = ceil(17 / 8) = 3 steps < 4, so chunks are 4 steps = 256 keys
    ch = S.bq_key_chunks([1000, 10, 0], 1, 256, 256, 8)
    assert ch == [(0, 0, 256), (0, 256, 256), (0, 512, 256), (0, 768, 232), (1, 0, 10), (2, 0, 0)]
    tiles, ptr, p = S.fwd_schedule([1000, 10, 0], 1, S.MODE_BROADCAST_Q, 256, 256, 8)
    # chunk costs 256, 256, 256, 232, 10, 0: one tile per program in sorted order
    assert p == 6 and tiles == [(0, 0, 0), (1, 0, 0), (2, 0, 0), (3, 0, 0), (4, 0, 0), (5, 0, 0)]
    assert ptr == [0, 1, 2, 3, 4, 5, 6]


@pytest.mark.parametrize("seed", range(4))
def test_bq_key_chunks_cover_every_key_once(seed):
    rng = np.random.default_rng(300 + seed)
    lengths = (rng.integers(0, 5000, size=20) * (rng.random(20) < 0.8)).tolist()
    h, mq, rows, nprog = int(rng.integers(1, 5)), int(rng.integers(1, 600)), 256, int(rng.integers(1, 300))
    ch = S.bq_key_chunks(lengths, h, mq, rows, nprog)
    steps = sum(_cdiv(n, 64) for n in lengths)
    keys = 64 * max(4, _cdiv(h * _cdiv(mq, rows) * steps, nprog))
    assert [c[0] for c in ch] == sorted(c[0] for c in ch)
    for b, n in enumerate(lengths):
        mine = [c for c in ch if c[0] == b]
        if n == 0:
            assert mine == [(b, 0, 0)]
            continue
        assert [c[1] for c in mine] == list(range(0, n, keys))
        assert sum(c[2] for c in mine) == n and all(0 < c[2] <= keys for c in mine)
    # every (chunk, head, query block) tile once
    tiles, ptr, p = S.fwd_schedule(lengths, h, S.MODE_BROADCAST_Q, mq, rows, nprog)
    assert sorted(tiles) == sorted((c, hh, i) for c in range(len(ch)) for hh in range(h)
                                   for i in range(_cdiv(mq, rows)))


def test_bq_fwd_schedule_unchunked_when_no_sequence_exceeds_a_share():
    lengths = [300, 0, 1, 129, 4000]
    h, mq, rows, nprog = 2, 300, 256, 1  # one program: its share is all the work
    assert S.bq_key_chunks(lengths, h, mq, rows, nprog) == [(b, 0, n) for b, n in enumerate(lengths)]
    tiles, _, _ = S.fwd_schedule(lengths, h, S.MODE_BROADCAST_Q, mq, rows, nprog, dynamic=True)
    assert tiles == S.sorted_cost_tiles(lengths, h, rows, lambda b: mq)


@pytest.mark.parametrize("seed", range(6))
def test_bq_cut_sequence_chunks_within_workspace_bound(seed):
    # The library sizes the forward's partial-result slots (chunks of sequences cut into
    # two or more) as min(2 P / (H ceil(Mq / 256)), 2 T / 256) + 1.  A cut sequence is
    # longer than the chunk, which is at least max(256, H ceil(Mq/256) T / P) keys.
    rng = np.random.default_rng(500 + seed)
    for _ in range(50):
        n = int(rng.integers(1, 80))
        lengths = (rng.integers(0, 6000, size=n) * (rng.random(n) < 0.9)).tolist()
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, n))] = int(rng.integers(20000, 60000))
        h, mq, p = int(rng.integers(1, 9)), int(rng.integers(1, 1200)), int(rng.integers(1, 600))
        ch = S.bq_key_chunks(lengths, h, mq, 256, p)
        per_seq = {}
        for c in ch:
            per_seq[c[0]] = per_seq.get(c[0], 0) + 1
        slots = sum(k for k in per_seq.values() if k > 1)
        bound = min(2 * p // (h * _cdiv(mq, 256)), 2 * sum(lengths) // 256) + 1
        assert slots <= bound


def test_self_key_chunks_hand_example():
    # one head, 256-row query tiles, 256 programs: key steps 16*64 + 1*2 + 8*32 = 1282,
    # share = ceil(1282 / 256) = 6 steps < 8, so chunks are 512 keys
    lengths = [4096, 128, 0, 2048]
    ch = S.self_key_chunks(lengths, 1, 256, 256)
    assert ch == [(0, k, 512) for k in range(0, 4096, 512)] + [(1, 0, 128)] + [(3, k, 512) for k in range(0, 2048, 512)]
    assert S.self_chunks_cut(lengths, 1, 256, 256)
    assert not S.self_chunks_cut([300, 65, 1], 2, 256, 256)  # 300 keys: under one 512-key chunk
    tiles, ptr, p = S.fwd_schedule(lengths, 1, S.MODE_SELF, 0, 256, 256)
    # tiles (chunk, 0, blk): 8 chunks x 16 blocks + 1 + 4 chunks x 8 blocks
    assert len(tiles) == 8 * 16 + 1 + 4 * 8 and p == 161
    assert all(blk < -(-lengths[ch[c][0]] // 256) for c, _, blk in tiles)


@pytest.mark.parametrize("seed", range(4))
def test_self_key_chunks_cover_every_key_and_query_once(seed):
    rng = np.random.default_rng(900 + seed)
    lengths = (rng.integers(0, 5000, size=12) * (rng.random(12) < 0.8)).tolist()
    h, rows, nprog = int(rng.integers(1, 5)), 256, int(rng.integers(16, 600))
    ch = S.self_key_chunks(lengths, h, rows, nprog)
    steps = sum(_cdiv(n, rows) * _cdiv(n, 64) for n in lengths)
    keys = 64 * max(8, _cdiv(h * steps, nprog))
    assert [c[0] for c in ch] == sorted(c[0] for c in ch)
    for b, n in enumerate(lengths):
        mine = [c for c in ch if c[0] == b]
        assert [c[1] for c in mine] == list(range(0, n, keys))
        assert sum(c[2] for c in mine) == n and all(0 < c[2] <= keys for c in mine)
    tiles, _, _ = S.fwd_schedule(lengths, h, S.MODE_SELF, 0, rows, nprog)
    if S.self_chunks_cut(lengths, h, rows, nprog):
        # every (chunk, head, query block of the chunk's sequence) once, so each (query
        # row, key) pair of every sequence is covered exactly once
        assert sorted(tiles) == sorted((c, hh, i) for c in range(len(ch)) for hh in range(h)
                                       for i in range(_cdiv(lengths[ch[c][0]], rows)))
    else:
        assert sorted(tiles) == sorted((b, hh, i) for b, n in enumerate(lengths) for hh in range(h)
                                       for i in range(_cdiv(n, rows)))


def test_self_schedule_unchunked_for_a_large_batch():
    # many sequences: the fair share exceeds every sequence's key steps
    rng = np.random.default_rng(5)
    lengths = np.clip(np.rint(np.exp(rng.normal(np.log(600.0), 1.0, size=1152))), 1, 4000).astype(int).tolist()
    assert not S.self_chunks_cut(lengths, 4, 256, 256)
    assert S.fwd_schedule(lengths, 4, S.MODE_SELF, 0, 256, 256)[0] == _deal_plain(lengths, 4, 256, 256)


def _deal_plain(lengths, h, rows, nprog):
    order = S.sorted_cost_tiles(lengths, h, rows, lambda b: int(lengths[b]))
    per = [[] for _ in range(min(nprog, len(order)))]
    for n, t in enumerate(order):
        per[S.zigzag_program(n, len(per))].append(t)
    return [t for lst in per for t in lst]


@pytest.mark.parametrize("seed", range(6))
def test_self_cut_chunks_within_workspace_bound(seed):
    # The library holds the partial rows of cut sequences in 2 * rows * P row-heads, the
    # chunks in B + 2 T / 256 + 1 entries and their tiles in H (T / rows + B + 1) + 2 P +
    # H (B + 2 T / 256 + 1).
    rng = np.random.default_rng(600 + seed)
    rows = 256
    for _ in range(60):
        n = int(rng.integers(1, 40))
        lengths = (rng.integers(0, 3000, size=n) * (rng.random(n) < 0.9)).tolist()
        if rng.random() < 0.5:
            lengths[int(rng.integers(0, n))] = int(rng.integers(5000, 40000))
        h, p = int(rng.integers(1, 9)), int(rng.integers(1, 600))
        ch = S.self_key_chunks(lengths, h, rows, p)
        per_seq = {}
        for c in ch:
            per_seq[c[0]] = per_seq.get(c[0], 0) + 1
        part = sum(k * lengths[b] for b, k in per_seq.items() if k > 1) * h
        assert part < 2 * rows * p
        t = sum(lengths)
        chunk_cap = n + 2 * t // 256 + 1
        assert len(ch) <= chunk_cap
        tiles, _, _ = S.fwd_schedule(lengths, h, S.MODE_SELF, 0, rows, p)
        assert len(tiles) <= h * (t // rows + n + 1) + 2 * p + h * chunk_cap
