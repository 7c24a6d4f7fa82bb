"""The tile scheduling rules, written out as the bit-exact specification of the host
scheduler.  Test infrastructure only (see the package docstring).

What the pages fix:

* Forward tiles cost in proportion to the key/value length of their sequence; the
  host sorts them by decreasing cost and deals them out in a zigzag: even passes from
  the first program to the last, odd passes back from the last to the first
  (aixai.ru page, "Tile balancing and Cluster Launch Control"; yuxiaoba page, "load
  balancing needs a static and a dynamic layer").
* Backward tiles cost about the same but their number varies; the host enumerates
  only the valid tiles and deals them round robin, ordered so that neighbouring tiles
  reuse the same data in L2 (same sections).
* Static pre-filtering removes empty tiles; a runtime counter then hands the next
  tile to whichever processor is free (same sections).
* min(#processors, #tiles) persistent programs; for fixed 64-token blocks each
  program gets a balanced contiguous range computed in closed form with divmod
  (bittide page, section 5).

Readings where the pages leave the rule open:

* Tiles are tuples (b, h, blk).  A forward tile is ``rows`` query rows of one (b, h);
  a self-attention backward tile is ``rows`` key rows of one (b, h).
* Cost key of a forward tile: L_kv(b) = L_b.  Ties are broken by (b, h, blk), so the
  sort key (-L_b, b, h, blk) is a total order.  Pass 0 runs left to right.
* Self-attention backward tiles cost in proportion to L_b as well (their loop runs
  over every query row of the sequence), so they take the forward rule.  The pages'
  round robin is applied where tiles really cost the same: the broadcast-Q backward,
  whose every tile loops over the same Mq shared queries.
* Broadcast-Q backward is head-pinned: the program count is rounded to a multiple of
  H, programs form H groups of P_h = P / H, and the n-th tile of head h (in (b, blk)
  order) goes to program h * P_h + (n mod P_h).  Every program then adds into one
  head's dQ only.
* Broadcast-Q forward keeps the tiles of empty sequences (they must still write
  O = 0 and lse = -inf); self and block-diagonal modes have no tile for them.
* Dynamic mode keeps the sorted order; program p starts with tile p of its group
  and then takes tiles from a per-group atomic counter.  The pages want neighbouring
  tiles to meet in one L2; a single counter would scatter one sequence's tiles over
  all L2s (each XCD has its own), so forward and self-attention backward schedules
  keep one counter per XCD: when P is a multiple of 8 the programs form 8 groups of
  P / 8 consecutive ids (one XCD each) and group g serves, in sorted order, the tiles
  the zigzag deal gives its programs; otherwise one group serves all tiles.  The
  output here is the tile list with one segment per counter group.
* Broadcast-Q forward key chunks: with a few hundred tiles (one per sequence, head and
  query block), zigzag dealing cannot help when the tiles of the longest sequence
  alone take longer than the average program's share, so such a sequence's keys are
  cut into chunks and every chunk is a tile "sequence" of its own (cost key: the
  chunk's keys); the chunks' partial outputs are merged by their log-sum-exp
  afterwards, which gives the same attention (the softmax over a union of key sets).
  A chunk is ``key_step * max(min_steps, share)`` keys, share = the key steps of one
  program's fair share of all tiles, ceil(H * ceil(Mq / rows) * sum_b
  ceil(L_b / key_step) / P).  Chunks are listed in sequence order; an empty sequence
  keeps one chunk of zero keys.  When no sequence is longer than one chunk the
  schedule is exactly the unchunked one.
* Self-attention forward key chunks: the same imbalance arises in self attention when
  a batch holds a few long sequences (their tiles are few and each walks all the
  sequence's keys), so the same rule applies with each sequence's own query tiles:
  share = ceil(H * sum_b ceil(L_b / rows) * ceil(L_b / key_step) / P), and a chunk of
  at least 8 key steps (each cut costs a merge pass that a shorter chunk does not
  repay; the pages give no number, this one is ours).  Empty sequences have no chunk.  When some sequence is cut, tiles are (chunk, h, blk) with
  blk < ceil(L_b / rows) for the chunk's sequence b, sorted by the chunk's keys;
  otherwise the schedule is exactly the unchunked one.

Every function returns plain Python lists so that a reader can compare them by eye.
"""

MODE_SELF = 0
MODE_BROADCAST_Q = 1
MODE_BLOCK_DIAG = 2


def _cdiv(a, b):
    return -(-a // b)


def zigzag_program(n, num_programs):
    """Program that receives the tile at sorted position n under zigzag dealing."""
    r, pos = divmod(n, num_programs)
    return pos if r % 2 == 0 else num_programs - 1 - pos


def sorted_cost_tiles(lengths, num_heads, rows, rows_of):
    """All (b, h, blk) tiles with blk < ceil(rows_of(b) / rows), sorted by the key
    (-L_b, b, h, blk)."""
    tiles = [(b, h, i)
             for b in range(len(lengths))
             for h in range(num_heads)
             for i in range(_cdiv(rows_of(b), rows))]
    return sorted(tiles, key=lambda t: (-int(lengths[t[0]]), t[0], t[1], t[2]))


XCDS = 8


def counter_groups(num_programs):
    """Counter groups of a dynamic forward or self-attention backward schedule."""
    return XCDS if num_programs >= XCDS and num_programs % XCDS == 0 else 1


def _deal_zigzag(order, num_programs, dynamic=False):
    n_tiles = len(order)
    p_used = min(num_programs, n_tiles)
    if p_used == 0:
        return [], ([0, 0] if dynamic else [0]), 0
    per_prog = [[] for _ in range(p_used)]
    for n, t in enumerate(order):
        per_prog[zigzag_program(n, p_used)].append(t)
    if dynamic:
        # one segment per group of p_used / G consecutive programs, in sorted order
        g = counter_groups(p_used)
        gsize = p_used // g
        rank = {t: n for n, t in enumerate(order)}
        segs = [sorted((t for lst in per_prog[k * gsize:(k + 1) * gsize] for t in lst), key=rank.__getitem__)
                for k in range(g)]
    else:
        segs = per_prog
    tiles, ptr = [], [0]
    for lst in segs:
        tiles.extend(lst)
        ptr.append(len(tiles))
    return tiles, ptr, p_used


def bq_key_chunks(lengths, num_heads, num_q, rows, num_programs, key_step=64, min_steps=4):
    """Key chunks of the broadcast-Q forward tiles: a list of (b, first_key, keys) in
    sequence order (see the module docstring for the rule)."""
    steps = sum(_cdiv(int(n), key_step) for n in lengths)
    share = _cdiv(num_heads * _cdiv(num_q, rows) * steps, max(1, num_programs))
    keys = key_step * max(min_steps, share)
    chunks = []
    for b, n in enumerate(lengths):
        n = int(n)
        if n == 0:
            chunks.append((b, 0, 0))
        for k0 in range(0, n, keys):
            chunks.append((b, k0, min(keys, n - k0)))
    return chunks


def self_key_chunks(lengths, num_heads, rows, num_programs, key_step=64, min_steps=8):
    """Key chunks of the self-attention forward tiles: a list of (b, first_key, keys)
    in sequence order, empty sequences skipped (see the module docstring)."""
    steps = sum(_cdiv(int(n), rows) * _cdiv(int(n), key_step) for n in lengths)
    share = _cdiv(num_heads * steps, max(1, num_programs))
    keys = key_step * max(min_steps, share)
    return [(b, k0, min(keys, int(n) - k0)) for b, n in enumerate(lengths) for k0 in range(0, int(n), keys)]


def self_chunks_cut(lengths, num_heads, rows, num_programs):
    """True when the self-attention forward cuts some sequence into key chunks."""
    chunks = self_key_chunks(lengths, num_heads, rows, num_programs)
    return len(chunks) != sum(1 for n in lengths if int(n) > 0)


def fwd_schedule(lengths, num_heads, mode, num_q, rows, num_programs, dynamic=False):
    """Forward schedule for MODE_SELF / MODE_BROADCAST_Q.

    Returns (tiles, segment_ptr, programs).  Static: tiles in program-major order and
    one segment per program.  Dynamic: one segment per counter group (counter_groups),
    each holding in sorted order the tiles the static deal gives its programs.  In
    broadcast-Q mode a tile's first entry is the index of its key chunk in
    bq_key_chunks(...) (the sequence index when no sequence is cut); in self mode it
    is the index in self_key_chunks(...) when some sequence is cut."""
    if mode == MODE_SELF and self_chunks_cut(lengths, num_heads, rows, num_programs):
        chunks = self_key_chunks(lengths, num_heads, rows, num_programs)
        order = sorted_cost_tiles([c[2] for c in chunks], num_heads, rows, lambda c: int(lengths[chunks[c][0]]))
    elif mode == MODE_SELF:
        order = sorted_cost_tiles(lengths, num_heads, rows, lambda b: int(lengths[b]))
    elif mode == MODE_BROADCAST_Q:
        keys = [c[2] for c in bq_key_chunks(lengths, num_heads, num_q, rows, num_programs)]
        order = sorted_cost_tiles(keys, num_heads, rows, lambda c: int(num_q))
    else:
        raise ValueError("fwd_schedule covers the self and broadcast-Q modes")
    return _deal_zigzag(order, num_programs, dynamic)


def bwd_schedule(lengths, num_heads, mode, rows, num_programs, dynamic=False):
    """Backward schedule for MODE_SELF / MODE_BROADCAST_Q over key/value tiles of
    ``rows`` keys.  Returns (tiles, segment_ptr, programs) as in fwd_schedule; the
    broadcast-Q dynamic form has one segment per head."""
    if mode == MODE_SELF:
        order = sorted_cost_tiles(lengths, num_heads, rows, lambda b: int(lengths[b]))
        return _deal_zigzag(order, num_programs, dynamic)
    if mode != MODE_BROADCAST_Q:
        raise ValueError("bwd_schedule covers the self and broadcast-Q modes")
    per_head = [[(b, h, j) for b in range(len(lengths)) for j in range(_cdiv(int(lengths[b]), rows))]
                for h in range(num_heads)]
    n_head = len(per_head[0]) if num_heads else 0
    if n_head == 0:
        return [], [0], 0
    p_h = max(1, min(num_programs // num_heads, n_head))
    if dynamic:
        tiles, ptr = [], [0]
        for lst in per_head:
            tiles.extend(lst)
            ptr.append(len(tiles))
        return tiles, ptr, p_h * num_heads
    per_prog = [[] for _ in range(p_h * num_heads)]
    for h, lst in enumerate(per_head):
        for n, t in enumerate(lst):
            per_prog[h * p_h + n % p_h].append(t)
    tiles, ptr = [], [0]
    for lst in per_prog:
        tiles.extend(lst)
        ptr.append(len(tiles))
    return tiles, ptr, p_h * num_heads


def blockdiag_schedule(lengths, num_heads, num_programs, block=64, min_tiles=1):
    """Block-diagonal schedule: tiles (b, h, j) for every block j < ceil(L_b / block),
    enumerated with the head fastest, so consecutive tiles cover one contiguous slab
    of the packed buffer.  Program p receives the contiguous range
    [p*q + min(p, r), (p+1)*q + min(p+1, r)) with (q, r) = divmod(N, P) and
    P = min(num_programs, ceil(N / min_tiles)) (min_tiles > 1 when a program is a group
    of workers that should each get a tile, as a workgroup of several waves)."""
    tiles = [(b, h, j)
             for b in range(len(lengths))
             for j in range(_cdiv(int(lengths[b]), block))
             for h in range(num_heads)]
    n_tiles = len(tiles)
    p_used = min(num_programs, _cdiv(n_tiles, min_tiles))
    if p_used == 0:
        return [], [0], 0
    q, r = divmod(n_tiles, p_used)
    ptr = [p * q + min(p, r) for p in range(p_used + 1)]
    return tiles, ptr, p_used
