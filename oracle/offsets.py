"""Offsets (cu_seqlens) arithmetic for the jagged layout, written out plainly.

Test infrastructure only (see the package docstring).

The jagged layout stores the valid tokens of all sequences back to back in one flat
buffer and records the sequence boundaries in an offsets array: offsets[0] = 0 and
offsets[b+1] - offsets[b] is the length of sequence b.  The worked example on the
explore.n1n.ai page (section on the performance defects of padded tensors) packs the
lengths [128, 4096, 512, 2048] into 6784 tokens with offsets [0, 128, 4224, 4736, 6784],
where padding to the longest sequence would need 4 * 4096 = 16384 token slots.
"""

import numpy as np


def offsets_from_lengths(lengths):
    """Exclusive prefix sum of the sequence lengths: offsets[0] = 0,
    offsets[b+1] = offsets[b] + lengths[b].  Returns int64 [B+1]."""
    lengths = [int(x) for x in lengths]
    out = [0]
    for n in lengths:
        if n < 0:
            raise ValueError("negative sequence length")
        out.append(out[-1] + n)
    return np.asarray(out, dtype=np.int64)


def validate_offsets(offsets, total_tokens=None):
    """Offsets intake: offsets[0] must be 0, the array must be non-decreasing and,
    when the packed token count T is given, offsets[B] must equal T.
    Raises ValueError naming the first violated rule."""
    off = [int(x) for x in np.asarray(offsets).reshape(-1)]
    if len(off) < 1:
        raise ValueError("offsets must hold B+1 >= 1 entries")
    if off[0] != 0:
        raise ValueError("offsets[0] must be 0")
    for b in range(len(off) - 1):
        if off[b + 1] < off[b]:
            raise ValueError(f"offsets decrease at index {b + 1}")
    if total_tokens is not None and off[-1] != int(total_tokens):
        raise ValueError("offsets[B] must equal the packed token count")
    return off


def lengths_from_offsets(offsets):
    """Per-sequence lengths L_b = offsets[b+1] - offsets[b] after validation."""
    off = validate_offsets(offsets)
    return np.asarray([off[b + 1] - off[b] for b in range(len(off) - 1)], dtype=np.int64)


def block_offsets(offsets, block=64):
    """Refine sequence boundaries into fixed-size diagonal blocks.

    Block-diagonal attention splits every sequence into consecutive groups of
    ``block`` tokens that attend only within themselves (bittide page, section 1 and
    section 2.1).  Block j of sequence b covers tokens
    [s + block*j, min(s + block*(j+1), e)) with s = offsets[b], e = offsets[b+1]; a
    trailing partial block attends within itself.  Empty sequences contribute no
    block.  Returns the refined int64 offsets."""
    off = validate_offsets(offsets)
    out = [0]
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        t = s
        while t < e:
            t = min(t + block, e)
            out.append(t)
    return np.asarray(out, dtype=np.int64)
