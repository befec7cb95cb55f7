"""Zero-communication mask localization for one context-parallel rank (oracle; test
infrastructure only).

FlashMask-3 page, §3.2: every rank holds every key column of the O(n) mask and only
renumbers each row bound into its own rows, by a purely local count.  A rank owning
the query chunks [O_i, O_i + C), i = 0 .. k-1 with O_0 < O_1 < ... (non-overlapping),
maps a global row bound x to

    x_local = number of the rank's rows before global row x = sum_i clip(x - O_i, 0, C).

The page prints this as max_i [clip(x - O_i, 0, C) + i C 1(clip > 0)] (garbled in the
extracted text); with sorted, non-overlapping chunks the two agree, which the tests
check.  Theorem 1 there: the localized intervals select exactly the global intervals'
rows, so the rank's kernel sees the global mask restricted to its rows.
"""
import numpy as np


def rank_rows(offsets, chunk_len):
    """Global row index of each local row of the rank, in local order."""
    return np.concatenate([np.arange(o, o + chunk_len, dtype=np.int64)
                           for o in sorted(int(x) for x in offsets)]) \
        if len(offsets) else np.zeros(0, dtype=np.int64)


def localize(x, offsets, chunk_len):
    """Sum form: x_local = sum_i clip(x - O_i, 0, C), elementwise over the array x."""
    x = np.asarray(x, dtype=np.int64)
    out = np.zeros_like(x)
    for o in offsets:
        out += np.clip(x - int(o), 0, chunk_len)
    return out


def localize_max_form(x, offsets, chunk_len):
    """The page's printed form: max over chunks i (ascending offsets) of
    clip(x - O_i, 0, C) + i C [clip > 0], and 0 when no chunk starts before x."""
    x = np.asarray(x, dtype=np.int64)
    out = np.zeros_like(x)
    for i, o in enumerate(sorted(int(v) for v in offsets)):
        c = np.clip(x - o, 0, chunk_len)
        out = np.maximum(out, c + i * chunk_len * (c > 0))
    return out


def localize_vectors(vectors, offsets, chunk_len):
    """All four vectors [B][N_k] of a batch: each bound renumbered into the rank's rows."""
    return tuple(localize(v, offsets, chunk_len).astype(np.int32) for v in vectors)
