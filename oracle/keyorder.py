"""Key reordering within super-blocks (oracle; test infrastructure only).

Softmax attention does not depend on the order of the key columns: permuting K, V and
the four column vectors together, and permuting dK and dV back, leaves O, LSE, dQ, dK and
dV unchanged.  The tile rule of the FlashMask-3 page (§3.1) classifies blocks of
*consecutive* columns from the min/max of their bounds, so a mask whose columns end at
scattered rows (the random-eviction mask of the page's §4 mask list: LTS_j drawn at
random) leaves almost every tile partial.  Grouping columns with similar bounds into the
same tile turns most of those tiles into skipped or unmasked ones.  The pages do not
describe this step; it is this library's own, and this module is its definition.

The rule, per mask row, over super-blocks of S consecutive keys [s0, s0 + S) (the last
one ragged):
  * candidate "sorted": the super-block's keys in ascending order of LTS, ties by key
    index (a stable sort);
  * spread(order) = sum over groups of G consecutive positions of that order (the last
    group ragged) and over the four vectors x of max(clip(x, 0, N_q)) - min(clip(x, 0,
    N_q)) over the group -- the number of query rows over which the group's tile is
    partial on each bound, summed;
  * the super-block takes the sorted order iff its spread is strictly smaller than the
    natural order's; otherwise it keeps the natural order.
perm[s0 + p] = the key placed at position s0 + p; keys never leave their super-block.
"""
import numpy as np


def spread(vectors, nq, group):
    """Sum over consecutive groups of `group` positions, and over the vectors, of the
    group's range max - min after clipping to [0, nq]."""
    total = 0
    n = len(vectors[0])
    for g0 in range(0, n, group):
        for x in vectors:
            seg = np.clip(np.asarray(x[g0:g0 + group], dtype=np.int64), 0, nq)
            total += int(seg.max() - seg.min())
    return total


def key_order(lts, lte, uts, ute, nq, span=2048, group=64):
    """The key permutation of one mask row (int64 [N_k]): position p holds key perm[p]."""
    vecs = [np.asarray(x, dtype=np.int64) for x in (lts, lte, uts, ute)]
    n = len(vecs[0])
    perm = np.arange(n, dtype=np.int64)
    for s0 in range(0, n, span):
        natural = np.arange(s0, min(s0 + span, n), dtype=np.int64)
        srt = natural[np.argsort(vecs[0][natural], kind="stable")]
        if spread([x[srt] for x in vecs], nq, group) < spread([x[natural] for x in vecs], nq, group):
            perm[s0:s0 + len(natural)] = srt
    return perm


def key_order_rows(lts, lte, uts, ute, nq, span=2048, group=64):
    """key_order over every mask row of [..., N_k] vectors; returns the same shape."""
    vecs = [np.asarray(x, dtype=np.int64) for x in (lts, lte, uts, ute)]
    shape = vecs[0].shape
    flat = [x.reshape(-1, shape[-1]) for x in vecs]
    out = np.stack([key_order(*(x[r] for x in flat), nq, span, group)
                    for r in range(flat[0].shape[0])]) if flat[0].shape[0] else \
        np.zeros((0, shape[-1]), dtype=np.int64)
    return out.reshape(shape)
