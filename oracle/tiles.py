"""Tile classification, queues, costs and LPT order (oracle; test infrastructure).

FlashMask-3 page, §3.1 ("A third warp role that reads the mask"): for a tile of
query rows [q0, q1) and a KV block, the block-wise max/min of the vectors decide
whether the tile is skipped, unmasked or partial; the KV Index Generator emits,
per Q-block, a queue of the KV blocks that are not skipped, each tagged partial or
unmasked, visited right to left.  §3.3: a tile costs 0 (skipped), alpha_p
(partial) or alpha_u (unmasked), with alpha_u = 1 and alpha_p = 1.3 given as
illustrative values.  The FlashMask Guide ("On-Chip Block-Skipping Logic") states
the same rule in the two-vector form.

The page prints the rule for the LTS/UTE pair only (it assumes LTE = N and
UTS = 0).  Reading adopted for all four vectors, which reduces to the printed rule
in that case and is sound for any vectors:

  skip     = (q0 >= max LTS and q1 <= min LTE) or (q0 >= max UTS and q1 <= min UTE)
  unmasked = (q1 <= min LTS or q0 >= max LTE) and (q1 <= min UTS or q0 >= max UTE)
  class    = 0 if skip, else 2 if unmasked, else 1 (partial)

q1 and the block's last column are clamped to N (ragged tails).  The class is the
rule's output: a tile the rule calls partial may still be hidden everywhere when
both intervals cover it together (the rule is conservative, never unsound).
"""
import numpy as np

from .mask import BLOCK, hidden_block_rows, hidden_multi_rows, masked_rows

SKIP, PARTIAL, UNMASKED = 0, 1, 2
# alpha_p : alpha_u in integer units.  The FlashMask-3 page (§3.3) calls its 1.3 : 1
# illustrative; the weights used here are the ratio measured on MI355X for these kernels
# (a partial tile with nothing hidden against an unmasked tile on identical work: 1.11
# forward, 1.08 dQ, 1.05 dK/dV), rounded to 1.1 : 1.
ALPHA_PARTIAL = 11
ALPHA_UNMASKED = 10


def _nblocks(n, b):
    return (n + b - 1) // b


def block_minmax(vec, bk):
    """min and max of one vector [B][N] over each KV block -> two arrays [B][nKB]."""
    vec = np.asarray(vec, dtype=np.int64)
    B, N = vec.shape
    nkb = _nblocks(N, bk)
    mn = np.zeros((B, nkb), dtype=np.int64)
    mx = np.zeros((B, nkb), dtype=np.int64)
    for b in range(B):
        for kb in range(nkb):
            seg = vec[b, kb * bk:min((kb + 1) * bk, N)]
            mn[b, kb] = seg.min()
            mx[b, kb] = seg.max()
    return mn, mx


def classify(lts, lte, uts, ute, bq, bk, nq=None):
    """Tile class [B][nQB][nKB] (uint8: 0 skip, 1 partial, 2 unmasked) for nq query
    rows (default: as many as key columns) and the vectors' key columns.

    For each batch row and KV block the rule is evaluated for all Q-blocks at once
    (q0, q1 as arrays)."""
    B, Nk = np.asarray(lts).shape
    N = Nk if nq is None else nq
    nqb, nkb = _nblocks(N, bq), _nblocks(Nk, bk)
    (mnLTS, mxLTS), (mnLTE, mxLTE), (mnUTS, mxUTS), (mnUTE, mxUTE) = (
        block_minmax(x, bk) for x in (lts, lte, uts, ute))
    q0 = np.arange(nqb, dtype=np.int64) * bq
    q1 = np.minimum(q0 + bq, N)
    cls = np.zeros((B, nqb, nkb), dtype=np.uint8)
    for b in range(B):
        for kb in range(nkb):
            skip = (((q0 >= mxLTS[b, kb]) & (q1 <= mnLTE[b, kb])) |
                    ((q0 >= mxUTS[b, kb]) & (q1 <= mnUTE[b, kb])))
            unmasked = (((q1 <= mnLTS[b, kb]) | (q0 >= mxLTE[b, kb])) &
                        ((q1 <= mnUTS[b, kb]) | (q0 >= mxUTE[b, kb])))
            cls[b, :, kb] = np.where(skip, SKIP, np.where(unmasked, UNMASKED, PARTIAL))
    return cls


def tile_truth(lts, lte, uts, ute, bq, bk, nq=None):
    """Brute force from the dense mask: 0 if every cell of the tile is hidden, 2 if
    none is, 1 otherwise.  The rule's class must agree wherever it says 0 or 2."""
    lts, lte, uts, ute = (np.asarray(x) for x in (lts, lte, uts, ute))
    B, Nk = lts.shape
    N = Nk if nq is None else nq
    nqb, nkb = _nblocks(N, bq), _nblocks(Nk, bk)
    out = np.zeros((B, nqb, nkb), dtype=np.uint8)
    for b in range(B):
        for qb in range(nqb):
            q0, q1 = qb * bq, min(qb * bq + bq, N)
            hid = masked_rows(lts[b], lte[b], uts[b], ute[b], q0, q1)
            for kb in range(nkb):
                t = hid[:, kb * bk:min(kb * bk + bk, Nk)]
                out[b, qb, kb] = SKIP if t.all() else (UNMASKED if not t.any() else PARTIAL)
    return out


def block_minmax_multi(starts, ends, bk):
    """Multi-interval form, starts/ends [R][M][N_k]: [R][nKB][4M] int64 holding, for
    each interval m, (min start, max start, min end, max end) over the block's columns."""
    starts = np.asarray(starts, dtype=np.int64)
    ends = np.asarray(ends, dtype=np.int64)
    R, M, _ = starts.shape
    parts = []
    for m in range(M):
        mn_s, mx_s = block_minmax(starts[:, m], bk)
        mn_e, mx_e = block_minmax(ends[:, m], bk)
        parts += [mn_s, mx_s, mn_e, mx_e]
    return np.stack(parts, axis=-1)


def classify_multi(starts, ends, bq, bk, nq=None):
    """Tile class [R][nQB][nKB] for the multi-interval form (FlashMask Guide,
    "Multi-Interval Sparse Masks": a column is visible on M <= 4 row intervals).  The
    Guide gives the skip test for one interval (skip when the rows lie past every
    column's end or before every column's start); reading adopted for M intervals,
    from the block min/max of each interval's starts and ends:

      skip     = for every m: q1 <= min start_m  or  q0 >= max end_m
                 (no interval reaches the tile in any column)
      unmasked = for some m:  q0 >= max start_m and q1 <= min end_m
                 (one interval holds the tile's rows in every column)
      class    = 0 if skip, else 2 if unmasked, else 1

    Sound for any vectors (empty or overlapping intervals only make it conservative)."""
    mm = block_minmax_multi(starts, ends, bk)
    R, M, Nk = np.asarray(starts).shape
    N = Nk if nq is None else nq
    nqb, nkb = _nblocks(N, bq), _nblocks(Nk, bk)
    q0 = np.arange(nqb, dtype=np.int64) * bq
    q1 = np.minimum(q0 + bq, N)
    cls = np.zeros((R, nqb, nkb), dtype=np.uint8)
    for r in range(R):
        for kb in range(nkb):
            skip = np.ones(nqb, dtype=bool)
            unmasked = np.zeros(nqb, dtype=bool)
            for m in range(M):
                mn_s, mx_s, mn_e, mx_e = mm[r, kb, 4 * m:4 * m + 4]
                skip &= (q1 <= mn_s) | (q0 >= mx_e)
                unmasked |= (q0 >= mx_s) & (q1 <= mn_e)
            cls[r, :, kb] = np.where(skip, SKIP, np.where(unmasked, UNMASKED, PARTIAL))
    return cls


def tile_truth_multi(starts, ends, bq, bk, nq=None):
    """Brute force from the dense multi-interval mask: 0 all hidden, 2 none, 1 else."""
    starts, ends = np.asarray(starts), np.asarray(ends)
    R, M, Nk = starts.shape
    N = Nk if nq is None else nq
    nqb, nkb = _nblocks(N, bq), _nblocks(Nk, bk)
    out = np.zeros((R, nqb, nkb), dtype=np.uint8)
    for r in range(R):
        for qb in range(nqb):
            q0, q1 = qb * bq, min(qb * bq + bq, N)
            hid = hidden_multi_rows(starts[r], ends[r], q0, q1)
            for kb in range(nkb):
                t = hid[:, kb * bk:min(kb * bk + bk, Nk)]
                out[r, qb, kb] = SKIP if t.all() else (UNMASKED if not t.any() else PARTIAL)
    return out


def classify_blocks(blocks, bq, bk, nq, nk):
    """Tile class [R][nQB][nKB] for the block-sparse form (blocks [R][ceil(nq/128)]
    [ceil(nk/128)]): a tile is skipped when every block it overlaps is hidden, unmasked
    when every one is visible, and partial otherwise (a tile that straddles blocks of
    both kinds).  Exact by construction: blocks are uniformly visible or hidden."""
    blocks = np.asarray(blocks)
    R = blocks.shape[0]
    nqb, nkb = _nblocks(nq, bq), _nblocks(nk, bk)
    cls = np.zeros((R, nqb, nkb), dtype=np.uint8)
    for r in range(R):
        for qb in range(nqb):
            b0, b1 = qb * bq // BLOCK, (min(qb * bq + bq, nq) - 1) // BLOCK + 1
            for kb in range(nkb):
                c0, c1 = kb * bk // BLOCK, (min(kb * bk + bk, nk) - 1) // BLOCK + 1
                sub = blocks[r, b0:b1, c0:c1]
                cls[r, qb, kb] = SKIP if not sub.any() else (UNMASKED if sub.all() else PARTIAL)
    return cls


def tile_truth_blocks(blocks, bq, bk, nq, nk):
    """Brute force from the dense block-sparse mask: 0 all hidden, 2 none, 1 else."""
    blocks = np.asarray(blocks)
    R = blocks.shape[0]
    nqb, nkb = _nblocks(nq, bq), _nblocks(nk, bk)
    out = np.zeros((R, nqb, nkb), dtype=np.uint8)
    for r in range(R):
        for qb in range(nqb):
            q0, q1 = qb * bq, min(qb * bq + bq, nq)
            hid = hidden_block_rows(blocks[r], q0, q1, nk)
            for kb in range(nkb):
                t = hid[:, kb * bk:min(kb * bk + bk, nk)]
                out[r, qb, kb] = SKIP if t.all() else (UNMASKED if not t.any() else PARTIAL)
    return out


def queues(cls):
    """Queues and counts from the class matrix.

    Forward (per Q-block, KV blocks visited right to left as in §3.1's example):
      q_queue[b][qb] = [kb | partial << 31 for kb = nKB-1 .. 0 if class != skip]
      q_count[b][qb] = (n_partial, n_unmasked)
    Backward (per KV block, Q-blocks in ascending order; a reading, the pages give
    no order for it):
      k_queue[b][kb] = [qb | partial << 31 for qb = 0 .. nQB-1 if class != skip]
      k_count[b][kb] = (n_partial, n_unmasked)
    Queues are returned as int32 arrays padded with -1 after their last entry."""
    cls = np.asarray(cls)
    B, nqb, nkb = cls.shape
    tag = np.int64(1 << 31)
    q_queue = np.full((B, nqb, nkb), -1, dtype=np.int64)
    q_count = np.zeros((B, nqb, 2), dtype=np.int32)
    k_queue = np.full((B, nkb, nqb), -1, dtype=np.int64)
    k_count = np.zeros((B, nkb, 2), dtype=np.int32)
    for b in range(B):
        for qb in range(nqb):
            row = cls[b, qb]
            kbs = np.nonzero(row != SKIP)[0][::-1]           # right to left
            q_queue[b, qb, :len(kbs)] = kbs + np.where(row[kbs] == PARTIAL, tag, 0)
            q_count[b, qb] = ((row == PARTIAL).sum(), (row == UNMASKED).sum())
        for kb in range(nkb):
            col = cls[b, :, kb]
            qbs = np.nonzero(col != SKIP)[0]                  # ascending
            k_queue[b, kb, :len(qbs)] = qbs + np.where(col[qbs] == PARTIAL, tag, 0)
            k_count[b, kb] = ((col == PARTIAL).sum(), (col == UNMASKED).sum())
    as_i32 = lambda a: np.where(a < 0, -1, a).astype(np.uint32).view(np.int32)
    return as_i32(q_queue), q_count, as_i32(k_queue), k_count


def tile_costs(count, alpha_p=ALPHA_PARTIAL, alpha_u=ALPHA_UNMASKED):
    """cost = alpha_p * n_partial + alpha_u * n_unmasked (skipped tiles cost 0)."""
    count = np.asarray(count, dtype=np.int64)
    return alpha_p * count[..., 0] + alpha_u * count[..., 1]


def lpt_order(costs):
    """Longest-processing-time-first order of the flattened items: indices sorted
    by cost descending, ties by ascending index (so (b, block) ascending)."""
    c = np.asarray(costs, dtype=np.int64).reshape(-1)
    idx = list(range(len(c)))
    idx.sort(key=lambda i: (-c[i], i))
    return np.asarray(idx, dtype=np.int32)
