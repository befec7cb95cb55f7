"""Dense expansion of the column-wise mask (oracle; test infrastructure only).

FlashMask-3 page, Overview: each key column j stores four query-row bounds
LTS_j, LTE_j, UTS_j, UTE_j.  Reading adopted (the page prints no membership
formula): the hidden rows of column j are the half-open intervals [LTS_j, LTE_j)
and [UTS_j, UTE_j); an interval whose start is not below its end is empty.
"""
import numpy as np


def masked_rows(lts, lte, uts, ute, r0, r1):
    """Boolean [r1-r0][N] block of the dense mask for one batch row: True = hidden.

    masked(i, j) = (LTS_j <= i < LTE_j) or (UTS_j <= i < UTE_j)."""
    i = np.arange(r0, r1, dtype=np.int64)[:, None]
    lts = np.asarray(lts, dtype=np.int64)[None, :]
    lte = np.asarray(lte, dtype=np.int64)[None, :]
    uts = np.asarray(uts, dtype=np.int64)[None, :]
    ute = np.asarray(ute, dtype=np.int64)[None, :]
    return ((lts <= i) & (i < lte)) | ((uts <= i) & (i < ute))


def dense_mask(lts, lte, uts, ute):
    """Full N x N dense mask for one batch row (small N only)."""
    n = len(lts)
    return masked_rows(lts, lte, uts, ute, 0, n)


def hidden_multi_rows(starts, ends, r0, r1):
    """Multi-interval form (FlashMask Guide, "Multi-Interval Sparse Masks"): each key
    column j carries M <= 4 active intervals, and row i sees key j iff
    starts[m][j] <= i < ends[m][j] for some m.  Reading adopted: half-open like the
    four-vector form (the Guide's inclusive end FME is ends = FME + 1); an interval
    whose start is not below its end is empty; the intervals need not be disjoint.
    Returns the boolean [r1-r0][N] block with True = hidden (no interval holds the row)."""
    starts = np.asarray(starts, dtype=np.int64)
    ends = np.asarray(ends, dtype=np.int64)
    i = np.arange(r0, r1, dtype=np.int64)[:, None]
    visible = np.zeros((r1 - r0, starts.shape[-1]), dtype=bool)
    for m in range(starts.shape[0]):
        visible |= (starts[m][None, :] <= i) & (i < ends[m][None, :])
    return ~visible


def dense_mask_multi(starts, ends, nq=None):
    """Full dense mask (True = hidden) of the multi-interval form, [N_q][N_k]."""
    n = np.asarray(starts).shape[-1] if nq is None else nq
    return hidden_multi_rows(starts, ends, 0, n)


def visible_interval_to_vectors(fms, fme, n):
    """FlashMask Guide, "Mathematical Formalization of Column-Wise Sparsity": key
    column j is visible to rows FMS_j <= i <= FME_j (inclusive).  In the four-vector
    form the hidden rows are [0, FMS_j) and [FME_j + 1, N):
    UTS = 0, UTE = FMS, LTS = FME + 1, LTE = N."""
    fms = np.asarray(fms, dtype=np.int64)
    fme = np.asarray(fme, dtype=np.int64)
    uts = np.zeros_like(fms)
    ute = fms.copy()
    lts = np.minimum(fme + 1, n)
    lte = np.full_like(fms, n)
    return lts, lte, uts, ute


def encode_causal(n):
    """Causal closed form (FlashMask Guide, same section): FMS_j = j, FME_j = N-1."""
    j = np.arange(n)
    return j.copy(), np.full(n, n - 1)


def encode_packed(lengths, causal=True):
    """Packed documents (FlashMask Guide, "Mathematical Formalization of Column-Wise
    Sparsity", the document closed form): a key j inside document k, which spans rows
    [s_k, e_k] (inclusive), is visible from FMS_j = j (causal) or s_k (bidirectional) down
    to FME_j = e_k.  Each document's start and last row are repeated over its keys."""
    lengths = np.asarray(lengths, dtype=np.int64)
    ends = np.cumsum(lengths)                       # one past each document's last row
    starts = ends - lengths
    doc_start = np.repeat(starts, lengths)          # s_k of the document holding key j
    fme = np.repeat(ends - 1, lengths)              # e_k
    fms = np.arange(int(ends[-1]) if len(ends) else 0, dtype=np.int64) if causal else doc_start
    return fms, fme


def encode_dpo(prompt, chosen, rejected):
    """DPO pair [prompt | chosen | rejected] (same section): prompt keys are
    visible from j to the end of the sequence; chosen keys from j to the end of
    the chosen span; rejected keys from j to the end of the sequence."""
    n = prompt + chosen + rejected
    fms = np.arange(n, dtype=np.int64)
    fme = np.empty(n, dtype=np.int64)
    fme[:prompt] = n - 1
    fme[prompt:prompt + chosen] = prompt + chosen - 1
    fme[prompt + chosen:] = n - 1
    return fms, fme


BLOCK = 128  # block edge of the block-sparse form


def hidden_block_rows(blocks, r0, r1, nk):
    """Block-sparse form (the block-sparse family the FlashMask-3 page lists among packed
    long-context masks): a grid of BLOCK x BLOCK blocks, blocks[qb][kb] = 1 if every
    (row, key) of the block is visible, 0 if every one is hidden; the last block row and
    column may be cut by N_q and N_k.  Returns the boolean [r1-r0][N_k] block of the
    dense mask, True = hidden."""
    blocks = np.asarray(blocks)
    qb = np.arange(r0, r1) // BLOCK
    kb = np.arange(nk) // BLOCK
    return blocks[qb][:, kb] == 0


def dense_mask_blocks(blocks, nq, nk):
    """Full dense mask (True = hidden) of the block-sparse form, [N_q][N_k]."""
    return hidden_block_rows(blocks, 0, nq, nk)
