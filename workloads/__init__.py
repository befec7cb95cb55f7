"""Seeded synthetic inputs for mask-aware attention: mask vectors and Q/K/V/dO.

This module is shared by the CPU oracle and the HIP path.  It builds inputs only:
it holds none of the method's arithmetic (no masking predicate, no tile rule, no
softmax).  Every workload is a procedure on a seed, so the same seed gives the same
bytes on every machine.

Mask encoding.  Each key column j carries four int32 row bounds
(LTS_j, LTE_j, UTS_j, UTE_j); the rows of column j that are hidden are the two
half-open intervals [LTS_j, LTE_j) and [UTS_j, UTE_j).  This is the column-wise
O(n) representation named in the Overview of "FlashMask-3: Efficient and Expressive
Mask-Aware Distributed Attention".  Unless a workload says otherwise UTS = 0 and
LTE = N, the common case in which the upper interval holds the rows above the
diagonal band and the lower interval the rows below it.

The mask families are the ones the pages list (document packing, prefix-LM,
share-question / DPO, sliding window with sinks, random eviction: FlashMask-3 page,
Overview and Results; FlashMask Guide, "The Diversity of Real-World Attention
Masks").  The pages give families, not procedures; the procedures below are the
plainest readings, fixed once so that runs are reproducible.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

HEAD_DIM = 128


@dataclass
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    lts: np.ndarray          # int32 [B][N], or [B][H_m][N] for per-head sets
    lte: np.ndarray
    uts: np.ndarray
    ute: np.ndarray
    seed: int
    info: dict = field(default_factory=dict)

    def vectors(self):
        return self.lts, self.lte, self.uts, self.ute

    @property
    def mask_heads(self) -> int:
        """Vector sets per batch row (1 unless the vectors are [B][H_m][N])."""
        return 1 if self.lts.ndim == 2 else self.lts.shape[1]


@dataclass
class MultiWorkload:
    """Multi-interval form: each key column is visible on up to 4 row intervals
    [start_m, end_m).  starts/ends are int32 [B][M][N] (shared by every head) or
    [B][H_m][M][N] (per-head sets)."""
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    starts: np.ndarray
    ends: np.ndarray
    seed: int
    info: dict = field(default_factory=dict)

    def intervals(self):
        return self.starts, self.ends

    @property
    def n_intervals(self) -> int:
        return self.starts.shape[-2]

    @property
    def mask_heads(self) -> int:
        return 1 if self.starts.ndim == 3 else self.starts.shape[1]


@dataclass
class BlockWorkload:
    """Block-sparse form: uint8 blocks [B][nQB][nKB] (or [B][H_m][nQB][nKB]) over 128 x 128
    blocks, 1 = visible, 0 = hidden; nQB = ceil(N / 128)."""
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    blocks: np.ndarray
    seed: int
    info: dict = field(default_factory=dict)

    @property
    def mask_heads(self) -> int:
        return 1 if self.blocks.ndim == 3 else self.blocks.shape[1]


BLOCK = 128


def _empty_vectors(batch: int, n: int):
    lts = np.full((batch, n), n, dtype=np.int64)
    lte = np.full((batch, n), n, dtype=np.int64)
    uts = np.zeros((batch, n), dtype=np.int64)
    ute = np.zeros((batch, n), dtype=np.int64)
    return lts, lte, uts, ute


def _finish(name, batch, hq, hkv, n, vecs, seed, info):
    lts, lte, uts, ute = (np.ascontiguousarray(v, dtype=np.int32) for v in vecs)
    return Workload(name, batch, hq, hkv, n, HEAD_DIM, lts, lte, uts, ute, seed, info)


def causal_doc(seed: int = 0, n: int = 1024, ndocs: int = 4, batch: int = 1,
               heads_q: int = 1, heads_kv: int = 1) -> Workload:
    """Causal document packing: `ndocs` documents whose lengths come from
    `ndocs-1` distinct sorted cut points.  Key j of document [s, e) is hidden
    from rows >= e (LTS=e, LTE=N) and from rows < j (UTS=0, UTE=j)."""
    rng = np.random.default_rng(seed)
    lts, lte, uts, ute = _empty_vectors(batch, n)
    docs = []
    for b in range(batch):
        cuts = np.sort(rng.choice(np.arange(1, n), ndocs - 1, replace=False))
        bounds = np.r_[0, cuts, n]
        docs.append(np.diff(bounds).tolist())
        for s, e in zip(bounds[:-1], bounds[1:]):
            j = np.arange(s, e)
            lts[b, s:e] = e
            ute[b, s:e] = j
    return _finish("causal_doc", batch, heads_q, heads_kv, n, (lts, lte, uts, ute), seed,
                   {"doc_lengths": docs})


def prefix_lm_doc(seed: int = 0, n: int = 8192, batch: int = 4, heads_q: int = 32,
                  heads_kv: int = 8, lo: int = 512, hi: int = 2048,
                  prefix_frac: float = 0.25) -> Workload:
    """Prefix-LM document packing.  Document lengths are drawn uniformly in
    [lo, hi] until they cover N; the last one is cut to fit.  Each document
    [s, e) has a bidirectional prefix of floor(L/4) keys (visible to every row
    of the document: UTE=s) followed by causal keys (UTE=j); no key is visible
    outside its document (LTS=e)."""
    rng = np.random.default_rng(seed)
    lts, lte, uts, ute = _empty_vectors(batch, n)
    docs = []
    for b in range(batch):
        s = 0
        lens = []
        while s < n:
            length = min(int(rng.integers(lo, hi + 1)), n - s)
            e = s + length
            p = int(length * prefix_frac)
            lts[b, s:e] = e
            ute[b, s:s + p] = s
            ute[b, s + p:e] = np.arange(s + p, e)
            lens.append(length)
            s = e
        docs.append(lens)
    return _finish("prefix_lm_doc", batch, heads_q, heads_kv, n, (lts, lte, uts, ute), seed,
                   {"doc_lengths": docs})


def share_question(seed: int = 0, n: int = 32768, batch: int = 1, heads_q: int = 64,
                   heads_kv: int = 1, samples: int = 4, answers: int = 3,
                   prompt_range=(2048, 4096), answer_range=(1024, 2048)) -> Workload:
    """Share-question (DPO-style) packing: `samples` packed samples, each a causal
    prompt followed by `answers` causal answers that see the prompt but not each
    other.  Lengths are redrawn together until they fit in N; the tail is padding
    whose keys are hidden from every row (UTE=N), so padding rows see nothing."""
    rng = np.random.default_rng(seed)
    lts, lte, uts, ute = _empty_vectors(batch, n)
    layout = []
    for b in range(batch):
        while True:
            P = rng.integers(prompt_range[0], prompt_range[1] + 1, samples)
            A = rng.integers(answer_range[0], answer_range[1] + 1, (samples, answers))
            if int(P.sum() + A.sum()) <= n:
                break
        s = 0
        for k in range(samples):
            e = s + int(P[k]) + int(A[k].sum())
            lts[b, s:s + P[k]] = e
            ute[b, s:s + P[k]] = np.arange(s, s + P[k])
            a0 = s + int(P[k])
            for a in range(answers):
                a1 = a0 + int(A[k, a])
                lts[b, a0:a1] = a1
                ute[b, a0:a1] = np.arange(a0, a1)
                a0 = a1
            s = e
        ute[b, s:] = n                    # padding keys: hidden from all rows
        layout.append({"prompts": P.tolist(), "answers": A.tolist(), "pad_start": s,
                       "pad": n - s})
    return _finish("share_question", batch, heads_q, heads_kv, n, (lts, lte, uts, ute), seed,
                   {"layout": layout})


def sliding_window_sinks(seed: int = 0, n: int = 131072, batch: int = 1, heads_q: int = 64,
                         heads_kv: int = 1, window: int = 4096, sinks: int = 64) -> Workload:
    """Causal sliding window plus global sink keys.  Key j is hidden from rows < j
    (UTE=j) and, unless it is one of the first `sinks` keys, from rows
    >= j + window (LTS=min(j+window, N)).  Deterministic; `seed` is recorded only."""
    lts, lte, uts, ute = _empty_vectors(batch, n)
    j = np.arange(n)
    for b in range(batch):
        ute[b] = j
        lts[b] = np.minimum(j + window, n)
        lts[b, :sinks] = n
    return _finish("sliding_window_sinks", batch, heads_q, heads_kv, n, (lts, lte, uts, ute),
                   seed, {"window": window, "sinks": sinks})


def random_eviction(seed: int = 0, n: int = 131072, batch: int = 1, heads_q: int = 64,
                    heads_kv: int = 1) -> Workload:
    """Random-eviction causal mask: key j is visible to rows j .. LTS_j-1, where
    LTS_j is uniform on [j+1, N] (one draw per key, in key order)."""
    rng = np.random.default_rng(seed)
    lts, lte, uts, ute = _empty_vectors(batch, n)
    j = np.arange(n)
    for b in range(batch):
        lts[b] = rng.integers(j + 1, n + 1)
        ute[b] = j
    return _finish("random_eviction", batch, heads_q, heads_kv, n, (lts, lte, uts, ute), seed, {})


def causal(n: int, batch: int = 1, heads_q: int = 1, heads_kv: int = 1) -> Workload:
    """Plain causal attention: key j hidden from rows < j only."""
    lts, lte, uts, ute = _empty_vectors(batch, n)
    ute[:] = np.arange(n)
    return _finish("causal", batch, heads_q, heads_kv, n, (lts, lte, uts, ute), 0, {})


def full_attention(n: int, batch: int = 1, heads_q: int = 1, heads_kv: int = 1) -> Workload:
    """No key hidden from any row: every tile is unmasked."""
    return _finish("full_attention", batch, heads_q, heads_kv, n, _empty_vectors(batch, n), 0, {})


def full_attention_partial_tiles(n: int, batch: int = 1, heads_q: int = 1,
                                 heads_kv: int = 1) -> Workload:
    """No key hidden from any row, yet every tile of at least two columns is classified
    partial: even columns carry the empty lower interval [0, 0) and odd columns [N, N),
    so each KV block's minimum LTS is 0 and its maximum LTE is N.  The same attention as
    full_attention() with the mask path switched on everywhere (timing the cost of a
    partial tile against an unmasked one)."""
    lts, lte, uts, ute = _empty_vectors(batch, n)
    odd = (np.arange(n) % 2) == 1
    lts[:, ~odd] = 0
    lte[:, ~odd] = 0
    return _finish("full_attention_partial_tiles", batch, heads_q, heads_kv, n,
                   (lts, lte, uts, ute), 0, {})


def random_intervals(seed: int, n: int, batch: int = 1, heads_q: int = 1,
                     heads_kv: int = 1, p_empty: float = 0.2, mask_heads: int = 0) -> Workload:
    """Adversarial vectors: both intervals of every column are random, may be
    empty (start >= end), may cover every row, and may overlap.  mask_heads > 0 draws
    that many independent sets per batch row ([B][H_m][N])."""
    rng = np.random.default_rng(seed)
    shape = (batch, n) if mask_heads <= 0 else (batch, mask_heads, n)
    a = rng.integers(0, n + 1, (4,) + shape)
    lts = np.minimum(a[0], a[1]); lte = np.maximum(a[0], a[1])
    uts = np.minimum(a[2], a[3]); ute = np.maximum(a[2], a[3])
    e1 = rng.random(shape) < p_empty
    e2 = rng.random(shape) < p_empty
    lts = np.where(e1, lte, lts)            # empty lower interval (start == end)
    uts = np.where(e2, ute + 1, uts)         # empty upper interval (start > end)
    uts = np.minimum(uts, n)
    return _finish("random_intervals", batch, heads_q, heads_kv, n, (lts, lte, uts, ute), seed, {})


def per_head_windows(seed: int = 0, n: int = 32768, batch: int = 1, heads_q: int = 32,
                     heads_kv: int = 8, mask_heads: int = 8, windows=None,
                     sinks: int = 64) -> Workload:
    """Per-head masks: causal sliding windows whose width differs by head, local heads
    next to global ones.  Set m hides key j from rows < j and, unless j is one of the
    first `sinks` keys, from rows >= j + W_m, with W_m = windows[m % len(windows)]
    (default n/64, n/32, n/16, n/8, n/4, n/2 and two global causal sets).  The work per
    head therefore differs by up to 30x.  Deterministic; `seed` is recorded only."""
    if windows is None:
        windows = [n // 64, n // 32, n // 16, n // 8, n // 4, n // 2, n, n]
    lts, lte, uts, ute = (np.repeat(x[:, None, :], mask_heads, axis=1)
                          for x in _empty_vectors(batch, n))
    j = np.arange(n)
    for m in range(mask_heads):
        w = int(windows[m % len(windows)])
        ute[:, m] = j
        lts[:, m] = np.minimum(j + w, n)
        lts[:, m, :sinks] = n
    return _finish("per_head_windows", batch, heads_q, heads_kv, n, (lts, lte, uts, ute), seed,
                   {"windows": [int(windows[m % len(windows)]) for m in range(mask_heads)],
                    "sinks": sinks})


def with_head_dim(w, d: int):
    """The same workload (mask, heads, lengths) at head dimension d."""
    return replace(w, head_dim=int(d), name=f"{w.name}_d{int(d)}")


def _finish_multi(name, batch, hq, hkv, n, starts, ends, seed, info):
    return MultiWorkload(name, batch, hq, hkv, n, HEAD_DIM,
                         np.ascontiguousarray(starts, dtype=np.int32),
                         np.ascontiguousarray(ends, dtype=np.int32), seed, info)


def random_multi_intervals(seed: int, n: int, batch: int = 1, heads_q: int = 1,
                           heads_kv: int = 1, n_intervals: int = 3, mask_heads: int = 0,
                           p_empty: float = 0.2) -> MultiWorkload:
    """Adversarial multi-interval columns: every interval random in [0, N], possibly
    empty (start >= end), covering every row, or overlapping another."""
    rng = np.random.default_rng(seed)
    shape = ((batch,) if mask_heads <= 0 else (batch, mask_heads)) + (n_intervals, n)
    a = rng.integers(0, n + 1, (2,) + shape)
    starts, ends = np.minimum(a[0], a[1]), np.maximum(a[0], a[1])
    empty = rng.random(shape) < p_empty
    starts = np.where(empty, ends, starts)
    return _finish_multi("random_multi_intervals", batch, heads_q, heads_kv, n, starts, ends,
                         seed, {})


def block_sparse_window(seed: int = 0, n: int = 32768, batch: int = 1, heads_q: int = 32,
                        heads_kv: int = 8, window: int = 2048, rand_blocks: int = 3,
                        block: int = 128, sinks: int = 64) -> MultiWorkload:
    """Causal local window plus random distant query blocks, written column-wise with
    four intervals (a block-sparse pattern of the kind the pages list, in the
    multi-interval form).  Key j sees rows [j, j + window) (interval 0; the first
    `sinks` keys see every row from j on); each block of `block` keys is also seen by
    `rand_blocks` query blocks of `block` rows drawn without replacement from those
    past its window (intervals 1..3, empty where there are too few)."""
    rng = np.random.default_rng(seed)
    M = 1 + rand_blocks
    starts = np.zeros((batch, M, n), dtype=np.int64)
    ends = np.zeros((batch, M, n), dtype=np.int64)
    j = np.arange(n)
    nb = n // block
    for b in range(batch):
        starts[b, 0] = j
        ends[b, 0] = np.minimum(j + window, n)
        ends[b, 0, :sinks] = n
        for kb in range(nb):
            first = (kb * block + block + window + block - 1) // block   # past the window
            cand = np.arange(first, nb)
            pick = np.sort(rng.choice(cand, size=min(rand_blocks, len(cand)), replace=False))
            for t, qb in enumerate(pick):
                starts[b, 1 + t, kb * block:(kb + 1) * block] = qb * block
                ends[b, 1 + t, kb * block:(kb + 1) * block] = (qb + 1) * block
    return _finish_multi("block_sparse_window", batch, heads_q, heads_kv, n, starts, ends, seed,
                         {"window": window, "rand_blocks": rand_blocks, "block": block,
                          "sinks": sinks})


def random_blocks(seed: int, n: int, batch: int = 1, heads_q: int = 1, heads_kv: int = 1,
                  density: float = 0.3, mask_heads: int = 0) -> BlockWorkload:
    """Adversarial block grids: every 128 x 128 block visible with probability `density`,
    including whole block rows that see nothing (ragged last row and column when N is not a
    multiple of 128)."""
    rng = np.random.default_rng(seed)
    nb = -(-n // BLOCK)
    shape = ((batch,) if mask_heads <= 0 else (batch, mask_heads)) + (nb, nb)
    blocks = (rng.random(shape) < density).astype(np.uint8)
    return BlockWorkload("random_blocks", batch, heads_q, heads_kv, n, HEAD_DIM,
                         np.ascontiguousarray(blocks), seed, {"density": density})


def bigbird_blocks(seed: int = 0, n: int = 32768, batch: int = 1, heads_q: int = 32,
                   heads_kv: int = 8, window: int = 1, globals_: int = 1,
                   randoms: int = 3) -> BlockWorkload:
    """Block-sparse pattern of the BigBird kind on 128 x 128 blocks: each block row sees the
    blocks within `window` of the diagonal, the first `globals_` block columns, and
    `randoms` further blocks drawn per row; the first `globals_` block rows see every
    block."""
    rng = np.random.default_rng(seed)
    nb = -(-n // BLOCK)
    blocks = np.zeros((batch, nb, nb), dtype=np.uint8)
    for b in range(batch):
        for qb in range(nb):
            blocks[b, qb, max(0, qb - window):min(nb, qb + window + 1)] = 1
            blocks[b, qb, :globals_] = 1
            rest = np.nonzero(blocks[b, qb] == 0)[0]
            pick = rng.choice(rest, size=min(randoms, len(rest)), replace=False)
            blocks[b, qb, pick] = 1
        blocks[b, :globals_, :] = 1
    return BlockWorkload("bigbird_blocks", batch, heads_q, heads_kv, n, HEAD_DIM, blocks, seed,
                         {"window": window, "globals": globals_, "randoms": randoms})


# The five benchmark workloads, in order.  Shapes and mask families follow the
# synthetic stand-ins for the mask families the FlashMask-3 page benchmarks.
CONFIGS = {
    "c1_causal_doc_1k": lambda seed=0: causal_doc(seed),
    "c2_prefix_lm_doc_8k": lambda seed=0: prefix_lm_doc(seed),
    "c3_share_question_32k": lambda seed=0: share_question(seed),
    "c4_sliding_window_128k": lambda seed=0: sliding_window_sinks(seed),
    "c5_random_eviction_128k": lambda seed=0: random_eviction(seed),
}
CONFIG_NAMES = list(CONFIGS)

# Variants beyond the five (widening the mask family the same kernels take).
VARIANTS = {
    # per-head masks: 32 query heads, 8 kv heads, one window per kv head's group
    "v1_per_head_windows_32k": lambda seed=0: per_head_windows(seed),
    # multi-interval columns: local window + three random distant query blocks per key block
    "v2_block_sparse_window_32k": lambda seed=0: block_sparse_window(seed),
    # head dimension 64: the prefix-LM document workload (B=4, 32/8 heads, N=8192) at d=64
    "v3_prefix_lm_doc_8k_d64": lambda seed=0: with_head_dim(prefix_lm_doc(seed), 64),
    # block-sparse masks: BigBird-style 128 x 128 block grid (window, global, random blocks)
    "v4_bigbird_blocks_32k": lambda seed=0: bigbird_blocks(seed),
    # head dimension 256: the prefix-LM document workload (B=4, 32/8 heads, N=8192) at d=256
    "v5_prefix_lm_doc_8k_d256": lambda seed=0: with_head_dim(prefix_lm_doc(seed), 256),
}
VARIANT_NAMES = list(VARIANTS)


def make_workload(name: str, seed: int = 0) -> Workload:
    return (CONFIGS[name] if name in CONFIGS else VARIANTS[name])(seed)


def make_tensors(w: Workload, seed: int | None = None, device: str = "cpu",
                 need_grad_inputs: bool = True):
    """Q, K, V, dO as bf16 drawn N(0,1) in that order, rounded to nearest even.

    On the CPU the draws come from torch's CPU generator seeded with `seed`; on a
    GPU device from that device's generator with the same seed (the large
    workloads are drawn where they live).  Callers hand the *same* tensors to the
    oracle (as host copies) and to the HIP path, so parity never depends on the
    two generators agreeing."""
    import torch
    seed = w.seed if seed is None else seed
    g = torch.Generator(device=device).manual_seed(seed)
    shp_q = (w.batch, w.heads_q, w.seqlen, w.head_dim)
    shp_k = (w.batch, w.heads_kv, w.seqlen, w.head_dim)

    def draw(shape):
        return torch.randn(shape, dtype=torch.float32, generator=g, device=device).to(torch.bfloat16)

    q = draw(shp_q)
    k = draw(shp_k)
    v = draw(shp_k)
    do = draw(shp_q) if need_grad_inputs else None
    return q, k, v, do


def mask_tensors(w, device: str = "cpu"):
    """The mask as tensors: the four int32 vectors of a Workload, (starts, ends) of a
    MultiWorkload, or (blocks,) (uint8) of a BlockWorkload."""
    import torch
    if isinstance(w, BlockWorkload):
        return (torch.from_numpy(np.ascontiguousarray(w.blocks)).to(device),)
    arrs = w.intervals() if isinstance(w, MultiWorkload) else w.vectors()
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(device) for x in arrs)


# Per-row factors of the mixed-magnitude inputs (applied to the shared half of each query
# row) and the values of the random halves: all exact in bf16, and every product and every
# sum of 128 products is exact in fp32 (multiples of 1/4 below 2^22).
MIXED_FACTORS = (-32.0, -24.0, -8.0, -1.0, 0.5, 1.0, 8.0, 24.0, 32.0)
RANDOM_HALF_VALUES = (-1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5)


def extreme_logit_tensors(w: Workload, kind: str, seed: int = 0, device: str = "cpu"):
    """Q, K, V, dO whose scores lie far from zero, for the numerics of the online softmax.

    The first d/2 dimensions of every key row of a kv head hold one random +-1 pattern
    (shared by all its keys); the other d/2 hold values drawn from RANDOM_HALF_VALUES per
    key.  A query row is [factor * pattern of its kv head, its own random half] (query
    head h uses kv head h // (H_q / H_kv)).  So q.k = factor * d/2 + r.k', an exact
    multiple of 1/4 in fp32, with r.k' of spread 8 giving the keys different weights:
      "low"   factor -32: q.k = -2048 + r.k' (|r.k'| <= 144), so at the default scale
              s * log2(e) / sqrt(128) lies in [-280, -243];
      "high"  factor +32: the same with the shared part's sign reversed;
      "mixed" a factor per query row drawn from MIXED_FACTORS.
    The random halves keep dQ = scale * sum_j dS_ij K_j away from the cancellation of the
    shared half (sum_j dS_ij = 0).  V and dO are N(0,1) rounded to bf16.  Draws come from
    one CPU generator seeded with `seed`."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    B, Hq, Hkv, N, d = w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim
    h = d // 2
    vals = torch.tensor(RANDOM_HALF_VALUES)
    pat = (torch.randint(0, 2, (B, Hkv, 1, h), generator=g) * 2 - 1).float()
    k = torch.cat([pat.expand(B, Hkv, N, h),
                   vals[torch.randint(0, len(vals), (B, Hkv, N, d - h), generator=g)]], dim=-1)
    qpat = pat.repeat_interleave(Hq // Hkv, dim=1).expand(B, Hq, N, h)
    if kind == "low":
        fac = torch.full((B, Hq, N, 1), -32.0)
    elif kind == "high":
        fac = torch.full((B, Hq, N, 1), 32.0)
    elif kind == "mixed":
        idx = torch.randint(0, len(MIXED_FACTORS), (B, Hq, N, 1), generator=g)
        fac = torch.tensor(MIXED_FACTORS)[idx]
    else:
        raise ValueError(f"unknown kind {kind!r}")
    q = torch.cat([fac * qpat,
                   vals[torch.randint(0, len(vals), (B, Hq, N, d - h), generator=g)]], dim=-1)
    v = torch.randn((B, Hkv, N, d), generator=g)
    do = torch.randn((B, Hq, N, d), generator=g)
    return tuple(t.to(torch.bfloat16).contiguous().to(device) for t in (q, k, v, do))
