"""CPU oracle for mask-aware (column-interval) attention.  TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy code in float64.  It shares no code with the
HIP library in `mask_aware_sparse_amd/`: no kernels, headers, tables, constants or
helpers, and neither side imports the other.  Only `tests/`, the `smoke()` check in
`__graft_entry__.py` and the `cpu_baseline` leg of `bench.py` may import it; the
product path never does.

Contents and the passage each part follows:

  mask.py       dense expansion of the four column vectors (FlashMask-3 page,
                Overview: per-key row bounds LTS/LTE/UTS/UTE); conversion from the
                two-vector visible-interval form and its closed-form encoders
                (FlashMask Guide, "Mathematical Formalization of Column-Wise
                Sparsity"); the multi-interval form, up to 4 active row intervals
                per column (same Guide, "Multi-Interval Sparse Masks"); the block-sparse
                form, a grid of 128 x 128 blocks each visible or hidden (the
                block-sparse family the FlashMask-3 page lists).
  attention.py  masked softmax attention forward (plain two-pass softmax) and its
                analytic backward (Flash MSA guide, "Why Standard Attention Broke"
                and "The Backward Pass: The Real Beast"; FlashMask Guide, dense
                additive-mask formula).
  tiles.py      block min/max, tile classification, per-block queues, tile costs
                and the cost-descending (LPT) order (FlashMask-3 page, §3.1 tile
                rule and KV Index Generator; §3.3 tile costs; FlashMask Guide,
                "On-Chip Block-Skipping Logic").
  localize.py   renumbering of the row bounds into one context-parallel rank's own
                rows (FlashMask-3 page, §3.2, Theorem 1).
  ipo.py        stage-1 chunk balancing over ranks: LPT, pairwise and three-rank
                repartition (FlashMask-3 page, §3.3 and the IPO ablation table).
  keyorder.py   reordering of the key columns within super-blocks so that columns
                with similar bounds share tiles (this library's own step; attention
                is invariant under a joint permutation of K, V and the vectors).
  schedule.py   list scheduling of weighted work items over P slots, the lower
                bound max(ceil(sum/P), max w) and a brute-force optimum
                (FlashMask-3 page, §3.3 and the IPO ablation table).

Readings taken where the pages are silent (the main ones): masked intervals are
half-open; rows masked everywhere give O = 0, LSE = -inf,
dQ = 0 and add nothing to dK/dV; query head h uses kv head h // (H_q/H_kv);
the softmax scale is 1/sqrt(d) and appears in dQ and dK by the chain rule.

Every function is pinned by a `-m "not gpu"` test against something other than
itself (printed mask pictures, closed forms, library routines on special cases,
brute force, invariants); see tests/test_oracle_*.py.  Full-size numeric outputs
have no printed values on the pages: beyond those pins they are parity unpinned.
"""
from .mask import (masked_rows, dense_mask, visible_interval_to_vectors,
                   encode_causal, encode_packed, encode_dpo, hidden_multi_rows,
                   dense_mask_multi, hidden_block_rows, dense_mask_blocks, BLOCK)
from .attention import (attention_fwd, attention_bwd, attention_rows, attention_cols,
                        attention_fwd_bwd, attention_fwd_multi, attention_fwd_bwd_multi,
                        attention_rows_multi, attention_cols_multi, attention_fwd_blocks,
                        attention_fwd_bwd_blocks, attention_rows_blocks, attention_cols_blocks)
from .tiles import (block_minmax, classify, tile_truth, queues, tile_costs, lpt_order,
                    block_minmax_multi, classify_multi, tile_truth_multi, classify_blocks,
                    tile_truth_blocks,
                    ALPHA_PARTIAL, ALPHA_UNMASKED)
from .schedule import list_schedule, lower_bound, brute_force_optimum
from .localize import rank_rows, localize, localize_max_form, localize_vectors
from .keyorder import key_order, key_order_rows, spread
from . import ipo

__all__ = [
    "masked_rows", "dense_mask", "visible_interval_to_vectors", "encode_causal",
    "encode_packed", "encode_dpo", "hidden_multi_rows", "dense_mask_multi",
    "hidden_block_rows", "dense_mask_blocks", "BLOCK", "attention_fwd_blocks",
    "attention_fwd_bwd_blocks", "attention_rows_blocks", "attention_cols_blocks",
    "classify_blocks", "tile_truth_blocks",
    "attention_fwd", "attention_bwd", "attention_rows", "attention_cols",
    "attention_fwd_bwd", "attention_fwd_multi", "attention_fwd_bwd_multi",
    "attention_rows_multi", "attention_cols_multi", "block_minmax", "classify",
    "tile_truth", "block_minmax_multi", "classify_multi", "tile_truth_multi",
    "queues", "tile_costs", "lpt_order", "ALPHA_PARTIAL", "ALPHA_UNMASKED",
    "list_schedule", "lower_bound", "brute_force_optimum", "rank_rows", "localize",
    "localize_max_form", "localize_vectors", "ipo", "key_order", "key_order_rows", "spread",
]
