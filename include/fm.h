/*
 * fm.h -- C ABI of libfm: mask-aware (column-interval) attention on AMD MI355X (gfx950).
 *
 * The operation.  Attention softmax(scale * Q K^T + M) V where the mask M is given in
 * the column-wise O(n) form of the FlashMask-3 project page ("FlashMask-3: Efficient
 * and Expressive Mask-Aware Distributed Attention", Overview): every key column j of a
 * batch row carries four int32 query-row bounds LTS_j, LTE_j, UTS_j, UTE_j, and query
 * row i is hidden from key j iff
 *
 *     LTS_j <= i < LTE_j   or   UTS_j <= i < UTE_j        (half-open intervals).
 *
 * Tiles of query rows x key columns are classified from the block-wise min/max of the
 * four vectors (same page, §3.1): fully hidden tiles are skipped, partial tiles get the
 * row-interval mask applied, unmasked tiles run plain.  The forward is the tiled
 * online-softmax attention of "Flash MSA Attention Kernel Implementation: A Practical
 * Guide for Production AI" ("The Flash Core"), returning O and the per-row log-sum-exp;
 * the backward recomputes the probabilities from that statistic (same guide, "The
 * Backward Pass").  Work items are dispatched longest-processing-time first by tile
 * cost {0, alpha_p, alpha_u} (FlashMask-3 page, §3.3).
 *
 * Conventions for every entry point:
 *  - Device pointers.  Every array argument is a pointer to device memory on the
 *    current HIP device, except the fm_problem / fm_mask / fm_tiles structs themselves,
 *    which are host structs (read during the call only).  The caller owns and allocates
 *    all memory: inputs, outputs and the workspace.  The library never allocates device
 *    memory and keeps no state between calls, with one exception: fm_attn_fwd_static
 *    works in a fixed device array the library holds on each GPU for the process.
 *  - Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    their kernels on it and return without synchronizing.
 *  - Layouts (all contiguous, row-major), with N_q = seqlen query rows and N_k =
 *    seqlen_kv keys (N_k = N_q for self-attention):
 *      Q, O, dO, dQ  bf16  [B][H_q][N_q][d]
 *      K, V, dK, dV  bf16  [B][H_kv][N_k][d]
 *      LSE           fp32  [B][H_q][N_q]    natural log; -inf for a row that sees no key
 *      LTS/LTE/UTS/UTE int32 [B][H_m][N_k]  query-row bounds in [0, N_q]; H_m =
 *                                           mask_heads sets per batch row (1: one set
 *                                           shared by all heads)
 *    N_q < N_k is one context-parallel rank's share of the query rows: its chunks,
 *    concatenated in ascending order, against every key, with the vectors renumbered
 *    into its own rows by fm_localize_mask (FlashMask-3 page, §3.2).
 *  - GQA.  Query head h reads kv head h / (H_q / H_kv).
 *  - Per-head masks (a variant the FlashMask-3 page lists among its extensions without
 *    defining it).  Query head h uses vector set h / (H_q / H_m): contiguous groups of
 *    query heads share a set, as for GQA; H_m = H_q gives every query head its own.
 *    Tiles are classified per mask row (b, m), B * H_m of them.
 *  - Rows that see no key get O = 0, LSE = -inf, dQ = 0 and add nothing to dK/dV.
 *  - Errors.  Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is launched and the outputs are untouched.  Vector values outside
 *    [0, N_q] are not checked by the attention calls and give unspecified (but memory-safe)
 *    results; fm_check_mask counts them on the device.  No C++ exception crosses this
 *    interface.
 */
#ifndef FM_H
#define FM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FM_OK = 0,
  FM_ERR_INVALID_ARG = -1, /* null pointer, negative size, H_q % H_kv != 0, bad tile shape */
  FM_ERR_UNSUPPORTED = -2, /* head_dim not 64, 128 or 256, or a size beyond the limits   */
  FM_ERR_WORKSPACE = -3,   /* ws_bytes smaller than fm_workspace_size() reports           */
  FM_ERR_HIP = -4          /* a HIP launch failed                                         */
} fm_status;

typedef enum { FM_OP_CLASSIFY = 0, FM_OP_FWD = 1, FM_OP_BWD = 2 } fm_op;

/* Problem shape.  batch, heads and the lengths may be 0 (nothing to do beyond zero
 * outputs, FM_OK); head_dim d must be 64, 128 or 256.  softmax_scale <= 0 selects 1/sqrt(d).
 * seqlen is N_q; seqlen_kv is N_k, with 0 meaning N_k = N_q (so N_q > 0 rows without
 * keys cannot be expressed; their result is O = 0, LSE = -inf).  mask_heads is H_m, the
 * vector sets per batch row; 0 means 1.  H_m must divide heads_q (when heads_q > 0) and
 * either divide heads_kv or be a multiple of it (so that one kv head's query heads never
 * straddle a mask set boundary partway); otherwise FM_ERR_INVALID_ARG.  Limits: N_q, N_k
 * <= 2^22 and batch * H_m * ceil(N_q/block_q) and batch * H_m * ceil(N_k/block_k) at
 * most 2^24 work blocks per sorted list (lists above 1024 blocks are sorted in chunks and
 * merged, in workspace); larger problems return FM_ERR_UNSUPPORTED. */
typedef struct {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t seqlen;
  int32_t head_dim;
  float softmax_scale;
  int32_t seqlen_kv;
  int32_t mask_heads;
  int32_t key_order; /* FM_KEYS_NATURAL (0) or FM_KEYS_SORTED (1), see fm_key_order */
  int32_t schedule;  /* FM_SCHEDULE_LPT (0) or FM_SCHEDULE_NATURAL (1), see below */
} fm_problem;

/* Dispatch order of the attention kernels' work items (fm_attn_fwd, fm_attn_bwd and their
 * _multi / _blocks / _static forms).  FM_SCHEDULE_LPT: cost-descending, the q_order /
 * k_order of fm_classify_tiles (FlashMask-3 page, §3.3, longest processing time first).
 * FM_SCHEDULE_NATURAL: index order (mask row, then block), for measuring what the LPT order
 * buys; the outputs are the same attention (O, LSE and dQ bit for bit; dK/dV up to the
 * fp32 summation order: the dK/dV split plan grants its extra segments in dispatch order,
 * and atomic additions follow it).
 * fm_classify_tiles always writes the LPT orders.  Other values: FM_ERR_INVALID_ARG. */
#define FM_SCHEDULE_LPT 0
#define FM_SCHEDULE_NATURAL 1

/* Key order of fm_attn_fwd / fm_attn_bwd (four-vector masks).  FM_KEYS_SORTED runs the
 * attention kernels over the keys in the order fm_key_order gives: K, V and the vectors are
 * gathered into that order in the workspace first, dK and dV scattered back after, so every
 * output is in the caller's key order and O, LSE, dQ, dK, dV are the same attention (up to
 * the fp32 summation order).  It pays where the columns' bounds are scattered (a
 * random-eviction mask); on masks whose sorted order is not narrower it only adds the
 * gathers.  With FM_KEYS_SORTED and head_dim = 128 the backward's dK/dV kernel takes 256
 * keys per workgroup (32 x 256 tiles, one 8-wave workgroup per CU): with scattered column
 * ends its Q/dO rows rarely stay in L2, and each row is then read once per 256 keys
 * instead of per 128.  FM_KEYS_SORTED is FM_ERR_UNSUPPORTED with the _multi and _blocks entry points
 * and when mask_heads > heads_kv (one kv head would need two orders).  fm_classify_tiles
 * ignores key_order (it classifies the vectors as given); values other than 0 and 1 are
 * FM_ERR_INVALID_ARG everywhere. */
#define FM_KEYS_NATURAL 0
#define FM_KEYS_SORTED 1

/* The four column vectors, each int32 [B][H_m][N_k] in device memory. */
typedef struct {
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
} fm_mask;

/* Outputs of fm_classify_tiles, all device memory, nQB = ceil(N_q/block_q),
 * nKB = ceil(N_k/block_k), R = B * H_m mask rows (r = b * H_m + m):
 *   block_minmax [R][nKB][8]  int32: min,max of LTS, LTE, UTS, UTE over the block's columns
 *   tile_class   [R][nQB][nKB] uint8: 0 skipped, 1 partial, 2 unmasked
 *   q_queue      [R][nQB][nKB] int32: per Q-block the non-skipped KV blocks, right to left
 *                (descending kb), each entry kb | (partial << 31); then -1 to the end
 *   q_count      [R][nQB][2]   int32: {n_partial, n_unmasked} per Q-block
 *   k_queue      [R][nKB][nQB] int32: per KV block the non-skipped Q-blocks, ascending,
 *                each entry qb | (partial << 31); then -1 to the end
 *   k_count      [R][nKB][2]   int32: {n_partial, n_unmasked} per KV block
 *   q_order      [R*nQB]       int32: Q-blocks (r*nQB + qb) sorted by cost
 *                11*n_partial + 10*n_unmasked descending, ties ascending
 *   k_order      [R*nKB]       int32: the same over KV blocks (r*nKB + kb)          */
typedef struct {
  int32_t* block_minmax;
  uint8_t* tile_class;
  int32_t* q_queue;
  int32_t* q_count;
  int32_t* k_queue;
  int32_t* k_count;
  int32_t* q_order;
  int32_t* k_order;
} fm_tiles;

/* Optional timing hook for fm_attn_fwd / fm_attn_bwd.  Each member is a hipEvent_t
 * created by the caller (hipEventCreate, timing enabled) or NULL.  fm_attn_fwd records
 * `start` immediately before and `stop` immediately after the launch of its attention
 * kernel; fm_attn_bwd records (start, stop) around its dK/dV kernel and (start2, stop2)
 * around its dQ kernel, so hipEventElapsedTime gives each kernel's duration on `stream`.
 * Pass NULL for no timing.  The library keeps no reference after the call returns. */
typedef struct {
  void* start;
  void* stop;
  void* start2;
  void* stop2;
} fm_kernel_events;

/* Workspace bytes an entry point needs for this problem.  For FM_OP_CLASSIFY the tile
 * shape is (block_q, block_k); for FM_OP_FWD / FM_OP_BWD those two arguments are ignored
 * (the kernels' own shapes, see fm_tile_shape, are used).  Writes *bytes; returns
 * FM_ERR_INVALID_ARG / FM_ERR_UNSUPPORTED for problems the op rejects. */
fm_status fm_workspace_size(const fm_problem* p, fm_op op, int32_t block_q, int32_t block_k,
                            size_t* bytes);
/* The same byte count as a return value: 0 when fm_workspace_size would return an error
 * (a problem that needs no workspace also gives 0, so callers that must tell the two apart
 * use fm_workspace_size). */
size_t fm_workspace_bytes(const fm_problem* p, fm_op op, int32_t block_q, int32_t block_k);

/* The tile shape (rows of Q, columns of K per tile) the forward or backward kernel uses
 * and classifies with: 128 x 64 for FM_OP_FWD (also the backward's dQ kernel), 32 x 128
 * for FM_OP_BWD (the dK/dV kernel; 32 x 256 when key_order = FM_KEYS_SORTED and
 * head_dim = 128, see below).  FM_OP_CLASSIFY is invalid here.  Where heads_q / heads_kv
 * and heads_q / mask_heads are both multiples of 4, four query heads of one kv head share
 * a forward (and dQ) workgroup, one per wave, over 32 rows: the forward's tile is then
 * 32 x 64 (same work per tile and workgroup, four times as many Q-blocks and queue rows). */
fm_status fm_tile_shape(fm_op op, int32_t* block_q, int32_t* block_k);

/* Tile classification (FlashMask-3 page, §3.1 tile rule, generalized to all four
 * vectors: skip = (q0 >= max LTS and q1 <= min LTE) or (q0 >= max UTS and q1 <= min UTE);
 * unmasked = (q1 <= min LTS or q0 >= max LTE) and (q1 <= min UTS or q0 >= max UTE);
 * q1 and the block's last column clamped to N), the per-block queues with their tags
 * (§3.1, KV Index Generator), tile costs and the LPT orders (§3.3).  block_q and block_k
 * must be powers of two in [8, 256].  Any N >= 0 is accepted (ragged tails allowed). */
fm_status fm_classify_tiles(const fm_problem* p, const fm_mask* m, int32_t block_q,
                            int32_t block_k, const fm_tiles* out, void* ws, size_t ws_bytes,
                            void* stream);

/* Forward: O (bf16) and LSE (fp32) from Q, K, V (bf16) under the mask.  Classifies
 * internally into `ws` (fm_workspace_size(p, FM_OP_FWD, ...) bytes), then runs the
 * attention kernel over the queued tiles only, in LPT order.  Any N >= 0. */
fm_status fm_attn_fwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const fm_mask* m, void* o, float* lse, void* ws, size_t ws_bytes,
                      void* stream, const fm_kernel_events* events);

/* Forward without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same problem, arguments, outputs and errors as fm_attn_fwd, but the workspace is a
 * device array of FM_STATIC_WORKSPACE_BYTES (16 MiB) that the library holds on every GPU
 * it runs on until the process ends; nothing is allocated or freed by the call.  A
 * problem whose forward workspace (fm_workspace_size(p, FM_OP_FWD, ...)) exceeds that
 * size returns FM_ERR_WORKSPACE and launches nothing: key_order = FM_KEYS_NATURAL covers
 * N_k up to 131072 keys with one mask row (about 8.6 MiB there) at the 128-row forward tile,
 * and up to 65536 keys at the 32-row tile of four packed query heads (about 8.4 MiB);
 * FM_KEYS_SORTED needs room for permuted copies of K and V and rarely fits.  All calls on one GPU share its array:
 * calls that overlap on one GPU (issued on different streams with no ordering between
 * them) race and give undefined results; calls on one stream are safe.  The first call on
 * a device resolves the array's address there (hipGetSymbolAddress); FM_ERR_HIP if that
 * fails, FM_ERR_UNSUPPORTED on a device index of 64 or more. */
#define FM_STATIC_WORKSPACE_BYTES (16u << 20)
fm_status fm_attn_fwd_static(const fm_problem* p, const void* q, const void* k, const void* v,
                             const fm_mask* m, void* o, float* lse, void* stream,
                             const fm_kernel_events* events);

/* Backward: dQ, dK, dV (bf16) from Q, K, V, the forward's O and LSE, and dO.  Classifies
 * internally at both tile shapes (fm_tile_shape(FM_OP_BWD) for dK/dV, FM_OP_FWD for dQ),
 * then runs two kernels that recompute P = exp(S - LSE) on queued tiles only: a
 * Q-block-outer one that also forms D = rowsum(dO * O) (fp32) and accumulates dQ in
 * registers (the forward's LPT order), and a KV-block-outer one accumulating dK and dV
 * (LPT order over KV blocks).  A dK/dV work item covers at most 4 query heads of one kv
 * head that share one mask set; when a kv head's KV block needs more than one item
 * (heads_q / heads_kv above 4, or per-head masks splitting the group), the items add into
 * fp32 accumulators in `ws`, converted to bf16 at the end; otherwise each workgroup stores
 * its bf16 rows directly.  Any N >= 0. */
fm_status fm_attn_bwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, const fm_mask* m,
                      void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream,
                      const fm_kernel_events* events);

/* Dense expansion of rows [row0, row1) of mask row b (b = batch row * H_m + mask set):
 * dense[(i-row0)*N_k + j] = 1 if the mask hides (i, j), else 0 -- the same predicate the
 * attention kernels apply on partial tiles.  For checking only.  0 <= b < batch * H_m,
 * 0 <= row0 <= row1 <= N_q. */
fm_status fm_debug_expand_mask(const fm_problem* p, const fm_mask* m, int32_t b, int32_t row0,
                               int32_t row1, uint8_t* dense, void* stream);

/* Mask localization for one context-parallel rank (FlashMask-3 page, §3.2): the rank
 * owns the query chunks [offsets[i], offsets[i] + chunk_len), i < n_chunks, offsets
 * strictly ascending by at least chunk_len (non-overlapping), and every key.  Each bound
 * x of the global vectors (`global`, int32 [B][H_m][N_k] with values in [0, N]) becomes
 * the number of the rank's rows before global row x, sum_i clamp(x - offsets[i], 0,
 * chunk_len), written to the arrays of `local` (int32 [B][H_m][N_k] each, values in
 * [0, n_chunks * chunk_len]).
 * Theorem 1 of the page: the local intervals select exactly the rank's rows of the global
 * intervals, so attention with p->seqlen = n_chunks * chunk_len local query rows (the
 * chunks' rows of Q concatenated in order) against all N_k keys gives those rows of the
 * global result.  p->seqlen_kv (or p->seqlen when 0) is N_k and p->mask_heads is H_m
 * (0 means 1, any H_m >= 1 accepted here); p->heads_* and head_dim are not used.  offsets: device int32 [n_chunks]; 1 <= n_chunks <= 4096, chunk_len >= 1.
 * Offsets that are not ascending and non-overlapping give unspecified (but memory-safe)
 * results. */
typedef struct {
  int32_t* lts;
  int32_t* lte;
  int32_t* uts;
  int32_t* ute;
} fm_mask_out;

fm_status fm_localize_mask(const fm_problem* p, const fm_mask* global, const int32_t* offsets,
                           int32_t n_chunks, int32_t chunk_len, const fm_mask_out* local,
                           void* stream);

/* Key order of each mask row (this library's own step; the pages classify blocks of
 * consecutive keys only).  Attention does not depend on the order of the key columns, but
 * the tile rule of the FlashMask-3 page (§3.1) sees a block of consecutive columns through
 * the min/max of their bounds, so columns that end at scattered rows (the page's
 * random-eviction mask, §4) leave nearly every tile partial.  Per mask row r and super-block
 * of FM_KEY_ORDER_SPAN consecutive keys [s0, s0 + FM_KEY_ORDER_SPAN) (the last one cut at
 * N_k), the keys are sorted by LTS, ties by key index; the super-block takes that order iff
 * its spread is strictly smaller than the natural order's, where spread = the sum, over
 * groups of FM_KEY_ORDER_GROUP consecutive positions (the last one cut) and over the four
 * vectors, of max - min of the bounds clipped to [0, N_q].  Keys never leave their
 * super-block.
 *   perm      device int32 [B][H_m][N_k], written: position p of row r holds key perm[p]
 *   permuted  NULL, or device arrays (int32 [B][H_m][N_k] each; members may be NULL)
 *             receiving the vectors in that order: permuted->lts[p] = lts[perm[p]], ...
 * p->seqlen (N_q), seqlen_kv, batch and mask_heads are used; heads and head_dim are not.
 * One workgroup per (mask row, super-block); asynchronous on `stream`.  Errors:
 * FM_ERR_INVALID_ARG for null pointers with a non-empty problem. */
#define FM_KEY_ORDER_SPAN 2048
#define FM_KEY_ORDER_GROUP 64
fm_status fm_key_order(const fm_problem* p, const fm_mask* m, int32_t* perm,
                       const fm_mask_out* permuted, void* stream);

/* ---- Multi-interval column masks -------------------------------------------------------
 * The FlashMask Guide ("Multi-Interval Sparse Masks") generalizes the column-wise form to
 * up to 4 active row intervals per key column: key j is visible to query row i iff
 *
 *     start[m][j] <= i < end[m][j]   for some m < n_intervals          (half-open)
 *
 * (the Guide's inclusive end FME is end = FME + 1).  Intervals may be empty (start >= end)
 * or overlap.  start and end are int32 [B][H_m][n_intervals][N_k] in device memory, values
 * in [0, N_q]; H_m = p->mask_heads as for the four-vector form.  Tile rule, from the
 * block-wise min/max of each interval's starts and ends: skip when every interval lies
 * outside the tile's rows in every column (q1 <= min start_m or q0 >= max end_m for all
 * m), unmasked when one interval holds them in every column (q0 >= max start_m and
 * q1 <= min end_m for some m), partial otherwise.
 *
 * The _multi entry points behave exactly as their four-vector counterparts (same problem,
 * arguments, workspace sizes, outputs and errors), except:
 *   - fm_tiles.block_minmax is [R][nKB][4 * n_intervals]: per interval {min start, max
 *     start, min end, max end};
 *   - FM_ERR_INVALID_ARG for n_intervals outside 1..4;
 *   - fm_localize_mask_multi renumbers every start and end (R * n_intervals * N_k each) into
 *     local_start / local_end (device int32, the same shape). */
typedef struct {
  const int32_t* start;
  const int32_t* end;
  int32_t n_intervals;
} fm_mask_multi;

fm_status fm_classify_tiles_multi(const fm_problem* p, const fm_mask_multi* m, int32_t block_q,
                                  int32_t block_k, const fm_tiles* out, void* ws,
                                  size_t ws_bytes, void* stream);
fm_status fm_attn_fwd_multi(const fm_problem* p, const void* q, const void* k, const void* v,
                            const fm_mask_multi* m, void* o, float* lse, void* ws,
                            size_t ws_bytes, void* stream, const fm_kernel_events* events);
fm_status fm_attn_bwd_multi(const fm_problem* p, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* dout,
                            const fm_mask_multi* m, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* stream, const fm_kernel_events* events);
fm_status fm_debug_expand_mask_multi(const fm_problem* p, const fm_mask_multi* m, int32_t b,
                                     int32_t row0, int32_t row1, uint8_t* dense, void* stream);
fm_status fm_localize_mask_multi(const fm_problem* p, const fm_mask_multi* global,
                                 const int32_t* offsets, int32_t n_chunks, int32_t chunk_len,
                                 int32_t* local_start, int32_t* local_end, void* stream);

/* ---- Block-sparse masks ------------------------------------------------------------------
 * The block-sparse family (listed on the FlashMask-3 page among the masks of packed
 * long-context batches): a grid of 128 x 128 blocks over (query rows, keys), each block
 * wholly visible (1) or wholly hidden (0); the last block row and column may be cut by N_q
 * and N_k.  blocks: uint8 [B][H_m][ceil(N_q/128)][ceil(N_k/128)] in device memory (H_m =
 * p->mask_heads, as for the other forms).  Every tile of the attention kernels lies inside
 * one block, so tiles are only skipped or unmasked (keys past N_k stay hidden); the
 * classifier's tile of up to 256 x 256 is partial when it straddles blocks of both kinds.
 * The _blocks entry points behave exactly as their four-vector counterparts (same problem,
 * arguments, workspace sizes, outputs and errors), except that fm_tiles.block_minmax is not
 * written (it must still be a valid pointer) and a null `blocks` with a non-empty grid is
 * FM_ERR_INVALID_ARG.  There is no localization for this form. */
typedef struct {
  const uint8_t* blocks;
} fm_mask_blocks;

fm_status fm_classify_tiles_blocks(const fm_problem* p, const fm_mask_blocks* m, int32_t block_q,
                                   int32_t block_k, const fm_tiles* out, void* ws,
                                   size_t ws_bytes, void* stream);
fm_status fm_attn_fwd_blocks(const fm_problem* p, const void* q, const void* k, const void* v,
                             const fm_mask_blocks* m, void* o, float* lse, void* ws,
                             size_t ws_bytes, void* stream, const fm_kernel_events* events);
fm_status fm_attn_bwd_blocks(const fm_problem* p, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout,
                             const fm_mask_blocks* m, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, void* stream, const fm_kernel_events* events);
fm_status fm_debug_expand_mask_blocks(const fm_problem* p, const fm_mask_blocks* m, int32_t b,
                                      int32_t row0, int32_t row1, uint8_t* dense, void* stream);

/* Range check of the mask (a debugging aid; the attention entry points do not check values).
 * Writes to *bad (device int32, cleared first) the number of row bounds outside [0, N_q]:
 * over the four vectors, or over the interval starts and ends of the multi-interval form
 * (R * n_intervals * N_k each).  Asynchronous on `stream`, no host synchronization and no
 * allocation; read *bad after the stream has reached it.  A nonzero count means the
 * attention results for that mask are unspecified (though memory-safe).  p->seqlen (N_q),
 * seqlen_kv, batch and mask_heads are used.  FM_ERR_INVALID_ARG for null pointers (the
 * arrays may be null only for an empty mask) and, for the multi form, n_intervals outside
 * 1..4. */
fm_status fm_check_mask(const fm_problem* p, const fm_mask* m, int32_t* bad, void* stream);
fm_status fm_check_mask_multi(const fm_problem* p, const fm_mask_multi* m, int32_t* bad,
                              void* stream);

/* Static description of a status code. */
const char* fm_status_string(fm_status s);

/* ---- Chunk balancing for context parallelism (host code, no GPU) ----------------------
 * Stage 1 of HCC-IPO (FlashMask-3 page, §3.3 "Balance the work, not the length", and its
 * IPO ablation table): n_chunks = ranks * kappa chunk loads are assigned to `ranks`
 * ranks, exactly kappa each, minimising the makespan (largest rank load).  Phases: LPT
 * under the cardinality constraint, exact pairwise repartition (P2, stages >= 2), and
 * exact three-rank repartition (P3, stages = 3), repeated until no move improves or the
 * makespan reaches LB = max(ceil(sum / ranks), max weight), which certifies optimality.
 * The page gives no pseudo-code; the move order and tie-breaks are fixed in fm_ipo.cpp.
 *
 *   weights  host, [n_chunks] int64, each >= 0 (e.g. summed tile costs of a query chunk)
 *   owner    host, [n_chunks] int32, written: the rank of each chunk
 *   report   host, written: lb, makespans after LPT / after the first P2 pass / final,
 *            certified (final == lb), moves (repartitions applied)
 * Errors: FM_ERR_INVALID_ARG for null pointers, ranks or n_chunks <= 0, n_chunks not a
 * multiple of ranks, a negative weight, stages outside 1..3; FM_ERR_UNSUPPORTED for
 * kappa > FM_IPO_MAX_KAPPA (the exact repartitions search 3 * kappa chunks).  Runs
 * synchronously on the calling thread; nothing is allocated on the device. */
#define FM_IPO_MAX_KAPPA 16
typedef struct {
  int64_t lb;
  int64_t makespan_lpt;
  int64_t makespan_p2;
  int64_t makespan;
  int32_t certified;
  int32_t moves;
} fm_ipo_report;

fm_status fm_ipo_balance(const int64_t* weights, int32_t n_chunks, int32_t ranks, int32_t stages,
                         int32_t* owner, fm_ipo_report* report);

#ifdef __cplusplus
}
#endif

#endif /* FM_H */
