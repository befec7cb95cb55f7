// Host-side declarations shared by the libfm translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fm {

// Head dimensions the kernels are built for.  D = 256 runs one workgroup per CU (its LDS
// tiles take 143 KB); the others two.
inline bool head_dim_supported(int d) { return d == 64 || d == 128 || d == 256; }

// Tile shapes of the attention kernels.  The forward (and the backward's dQ kernel) uses
// 128 query rows (4 waves x 32) by 64 keys; the backward's dK/dV kernel 32 query rows by
// 128 keys (4 waves x 32 keys, two workgroups per CU).
constexpr int kFwdBlockQ = 128;
constexpr int kFwdBlockK = 64;
constexpr int kBwdBlockQ = 32;
constexpr int kBwdBlockK = 128;
// With sorted keys at D = 128 the dK/dV kernel takes 256 keys per workgroup (8 waves, one
// workgroup per CU): the Q/dO rows of its steps rarely stay in L2 there, and reading each
// row once per 256 keys halves those bytes.
constexpr int kBwdBlockKWide = 256;
inline int bwd_block_k(int D, bool sorted_keys) {
  return sorted_keys && D == 128 ? kBwdBlockKWide : kBwdBlockK;
}
// Forward and dQ workgroups are 4 waves of 32 query rows.  Where every four consecutive
// query heads share a kv head and a mask set, a workgroup takes the same 32 rows of four
// heads (one per wave) instead of 128 rows of one head: Q-blocks of 32 rows, so tiles of
// 32 x 64 that follow the mask more closely, at the same work per workgroup and tile.
constexpr int kFwdPack = 4;
inline int fwd_pack(int Hq, int Hkv, int Hm) {
  if (Hq <= 0 || Hkv <= 0 || Hm <= 0) return 1;
  return (Hq / Hkv) % kFwdPack == 0 && (Hq / Hm) % kFwdPack == 0 ? kFwdPack : 1;
}
inline int fwd_block_q(int pack) { return kFwdBlockQ / pack; }
// Query heads handled by one backward work item (dK/dV of a KV block are summed over
// these heads in registers, then added across items with fp32 atomics).
constexpr int kBwdHeadChunk = 4;
// Tile costs in integer units, alpha_partial : alpha_unmasked = 1.1 : 1: the FlashMask-3
// page's 1.3 : 1 (§3.3) is illustrative; 1.1 is the measured cost of a partial tile of these
// kernels against an unmasked one on identical work (1.11 fwd, 1.08 dQ, 1.05 dK/dV).
constexpr int kAlphaPartial = 11;
constexpr int kAlphaUnmasked = 10;
// The LPT sort: up to 1024 64-bit keys in one workgroup's LDS; longer lists in chunks of
// that size, merged pass by pass through a scratch buffer of lpt_sort_scratch_bytes(count)
// bytes.  Lists are limited to kMaxWorkItems entries.  The dK/dV split plan runs in one
// workgroup over at most kMaxSortItems (mask row, KV block) pairs.
constexpr int kMaxSortItems = 8192;
constexpr int64_t kMaxWorkItems = 1 << 24;
// Splitting of long dK/dV work items.  A (mask row, KV block) pair whose queue is long
// against the average load per workgroup slot is cut into at most kSplitMaxSegs segments
// of its queue; at most kSplitExtraUnits extra workgroups are added per launch.  Where the
// kernel would store bf16 directly, the segments write fp32 partial sums (one slot of
// kBwdBlockK x D per segment and tensor) that a reduction kernel adds in segment order.
constexpr int kSplitMaxSegs = 16;
constexpr int kSplitExtraUnits = 512;
constexpr int kSplitMinSteps = 16;   // no segment shorter than this many tile steps

// How query heads, kv heads and mask sets relate.  The vectors are [B][Hm][Nk]; query
// head h uses set h / (Hq / Hm), and Hm divides Hkv or is a multiple of it.  Tiles are
// classified per mask row (b, m).  A dK/dV work item is (mask row, KV block, kv head of
// that set, chunk of at most kBwdHeadChunk query heads of that kv head and set).
struct HeadMap {
  int Hm;       // mask sets per batch row
  int qpm;      // query heads per set
  int kvpm;     // kv heads per set (1 when a set covers part of one kv head's group)
  int gq;       // query heads of one (kv head, set) pair
  int hc;       // query heads per dK/dV item
  int cpk;      // dK/dV items per (mask row, kv head, KV block)
  int writers;  // dK/dV items writing one kv head's KV block (> 1: fp32 accumulators)
};
inline bool head_map_valid(int Hq, int Hkv, int Hm) {
  if (Hm < 1 || Hkv < 1) return false;
  if (Hq > 0 && Hq % Hm != 0) return false;
  return Hkv % Hm == 0 || Hm % Hkv == 0;
}
inline HeadMap head_map(int Hq, int Hkv, int Hm) {
  HeadMap m{};
  m.Hm = Hm;
  m.qpm = Hq / Hm;
  m.kvpm = Hm <= Hkv ? Hkv / Hm : 1;
  const int g = Hq / Hkv;
  m.gq = g < m.qpm ? g : m.qpm;
  m.hc = m.gq < kBwdHeadChunk ? (m.gq > 0 ? m.gq : 1) : kBwdHeadChunk;
  m.cpk = (m.gq + m.hc - 1) / m.hc;
  m.writers = m.gq > 0 ? (g / m.gq) * m.cpk : 0;
  return m;
}

struct MaskPtrs {
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
};

// The mask as the kernels take it: the four-vector form (n == 0; rows of Nk per vector),
// the multi-interval form (n = 1..4 visible intervals per column; start/end [rows][n][Nk])
// or, for the classifier only, the block-sparse form (n == kBlocksMode; blocks [rows]
// [ceil(Nq/128)][ceil(Nk/128)], 1 = visible).  The attention kernels run a block-sparse
// mask as the four-vector form with all-zero vectors (nothing hidden inside a block; keys
// past Nk are hidden by the kernels' own bound).
constexpr int kMaxIntervals = 4;
constexpr int kBlocksMode = -1;
constexpr int kMaskBlock = 128;
struct MaskArgs {
  MaskPtrs v;
  const int32_t* start;
  const int32_t* end;
  int n;
  const uint8_t* blocks;
  int grid_rows;  // block rows of the grid: ceil(Nq / kMaskBlock)
};
// int32 values per KV block in the block min/max array: 8 (min, max of each of the four
// vectors) or 4 n (min start, max start, min end, max end of each interval).  Workspaces
// reserve the largest.
inline int minmax_width(int n) { return n == 0 ? 8 : 4 * n; }
constexpr int kMaxMinmaxWidth = 4 * kMaxIntervals;

// Classification outputs (B here counts mask rows); any of the optional outputs may be null.
struct TileOut {
  int32_t* minmax;       // [B][nKB][minmax_width(n)]  (required)
  uint8_t* tile_class;   // [B][nQB][nKB]              (optional)
  int32_t* q_queue;      // [B][nQB][nKB]              (optional)
  int32_t* q_count;      // [B][nQB][2]                (required if q_queue)
  int32_t* q_cost;       // [B*nQB]                    (required if q_queue)
  int32_t* k_queue;      // [B][nKB][nQB]              (optional)
  int32_t* k_count;      // [B][nKB][2]                (required if k_queue)
  int32_t* k_cost;       // [B*nKB]                    (required if k_queue)
};

// Nq query rows (Q-blocks of bq), Nk keys (KV blocks of bk); B mask rows.
hipError_t launch_classify(const MaskArgs& m, int B, int Nq, int Nk, int bq, int bk,
                           const TileOut& out, hipStream_t s);
// The backward's two classifications in fewer launches: K-side queues (out_k.k_queue) at
// bq_k x bk_k and Q-side queues (out_q.q_queue) at bq_q x bk_q; one block min/max pass
// where the K side's blocks are a multiple of the Q side's, then one classify launch.
hipError_t launch_classify_pair(const MaskArgs& m, int B, int Nq, int Nk, int bq_k, int bk_k,
                                const TileOut& out_k, int bq_q, int bk_q, const TileOut& out_q,
                                hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, size_t n, hipStream_t s);
// order[i] = i for i < n: the natural dispatch order (fm_problem.schedule)
hipError_t launch_iota_i32(int32_t* p, int n, hipStream_t s);
size_t lpt_sort_scratch_bytes(int64_t count);
hipError_t launch_lpt_sort(const int32_t* cost, int32_t* order, int count, void* scratch,
                           hipStream_t s);
// Two LPT orders; one launch when both lists are short (at most 1024 items), else two sorts.
hipError_t launch_lpt_sort_pair(const int32_t* cost0, int32_t* order0, int count0,
                                const int32_t* cost1, int32_t* order1, int count1,
                                void* scratch, hipStream_t s);
hipError_t launch_expand_mask(const MaskArgs& m, int b, int Nk, int row0, int row1,
                              uint8_t* dense, hipStream_t s);

struct MaskOut {
  int32_t* lts;
  int32_t* lte;
  int32_t* uts;
  int32_t* ute;
};
// Renumber `cols` row bounds of each of the first `arrays` (2 or 4) arrays of g into the
// rank's rows.
// Number of values of `arrays` (2 or 4) arrays of `cols` int32 outside [0, hi] into *bad.
hipError_t launch_check_bounds(const MaskPtrs& g, int arrays, int64_t cols, int hi, int32_t* bad,
                               hipStream_t s);
hipError_t launch_localize(const MaskPtrs& g, int arrays, const int32_t* offsets, int n_chunks,
                           int chunk_len, const MaskOut& out, int64_t cols, hipStream_t s);

// Key reordering (an option of the attention entry points): per mask row and super-block
// of kKeyOrderSpan keys, the keys sorted by LTS where that narrows the spread of bounds
// over groups of kKeyOrderGroup positions.  perm [rows][Nk]: position p holds key
// perm[p]; `permuted` (members may be null) receives the vectors in that order.
constexpr int kKeyOrderSpan = 2048;
constexpr int kKeyOrderGroup = 64;
hipError_t launch_key_order(const MaskPtrs& m, int rows, int Nq, int Nk, int32_t* perm,
                            const MaskOut& permuted, hipStream_t s);
// Rows of two [B][Hkv][Nk][D] bf16 tensors moved into (gather) or out of (scatter) the key
// order of perm; kv head h uses mask set h / (Hkv / Hm), Hm dividing Hkv.
hipError_t launch_permute_rows(bool scatter, const void* src0, const void* src1, void* dst0,
                               void* dst1, const int32_t* perm, int B, int Hkv, int Hm, int Nk,
                               int D, hipStream_t s);

// Compute units of the current device (queried once per device and cached).
int device_cu_count();

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  MaskArgs m;
  void* o;
  float* lse;
  const int32_t* q_queue;
  const int32_t* q_count;
  const int32_t* q_order;
  int B, Hq, Hkv, Hm, Nq, Nk, nQB, nKB;  // Hm: mask sets per batch row
  int D;                                 // head dimension: 64, 128 or 256
  int pack;                              // query heads per workgroup: fwd_pack(...)
  float scale;
};
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  MaskArgs m;
  void* dq;
  void* dk;
  void* dv;
  // KV-block-outer tiles (dK/dV kernel): tile kBwdBlockQ x kBwdBlockK
  const int32_t* k_queue;
  const int32_t* k_count;
  const int32_t* k_order;
  // Q-block-outer tiles (dQ kernel): the forward's tile fwd_block_q(pack) x kFwdBlockK
  const int32_t* q_queue;
  const int32_t* q_count;
  const int32_t* q_order;
  float* lse2;   // [B][Hq][Nq] log2-domain LSE (+inf for rows that see nothing)
  float* delta;  // [B][Hq][Nq] rowsum(dO * O)
  float* dk_acc; // [B][Hkv][Nk][D] fp32, only when head_map(...).writers > 1 (else null)
  float* dv_acc; // [B][Hkv][Nk][D] fp32, likewise
  // dK/dV work units (split plan): unit_pair / unit_slot [pairs + extra], split_pair /
  // split_slot [extra], counts[2] = {units, split pairs}; partials [2][slots][BK][D] fp32
  // (only when writers == 1)
  int32_t* unit_pair;
  int32_t* unit_slot;
  int32_t* split_pair;
  int32_t* split_slot;
  int32_t* split_counts;
  float* partials;
  int split_extra;   // extra pair units allowed (0: no splitting)
  int B, Hq, Hkv, Hm, Nq, Nk;
  int D;             // head dimension: 64 or 128
  int bk;            // keys per dK/dV workgroup: bwd_block_k(D, sorted keys)
  int nQB_k, nKB_k;  // block counts at the dK/dV tile
  int nQB_q, nKB_q;  // block counts at the dQ (forward) tile
  int pack;          // query heads per dQ workgroup: fwd_pack(...)
  float scale;
};
// Extra pair units of the split plan for `per` workgroups per pair, and the partial slots
// it can use (each split pair takes s >= 2 segments of `per` slots, s - 1 of them extra).
inline int split_extra_pairs(int per, int64_t pair_units) {
  if (per <= 0 || pair_units > kMaxSortItems) return 0;  // the plan runs in one workgroup
  int64_t e = kSplitExtraUnits / per;
  const int64_t cap = pair_units;  // never more than doubles the work units
  return (int)(e < cap ? e : cap);
}
inline int split_slots(int per, int extra) { return 2 * extra * per; }

struct BwdEvents {
  hipEvent_t dkdv_start, dkdv_stop, dq_start, dq_stop;
};
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s, const BwdEvents& ev);

}  // namespace fm
