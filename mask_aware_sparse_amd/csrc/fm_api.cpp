// libfm C ABI: argument validation, workspace layout, kernel launch sequences.
// The declarations and their contracts are in include/fm.h.
#include "fm.h"
#include "fm_internal.h"

#include <cmath>
#include <cstdint>
#include <type_traits>

namespace {

using fm::MaskPtrs;

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }
inline bool pow2_in(int32_t x, int32_t lo, int32_t hi) {
  return x >= lo && x <= hi && (x & (x - 1)) == 0;
}
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// N_q (query rows) and N_k (keys); N_k = N_q unless seqlen_kv is set.
inline int32_t nq_of(const fm_problem* p) { return p->seqlen; }
inline int32_t nk_of(const fm_problem* p) { return p->seqlen_kv > 0 ? p->seqlen_kv : p->seqlen; }
// H_m mask sets per batch row (0 means 1) and the mask rows B * H_m the tiles are built for.
inline int32_t hm_of(const fm_problem* p) { return p->mask_heads > 0 ? p->mask_heads : 1; }
inline int64_t mask_rows(const fm_problem* p) { return (int64_t)p->batch * hm_of(p); }

// Problem checks shared by every entry point.
fm_status check_problem(const fm_problem* p) {
  if (!p) return FM_ERR_INVALID_ARG;
  if (p->batch < 0 || p->heads_q < 0 || p->heads_kv < 1 || p->seqlen < 0 || p->seqlen_kv < 0 ||
      p->mask_heads < 0)
    return FM_ERR_INVALID_ARG;
  if (p->heads_q % p->heads_kv != 0) return FM_ERR_INVALID_ARG;
  if (!fm::head_map_valid(p->heads_q, p->heads_kv, hm_of(p))) return FM_ERR_INVALID_ARG;
  if (!(p->softmax_scale <= 0.f || std::isfinite(p->softmax_scale))) return FM_ERR_INVALID_ARG;
  if (p->key_order != FM_KEYS_NATURAL && p->key_order != FM_KEYS_SORTED) return FM_ERR_INVALID_ARG;
  if (p->schedule != FM_SCHEDULE_LPT && p->schedule != FM_SCHEDULE_NATURAL)
    return FM_ERR_INVALID_ARG;
  if (!fm::head_dim_supported(p->head_dim)) return FM_ERR_UNSUPPORTED;
  // per-head buffers < 2 GiB
  if (nq_of(p) > (1 << 22) || nk_of(p) > (1 << 22)) return FM_ERR_UNSUPPORTED;
  return FM_OK;
}

// Nothing to compute or write at all.  (N_q = 0 with keys still zeroes dK/dV; N_k = 0
// with rows still writes O = 0 and LSE = -inf.)
bool empty_problem(const fm_problem* p) {
  return p->batch == 0 || p->heads_q == 0 || (nq_of(p) == 0 && nk_of(p) == 0);
}

fm_status check_mask(const fm_problem* p, const fm_mask* m) {
  if (!m) return FM_ERR_INVALID_ARG;
  if (mask_rows(p) * nk_of(p) == 0) return FM_OK;
  if (!m->lts || !m->lte || !m->uts || !m->ute) return FM_ERR_INVALID_ARG;
  return FM_OK;
}

fm_status check_mask(const fm_problem* p, const fm_mask_multi* m) {
  if (!m) return FM_ERR_INVALID_ARG;
  if (m->n_intervals < 1 || m->n_intervals > fm::kMaxIntervals) return FM_ERR_INVALID_ARG;
  if (mask_rows(p) * nk_of(p) == 0) return FM_OK;
  if (!m->start || !m->end) return FM_ERR_INVALID_ARG;
  if (mask_rows(p) * m->n_intervals * nk_of(p) > INT32_MAX) return FM_ERR_UNSUPPORTED;
  return FM_OK;
}

fm_status check_mask(const fm_problem* p, const fm_mask_blocks* m) {
  if (!m) return FM_ERR_INVALID_ARG;
  const int64_t nb = fm::kMaskBlock;
  if (mask_rows(p) * ((nq_of(p) + nb - 1) / nb) * ((nk_of(p) + nb - 1) / nb) == 0) return FM_OK;
  if (!m->blocks) return FM_ERR_INVALID_ARG;
  return FM_OK;
}

// The dispatch order of the attention kernels' work items: cost-descending (LPT, the sort)
// or index order (FM_SCHEDULE_NATURAL, for measuring what the LPT order buys).
hipError_t dispatch_order(const fm_problem* p, const int32_t* cost, int32_t* order, int count,
                          void* scratch, hipStream_t s) {
  if (p->schedule == FM_SCHEDULE_NATURAL) return fm::launch_iota_i32(order, count, s);
  return fm::launch_lpt_sort(cost, order, count, scratch, s);
}

// The key-order option: four-vector masks only, and each kv head in one mask set.
inline bool sorted_keys(const fm_problem* p) { return p->key_order == FM_KEYS_SORTED; }
// Keys per dK/dV workgroup (and the KV block of its tiles) for this problem.
inline int bwd_bk(const fm_problem* p) { return fm::bwd_block_k(p->head_dim, sorted_keys(p)); }
// Query heads per forward / dQ workgroup, and the rows of their Q-blocks.
inline int fwd_pack_of(const fm_problem* p) {
  return fm::fwd_pack(p->heads_q, p->heads_kv, hm_of(p));
}
inline int fwd_bq(const fm_problem* p) { return fm::fwd_block_q(fwd_pack_of(p)); }
template <typename MaskT>
fm_status check_key_order(const fm_problem* p) {
  if (!sorted_keys(p)) return FM_OK;
  if (!std::is_same<MaskT, fm_mask>::value) return FM_ERR_UNSUPPORTED;
  if (hm_of(p) > p->heads_kv) return FM_ERR_UNSUPPORTED;
  return FM_OK;
}

fm::MaskArgs mask_args(const fm_problem*, const fm_mask* m) {
  return fm::MaskArgs{fm::MaskPtrs{m->lts, m->lte, m->uts, m->ute}, nullptr, nullptr, 0,
                      nullptr, 0};
}
fm::MaskArgs mask_args(const fm_problem*, const fm_mask_multi* m) {
  return fm::MaskArgs{fm::MaskPtrs{nullptr, nullptr, nullptr, nullptr}, m->start, m->end,
                      m->n_intervals, nullptr, 0};
}
fm::MaskArgs mask_args(const fm_problem* p, const fm_mask_blocks* m) {
  return fm::MaskArgs{fm::MaskPtrs{nullptr, nullptr, nullptr, nullptr}, nullptr, nullptr,
                      fm::kBlocksMode, m->blocks,
                      (int)((nq_of(p) + fm::kMaskBlock - 1) / fm::kMaskBlock)};
}
// The mask the attention kernels read: a block grid runs as all-zero four vectors (the
// tiles come from the grid's queues; inside a visible block nothing is hidden).
fm::MaskArgs kernel_mask(const fm::MaskArgs& ma, int32_t* zeros) {
  if (ma.n != fm::kBlocksMode) return ma;
  fm::MaskArgs k = ma;
  k.n = 0;
  k.v = fm::MaskPtrs{zeros, zeros, zeros, zeros};
  return k;
}

float scale_of(const fm_problem* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
}

struct Blocks {
  int64_t nQB, nKB;
};
Blocks blocks(const fm_problem* p, int bq, int bk) {
  return {cdiv(nq_of(p), bq), cdiv(nk_of(p), bk)};
}

fm_status check_sort_limits(const fm_problem* p, const Blocks& nb) {
  if (mask_rows(p) * nb.nQB > fm::kMaxWorkItems) return FM_ERR_UNSUPPORTED;
  if (mask_rows(p) * nb.nKB > fm::kMaxWorkItems) return FM_ERR_UNSUPPORTED;
  return FM_OK;
}
inline int64_t max2(int64_t a, int64_t b) { return a > b ? a : b; }

// ---- workspace layouts ------------------------------------------------------------
struct ClassifyWs { size_t q_cost, k_cost, sort, total; };
ClassifyWs classify_ws(const fm_problem* p, const Blocks& nb) {
  ClassifyWs w{};
  size_t off = 0;
  w.q_cost = off; off += align_up((size_t)mask_rows(p) * nb.nQB * 4);
  w.k_cost = off; off += align_up((size_t)mask_rows(p) * nb.nKB * 4);
  w.sort = off;
  off += align_up(fm::lpt_sort_scratch_bytes(max2(mask_rows(p) * nb.nQB, mask_rows(p) * nb.nKB)));
  w.total = off;
  return w;
}

// Buffers of the key-order option: the permutation, the vectors, K and V in that order,
// and (backward) dK and dV in that order before they are scattered back.
struct KeyWs { size_t perm, vec[4], k, v, dk, dv; };
size_t key_ws(const fm_problem* p, size_t off, bool grads, KeyWs* w) {
  if (!sorted_keys(p)) return off;
  const size_t cols = (size_t)mask_rows(p) * nk_of(p);
  const size_t rows = (size_t)p->batch * p->heads_kv * nk_of(p) * p->head_dim * 2;
  w->perm = off; off += align_up(cols * 4);
  for (int x = 0; x < 4; ++x) { w->vec[x] = off; off += align_up(cols * 4); }
  w->k = off; off += align_up(rows);
  w->v = off; off += align_up(rows);
  if (grads) {
    w->dk = off; off += align_up(rows);
    w->dv = off; off += align_up(rows);
  }
  return off;
}

struct FwdWs { size_t mm, q_queue, q_count, q_cost, q_order, sort, zeros, total; KeyWs key; };
FwdWs fwd_ws(const fm_problem* p, const Blocks& nb) {
  FwdWs w{};
  const size_t B = mask_rows(p);  // tile structures are per mask row
  size_t off = 0;
  w.mm = off; off += align_up(B * nb.nKB * fm::kMaxMinmaxWidth * 4);
  w.q_queue = off; off += align_up(B * nb.nQB * nb.nKB * 4);
  w.q_count = off; off += align_up(B * nb.nQB * 2 * 4);
  w.q_cost = off; off += align_up(B * nb.nQB * 4);
  w.q_order = off; off += align_up(B * nb.nQB * 4);
  w.sort = off; off += align_up(fm::lpt_sort_scratch_bytes((int64_t)B * nb.nQB));
  w.zeros = off; off += align_up(B * nk_of(p) * 4);  // block-sparse masks only
  w.total = key_ws(p, off, false, &w.key);
  return w;
}

struct BwdWs {
  size_t mm_k, k_queue, k_count, k_cost, k_order;   // dK/dV tiles
  size_t mm_q, q_queue, q_count, q_cost, q_order;   // dQ (forward) tiles
  size_t lse2, delta, dk, dv;
  size_t unit_pair, unit_slot, split_pair, split_slot, split_counts, partials;  // split plan
  size_t sort;   // LPT sort scratch (lists longer than one workgroup sorts)
  size_t zeros;  // all-zero vectors standing for a block-sparse mask in the kernels
  KeyWs key;     // key-order buffers
  size_t total;
  bool acc;   // fp32 dK/dV accumulators present
  int extra;  // extra pair units of the split plan
};
BwdWs bwd_ws(const fm_problem* p, const Blocks& nk, const Blocks& nq) {
  BwdWs w{};
  const size_t rq = (size_t)p->batch * p->heads_q * nq_of(p);
  const size_t rk = (size_t)p->batch * p->heads_kv * nk_of(p);
  const size_t B = mask_rows(p);  // tile structures are per mask row
  size_t off = 0;
  w.mm_k = off; off += align_up(B * nk.nKB * fm::kMaxMinmaxWidth * 4);
  w.k_queue = off; off += align_up(B * nk.nKB * nk.nQB * 4);
  w.k_count = off; off += align_up(B * nk.nKB * 2 * 4);
  w.k_cost = off; off += align_up(B * nk.nKB * 4);
  w.k_order = off; off += align_up(B * nk.nKB * 4);
  w.mm_q = off; off += align_up(B * nq.nKB * fm::kMaxMinmaxWidth * 4);
  w.q_queue = off; off += align_up(B * nq.nQB * nq.nKB * 4);
  w.q_count = off; off += align_up(B * nq.nQB * 2 * 4);
  w.q_cost = off; off += align_up(B * nq.nQB * 4);
  w.q_order = off; off += align_up(B * nq.nQB * 4);
  w.lse2 = off; off += align_up(rq * 4);
  w.delta = off; off += align_up(rq * 4);
  // fp32 dK/dV accumulators only when several workgroups write one kv head's KV block
  // (query-head groups larger than one head chunk, or split by per-head mask sets);
  // otherwise the kernel stores bf16 directly
  const fm::HeadMap hm = fm::head_map(p->heads_q, p->heads_kv, hm_of(p));
  w.acc = hm.writers > 1;
  if (w.acc) {
    w.dk = off; off += align_up(rk * p->head_dim * 4);
    w.dv = off; off += align_up(rk * p->head_dim * 4);
  }
  // split plan of the dK/dV work units; partial sums only where bf16 is stored directly
  const int64_t pairs = (int64_t)B * nk.nKB;
  const int per = hm.kvpm * hm.cpk;
  w.extra = fm::split_extra_pairs(per, pairs);
  w.unit_pair = off; off += align_up((size_t)(pairs + w.extra) * 4);
  w.unit_slot = off; off += align_up((size_t)(pairs + w.extra) * 4);
  w.split_pair = off; off += align_up((size_t)w.extra * 4);
  w.split_slot = off; off += align_up((size_t)w.extra * 4);
  w.split_counts = off; off += align_up(2 * 4);
  w.sort = off;
  off += align_up(fm::lpt_sort_scratch_bytes(max2((int64_t)B * nk.nKB, (int64_t)B * nq.nQB)));
  w.zeros = off; off += align_up(B * nk_of(p) * 4);
  if (!w.acc) {
    w.partials = off;
    off += align_up((size_t)2 * fm::split_slots(per, w.extra) * bwd_bk(p) * p->head_dim * 4);
  }
  w.total = key_ws(p, off, true, &w.key);
  return w;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

hipEvent_t ev_start(const fm_kernel_events* e) {
  return e ? static_cast<hipEvent_t>(e->start) : nullptr;
}
hipEvent_t ev_stop(const fm_kernel_events* e) {
  return e ? static_cast<hipEvent_t>(e->stop) : nullptr;
}

fm_status hip_status(hipError_t e) { return e == hipSuccess ? FM_OK : FM_ERR_HIP; }

fm_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return FM_OK;
  if (!ws) return FM_ERR_INVALID_ARG;
  if (!aligned16(ws)) return FM_ERR_INVALID_ARG;
  if (have < need) return FM_ERR_WORKSPACE;
  return FM_OK;
}

fm_status check_grid(const fm_problem* p, const Blocks& fwd, const Blocks& bwd) {
  const fm::HeadMap hm = fm::head_map(p->heads_q, p->heads_kv, hm_of(p));
  if ((int64_t)p->batch * fwd.nQB * p->heads_q >= INT32_MAX) return FM_ERR_UNSUPPORTED;
  if ((mask_rows(p) * bwd.nKB + fm::kSplitExtraUnits) * hm.kvpm * hm.cpk >= INT32_MAX)
    return FM_ERR_UNSUPPORTED;
  return FM_OK;
}

}  // namespace

namespace fm {
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
}  // namespace fm

extern "C" {

const char* fm_status_string(fm_status s) {
  switch (s) {
    case FM_OK: return "FM_OK";
    case FM_ERR_INVALID_ARG: return "FM_ERR_INVALID_ARG: invalid argument";
    case FM_ERR_UNSUPPORTED: return "FM_ERR_UNSUPPORTED: unsupported problem";
    case FM_ERR_WORKSPACE: return "FM_ERR_WORKSPACE: workspace too small";
    case FM_ERR_HIP: return "FM_ERR_HIP: HIP launch failed";
  }
  return "unknown fm_status";
}

fm_status fm_tile_shape(fm_op op, int32_t* block_q, int32_t* block_k) {
  if (!block_q || !block_k) return FM_ERR_INVALID_ARG;
  if (op == FM_OP_FWD) { *block_q = fm::kFwdBlockQ; *block_k = fm::kFwdBlockK; return FM_OK; }
  if (op == FM_OP_BWD) { *block_q = fm::kBwdBlockQ; *block_k = fm::kBwdBlockK; return FM_OK; }
  return FM_ERR_INVALID_ARG;
}

fm_status fm_workspace_size(const fm_problem* p, fm_op op, int32_t block_q, int32_t block_k,
                            size_t* bytes) {
  if (!bytes) return FM_ERR_INVALID_ARG;
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  switch (op) {
    case FM_OP_CLASSIFY: {
      if (!pow2_in(block_q, 8, 256) || !pow2_in(block_k, 8, 256)) return FM_ERR_INVALID_ARG;
      Blocks nb = blocks(p, block_q, block_k);
      if ((st = check_sort_limits(p, nb)) != FM_OK) return st;
      *bytes = classify_ws(p, nb).total;
      return FM_OK;
    }
    case FM_OP_FWD: {
      Blocks nb = blocks(p, fwd_bq(p), fm::kFwdBlockK);
      if ((st = check_sort_limits(p, nb)) != FM_OK) return st;
      *bytes = fwd_ws(p, nb).total;
      return FM_OK;
    }
    case FM_OP_BWD: {
      Blocks nk = blocks(p, fm::kBwdBlockQ, bwd_bk(p));
      Blocks nq = blocks(p, fwd_bq(p), fm::kFwdBlockK);
      if ((st = check_sort_limits(p, nk)) != FM_OK) return st;
      if ((st = check_sort_limits(p, nq)) != FM_OK) return st;
      *bytes = bwd_ws(p, nk, nq).total;
      return FM_OK;
    }
  }
  return FM_ERR_INVALID_ARG;
}

size_t fm_workspace_bytes(const fm_problem* p, fm_op op, int32_t block_q, int32_t block_k) {
  size_t n = 0;
  return fm_workspace_size(p, op, block_q, block_k, &n) == FM_OK ? n : 0;
}

}  // extern "C"

namespace {

// The key-order option: the permutation and the permuted vectors into the workspace, then K
// and V gathered into that order; `ma`, `k` and `v` are redirected to the permuted copies.
hipError_t order_keys(const fm_problem* p, void* ws, const KeyWs& w, fm::MaskArgs& ma,
                      const void*& k, const void*& v, hipStream_t s) {
  int32_t* perm = at<int32_t>(ws, w.perm);
  const fm::MaskOut pv{at<int32_t>(ws, w.vec[0]), at<int32_t>(ws, w.vec[1]),
                       at<int32_t>(ws, w.vec[2]), at<int32_t>(ws, w.vec[3])};
  hipError_t e = fm::launch_key_order(ma.v, (int)mask_rows(p), nq_of(p), nk_of(p), perm, pv, s);
  void* kp = at<char>(ws, w.k);
  void* vp = at<char>(ws, w.v);
  if (e == hipSuccess)
    e = fm::launch_permute_rows(false, k, v, kp, vp, perm, p->batch, p->heads_kv, hm_of(p),
                                nk_of(p), p->head_dim, s);
  ma.v = MaskPtrs{pv.lts, pv.lte, pv.uts, pv.ute};
  k = kp;
  v = vp;
  return e;
}

template <typename MaskT>
fm_status classify_impl(const fm_problem* p, const MaskT* m, int32_t block_q, int32_t block_k,
                        const fm_tiles* out, void* ws, size_t ws_bytes, void* stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if ((st = check_mask(p, m)) != FM_OK) return st;
  if (!pow2_in(block_q, 8, 256) || !pow2_in(block_k, 8, 256)) return FM_ERR_INVALID_ARG;
  if (!out) return FM_ERR_INVALID_ARG;
  Blocks nb = blocks(p, block_q, block_k);
  if ((st = check_sort_limits(p, nb)) != FM_OK) return st;
  if (p->batch == 0 || (nq_of(p) == 0 && nk_of(p) == 0)) return FM_OK;
  if (!out->block_minmax || !out->tile_class || !out->q_queue || !out->q_count ||
      !out->k_queue || !out->k_count || !out->q_order || !out->k_order)
    return FM_ERR_INVALID_ARG;
  ClassifyWs w = classify_ws(p, nb);
  if ((st = check_ws(ws, ws_bytes, w.total)) != FM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  fm::TileOut t{};
  t.minmax = out->block_minmax;
  t.tile_class = out->tile_class;
  t.q_queue = out->q_queue;
  t.q_count = out->q_count;
  t.q_cost = at<int32_t>(ws, w.q_cost);
  t.k_queue = out->k_queue;
  t.k_count = out->k_count;
  t.k_cost = at<int32_t>(ws, w.k_cost);
  const int R = (int)mask_rows(p);
  hipError_t e = fm::launch_classify(mask_args(p, m), R, nq_of(p), nk_of(p), block_q, block_k, t, s);
  void* scr = at<char>(ws, w.sort);
  if (e == hipSuccess) e = fm::launch_lpt_sort(t.q_cost, out->q_order, (int)(R * nb.nQB), scr, s);
  if (e == hipSuccess) e = fm::launch_lpt_sort(t.k_cost, out->k_order, (int)(R * nb.nKB), scr, s);
  return hip_status(e);
}

template <typename MaskT>
fm_status fwd_impl(const fm_problem* p, const void* q, const void* k, const void* v,
                   const MaskT* m, void* o, float* lse, void* ws, size_t ws_bytes, void* stream,
                   const fm_kernel_events* events) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if ((st = check_mask(p, m)) != FM_OK) return st;
  if ((st = check_key_order<MaskT>(p)) != FM_OK) return st;
  Blocks nb = blocks(p, fwd_bq(p), fm::kFwdBlockK);
  if ((st = check_sort_limits(p, nb)) != FM_OK) return st;
  if ((st = check_grid(p, nb, blocks(p, fm::kBwdBlockQ, bwd_bk(p)))) != FM_OK) return st;
  if (empty_problem(p)) return FM_OK;
  // query-side arrays are needed when there are rows, key-side ones when there are keys
  if (nq_of(p) > 0 && (!q || !o || !lse)) return FM_ERR_INVALID_ARG;
  if (nk_of(p) > 0 && (!k || !v)) return FM_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FM_ERR_INVALID_ARG;
  FwdWs w = fwd_ws(p, nb);
  if ((st = check_ws(ws, ws_bytes, w.total)) != FM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  fm::MaskArgs ma = mask_args(p, m);
  hipError_t e = hipSuccess;
  if (sorted_keys(p)) e = order_keys(p, ws, w.key, ma, k, v, s);
  fm::TileOut t{};
  t.minmax = at<int32_t>(ws, w.mm);
  t.q_queue = at<int32_t>(ws, w.q_queue);
  t.q_count = at<int32_t>(ws, w.q_count);
  t.q_cost = at<int32_t>(ws, w.q_cost);
  const int R = (int)mask_rows(p);
  if (e == hipSuccess)
    e = fm::launch_classify(ma, R, nq_of(p), nk_of(p), fwd_bq(p), fm::kFwdBlockK, t, s);
  int32_t* order = at<int32_t>(ws, w.q_order);
  if (e == hipSuccess)
    e = dispatch_order(p, t.q_cost, order, (int)(R * nb.nQB), at<char>(ws, w.sort), s);
  if (e == hipSuccess && ma.n == fm::kBlocksMode)
    e = fm::launch_zero_i32(at<int32_t>(ws, w.zeros), (size_t)R * nk_of(p), s);
  if (e == hipSuccess) {
    fm::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.m = kernel_mask(ma, at<int32_t>(ws, w.zeros)); a.o = o;
    a.lse = lse;
    a.q_queue = t.q_queue; a.q_count = t.q_count; a.q_order = order;
    a.B = p->batch; a.Hq = p->heads_q; a.Hkv = p->heads_kv; a.Hm = hm_of(p);
    a.Nq = nq_of(p); a.Nk = nk_of(p); a.D = p->head_dim;
    a.nQB = (int)nb.nQB; a.nKB = (int)nb.nKB;
    a.pack = fwd_pack_of(p);
    a.scale = scale_of(p);
    e = fm::launch_fwd(a, s, ev_start(events), ev_stop(events));
  }
  return hip_status(e);
}

template <typename MaskT>
fm_status bwd_impl(const fm_problem* p, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dout, const MaskT* m, void* dq,
                   void* dk, void* dv, void* ws, size_t ws_bytes, void* stream,
                   const fm_kernel_events* events) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if ((st = check_mask(p, m)) != FM_OK) return st;
  if ((st = check_key_order<MaskT>(p)) != FM_OK) return st;
  Blocks nk = blocks(p, fm::kBwdBlockQ, bwd_bk(p));
  Blocks nq = blocks(p, fwd_bq(p), fm::kFwdBlockK);
  if ((st = check_sort_limits(p, nk)) != FM_OK) return st;
  if ((st = check_sort_limits(p, nq)) != FM_OK) return st;
  if ((st = check_grid(p, nq, nk)) != FM_OK) return st;
  if (empty_problem(p)) return FM_OK;
  if (nq_of(p) > 0 && (!q || !o || !lse || !dout || !dq)) return FM_ERR_INVALID_ARG;
  if (nk_of(p) > 0 && (!k || !v || !dk || !dv)) return FM_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FM_ERR_INVALID_ARG;
  BwdWs w = bwd_ws(p, nk, nq);
  if ((st = check_ws(ws, ws_bytes, w.total)) != FM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  fm::MaskArgs ma = mask_args(p, m);
  hipError_t e = hipSuccess;
  // key order: K, V and the vectors gathered here; dK, dV written in that order into the
  // workspace and scattered to the caller's after the kernels
  void* dk_out = dk;
  void* dv_out = dv;
  if (sorted_keys(p)) {
    e = order_keys(p, ws, w.key, ma, k, v, s);
    dk = at<char>(ws, w.key.dk);
    dv = at<char>(ws, w.key.dv);
  }
  fm::TileOut tk{};
  tk.minmax = at<int32_t>(ws, w.mm_k);
  tk.k_queue = at<int32_t>(ws, w.k_queue);
  tk.k_count = at<int32_t>(ws, w.k_count);
  tk.k_cost = at<int32_t>(ws, w.k_cost);
  fm::TileOut tq{};
  tq.minmax = at<int32_t>(ws, w.mm_q);
  tq.q_queue = at<int32_t>(ws, w.q_queue);
  tq.q_count = at<int32_t>(ws, w.q_count);
  tq.q_cost = at<int32_t>(ws, w.q_cost);
  int32_t* k_order = at<int32_t>(ws, w.k_order);
  int32_t* q_order = at<int32_t>(ws, w.q_order);
  const int R = (int)mask_rows(p);
  // both tile shapes' classifications (the dK/dV kernel's per-KV-block queues, the dQ
  // kernel's per-Q-block queues) in shared launches: one block min/max pass, one classify
  // launch, one sort launch for short lists
  if (e == hipSuccess)
    e = fm::launch_classify_pair(ma, R, nq_of(p), nk_of(p), fm::kBwdBlockQ, bwd_bk(p), tk,
                                 fwd_bq(p), fm::kFwdBlockK, tq, s);
  void* scr = at<char>(ws, w.sort);
  if (e == hipSuccess) {
    if (p->schedule == FM_SCHEDULE_NATURAL) {
      e = dispatch_order(p, tk.k_cost, k_order, (int)(R * nk.nKB), scr, s);
      if (e == hipSuccess) e = dispatch_order(p, tq.q_cost, q_order, (int)(R * nq.nQB), scr, s);
    } else {
      e = fm::launch_lpt_sort_pair(tk.k_cost, k_order, (int)(R * nk.nKB), tq.q_cost, q_order,
                                   (int)(R * nq.nQB), scr, s);
    }
  }
  if (e == hipSuccess && ma.n == fm::kBlocksMode)
    e = fm::launch_zero_i32(at<int32_t>(ws, w.zeros), (size_t)R * nk_of(p), s);
  if (e == hipSuccess) {
    fm::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
    a.m = kernel_mask(ma, at<int32_t>(ws, w.zeros));
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.k_queue = tk.k_queue; a.k_count = tk.k_count; a.k_order = k_order;
    a.q_queue = tq.q_queue; a.q_count = tq.q_count; a.q_order = q_order;
    a.lse2 = at<float>(ws, w.lse2); a.delta = at<float>(ws, w.delta);
    if (w.acc) { a.dk_acc = at<float>(ws, w.dk); a.dv_acc = at<float>(ws, w.dv); }
    a.unit_pair = at<int32_t>(ws, w.unit_pair);
    a.unit_slot = at<int32_t>(ws, w.unit_slot);
    a.split_pair = at<int32_t>(ws, w.split_pair);
    a.split_slot = at<int32_t>(ws, w.split_slot);
    a.split_counts = at<int32_t>(ws, w.split_counts);
    a.partials = w.acc ? nullptr : at<float>(ws, w.partials);
    a.split_extra = w.extra;
    a.B = p->batch; a.Hq = p->heads_q; a.Hkv = p->heads_kv; a.Hm = hm_of(p);
    a.Nq = nq_of(p); a.Nk = nk_of(p); a.D = p->head_dim;
    a.bk = bwd_bk(p);
    a.nQB_k = (int)nk.nQB; a.nKB_k = (int)nk.nKB;
    a.nQB_q = (int)nq.nQB; a.nKB_q = (int)nq.nKB;
    a.pack = fwd_pack_of(p);
    a.scale = scale_of(p);
    fm::BwdEvents ev{};
    if (events) {
      ev.dkdv_start = static_cast<hipEvent_t>(events->start);
      ev.dkdv_stop = static_cast<hipEvent_t>(events->stop);
      ev.dq_start = static_cast<hipEvent_t>(events->start2);
      ev.dq_stop = static_cast<hipEvent_t>(events->stop2);
    }
    e = fm::launch_bwd(a, s, ev);
  }
  if (e == hipSuccess && sorted_keys(p))
    e = fm::launch_permute_rows(true, dk, dv, dk_out, dv_out, at<int32_t>(ws, w.key.perm),
                                p->batch, p->heads_kv, hm_of(p), nk_of(p), p->head_dim, s);
  return hip_status(e);
}

template <typename MaskT>
fm_status expand_impl(const fm_problem* p, const MaskT* m, int32_t b, int32_t row0, int32_t row1,
                      uint8_t* dense, void* stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if ((st = check_mask(p, m)) != FM_OK) return st;
  if (b < 0 || b >= mask_rows(p) || row0 < 0 || row1 < row0 || row1 > nq_of(p))
    return FM_ERR_INVALID_ARG;
  if (row1 == row0 || nk_of(p) == 0) return FM_OK;
  if (!dense) return FM_ERR_INVALID_ARG;
  return hip_status(fm::launch_expand_mask(mask_args(p, m), b, nk_of(p), row0, row1, dense,
                                           static_cast<hipStream_t>(stream)));
}

// Shared checks of the localization entry points; `cols` = bounds per array.
fm_status check_localize(const fm_problem* p, const int32_t* offsets, int32_t n_chunks,
                         int32_t chunk_len, int64_t cols) {
  if (n_chunks < 1 || chunk_len < 1) return FM_ERR_INVALID_ARG;
  if (n_chunks > 4096 || nk_of(p) > (1 << 22)) return FM_ERR_UNSUPPORTED;
  if ((int64_t)n_chunks * chunk_len > (1 << 22)) return FM_ERR_UNSUPPORTED;
  if (cols > INT32_MAX) return FM_ERR_UNSUPPORTED;
  if (cols > 0 && !offsets) return FM_ERR_INVALID_ARG;
  return FM_OK;
}

}  // namespace

extern "C" {

fm_status fm_classify_tiles(const fm_problem* p, const fm_mask* m, int32_t block_q,
                            int32_t block_k, const fm_tiles* out, void* ws, size_t ws_bytes,
                            void* stream) {
  return classify_impl(p, m, block_q, block_k, out, ws, ws_bytes, stream);
}

fm_status fm_classify_tiles_multi(const fm_problem* p, const fm_mask_multi* m, int32_t block_q,
                                  int32_t block_k, const fm_tiles* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  return classify_impl(p, m, block_q, block_k, out, ws, ws_bytes, stream);
}

fm_status fm_attn_fwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const fm_mask* m, void* o, float* lse, void* ws, size_t ws_bytes,
                      void* stream, const fm_kernel_events* events) {
  return fwd_impl(p, q, k, v, m, o, lse, ws, ws_bytes, stream, events);
}

fm_status fm_attn_fwd_multi(const fm_problem* p, const void* q, const void* k, const void* v,
                            const fm_mask_multi* m, void* o, float* lse, void* ws,
                            size_t ws_bytes, void* stream, const fm_kernel_events* events) {
  return fwd_impl(p, q, k, v, m, o, lse, ws, ws_bytes, stream, events);
}

fm_status fm_attn_bwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, const fm_mask* m,
                      void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream,
                      const fm_kernel_events* events) {
  return bwd_impl(p, q, k, v, o, lse, dout, m, dq, dk, dv, ws, ws_bytes, stream, events);
}

fm_status fm_attn_bwd_multi(const fm_problem* p, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* dout,
                            const fm_mask_multi* m, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* stream, const fm_kernel_events* events) {
  return bwd_impl(p, q, k, v, o, lse, dout, m, dq, dk, dv, ws, ws_bytes, stream, events);
}

fm_status fm_debug_expand_mask(const fm_problem* p, const fm_mask* m, int32_t b, int32_t row0,
                               int32_t row1, uint8_t* dense, void* stream) {
  return expand_impl(p, m, b, row0, row1, dense, stream);
}

fm_status fm_debug_expand_mask_multi(const fm_problem* p, const fm_mask_multi* m, int32_t b,
                                     int32_t row0, int32_t row1, uint8_t* dense, void* stream) {
  return expand_impl(p, m, b, row0, row1, dense, stream);
}

fm_status fm_classify_tiles_blocks(const fm_problem* p, const fm_mask_blocks* m, int32_t block_q,
                                   int32_t block_k, const fm_tiles* out, void* ws,
                                   size_t ws_bytes, void* stream) {
  return classify_impl(p, m, block_q, block_k, out, ws, ws_bytes, stream);
}

fm_status fm_attn_fwd_blocks(const fm_problem* p, const void* q, const void* k, const void* v,
                             const fm_mask_blocks* m, void* o, float* lse, void* ws,
                             size_t ws_bytes, void* stream, const fm_kernel_events* events) {
  return fwd_impl(p, q, k, v, m, o, lse, ws, ws_bytes, stream, events);
}

fm_status fm_attn_bwd_blocks(const fm_problem* p, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout,
                             const fm_mask_blocks* m, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, void* stream, const fm_kernel_events* events) {
  return bwd_impl(p, q, k, v, o, lse, dout, m, dq, dk, dv, ws, ws_bytes, stream, events);
}

fm_status fm_debug_expand_mask_blocks(const fm_problem* p, const fm_mask_blocks* m, int32_t b,
                                      int32_t row0, int32_t row1, uint8_t* dense,
                                      void* stream) {
  return expand_impl(p, m, b, row0, row1, dense, stream);
}

fm_status fm_localize_mask(const fm_problem* p, const fm_mask* global, const int32_t* offsets,
                           int32_t n_chunks, int32_t chunk_len, const fm_mask_out* local,
                           void* stream) {
  if (!p || !global || !local) return FM_ERR_INVALID_ARG;
  if (p->batch < 0 || p->seqlen < 0 || p->seqlen_kv < 0 || p->mask_heads < 0)
    return FM_ERR_INVALID_ARG;
  const int64_t cols = mask_rows(p) * nk_of(p);
  fm_status st = check_localize(p, offsets, n_chunks, chunk_len, cols);
  if (st != FM_OK || cols == 0) return st;
  if (!global->lts || !global->lte || !global->uts || !global->ute || !local->lts ||
      !local->lte || !local->uts || !local->ute)
    return FM_ERR_INVALID_ARG;
  return hip_status(fm::launch_localize(
      fm::MaskPtrs{global->lts, global->lte, global->uts, global->ute}, 4, offsets, n_chunks,
      chunk_len, fm::MaskOut{local->lts, local->lte, local->uts, local->ute}, cols,
      static_cast<hipStream_t>(stream)));
}

fm_status fm_check_mask(const fm_problem* p, const fm_mask* m, int32_t* bad, void* stream) {
  if (!p || !m || !bad) return FM_ERR_INVALID_ARG;
  if (p->batch < 0 || p->seqlen < 0 || p->seqlen_kv < 0 || p->mask_heads < 0)
    return FM_ERR_INVALID_ARG;
  const int64_t cols = mask_rows(p) * nk_of(p);
  if (cols > 0 && (!m->lts || !m->lte || !m->uts || !m->ute)) return FM_ERR_INVALID_ARG;
  return hip_status(fm::launch_check_bounds(MaskPtrs{m->lts, m->lte, m->uts, m->ute}, 4, cols,
                                            nq_of(p), bad, static_cast<hipStream_t>(stream)));
}

fm_status fm_check_mask_multi(const fm_problem* p, const fm_mask_multi* m, int32_t* bad,
                              void* stream) {
  if (!p || !m || !bad) return FM_ERR_INVALID_ARG;
  if (p->batch < 0 || p->seqlen < 0 || p->seqlen_kv < 0 || p->mask_heads < 0)
    return FM_ERR_INVALID_ARG;
  if (m->n_intervals < 1 || m->n_intervals > fm::kMaxIntervals) return FM_ERR_INVALID_ARG;
  const int64_t cols = mask_rows(p) * m->n_intervals * nk_of(p);
  if (cols > 0 && (!m->start || !m->end)) return FM_ERR_INVALID_ARG;
  return hip_status(fm::launch_check_bounds(MaskPtrs{m->start, m->end, nullptr, nullptr}, 2,
                                            cols, nq_of(p), bad,
                                            static_cast<hipStream_t>(stream)));
}

fm_status fm_key_order(const fm_problem* p, const fm_mask* m, int32_t* perm,
                       const fm_mask_out* permuted, void* stream) {
  if (!p || !m) return FM_ERR_INVALID_ARG;
  if (p->batch < 0 || p->seqlen < 0 || p->seqlen_kv < 0 || p->mask_heads < 0)
    return FM_ERR_INVALID_ARG;
  if (nq_of(p) > (1 << 22) || nk_of(p) > (1 << 22)) return FM_ERR_UNSUPPORTED;
  const int64_t cols = mask_rows(p) * nk_of(p);
  if (cols == 0) return FM_OK;
  if (cols > INT32_MAX) return FM_ERR_UNSUPPORTED;
  if (!m->lts || !m->lte || !m->uts || !m->ute || !perm) return FM_ERR_INVALID_ARG;
  const fm::MaskOut out = permuted ? fm::MaskOut{permuted->lts, permuted->lte, permuted->uts,
                                                 permuted->ute}
                                   : fm::MaskOut{nullptr, nullptr, nullptr, nullptr};
  return hip_status(fm::launch_key_order(MaskPtrs{m->lts, m->lte, m->uts, m->ute},
                                         (int)mask_rows(p), nq_of(p), nk_of(p), perm, out,
                                         static_cast<hipStream_t>(stream)));
}

fm_status fm_localize_mask_multi(const fm_problem* p, const fm_mask_multi* global,
                                 const int32_t* offsets, int32_t n_chunks, int32_t chunk_len,
                                 int32_t* local_start, int32_t* local_end, void* stream) {
  if (!p || !global) return FM_ERR_INVALID_ARG;
  if (p->batch < 0 || p->seqlen < 0 || p->seqlen_kv < 0 || p->mask_heads < 0)
    return FM_ERR_INVALID_ARG;
  if (global->n_intervals < 1 || global->n_intervals > fm::kMaxIntervals)
    return FM_ERR_INVALID_ARG;
  const int64_t cols = mask_rows(p) * global->n_intervals * nk_of(p);
  fm_status st = check_localize(p, offsets, n_chunks, chunk_len, cols);
  if (st != FM_OK || cols == 0) return st;
  if (!global->start || !global->end || !local_start || !local_end) return FM_ERR_INVALID_ARG;
  return hip_status(fm::launch_localize(
      fm::MaskPtrs{global->start, global->end, nullptr, nullptr}, 2, offsets, n_chunks,
      chunk_len, fm::MaskOut{local_start, local_end, nullptr, nullptr}, cols,
      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
