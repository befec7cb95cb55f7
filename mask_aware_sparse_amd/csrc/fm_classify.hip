// Tile classification, queues, costs and the LPT order (gfx950).
//
// FlashMask-3 page, §3.1: the block-wise min/max of the column vectors decide for each
// (Q-block, KV-block) tile whether it is skipped, partial or unmasked, and the KV
// Index Generator emits per Q-block a queue of the KV blocks to visit (right to left),
// each tagged partial or unmasked.  §3.3: a tile costs 0, alpha_p or alpha_u; work is
// balanced by those costs.  Here the queues are built by one HBM pass over the
// vectors plus one pass per queue row; the LPT order is a rank sort in LDS (merged
// across workgroups for long lists).
#include "fm_device.h"
#include "fm_internal.h"

#include <climits>

namespace fm {

// ---- A2: block min/max of the four vectors -------------------------------------
// A wave takes 256 columns of one mask row at a time (four waves per workgroup striding
// over all of them): lane l loads columns 4l .. 4l + 3 of each vector, sixteen independent
// loads in flight, and the bk / 4 lanes of each KV block reduce among themselves.  With
// mm2, the min/max of the smaller blocks of bk2 < bk keys is written on the way (the
// backward needs both of its tile shapes' block bounds: one pass instead of two).
__global__ __launch_bounds__(256) void k_block_minmax(MaskPtrs m, int Nk, int nKB, int bk,
                                                      int n_sc, int total,
                                                      int32_t* __restrict__ mm, int bk2,
                                                      int nKB2, int32_t* __restrict__ mm2) {
  const int lane = threadIdx.x & 63;
  const int G = bk >> 2;  // lanes per KV block (2 .. 64)
  const int G2 = mm2 ? bk2 >> 2 : 0;  // lanes per smaller block (1 .. G / 2), 0: none
  // 16-byte loads where every row starts on a 16-byte boundary
  const bool vec4 = (Nk & 3) == 0 &&
                    ((reinterpret_cast<uintptr_t>(m.lts) | reinterpret_cast<uintptr_t>(m.lte) |
                      reinterpret_cast<uintptr_t>(m.uts) | reinterpret_cast<uintptr_t>(m.ute)) &
                     15) == 0;
  for (int sc = blockIdx.x * 4 + (threadIdx.x >> 6); sc < total; sc += gridDim.x * 4) {
    const int b = sc / n_sc, c0 = (sc - b * n_sc) * 256 + 4 * lane;
    const size_t rowoff = (size_t)b * Nk;
    int x[4][4];
    if (vec4 && c0 + 3 < Nk) {
      // whole aligned quad: one 16-byte load per vector
      const int32_t* src[4] = {m.lts, m.lte, m.uts, m.ute};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int4 q = *reinterpret_cast<const int4*>(src[t] + rowoff + c0);
        x[t][0] = q.x; x[t][1] = q.y; x[t][2] = q.z; x[t][3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = c0 + j < Nk;
        const size_t o = rowoff + (in ? c0 + j : 0);
        x[0][j] = in ? m.lts[o] : INT_MAX;
        x[1][j] = in ? m.lte[o] : INT_MAX;
        x[2][j] = in ? m.uts[o] : INT_MAX;
        x[3][j] = in ? m.ute[o] : INT_MAX;
      }
    }
    int v[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      int lo = INT_MAX, hi = INT_MIN;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c0 + j < Nk) { lo = min(lo, x[t][j]); hi = max(hi, x[t][j]); }
      }
      v[2 * t] = lo;
      v[2 * t + 1] = hi;
    }
    for (int off = 1; off < G; off <<= 1) {
      if (off == G2) {
        // lanes of each bk2-block have combined their columns: its first lane writes them
        const int kb2 = c0 / bk2;
        if ((lane & (G2 - 1)) == 0 && kb2 < nKB2) {
          int32_t* dst = mm2 + ((size_t)b * nKB2 + kb2) * 8;
#pragma unroll
          for (int t = 0; t < 8; ++t) dst[t] = v[t];
        }
      }
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        v[t] = min(v[t], __shfl_xor(v[t], off));
        v[t + 1] = max(v[t + 1], __shfl_xor(v[t + 1], off));
      }
    }
    const int kb = c0 / bk;
    if ((lane & (G - 1)) == 0 && kb < nKB) {
      int32_t* dst = mm + ((size_t)b * nKB + kb) * 8;
#pragma unroll
      for (int t = 0; t < 8; ++t) dst[t] = v[t];
    }
  }
}

// Multi-interval form: one wave per (mask row, kb); for each interval m < n the min and
// max of its starts and of its ends, written as [row][kb][4n].
__global__ __launch_bounds__(64) void k_block_minmax_multi(const int32_t* __restrict__ start,
                                                           const int32_t* __restrict__ end,
                                                           int n, int Nk, int nKB, int bk,
                                                           int32_t* __restrict__ mm) {
  const int bkb = blockIdx.x;
  const int b = bkb / nKB, kb = bkb - b * nKB;
  const int lane = threadIdx.x;
  const int c0 = kb * bk, c1 = min(c0 + bk, Nk);
  int v[4 * kMaxIntervals];
#pragma unroll
  for (int m = 0; m < kMaxIntervals; ++m) {
    v[4 * m] = INT_MAX; v[4 * m + 1] = INT_MIN; v[4 * m + 2] = INT_MAX; v[4 * m + 3] = INT_MIN;
    if (m < n) {
      const size_t rowoff = ((size_t)b * n + m) * Nk;
      for (int c = c0 + lane; c < c1; c += 64) {
        const int xs = start[rowoff + c], xe = end[rowoff + c];
        v[4 * m] = min(v[4 * m], xs); v[4 * m + 1] = max(v[4 * m + 1], xs);
        v[4 * m + 2] = min(v[4 * m + 2], xe); v[4 * m + 3] = max(v[4 * m + 3], xe);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
#pragma unroll
    for (int t = 0; t < 4 * kMaxIntervals; t += 2) {
      v[t] = min(v[t], __shfl_xor(v[t], off));
      v[t + 1] = max(v[t + 1], __shfl_xor(v[t + 1], off));
    }
  }
  if (lane < 4 * n) {
    int out = v[0];
#pragma unroll
    for (int t = 1; t < 4 * kMaxIntervals; ++t) out = (lane == t) ? v[t] : out;
    mm[(size_t)bkb * 4 * n + lane] = out;
  }
}

// The block-sparse grid (only read in kBlocksMode): blocks [rows][nqb][nkb] of kMaskBlock.
struct GridArgs {
  const uint8_t* g;
  int nqb, nkb;  // grid blocks per row and column
  int bk, Nk, nKB;
};

// The block min/max of one KV block, and the tile rule of the mask form on it.  kMode: 0
// four vectors, 1 intervals, 2 block grid (the tile's class read from the blocks it
// overlaps: skipped if all hidden, unmasked if all visible, partial otherwise).
template <int kMode>
struct BlockBounds {
  int v[kMode == 1 ? 4 * kMaxIntervals : 8];
  int n;
  int r, kb;
  const GridArgs* ga;
  __device__ __forceinline__ void load(const int32_t* __restrict__ mm, size_t idx, int n_,
                                       const GridArgs* ga_) {
    n = n_;
    ga = ga_;
    if constexpr (kMode == 2) {
      r = (int)(idx / ga->nKB);
      kb = (int)(idx - (size_t)r * ga->nKB);
    } else if constexpr (kMode == 0) {
      const int4* p = reinterpret_cast<const int4*>(mm + idx * 8);
      const int4 a = p[0], c = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    } else {
#pragma unroll
      for (int t = 0; t < 4 * kMaxIntervals; ++t) v[t] = t < 4 * n ? mm[idx * 4 * n + t] : 0;
    }
  }
  __device__ __forceinline__ int cls(int q0, int q1) const {
    if constexpr (kMode == 0) return tile_class(v, q0, q1);
    else if constexpr (kMode == 1) return tile_class_multi(v, n, q0, q1);
    else {
      const uint8_t* row = ga->g + (size_t)r * ga->nqb * ga->nkb;
      const int b0 = q0 / kMaskBlock, b1 = (q1 - 1) / kMaskBlock;
      const int k0 = kb * ga->bk;
      const int c0 = k0 / kMaskBlock, c1 = (min(k0 + ga->bk, ga->Nk) - 1) / kMaskBlock;
      bool any = false, all = true;
      for (int br = b0; br <= b1; ++br)
        for (int bc = c0; bc <= c1; ++bc) {
          const bool vis = row[(size_t)br * ga->nkb + bc] != 0;
          any = any || vis;
          all = all && vis;
        }
      return !any ? 0 : (all ? 2 : 1);
    }
  }
};

// Workgroup-wide ordered compaction helper: returns (exclusive offset of this
// thread among flagged threads, total flagged, total of `sub` among flagged).
struct ScanResult { int off; int total; int sub; };
__device__ __forceinline__ ScanResult block_scan_256(bool flag, bool sub, int* sh_cnt,
                                                     int* sh_sub) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  unsigned long long bal = __ballot(flag);
  unsigned long long bsub = __ballot(flag && sub);
  if (lane == 0) { sh_cnt[w] = __popcll(bal); sh_sub[w] = __popcll(bsub); }
  __syncthreads();
  ScanResult r{0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) r.off += sh_cnt[i];
    r.total += sh_cnt[i];
    r.sub += sh_sub[i];
  }
  r.off += __popcll(bal & ((1ull << lane) - 1ull));
  __syncthreads();
  return r;
}

// ---- A3: classes and per-Q-block queues (KV blocks right to left) --------------
// One workgroup per kR consecutive Q-blocks of one mask row: each chunk of 256 KV blocks
// has its bounds loaded once and classified against the kR Q-blocks, and one exclusive
// scan over the workgroup (two barriers) places the queued tiles of all kR rows.  kR > 1
// only for long lists (many mask rows), where reading every KV block's bounds once per
// Q-block made the kernel bound by L2 reads.
struct ClassifyQArgs {
  const int32_t* mm;
  GridArgs ga;
  int Nq, nQB, nKB, bq, groups;
  uint8_t* cls;
  int32_t* q_queue;
  int32_t* q_count;
  int32_t* q_cost;
};
struct ClassifyKArgs {
  const int32_t* mm;
  GridArgs ga;
  int Nq, nQB, nKB, bq;
  int32_t* k_queue;
  int32_t* k_count;
  int32_t* k_cost;
};

template <int kMode, int kR>
__device__ __forceinline__ void classify_q_body(const ClassifyQArgs& a, int n, int blk) {
  __shared__ int sh_cnt[kR][4], sh_sub[kR][4];
  const int32_t* __restrict__ mm = a.mm;
  const GridArgs ga = a.ga;
  const int Nq = a.Nq, nQB = a.nQB, nKB = a.nKB, bq = a.bq, groups = a.groups;
  uint8_t* __restrict__ cls = a.cls;
  int32_t* __restrict__ q_queue = a.q_queue;
  int32_t* __restrict__ q_count = a.q_count;
  int32_t* __restrict__ q_cost = a.q_cost;
  const int b = blk / groups, qb0 = (blk - b * groups) * kR;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int base[kR], np[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) { base[r] = 0; np[r] = 0; }
  for (int c0 = 0; c0 < nKB; c0 += 256) {
    const int idx = c0 + tid;
    const bool valid = idx < nKB;
    const int kb = nKB - 1 - idx;
    BlockBounds<kMode> bb;
    if (valid) bb.load(mm, (size_t)b * nKB + kb, n, &ga);
    int c[kR];
    unsigned long long bal[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int qb = qb0 + r;
      c[r] = 0;
      if (valid && qb < nQB) {
        const int q0 = qb * bq;
        c[r] = bb.cls(q0, min(q0 + bq, Nq));
        if (cls) cls[((size_t)b * nQB + qb) * nKB + kb] = (uint8_t)c[r];
      }
      bal[r] = __ballot(c[r] != 0);
      const unsigned long long bsub = __ballot(c[r] == 1);
      if (lane == 0) { sh_cnt[r][w] = __popcll(bal[r]); sh_sub[r][w] = __popcll(bsub); }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      int off = __popcll(bal[r] & ((1ull << lane) - 1ull)), total = 0, sub = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < w) off += sh_cnt[r][i];
        total += sh_cnt[r][i];
        sub += sh_sub[r][i];
      }
      if (q_queue && c[r] != 0)
        q_queue[((size_t)b * nQB + qb0 + r) * nKB + base[r] + off] =
            kb | (c[r] == 1 ? (int)0x80000000 : 0);
      base[r] += total;
      np[r] += sub;
    }
    __syncthreads();  // the counts are rewritten by the next chunk
  }
  if (q_queue) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int qb = qb0 + r;
      if (qb >= nQB) break;
      const size_t row = (size_t)b * nQB + qb;
      for (int p = base[r] + tid; p < nKB; p += 256) q_queue[row * nKB + p] = -1;
      if (tid == 0) {
        q_count[row * 2] = np[r];
        q_count[row * 2 + 1] = base[r] - np[r];
        q_cost[row] = kAlphaPartial * np[r] + kAlphaUnmasked * (base[r] - np[r]);
      }
    }
  }
}

template <int kMode, int kR>
__global__ __launch_bounds__(256) void k_classify_q(ClassifyQArgs a, int n) {
  classify_q_body<kMode, kR>(a, n, (int)blockIdx.x);
}

// ---- A3 (backward direction): per-KV-block queues of Q-blocks, ascending -----------
template <int kMode>
__device__ __forceinline__ void classify_k_body(const ClassifyKArgs& a, int n, int row) {
  __shared__ int sh_cnt[4], sh_sub[4];
  const int32_t* __restrict__ mm = a.mm;
  const GridArgs ga = a.ga;
  const int Nq = a.Nq, nQB = a.nQB, bq = a.bq;
  int32_t* __restrict__ k_queue = a.k_queue;
  int32_t* __restrict__ k_count = a.k_count;
  int32_t* __restrict__ k_cost = a.k_cost;
  // row = b * nKB + kb
  const int tid = threadIdx.x;
  BlockBounds<kMode> bb;
  bb.load(mm, (size_t)row, n, &ga);
  int base = 0, np = 0;
  for (int c0 = 0; c0 < nQB; c0 += 256) {
    const int qb = c0 + tid;
    const bool valid = qb < nQB;
    int c = 0;
    if (valid) c = bb.cls(qb * bq, min(qb * bq + bq, Nq));
    ScanResult s = block_scan_256(valid && c != 0, c == 1, sh_cnt, sh_sub);
    if (valid && c != 0)
      k_queue[(size_t)row * nQB + base + s.off] = qb | (c == 1 ? (int)0x80000000 : 0);
    base += s.total;
    np += s.sub;
  }
  for (int p = base + tid; p < nQB; p += 256) k_queue[(size_t)row * nQB + p] = -1;
  if (tid == 0) {
    k_count[(size_t)row * 2] = np;
    k_count[(size_t)row * 2 + 1] = base - np;
    k_cost[row] = kAlphaPartial * np + kAlphaUnmasked * (base - np);
  }
}

template <int kMode>
__global__ __launch_bounds__(256) void k_classify_k(ClassifyKArgs a, int n) {
  classify_k_body<kMode>(a, n, (int)blockIdx.x);
}

// Both directions in one launch (the backward's two tile shapes): workgroups below nk run
// the per-KV-block queues of `ka`, the rest the per-Q-block queues of `qa`.
template <int kMode, int kR>
__global__ __launch_bounds__(256) void k_classify_pair(ClassifyKArgs ka, ClassifyQArgs qa,
                                                       int n, int nk) {
  const int blk = (int)blockIdx.x;
  if (blk < nk) classify_k_body<kMode>(ka, n, blk);
  else classify_q_body<kMode, kR>(qa, n, blk - nk);
}

// ---- A4: longest-processing-time-first order ----------------------------------
// Keys (~cost << 32 | index) sorted ascending = cost descending, index ascending.  Lists of
// up to kRankSortItems keys sort in one workgroup; longer lists are sorted in chunks of
// that size (one workgroup each) and then merged pairwise, run length doubling per pass:
// keys are unique (they contain the index), so an element's place in the merged run is its
// place in its own run plus the number of keys below it in the other run (a binary
// search), and every element is placed independently.
__device__ __forceinline__ unsigned long long lpt_key(const int32_t* __restrict__ cost, int i) {
  return ((unsigned long long)(0xFFFFFFFFu - (unsigned)cost[i]) << 32) | (unsigned)i;
}

// One key per thread: the keys are unique, so each key's place in its chunk's sorted order
// is the number of the chunk's keys below it, counted against all of them in LDS after one
// barrier.  Chunk blockIdx.x holds keys [c0, c0 + n); its kRankSortItems / 256 workgroups
// (blockIdx.y) each load the whole chunk and rank 256 of its keys, so one chunk's counting
// spreads over several CUs.  A single chunk writes the item indices to `order`, several
// write their sorted keys to `run` for merging.
constexpr int kRankSortItems = 1024;
constexpr int kRankThreads = 256;
__device__ __forceinline__ void lpt_rank_body(const int32_t* __restrict__ cost,
                                              int32_t* __restrict__ order,
                                              unsigned long long* __restrict__ run, int count,
                                              int chunk) {
  __shared__ __align__(16) unsigned long long keys[kRankSortItems];
  const int tid = threadIdx.x;
  const int c0 = chunk * kRankSortItems;
  const int n = min(kRankSortItems, count - c0);
#pragma unroll
  for (int i = tid; i < kRankSortItems; i += kRankThreads)
    keys[i] = i < n ? lpt_key(cost, c0 + i) : ~0ull;
  __syncthreads();
  const int me = blockIdx.y * kRankThreads + tid;  // this thread's key in the chunk
  if (me < n) {
    const unsigned long long mine = keys[me];
    // past n the keys are ~0, above every real key: count up to n rounded to 8, two keys
    // per 16-byte read, four reads in flight
    const int n8 = (n + 7) & ~7;
    const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(keys);
    int rank = 0;
    for (int i = 0; i < n8 / 2; i += 4) {
      ulonglong2 a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = k2[i + j];
#pragma unroll
      for (int j = 0; j < 4; ++j) rank += (a[j].x < mine ? 1 : 0) + (a[j].y < mine ? 1 : 0);
    }
    if (run) run[c0 + rank] = mine;
    else order[rank] = me;
  }
}

__global__ __launch_bounds__(kRankThreads) void k_lpt_rank(const int32_t* __restrict__ cost,
                                                           int32_t* __restrict__ order,
                                                           unsigned long long* __restrict__ run,
                                                           int count) {
  lpt_rank_body(cost, order, run, count, (int)blockIdx.x);
}

// Two lists of at most kRankSortItems keys each, sorted in one launch (blockIdx.x = list).
__global__ __launch_bounds__(kRankThreads) void k_lpt_rank_pair(
    const int32_t* __restrict__ cost0, int32_t* __restrict__ order0, int count0,
    const int32_t* __restrict__ cost1, int32_t* __restrict__ order1, int count1) {
  if (blockIdx.x == 0) lpt_rank_body(cost0, order0, nullptr, count0, 0);
  else lpt_rank_body(cost1, order1, nullptr, count1, 0);
}

// Number of keys in sorted a[0, n) below x.
__device__ __forceinline__ int rank_below(const unsigned long long* __restrict__ a, int n,
                                          unsigned long long x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// One merge pass: runs of `len` sorted keys in src, merged pairwise into dst; the last
// pass writes the item indices to `order` instead.
__global__ __launch_bounds__(256) void k_lpt_merge(const unsigned long long* __restrict__ src,
                                                   unsigned long long* __restrict__ dst,
                                                   int32_t* __restrict__ order, int count,
                                                   int len) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < count; i += gridDim.x * 256) {
    const int base = (i / (2 * len)) * (2 * len);
    const int na = min(len, count - base);
    const int nb = max(0, min(len, count - base - len));
    const unsigned long long x = src[i];
    const int pos = i - base < len ? (i - base) + rank_below(src + base + len, nb, x)
                                   : (i - base - len) + rank_below(src + base, na, x);
    if (order) order[base + pos] = (int32_t)(x & 0xFFFFFFFFull);
    else dst[base + pos] = x;
  }
}

// ---- Dense expansion through the kernels' own predicate (checking only) ----------
__global__ __launch_bounds__(256) void k_expand_mask(MaskArgs m, int b, int Nk, int row0,
                                                     int row1, uint8_t* __restrict__ dense) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= Nk) return;
  if (m.n == kBlocksMode) {
    // block grid of this mask row: grid_rows x ceil(Nk / 128) blocks
    const int nkb = (Nk + kMaskBlock - 1) / kMaskBlock;
    const uint8_t* g = m.blocks + (size_t)b * m.grid_rows * nkb;
    for (int i = row0 + blockIdx.y; i < row1; i += gridDim.y)
      dense[(size_t)(i - row0) * Nk + j] = g[(size_t)(i / kMaskBlock) * nkb + j / kMaskBlock] ? 0 : 1;
    return;
  }
  int lts = 0, lte = 0, uts = 0, ute = 0;
  int sv[kMaxIntervals] = {0, 0, 0, 0}, ev[kMaxIntervals] = {0, 0, 0, 0};
  if (m.n == 0) {
    const size_t o = (size_t)b * Nk + j;
    lts = m.v.lts[o]; lte = m.v.lte[o]; uts = m.v.uts[o]; ute = m.v.ute[o];
  } else {
    const size_t o = (size_t)b * m.n * Nk + j;
#pragma unroll
    for (int t = 0; t < kMaxIntervals; ++t) {
      if (t < m.n) {
        sv[t] = m.start[o + (size_t)t * Nk];
        ev[t] = m.end[o + (size_t)t * Nk];
      }
    }
  }
  const int4 s = {sv[0], sv[1], sv[2], sv[3]}, e = {ev[0], ev[1], ev[2], ev[3]};
  for (int w = blockIdx.y; row0 + 32 * w < row1; w += gridDim.y) {
    const int r0 = row0 + 32 * w;
    const uint32_t word = m.n == 0 ? hidden_rows32(lts, lte, uts, ute, r0)
                                   : hidden_rows32_multi(s, e, r0);
    const int nr = min(32, row1 - r0);
    for (int r = 0; r < nr; ++r)
      dense[(size_t)(r0 - row0 + r) * Nk + j] = (uint8_t)((word >> r) & 1u);
  }
}

// ---- host launchers --------------------------------------------------------------
namespace {

// Rows of Q-blocks per k_classify_q workgroup: 1 up to 4096 queue rows (every attention call
// at its own tile shapes), more for longer lists, keeping at least 2048 workgroups.
int classify_rows_per_wg(int64_t rows) {
  return rows >= 16384 ? 8 : rows >= 8192 ? 4 : rows > 4096 ? 2 : 1;
}

template <int kMode>
void* classify_q_kernel(int R) {
  return R == 8 ? (void*)k_classify_q<kMode, 8>
         : R == 4 ? (void*)k_classify_q<kMode, 4>
         : R == 2 ? (void*)k_classify_q<kMode, 2>
                  : (void*)k_classify_q<kMode, 1>;
}
template <int kMode>
void* classify_pair_kernel(int R) {
  return R == 8 ? (void*)k_classify_pair<kMode, 8>
         : R == 4 ? (void*)k_classify_pair<kMode, 4>
         : R == 2 ? (void*)k_classify_pair<kMode, 2>
                  : (void*)k_classify_pair<kMode, 1>;
}
int mask_mode(const MaskArgs& m) { return m.n == kBlocksMode ? 2 : (m.n > 0 ? 1 : 0); }

// Block min/max of B mask rows at bk keys per block into mm; with mm2 (four-vector form
// only), also at bk2 < bk into mm2 in the same pass.
void launch_minmax(const MaskArgs& m, int B, int Nk, int bk, int32_t* mm, int bk2,
                   int32_t* mm2, hipStream_t s) {
  const int nKB = (Nk + bk - 1) / bk;
  if (nKB == 0) return;
  const int mode = mask_mode(m);
  if (mode == 1) {
    hipLaunchKernelGGL(k_block_minmax_multi, dim3(B * nKB), dim3(64), 0, s, m.start, m.end,
                       m.n, Nk, nKB, bk, mm);
  } else if (mode == 0) {
    const int n_sc = (Nk + 255) / 256, total = B * n_sc;
    const int grid = min((total + 3) / 4, 2048);
    const int nKB2 = mm2 ? (Nk + bk2 - 1) / bk2 : 0;
    hipLaunchKernelGGL(k_block_minmax, dim3(grid), dim3(256), 0, s, m.v, Nk, nKB, bk, n_sc,
                       total, mm, bk2, nKB2, mm2);
  }
}

}  // namespace

hipError_t launch_classify(const MaskArgs& m, int B, int Nq, int Nk, int bq, int bk,
                           const TileOut& out, hipStream_t s) {
  const int nQB = (Nq + bq - 1) / bq, nKB = (Nk + bk - 1) / bk;
  if (B == 0) return hipSuccess;
  const int mode = mask_mode(m);
  GridArgs ga{m.blocks, (Nq + kMaskBlock - 1) / kMaskBlock, (Nk + kMaskBlock - 1) / kMaskBlock,
              bk, Nk, nKB};
  launch_minmax(m, B, Nk, bk, out.minmax, 0, nullptr, s);
  // with no KV block a Q-block's queue is empty; with no Q-block a KV block's is
  if ((out.tile_class || out.q_queue) && nQB > 0) {
    const int R = classify_rows_per_wg((int64_t)B * nQB);
    const int groups = (nQB + R - 1) / R;
    ClassifyQArgs qa{out.minmax, ga, Nq, nQB, nKB, bq, groups, out.tile_class, out.q_queue,
                     out.q_count, out.q_cost};
    void* kq = mode == 2 ? classify_q_kernel<2>(R)
               : mode == 1 ? classify_q_kernel<1>(R) : classify_q_kernel<0>(R);
    hipLaunchKernelGGL((void (*)(ClassifyQArgs, int))kq, dim3(B * groups), dim3(256), 0, s, qa,
                       m.n);
  }
  if (out.k_queue && nKB > 0) {
    ClassifyKArgs ka{out.minmax, ga, Nq, nQB, nKB, bq, out.k_queue, out.k_count, out.k_cost};
    auto kk = mode == 2 ? k_classify_k<2> : (mode == 1 ? k_classify_k<1> : k_classify_k<0>);
    hipLaunchKernelGGL(kk, dim3(B * nKB), dim3(256), 0, s, ka, m.n);
  }
  return hipGetLastError();
}

hipError_t launch_classify_pair(const MaskArgs& m, int B, int Nq, int Nk, int bq_k, int bk_k,
                                const TileOut& out_k, int bq_q, int bk_q, const TileOut& out_q,
                                hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int mode = mask_mode(m);
  const int nQB_k = (Nq + bq_k - 1) / bq_k, nKB_k = (Nk + bk_k - 1) / bk_k;
  const int nQB_q = (Nq + bq_q - 1) / bq_q, nKB_q = (Nk + bk_q - 1) / bk_q;
  // block bounds at both block sizes: one pass over the vectors when the K side's blocks
  // are the larger ones
  if (mode == 0 && bk_q < bk_k && bk_k % bk_q == 0) {
    launch_minmax(m, B, Nk, bk_k, out_k.minmax, bk_q, out_q.minmax, s);
  } else {
    launch_minmax(m, B, Nk, bk_k, out_k.minmax, 0, nullptr, s);
    launch_minmax(m, B, Nk, bk_q, out_q.minmax, 0, nullptr, s);
  }
  const int nk = (out_k.k_queue && nKB_k > 0) ? B * nKB_k : 0;  // K-side workgroups
  const bool q_side = (out_q.tile_class || out_q.q_queue) && nQB_q > 0;
  const int R = classify_rows_per_wg((int64_t)B * nQB_q);
  const int groups = (nQB_q + R - 1) / R;
  const int nq = q_side ? B * groups : 0;
  if (nk + nq == 0) return hipGetLastError();
  GridArgs ga_k{m.blocks, (Nq + kMaskBlock - 1) / kMaskBlock,
                (Nk + kMaskBlock - 1) / kMaskBlock, bk_k, Nk, nKB_k};
  GridArgs ga_q{m.blocks, (Nq + kMaskBlock - 1) / kMaskBlock,
                (Nk + kMaskBlock - 1) / kMaskBlock, bk_q, Nk, nKB_q};
  ClassifyKArgs ka{out_k.minmax, ga_k, Nq, nQB_k, nKB_k, bq_k, out_k.k_queue, out_k.k_count,
                   out_k.k_cost};
  ClassifyQArgs qa{out_q.minmax, ga_q, Nq, nQB_q, nKB_q, bq_q, groups, out_q.tile_class,
                   out_q.q_queue, out_q.q_count, out_q.q_cost};
  void* kp = mode == 2 ? classify_pair_kernel<2>(R)
             : mode == 1 ? classify_pair_kernel<1>(R) : classify_pair_kernel<0>(R);
  hipLaunchKernelGGL((void (*)(ClassifyKArgs, ClassifyQArgs, int, int))kp, dim3(nk + nq),
                     dim3(256), 0, s, ka, qa, m.n, nk);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero_i32(int32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_zero_i32, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     p, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_iota_i32(int32_t* __restrict__ p, int n) {
  for (int i = (int)(blockIdx.x * 256 + threadIdx.x); i < n; i += (int)(gridDim.x * 256)) p[i] = i;
}

hipError_t launch_iota_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_iota_i32, dim3(blocks < 4096 ? blocks : 4096), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

size_t lpt_sort_scratch_bytes(int64_t count) {
  return count > kRankSortItems ? 2 * (size_t)count * sizeof(unsigned long long) : 0;
}

hipError_t launch_lpt_sort(const int32_t* cost, int32_t* order, int count, void* scratch,
                           hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (count <= kRankSortItems) {
    const unsigned parts = (unsigned)((count + kRankThreads - 1) / kRankThreads);
    hipLaunchKernelGGL(k_lpt_rank, dim3(1, parts), dim3(kRankThreads), 0, s, cost, order,
                       (unsigned long long*)nullptr, count);
    return hipGetLastError();
  }
  unsigned long long* a = static_cast<unsigned long long*>(scratch);
  unsigned long long* b = a + count;
  const int chunks = (count + kRankSortItems - 1) / kRankSortItems;
  hipLaunchKernelGGL(k_lpt_rank, dim3(chunks, kRankSortItems / kRankThreads), dim3(kRankThreads),
                     0, s, cost, (int32_t*)nullptr, a, count);
  const unsigned grid = (unsigned)min((count + 255) / 256, 4096);
  for (int len = kRankSortItems; len < count; len *= 2) {
    const bool last = 2 * (int64_t)len >= count;
    hipLaunchKernelGGL(k_lpt_merge, dim3(grid), dim3(256), 0, s, a, b, last ? order : nullptr,
                       count, len);
    unsigned long long* t = a; a = b; b = t;
  }
  return hipGetLastError();
}

hipError_t launch_lpt_sort_pair(const int32_t* cost0, int32_t* order0, int count0,
                                const int32_t* cost1, int32_t* order1, int count1,
                                void* scratch, hipStream_t s) {
  if (count0 <= 0 || count1 <= 0 || count0 > kRankSortItems || count1 > kRankSortItems) {
    hipError_t e = launch_lpt_sort(cost0, order0, count0, scratch, s);
    if (e == hipSuccess) e = launch_lpt_sort(cost1, order1, count1, scratch, s);
    return e;
  }
  const unsigned parts = (unsigned)((max(count0, count1) + kRankThreads - 1) / kRankThreads);
  hipLaunchKernelGGL(k_lpt_rank_pair, dim3(2, parts), dim3(kRankThreads), 0, s, cost0, order0,
                     count0, cost1, order1, count1);
  return hipGetLastError();
}

hipError_t launch_expand_mask(const MaskArgs& m, int b, int Nk, int row0, int row1,
                              uint8_t* dense, hipStream_t s) {
  if (Nk == 0 || row1 <= row0) return hipSuccess;
  const int windows = (row1 - row0 + 31) / 32;
  dim3 grid((Nk + 255) / 256, (unsigned)min(windows, 65535));
  hipLaunchKernelGGL(k_expand_mask, grid, dim3(256), 0, s, m, b, Nk, row0, row1, dense);
  return hipGetLastError();
}

// ---- Mask localization for one context-parallel rank (FlashMask-3 page, §3.2) ----
// x_local = sum_i clamp(x - offsets[i], 0, C): the rank's rows before global row x.  The
// chunk offsets are staged once per workgroup in LDS.
// `four` selects the four arrays of the four-vector form, else the first two (start, end).
__global__ __launch_bounds__(256) void k_localize(MaskPtrs g, int four,
                                                  const int32_t* __restrict__ offsets,
                                                  int n_chunks, int C, MaskOut out,
                                                  int64_t cols) {
  __shared__ int32_t offs[4096];
  for (int i = threadIdx.x; i < n_chunks; i += 256) offs[i] = offsets[i];
  __syncthreads();
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < cols;
       c += (int64_t)gridDim.x * 256) {
    const int x0 = g.lts[c], x1 = g.lte[c];
    const int x2 = four ? g.uts[c] : 0, x3 = four ? g.ute[c] : 0;
    int y0 = 0, y1 = 0, y2 = 0, y3 = 0;
    for (int i = 0; i < n_chunks; ++i) {
      const int o = offs[i];
      y0 += min(max(x0 - o, 0), C);
      y1 += min(max(x1 - o, 0), C);
      y2 += min(max(x2 - o, 0), C);
      y3 += min(max(x3 - o, 0), C);
    }
    out.lts[c] = y0;
    out.lte[c] = y1;
    if (four) {
      out.uts[c] = y2;
      out.ute[c] = y3;
    }
  }
}

hipError_t launch_localize(const MaskPtrs& g, int arrays, const int32_t* offsets, int n_chunks,
                           int chunk_len, const MaskOut& out, int64_t cols, hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  const int64_t blocks = (cols + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 2048 ? blocks : 2048);
  hipLaunchKernelGGL(k_localize, dim3(grid), dim3(256), 0, s, g, arrays == 4 ? 1 : 0, offsets,
                     n_chunks, chunk_len, out, cols);
  return hipGetLastError();
}

// ---- Range check of the row bounds ----
// Counts the values of `arrays` int32 arrays of `cols` entries each that lie outside
// [0, hi]; one global atomic per workgroup.  `bad` must start at zero (the launcher clears
// it with a fill kernel first).
__global__ __launch_bounds__(256) void k_check_bounds(MaskPtrs g, int arrays, int64_t cols,
                                                      int hi, int32_t* __restrict__ bad) {
  __shared__ int count;
  if (threadIdx.x == 0) count = 0;
  __syncthreads();
  int mine = 0;
  const int32_t* a[4] = {g.lts, g.lte, g.uts, g.ute};
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < cols;
       c += (int64_t)gridDim.x * 256) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (x < arrays) {
        const int v = a[x][c];
        mine += (v < 0 || v > hi) ? 1 : 0;
      }
    }
  }
  if (mine) atomicAdd(&count, mine);
  __syncthreads();
  if (threadIdx.x == 0 && count) atomicAdd(bad, count);
}

hipError_t launch_check_bounds(const MaskPtrs& g, int arrays, int64_t cols, int hi, int32_t* bad,
                               hipStream_t s) {
  hipError_t e = launch_zero_i32(bad, 1, s);
  if (e != hipSuccess || cols <= 0) return e;
  const int64_t blocks = (cols + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 2048 ? blocks : 2048);
  hipLaunchKernelGGL(k_check_bounds, dim3(grid), dim3(256), 0, s, g, arrays, cols, hi, bad);
  return hipGetLastError();
}

}  // namespace fm
