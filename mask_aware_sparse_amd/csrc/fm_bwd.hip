// Mask-aware attention backward (gfx950, bf16 MFMA 32x32x16).
//
// Recomputation backward of the Flash MSA guide ("The Backward Pass: The Real Beast"):
// with the forward's statistic LSE, P = exp(S - LSE) is recomputed per tile, then
//   dV += P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK += scale dS^T Q,
//   dQ += scale dS K,   D_i = sum_j P_ij dP_ij = rowsum(dO o O).
// (The guide writes dQ and dK without the softmax scale; the chain rule through
// S = scale Q K^T puts it there.)
//
// Work split.  dK/dV sum over query rows and dQ over keys, so no single tile order
// serves both without a reduction through memory.  Adding dQ partials with fp32
// atomics from a KV-block-outer kernel is bound by the L2's atomic rate on MI355X, so
// the two sums run in two kernels that each own their output tile:
//   k_attn_bwd_dq    one workgroup per (b, 128-row Q-block, query head), numbered in the
//                    forward's LPT order.  It first forms D = rowsum(dO o O) and LSE in
//                    log2 units (+inf for rows that see nothing, so P = 0 there) for its
//                    rows and writes both for the dK/dV kernel; then it walks the forward's
//                    queue of 64-key blocks, recomputes S^T and dP^T, and accumulates
//                    dQ^T = K^T dS^T in registers (a lane owns one query row, as in the
//                    forward); dQ is written once.
//   k_attn_bwd_dkdv  one workgroup per (b, kv head, 128-key KV block, chunk of <= 4 query
//                    heads), numbered in LPT order of the KV blocks' tile costs; each of
//                    the 4 waves owns 32 keys; the workgroup walks the block's queue of
//                    32-row Q-blocks (partial tiles masked), recomputes S and dP, and keeps
//                    dK/dV in registers.  With one head chunk per KV head the workgroup
//                    owns its dK/dV rows and stores them as bf16; with several (GQA/MQA
//                    groups above 4 heads) it adds them to fp32 accumulators, which
//                    k_zero clears before and k_bwd_convert turns into bf16 after.
//   k_plan_split     one workgroup: the dK/dV work units.  A (mask row, KV block) pair
//                    whose queue is long against the average load of a workgroup slot is
//                    cut into segments of its queue (the sink keys of a window mask are
//                    seen by every row, so their block would otherwise be one serial chain
//                    longer than the rest of the launch).  Segments of a pair that would
//                    store bf16 directly write fp32 partial sums instead, and
//   k_dkdv_reduce    adds them in segment order (deterministic) and stores bf16.
#include "fm_device.h"
#include "fm_internal.h"

#include <type_traits>

namespace fm {
namespace {


__global__ __launch_bounds__(256) void k_zero(float4* __restrict__ p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = float4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(256) void k_bwd_convert(const float* __restrict__ src,
                                                     bf16* __restrict__ dst, float mul,
                                                     size_t n8) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
    u32x4 w;
    w[0] = pack_bf16x2(a.x * mul, a.y * mul);
    w[1] = pack_bf16x2(a.z * mul, a.w * mul);
    w[2] = pack_bf16x2(b.x * mul, b.y * mul);
    w[3] = pack_bf16x2(b.z * mul, b.w * mul);
    reinterpret_cast<u32x4*>(dst)[i] = w;
  }
}

// A-operand row permutation (bits 2 and 3 of the row index swapped): the accumulator
// rows a lane then owns are runs of 8 consecutive rows of the source, which is the
// k-ordering the next product wants for its register operand.
__device__ __forceinline__ int perm_rows(int a) {
  return (a & 0x13) | ((a & 4) << 1) | ((a & 8) >> 1);
}

// ---- KE: dK / dV (KV-block outer) -------------------------------------------------------
// kW waves x 32 keys per workgroup.  kW = 4: one 128-key block per workgroup, two
// workgroups per CU (78 KB of LDS each), so the two waves on a SIMD belong to different
// workgroups and their MFMA and softmax phases drift apart instead of meeting at the same
// barriers.  kW = 8 (sorted keys, D <= 128): one 256-key block per workgroup and CU, which
// reads each Q/dO row once per 256 keys instead of per 128 (half the bytes from HBM where
// the rows do not stay in L2).  Steps are 32-row Q-blocks, which keeps the live registers
// of a wave within 256.
namespace dkdv {
constexpr int BQ = kBwdBlockQ;  // 32 query rows per step

// Q / dO tiles use the swizzled layout (row reads and transposing reads; 320-byte rows at
// D <= 128), K rows are read row-wise only (272 bytes).
template <int D, bool kMulti, int BK>
struct __attribute__((aligned(16))) Smem {
  bf16 q[2][BQ * LdsRows<D>::SWZ];
  bf16 dO[2][BQ * LdsRows<D>::SWZ];
  bf16 k[BK * LdsRows<D>::KS];
  // per key of the block: the four row bounds, or the interval starts ([0]) and ends ([1])
  int4 mv[kMulti ? 2 : 1][BK];
  float lse2[2][BQ];
  float dl[2][BQ];
};
}  // namespace dkdv

struct DkdvParams {
  const bf16* __restrict__ q;
  const bf16* __restrict__ k;
  const bf16* __restrict__ v;
  const bf16* __restrict__ dout;
  const float* __restrict__ lse2;
  const float* __restrict__ delta;
  MaskArgs m;
  const int32_t* __restrict__ k_queue;
  const int32_t* __restrict__ k_count;
  const int32_t* __restrict__ k_order;
  float* __restrict__ dk_acc;  // fp32 accumulators (writers > 1)
  float* __restrict__ dv_acc;
  bf16* __restrict__ dk;       // bf16 outputs (writers == 1)
  bf16* __restrict__ dv;
  int B, Hq, Hkv, Nq, Nk, nQB, nKB;  // Nq query rows, Nk keys
  HeadMap hm;                        // mask sets, chunking and writers per KV block
  const int32_t* __restrict__ unit_pair;     // work units (split plan)
  const int32_t* __restrict__ unit_slot;
  const int32_t* __restrict__ split_counts;  // {units, split pairs}
  float* __restrict__ partials;              // [2][nslots][BK][D] fp32 (dK then dV)
  int nslots;
  float c;      // scale * log2(e)
  float scale;  // softmax scale (applied to dK)
};

// The query heads and kv head of one dK/dV workgroup: pair (mask row, KV block) `item`,
// then the rem-th (kv head of the set, head chunk) of that pair.
struct DkdvItem {
  int mr, kb, b, kvh, h0, nh;
};
__device__ __forceinline__ DkdvItem dkdv_item(const HeadMap& hm, int Hq, int Hkv, int nKB,
                                              int item, int rem) {
  DkdvItem it;
  const int kvl = rem / hm.cpk, ch = rem - kvl * hm.cpk;
  it.mr = item / nKB;
  it.kb = item - it.mr * nKB;
  it.b = it.mr / hm.Hm;
  const int g = Hq / Hkv;
  const int hq0 = (it.mr - it.b * hm.Hm) * hm.qpm;  // first query head of the set
  it.kvh = hq0 / g + kvl;
  const int hs = max(it.kvh * g, hq0);             // first query head of (kv head, set)
  it.h0 = hs + ch * hm.hc;
  it.nh = min(hm.hc, hs + hm.gq - it.h0);
  return it;
}

// ---- Split plan of the dK/dV work units (one workgroup of kPlanThreads) ---------------
// Pairs r = 0 .. npairs-1 in LPT order.  Each of a pair's `per` workgroups walks
// u_r = (queue length) x hc tile steps, and the average load of a workgroup slot is
// L = per * sum_r u_r / slots.  A pair with u_r > L / 2 is cut into
// s_r = min(kSplitMaxSegs, ceil(2 u_r / L), queue length, u_r / kSplitMinSteps) segments,
// the extra segments granted in pair order while they fit in `extra`.  Unit table, pairs in
// LPT order and the segments of a pair consecutive:
//   unit_pair[u] = r | seg << 24 | (s_r - 1) << 28 (r < 2^24);  unit_slot[u] = first partial slot of the
//   segment (its `per` workgroups use slot + rem) or -1 when unsplit or with_slots == 0;
//   split_pair[j] = r | (s_r - 1) << 28, split_slot[j] = the pair's first slot;
//   counts = {units, split pairs}.
constexpr int kPlanThreads = 1024;
constexpr int kPlanPerThread = (kMaxSortItems + kPlanThreads - 1) / kPlanThreads;

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of x over the workgroup's threads in thread order; *total = the sum.
__device__ int block_excl_scan(int x, int* sh, int* total) {
  constexpr int kW = kPlanThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int inc = wave_incl_scan(x);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < kW; ++i) {
      const int t = sh[i];
      sh[i] = acc;
      acc += t;
    }
    sh[kW] = acc;
  }
  __syncthreads();
  const int r = sh[w] + inc - x;
  *total = sh[kW];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void k_plan_split(
    const int32_t* __restrict__ k_count, const int32_t* __restrict__ k_order, int npairs, int per,
    int hc, int slots, int extra, int with_slots, int32_t* __restrict__ unit_pair,
    int32_t* __restrict__ unit_slot, int32_t* __restrict__ split_pair,
    int32_t* __restrict__ split_slot, int32_t* __restrict__ counts) {
  __shared__ long long red[kPlanThreads];
  __shared__ int sh[kPlanThreads / 64 + 1];
  const int tid = threadIdx.x;
  if (npairs > kPlanThreads * kPlanPerThread) {
    // more pairs than the plan handles in one workgroup: one unit per pair, no split
    for (int r = tid; r < npairs; r += kPlanThreads) {
      unit_pair[r] = r;
      unit_slot[r] = -1;
    }
    if (tid == 0) {
      counts[0] = npairs;
      counts[1] = 0;
    }
    return;
  }
  const int c = (npairs + kPlanThreads - 1) / kPlanThreads;  // pairs of this thread (<= 8)
  const int r0 = tid * c;
  int nq[kPlanPerThread];
  long long mine = 0;
#pragma unroll
  for (int i = 0; i < kPlanPerThread; ++i) {
    const int r = r0 + i;
    nq[i] = 0;
    if (i < c && r < npairs) {
      const int item = k_order[r];
      nq[i] = k_count[2 * item] + k_count[2 * item + 1];
      mine += (long long)nq[i] * hc;
    }
  }
  red[tid] = mine;
  __syncthreads();
  for (int st = kPlanThreads / 2; st > 0; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  // split above half the average slot load; where segments need the partial-sum reduction
  // (with_slots), only above the full average load
  long long half = red[0] * per / ((with_slots ? 1LL : 2LL) * slots);
  if (half < kSplitMinSteps) half = kSplitMinSteps;

  int want[kPlanPerThread];
  int my_want = 0;
#pragma unroll
  for (int i = 0; i < kPlanPerThread; ++i) {
    const long long u = (long long)nq[i] * hc;
    long long sg = 1;
    if (u > half) {
      sg = (u + half - 1) / half;
      sg = sg < kSplitMaxSegs ? sg : kSplitMaxSegs;
      sg = sg < nq[i] ? sg : nq[i];
      sg = sg < u / kSplitMinSteps ? sg : u / kSplitMinSteps;
      sg = sg > 1 ? sg : 1;
    }
    want[i] = (int)sg - 1;
    my_want += want[i];
  }
  int total;
  int before = block_excl_scan(my_want, sh, &total);
  int segs[kPlanPerThread];
  int my_units = 0, my_split = 0, my_slots = 0;
#pragma unroll
  for (int i = 0; i < kPlanPerThread; ++i) {
    const int allowed = max(0, min(want[i], extra - before));
    before += want[i];
    segs[i] = 1 + allowed;
    if (i < c && r0 + i < npairs) {
      my_units += segs[i];
      if (segs[i] > 1) {
        my_split += 1;
        my_slots += segs[i] * per;
      }
    }
  }
  int units_total, split_total, slots_total;
  int u_pos = block_excl_scan(my_units, sh, &units_total);
  int j_pos = block_excl_scan(my_split, sh, &split_total);
  int s_pos = block_excl_scan(my_slots, sh, &slots_total);
#pragma unroll
  for (int i = 0; i < kPlanPerThread; ++i) {
    const int r = r0 + i;
    if (i < c && r < npairs) {
      const int sg = segs[i];
      for (int q = 0; q < sg; ++q) {
        unit_pair[u_pos + q] = (int32_t)((unsigned)r | ((unsigned)q << 24) | ((unsigned)(sg - 1) << 28));
        unit_slot[u_pos + q] = (sg > 1 && with_slots) ? s_pos + q * per : -1;
      }
      if (sg > 1) {
        split_pair[j_pos] = (int32_t)((unsigned)r | ((unsigned)(sg - 1) << 28));
        split_slot[j_pos] = with_slots ? s_pos : -1;
        ++j_pos;
        s_pos += sg * per;
      }
      u_pos += sg;
    }
  }
  if (tid == 0) {
    counts[0] = units_total;
    counts[1] = split_total;
  }
}

// kMulti: the mask is the multi-interval form (else the four-vector form).  kW: waves (of
// 32 keys each) per workgroup, 4 or 8.
template <int D, bool kMulti, int kW>
__global__ __launch_bounds__(64 * kW, (D > 128 || kW > 4) ? 1 : 2) void k_attn_bwd_dkdv(DkdvParams p) {
  using namespace dkdv;
  constexpr int kWaves = kW;
  constexpr int BK = 32 * kW;  // keys per workgroup
  constexpr int KS = LdsRows<D>::KS;    // K row stride in LDS (elements)
  constexpr int kRow = LdsRows<D>::SWZ;  // swizzled Q / dO row stride
  constexpr int kS = D / 16;   // k-steps of a 32x32x16 product over D
  constexpr int kDB = D / 32;  // 32-column blocks of dK / dV
  constexpr int kCh = D / 8;   // 16-byte chunks per row
  __shared__ Smem<D, kMulti, BK> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int N = p.Nk, Nq = p.Nq;  // N: keys (and mask columns)

  // workgroup: work unit (a segment of the queue of an LPT pair (mask row, KV block)),
  // then a kv head of that mask set and a chunk of at most hc of its query heads
  const int per = p.hm.kvpm * p.hm.cpk;
  const int pu = blockIdx.x / per, rem = blockIdx.x - pu * per;
  if (pu >= p.split_counts[0]) return;  // the grid covers the largest possible plan
  const int ue = p.unit_pair[pu];
  const int seg = (int)(((unsigned)ue >> 24) & 15u), nseg = (int)((unsigned)ue >> 28) + 1;
  const int slot = p.unit_slot[pu];     // >= 0: a segment writing fp32 partial sums
  const int item = p.k_order[ue & 0xFFFFFF];
  const DkdvItem wi = dkdv_item(p.hm, p.Hq, p.Hkv, p.nKB, item, rem);
  const int mr = wi.mr, kb = wi.kb, b = wi.b, kvh = wi.kvh, h0 = wi.h0, nh = wi.nh;
  const bool direct = p.hm.writers == 1;
  const int nq_all = p.k_count[2 * item] + p.k_count[2 * item + 1];
  const int q_lo = seg * nq_all / nseg;
  const int nq = (seg + 1) * nq_all / nseg - q_lo;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const uint32_t acc_bytes = (uint32_t)N * D * 4;
  const size_t kvbase = (size_t)(b * p.Hkv + kvh) * N * D;
  if (nh <= 0) return;
  if (nq == 0) {
    // no query row sees these keys: dK = dV = 0 (the accumulators start at zero)
    if (direct) {
      const rsrc_t dkr = make_rsrc(p.dk + kvbase, head_bytes);
      const rsrc_t dvr = make_rsrc(p.dv + kvbase, head_bytes);
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < BK * D * 2 / (16 * 64 * kWaves); ++i) {
        const uint32_t off = (uint32_t)kb * (BK * D * 2) + (uint32_t)(i * 64 * kWaves + tid) * 16;
        buf_store16(z, dkr, off, 0);
        buf_store16(z, dvr, off, 0);
      }
    }
    return;
  }
  const int32_t* queue = p.k_queue + (size_t)item * p.nQB + q_lo;
  const bool ragged_k = (N % BK) != 0 && kb == p.nKB - 1;

  // ---- K of the block into LDS (B operand of S = Q K^T), V resident in registers
  const int key = kb * BK + wave * 32 + l32;
  bf16x8 vr[kS];
  {
    const rsrc_t kr_ = make_rsrc(p.k + kvbase, head_bytes);
    const rsrc_t vr_ = make_rsrc(p.v + kvbase, head_bytes);
    const uint32_t off = (uint32_t)key * (D * 2) + hh * 16;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      vr[s] = __builtin_bit_cast(bf16x8, buf_load16(vr_, off, s * 32));
      *reinterpret_cast<u32x4*>(&sm.k[(wave * 32 + l32) * KS + s * 16 + hh * 8]) =
          buf_load16(kr_, off, s * 32);
    }
  }
  if constexpr (!kMulti) {
    if (hh == 0) {
      const uint32_t vb = (uint32_t)N * 4, vo = (uint32_t)key * 4;
      const size_t mrow = (size_t)mr * N;
      sm.mv[0][wave * 32 + l32] = int4{(int)buf_load4(make_rsrc(p.m.v.lts + mrow, vb), vo, 0),
                                       (int)buf_load4(make_rsrc(p.m.v.lte + mrow, vb), vo, 0),
                                       (int)buf_load4(make_rsrc(p.m.v.uts + mrow, vb), vo, 0),
                                       (int)buf_load4(make_rsrc(p.m.v.ute + mrow, vb), vo, 0)};
    }
  } else {
    // lanes of the first half load the key's interval starts, the second half its ends;
    // absent intervals read past the row's bounds and load 0 (the empty interval)
    const uint32_t vb = (uint32_t)N * 4, vo = (uint32_t)key * 4;
    const size_t mrow = (size_t)mr * p.m.n * N;
    const rsrc_t rs = make_rsrc((hh ? p.m.end : p.m.start) + mrow, (uint32_t)p.m.n * vb);
    sm.mv[hh][wave * 32 + l32] = int4{(int)buf_load4(rs, vo, 0), (int)buf_load4(rs, vo + vb, 0),
                                      (int)buf_load4(rs, vo + 2 * vb, 0),
                                      (int)buf_load4(rs, vo + 3 * vb, 0)};
  }
  const bool key_ok = key < N;

  f32x16 dk[kDB], dv[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) { dk[d] = f32x16{}; dv[d] = f32x16{}; }

  // ---- staging of the Q / dO tiles: thread copies rows tid/kCh + kCpRows*i, chunk tid%kCh
  constexpr int kCp = BQ * kCh / (64 * kWaves);  // 16-byte chunks per thread and tensor
  constexpr int kCpRows = 64 * kWaves / kCh;
  static_assert(kCp * 64 * kWaves == BQ * kCh, "whole chunks per thread");
  const int cp_row = tid / kCh, cp_ch = tid % kCh;
  u32x4 qst[kCp], ost[kCp];
  uint32_t lst = 0u, dst_ = 0u;
  const int nsteps = nh * nq;

  auto load_step = [&](int hi, int it) {
    const int h = h0 + hi;
    const int qb = queue[it] & 0x7fffffff;
    const size_t base = (size_t)(b * p.Hq + h) * Nq;
    const uint32_t q_bytes = (uint32_t)Nq * D * 2;
    const rsrc_t qrs = make_rsrc(p.q + base * D, q_bytes);
    const rsrc_t ors = make_rsrc(p.dout + base * D, q_bytes);
    const uint32_t off = (uint32_t)(qb * BQ + cp_row) * (D * 2) + cp_ch * 16;
#pragma unroll
    for (int i = 0; i < kCp; ++i) {
      qst[i] = buf_load16(qrs, off, i * kCpRows * D * 2);
      ost[i] = buf_load16(ors, off, i * kCpRows * D * 2);
    }
    if (tid < BQ) {
      const uint32_t ro = (uint32_t)(qb * BQ + tid) * 4;
      lst = buf_load4(make_rsrc(p.lse2 + base, (uint32_t)Nq * 4), ro, 0);
      dst_ = buf_load4(make_rsrc(p.delta + base, (uint32_t)Nq * 4), ro, 0);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kCp; ++i) {
      const int o = swz<kRow>(cp_row + i * kCpRows, cp_ch);
      *reinterpret_cast<u32x4*>(&sm.q[buf][o]) = qst[i];
      *reinterpret_cast<u32x4*>(&sm.dO[buf][o]) = ost[i];
    }
    if (tid < BQ) {
      sm.lse2[buf][tid] = __uint_as_float(lst);
      sm.dl[buf][tid] = -__uint_as_float(dst_);  // -D: the dP products start from it
    }
  };

  load_step(0, 0);
  store_step(0);
  lds_barrier();

  const int arow = perm_rows(l32);
  const SwzRowRead<kRow> rr(arow, hh);
  const SwzTrRead<kRow> tr(lane, hh);
  const bf16* kp = &sm.k[(wave * 32 + l32) * KS + hh * 8];

  // steps walk (head hi, queue entry it) with it fastest
  int hi = 0, it = 0;
  auto step = [&](auto cur_c, int st) {
    const int cur = cur_c;  // the step's LDS buffer (a constant in the unrolled loop below)
    const int e = queue[it];
    const int qb = e & 0x7fffffff;
    const bool partial = (e < 0) || ragged_k;
    if (++it == nq) { it = 0; ++hi; }
    const bool has_next = st + 1 < nsteps;
    if (has_next) load_step(hi, it);

    // Hidden-row word of this lane's key over the step's 32 rows (partial steps only).
    auto mask_word = [&]() {
      const int r0 = qb * BQ;
      uint32_t w;
      if constexpr (!kMulti) {
        const int4 mv = sm.mv[0][wave * 32 + l32];
        w = hidden_rows32(mv.x, mv.y, mv.z, mv.w, r0);
      } else {
        w = hidden_rows32_multi(sm.mv[0][wave * 32 + l32], sm.mv[1][wave * 32 + l32], r0);
      }
      return key_ok ? w : 0xFFFFFFFFu;
    };
    // At D <= 128 a wave whose 32 keys are hidden from all 32 rows of a partial step adds
    // nothing to dK/dV there and skips the step's products and softmax gradient, leaving
    // the cycles to the other wave on its SIMD.  (At D = 256 the word is formed inside the
    // softmax gradient: kept live across the larger products it would spill.)
    constexpr bool kSkipDead = D <= 128;
    uint32_t word = 0u;
    bool live = true;
    if constexpr (kSkipDead) {
      if (partial) {
        word = mask_word();
        live = __builtin_amdgcn_ballot_w64(word != 0xFFFFFFFFu) != 0;
      }
    }
    if (live) {
      constexpr int qblk = 0;
      // ---- S = Q K^T and dP = dO V^T for 32 query rows x this wave's 32 keys.  Step s
      // reads its K, Q and dO fragments one step ahead; the scheduling barriers keep the
      // reads ahead of the products. ----
      // dP - D in one: the dP products accumulate onto -D of each row, which lies in LDS in
      // the accumulator's element order (element j*8 + t: row j*16 + hh*8 + t)
      f32x16 sacc, pacc;
      {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int q0 = qblk * 32 + j * 16 + hh * 8;
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sm.dl[cur][q0]);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sm.dl[cur][q0 + 4]);
#pragma unroll
          for (int t = 0; t < 4; ++t) { pacc[j * 8 + t] = d0[t]; pacc[j * 8 + 4 + t] = d1[t]; }
        }
      }
      {
        bf16x8 kf[2], qf[2], of[2];
        auto rd = [&](int s, int slot) {
          const int o = rr.at(s) + qblk * 32 * kRow;
          kf[slot] = *reinterpret_cast<const bf16x8*>(kp + s * 16);
          qf[slot] = *reinterpret_cast<const bf16x8*>(&sm.q[cur][o]);
          of[slot] = *reinterpret_cast<const bf16x8*>(&sm.dO[cur][o]);
        };
        rd(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < kS; ++s) {
          if (s + 1 < kS) rd(s + 1, (s + 1) & 1);
          sacc = mfma32(qf[s & 1], kf[s & 1], s == 0 ? f32x16{} : sacc);
          pacc = mfma32(of[s & 1], vr[s], pacc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- P = exp2(S c - LSE2), masked on partial tiles; dS = P (dP - D) ----
      bf16x8 pa[2], sa[2];
      auto softmax_grad = [&](auto masked) {
        constexpr bool kMasked = decltype(masked)::value;
        if constexpr (kMasked && !kSkipDead) word = mask_word();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int q0 = qblk * 32 + j * 16 + hh * 8;
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(&sm.lse2[cur][q0]);
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(&sm.lse2[cur][q0 + 4]);
          u32x4 pw, sw;
#pragma unroll
          for (int t = 0; t < 8; t += 2) {
            float pv[2], sv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int tt = t + u;
              const float l = tt < 4 ? l0[tt] : l1[tt - 4];
              float pp = __builtin_amdgcn_exp2f(fmaf(sacc[j * 8 + tt], p.c, -l));
              if (kMasked) pp = mask_zero(pp, word, (uint32_t)(j * 16 + hh * 8 + tt));
              pv[u] = pp;
              sv[u] = pp * pacc[j * 8 + tt];
            }
            pw[t / 2] = pack_bf16x2(pv[0], pv[1]);
            sw[t / 2] = pack_bf16x2(sv[0], sv[1]);
          }
          pa[j] = __builtin_bit_cast(bf16x8, pw);
          sa[j] = __builtin_bit_cast(bf16x8, sw);
        }
      };
      if (partial) softmax_grad(std::true_type{});
      else softmax_grad(std::false_type{});

      // ---- dV += P^T dO, dK += dS^T Q over these 32 rows (transposing reads) ----
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ks = qblk * 2 + j;
#pragma unroll
        for (int d = 0; d < kDB; ++d) {
          const int o0 = tr.at(0, ks, d), o1 = tr.at(1, ks, d);
          const bf16* op = sm.dO[cur];
          const bf16* qp = sm.q[cur];
          dv[d] = mfma32(pa[j], join_tr(lds_read_tr16(op + o0), lds_read_tr16(op + o1)), dv[d]);
          dk[d] = mfma32(sa[j], join_tr(lds_read_tr16(qp + o0), lds_read_tr16(qp + o1)), dk[d]);
        }
      }
    }

    if (has_next) store_step(cur ^ 1);
    lds_barrier();  // next buffer complete, current buffer free
  };
  if constexpr (kW == 8 && D <= 128) {
    // the 256-key kernel takes two steps per trip, so that each step's buffer is a constant
    // and its LDS addresses fold into immediate offsets (dK/dV 1.2% faster on the
    // random-eviction workload despite 4 spilled registers; the 128-key kernel spills 8 in
    // its loop that way and runs 7-12% slower, so it keeps one step per trip)
    for (int st = 0; st < nsteps; st += 2) {
      step(std::integral_constant<int, 0>{}, st);
      if (st + 1 < nsteps) step(std::integral_constant<int, 1>{}, st + 1);
    }
  } else {
    for (int st = 0; st < nsteps; ++st) step(st & 1, st);
  }

  // ---- dK, dV of this workgroup's keys (keys past N dropped by the buffer bounds).  A
  // lane holds dimension d*32 + l32 of keys wave*32 + hh*4 + (i/4)*8 + i%4.
  const uint32_t kl = (uint32_t)((kb * BK + wave * 32 + hh * 4) * D + l32);
  if (slot >= 0) {
    // one segment of a split pair: fp32 partial sums into its slot, reduced in segment
    // order by k_dkdv_reduce (scale applied there)
    const size_t so = (size_t)(slot + rem) * BK * D, half = (size_t)p.nslots * BK * D;
    float* pk = p.partials + so;
    float* pv = p.partials + half + so;
    const int kr = wave * 32 + hh * 4;
#pragma unroll
    for (int d = 0; d < kDB; ++d) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int o = (kr + (i >> 2) * 8 + (i & 3)) * D + d * 32 + l32;
        pk[o] = dk[d][i];
        pv[o] = dv[d][i];
      }
    }
  } else if (direct) {
    const rsrc_t dkr = make_rsrc(p.dk + kvbase, head_bytes);
    const rsrc_t dvr = make_rsrc(p.dv + kvbase, head_bytes);
#pragma unroll
    for (int d = 0; d < kDB; ++d) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t so = (uint32_t)(((i >> 2) * 8 + (i & 3)) * D + d * 32) * 2;
        buf_store2(bf16_bits(dk[d][i] * p.scale), dkr, kl * 2, so);
        buf_store2(bf16_bits(dv[d][i]), dvr, kl * 2, so);
      }
    }
  } else {
    const rsrc_t dkr = make_rsrc(p.dk_acc + kvbase, acc_bytes);
    const rsrc_t dvr = make_rsrc(p.dv_acc + kvbase, acc_bytes);
#pragma unroll
    for (int d = 0; d < kDB; ++d) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t so = (uint32_t)(((i >> 2) * 8 + (i & 3)) * D + d * 32) * 4;
        buf_atomic_add(dk[d][i], dkr, kl * 4, so);
        buf_atomic_add(dv[d][i], dvr, kl * 4, so);
      }
    }
  }
}

// ---- KF: dQ (Q-block outer, same tiling and queues as the forward) ----------------------
namespace dqk {
constexpr int BQ = kFwdBlockQ;  // 128 query rows: 4 waves x 32
constexpr int BK = kFwdBlockK;  // 64 keys per tile

// K tiles use the swizzled layout (row reads and transposing reads; 320-byte rows at D <=
// 128), V rows are read row-wise only (272 bytes).
template <int D>
struct __attribute__((aligned(16))) Smem {
  bf16 k[2][BK * LdsRows<D>::SWZ];
  bf16 v[2][BK * LdsRows<D>::KS];
  uint32_t mw[2][4][BK];  // hidden-row words: [buffer][wave][key]
};
}  // namespace dqk

struct DqParams {
  const bf16* __restrict__ q;
  const bf16* __restrict__ k;
  const bf16* __restrict__ v;
  const bf16* __restrict__ o;
  const bf16* __restrict__ dout;
  const float* __restrict__ lse;  // natural-log LSE from the forward
  float* __restrict__ lse2;       // written: LSE in log2 units (+inf where LSE = -inf)
  float* __restrict__ delta;      // written: rowsum(dO o O)
  MaskArgs m;
  bf16* __restrict__ dq;
  const int32_t* __restrict__ q_queue;
  const int32_t* __restrict__ q_count;
  const int32_t* __restrict__ q_order;
  int B, Hq, Hkv, Hm, Nq, Nk, nQB, nKB;  // Nq query rows, Nk keys, Hm mask sets per batch row
  int pack;     // query heads per workgroup: 1 (128 rows of one head) or 4 (32 rows of four)
  float c;      // scale * log2(e)
  float scale;  // softmax scale (applied to dQ)
};

template <int D, bool kMulti>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void k_attn_bwd_dq(DqParams p) {
  using namespace dqk;
  constexpr int kRow = LdsRows<D>::SWZ;  // swizzled K row stride (elements)
  constexpr int VS = LdsRows<D>::KS;     // V row stride (row reads only)
  constexpr int kS = D / 16;               // k-steps of a 32x32x16 product over D
  constexpr int kDB = D / 32;              // 32-column blocks of dQ
  constexpr int kCh = D / 8;               // 16-byte chunks per row
  constexpr int kRowsPass = 256 / kCh;     // rows one pass of the tile copy covers
  constexpr int kPasses = BK / kRowsPass;  // passes per 64-row tile
  __shared__ Smem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // workgroup L: the (L % gpi)-th group of p.pack query heads of the mask set of LPT item
  // L / gpi, the forward's decode: packed, wave w takes head 4 g + w over the Q-block's 32
  // rows; else the one head's 128 rows, 32 per wave.
  const int L = xcd_logical((int)blockIdx.x, (int)gridDim.x);
  const int qpm = p.Hq / p.Hm;
  const int gpi = qpm / p.pack;
  const int r = L / gpi;
  const int item = p.q_order[r];
  const int mr = item / p.nQB, qb = item - mr * p.nQB;  // mask row (b, set) and Q-block
  const int b = mr / p.Hm;
  const bool packed = p.pack > 1;
  const int hg = (mr - b * p.Hm) * qpm + (L - r * gpi) * p.pack;  // first head of the group
  const int kvh = hg / (p.Hq / p.Hkv);
  const int h = hg + (packed ? __builtin_amdgcn_readfirstlane(wave) : 0);  // this wave's
  const int bq = packed ? BQ / kFwdPack : BQ;  // rows of the Q-block
  const int n_tiles = p.q_count[2 * item] + p.q_count[2 * item + 1];
  const const_i32_ptr queue = const_view(p.q_queue + (size_t)item * p.nKB);
  const int N = p.Nk, Nq = p.Nq;  // N: keys (and mask columns)
  const uint32_t head_bytes = (uint32_t)N * D * 2, q_bytes = (uint32_t)Nq * D * 2;
  const size_t qbase = (size_t)(b * p.Hq + h) * Nq;
  const rsrc_t kr_ = make_rsrc(p.k + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const rsrc_t vr_ = make_rsrc(p.v + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const i32x4_t kw_ = rsrc_words(p.k + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const i32x4_t vw_ = rsrc_words(p.v + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const uint32_t vec_bytes = (uint32_t)N * 4, row_bytes = (uint32_t)Nq * 4;
  // mask row mr (multi-interval form: absent intervals load 0, the empty interval)
  rsrc_t m0, m1, m2, m3;
  if constexpr (!kMulti) {
    const size_t mrow = (size_t)mr * N;
    m0 = make_rsrc(p.m.v.lts + mrow, vec_bytes); m1 = make_rsrc(p.m.v.lte + mrow, vec_bytes);
    m2 = make_rsrc(p.m.v.uts + mrow, vec_bytes); m3 = make_rsrc(p.m.v.ute + mrow, vec_bytes);
  } else {
    const size_t mrow = (size_t)mr * p.m.n * N;
    m0 = make_rsrc(p.m.start + mrow, (uint32_t)p.m.n * vec_bytes);
    m1 = make_rsrc(p.m.end + mrow, (uint32_t)p.m.n * vec_bytes);
    m2 = m0; m3 = m1;
  }
  const bool ragged = (N % BK) != 0;

  const int row = qb * bq + (packed ? 0 : wave * 32) + l32;

  f32x16 qacc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) qacc[d] = f32x16{};

  const int cp_row = tid / kCh, cp_ch = (tid % kCh) * 8;
  const int mk_key = lane, mk_wave = __builtin_amdgcn_readfirstlane(wave);
  // D >= 128: tiles go from memory straight into LDS, one 16-byte slot per lane and load
  // (load j, lane l: slot 64 j + l of the padded tile; at D = 128 K rows hold 20 slots, 16
  // of them data under the XOR swizzle, V rows 17; at D = 256, 36 (32) and 33), pad slots
  // taking a copy of the row's first chunk.  Wave w issues loads j = w, w + 4, ...
  constexpr bool kDma = D >= 128;
  constexpr int kKSlots = kRow * 2 / 16, kVSlots = VS * 2 / 16;
  constexpr int kKLoads = BK * kKSlots / 64, kVLoads = BK * kVSlots / 64;
  constexpr int kDmaPer = (kKLoads + 3) / 4;
  uint32_t koff[kDma ? kDmaPer : 1], voff[kDma ? kDmaPer : 1];
  if constexpr (kDma) {
#pragma unroll
    for (int i = 0; i < kDmaPer; ++i) {
      const int pp = (wave + 4 * i) * 64 + lane;
      const int rk = pp / kKSlots, ck = pp - rk * kKSlots;
      const int rv = pp / kVSlots, cv = pp - rv * kVSlots;
      koff[i] = (uint32_t)(rk * D * 2 + (ck < D / 8 ? (ck ^ ((rk >> 2) & 3)) * 16 : 0));
      voff[i] = (uint32_t)(rv * D * 2 + (cv < D / 8 ? cv * 16 : 0));
    }
  }
  u32x4 kst[kDma ? 1 : kPasses], vst[kDma ? 1 : kPasses];
  uint32_t vec[kMulti ? 2 * kMaxIntervals : 4];

  // load_tile(e, buf): D >= 128 writes buffer buf directly; otherwise stages in registers
  // for store_tile
  auto load_tile = [&](int e, int buf) {
    const int kb = e & 0x7fffffff;
    if constexpr (kDma) {
      // the tile's resources in scalar registers: the per-lane offsets stay constant
      const uint32_t tb = (uint32_t)kb * BK * D * 2;
      const i32x4_t kt_ = rsrc_advance(kw_, tb), vt_ = rsrc_advance(vw_, tb);
#pragma unroll
      for (int i = 0; i < kDmaPer; ++i) {
        const int j = mk_wave + 4 * i;
        if (i < kKLoads / 4 || j < kKLoads)
          lds_load16_untracked(kt_, koff[i], lds_addr(&sm.k[buf][j * 512]));
        if (i < kVLoads / 4 || j < kVLoads)
          lds_load16_untracked(vt_, voff[i], lds_addr(&sm.v[buf][j * 512]));
      }
    } else {
      const uint32_t base = (uint32_t)(kb * BK + cp_row) * (D * 2) + cp_ch * 2;
#pragma unroll
      for (int i = 0; i < kPasses; ++i) {
        kst[i] = buf_load16(kr_, base, i * kRowsPass * D * 2);
        vst[i] = buf_load16(vr_, base, i * kRowsPass * D * 2);
      }
    }
    const bool part = (e < 0) || (ragged && kb == p.nKB - 1);
    if (part) {
      const uint32_t vo = (uint32_t)(kb * BK + mk_key) * 4;
      if constexpr (!kMulti) {
        vec[0] = buf_load4(m0, vo, 0); vec[1] = buf_load4(m1, vo, 0);
        vec[2] = buf_load4(m2, vo, 0); vec[3] = buf_load4(m3, vo, 0);
      } else {
#pragma unroll
        for (int t = 0; t < kMaxIntervals; ++t) {
          vec[2 * t] = buf_load4(m0, vo + t * vec_bytes, 0);
          vec[2 * t + 1] = buf_load4(m1, vo + t * vec_bytes, 0);
        }
      }
    }
  };
  auto store_tile = [&](int e, int buf) {
    if constexpr (!kDma) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i) {
        *reinterpret_cast<u32x4*>(&sm.k[buf][swz<kRow>(cp_row + kRowsPass * i, cp_ch >> 3)]) = kst[i];
        *reinterpret_cast<u32x4*>(&sm.v[buf][(cp_row + kRowsPass * i) * VS + cp_ch]) = vst[i];
      }
    }
    const int kb = e & 0x7fffffff;
    const bool part = (e < 0) || (ragged && kb == p.nKB - 1);
    if (part) {
      const int key = kb * BK + mk_key;
      const int r0 = qb * bq + (packed ? 0 : mk_wave * 32);
      uint32_t w;
      if constexpr (!kMulti)
        w = hidden_rows32((int)vec[0], (int)vec[1], (int)vec[2], (int)vec[3], r0);
      else
        w = hidden_rows32_multi(int4{(int)vec[0], (int)vec[2], (int)vec[4], (int)vec[6]},
                                int4{(int)vec[1], (int)vec[3], (int)vec[5], (int)vec[7]}, r0);
      sm.mw[buf][mk_wave][mk_key] = key < N ? w : 0xFFFFFFFFu;
    }
  };

  // Q^T and dO^T operands: lane holds row `row`, d = s*16 + hh*8 .. +7 (rows past Nq read 0)
  bf16x8 qr[kS], orr[kS];
  {
    const rsrc_t qrs = make_rsrc(p.q + qbase * D, q_bytes);
    const rsrc_t ors = make_rsrc(p.dout + qbase * D, q_bytes);
    const uint32_t off = (uint32_t)row * (D * 2) + hh * 16;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      qr[s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, off, s * 32));
      orr[s] = __builtin_bit_cast(bf16x8, buf_load16(ors, off, s * 32));
    }
  }
  // the first tile's loads go out now, so their latency overlaps that of Q, dO and O
  if (n_tiles > 0) load_tile(queue[0], 0);
  // D = rowsum(dO o O) for this lane's row (the two half-waves hold the two halves of each
  // 16-wide d slice) and the LSE in log2 units; both go to memory for the dK/dV kernel.
  float d_row;
  {
    const rsrc_t ors = make_rsrc(p.o + qbase * D, q_bytes);
    const uint32_t off = (uint32_t)row * (D * 2) + hh * 16;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const u32x4 ov = buf_load16(ors, off, s * 32);
      const u32x4 gv = __builtin_bit_cast(u32x4, orr[s]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        part += bf16lo_to_f32(ov[t]) * bf16lo_to_f32(gv[t]) +
                bf16hi_to_f32(ov[t]) * bf16hi_to_f32(gv[t]);
    }
    d_row = sum_with_partner32(part);
  }
  const float lse_nat =
      __uint_as_float(buf_load4(make_rsrc(p.lse + qbase, row_bytes), (uint32_t)row * 4, 0));
  const float lse_row = lse_nat == -INFINITY ? INFINITY : lse_nat * kLog2e;

  if (n_tiles > 0) store_tile(queue[0], 0);  // its loads were issued with Q and dO
  if constexpr (kDma) asm volatile("s_waitcnt vmcnt(0)");  // loads into LDS have landed
  lds_barrier();

  const int arow = perm_rows(l32);
  const SwzRowRead<kRow> rr(arow, hh);
  const SwzTrRead<kRow> tr(lane, hh);

  int e = n_tiles > 0 ? queue[0] : 0;
  auto tile = [&](auto cur_c, int it) {
    const int cur = cur_c;  // the tile's LDS buffer (a constant in the unrolled loop below)
    const int kb = e & 0x7fffffff;
    const bool partial = (e < 0) || (ragged && kb == p.nKB - 1);
    int en = 0;
    const bool has_next = it + 1 < n_tiles;
    if (has_next) {
      en = queue[it + 1];
      load_tile(en, cur ^ 1);
    }

    // ---- S^T = K Q^T and dP^T = V dO^T (a lane owns one query row).  Step i (key half
    // i / kS, d-step i % kS) reads its K and V fragments two steps ahead; the scheduling
    // barriers keep the reads ahead of the products. ----
    f32x16 sacc[2], pacc[2];
    {
      constexpr int kSt = 2 * kS;
      auto kread = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(
            &sm.k[cur][rr.at(i % kS) + (i / kS) * 32 * kRow]);
      };
      auto vread = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(
            &sm.v[cur][((i / kS) * 32 + arow) * VS + hh * 8 + (i % kS) * 16]);
      };
      bf16x8 kf[3], vf[3];
      kf[0] = kread(0); vf[0] = vread(0);
      kf[1] = kread(1); vf[1] = vread(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kSt; ++i) {
        if (i + 2 < kSt) {
          kf[(i + 2) % 3] = kread(i + 2);
          vf[(i + 2) % 3] = vread(i + 2);
        }
        const int blk = i / kS, st = i % kS;
        sacc[blk] = mfma32(kf[i % 3], qr[st], st == 0 ? f32x16{} : sacc[blk]);
        pacc[blk] = mfma32(vf[i % 3], orr[st], st == 0 ? f32x16{} : pacc[blk]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if (partial) {
      const uint32_t* mw = sm.mw[cur][wave];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 w0 = *reinterpret_cast<const u32x4*>(mw + blk * 32 + j * 16 + hh * 8);
          const u32x4 w1 = *reinterpret_cast<const u32x4*>(mw + blk * 32 + j * 16 + hh * 8 + 4);
#pragma unroll
          for (int t = 0; t < 8; ++t)
            sacc[blk][j * 8 + t] = mask_neg_inf(sacc[blk][j * 8 + t], t < 4 ? w0[t] : w1[t - 4],
                                                (uint32_t)l32);
        }
      }
    }

    // ---- dS^T = P^T o (dP^T - D), P^T = exp2(S^T c - LSE2), then dQ^T += K^T dS^T, one
    // 32-key half at a time so the VALU work of a half overlaps MFMAs of the other ----
    const bf16* kt = sm.k[cur];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      bf16x8 dsb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 packed;
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const int i0 = j * 8 + t;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[blk][i0], p.c, -lse_row));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[blk][i0 + 1], p.c, -lse_row));
          packed[t / 2] =
              pack_bf16x2(p0 * (pacc[blk][i0] - d_row), p1 * (pacc[blk][i0 + 1] - d_row));
        }
        dsb[j] = __builtin_bit_cast(bf16x8, packed);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ks = blk * 2 + j;
#pragma unroll
        for (int d = 0; d < kDB; ++d) {
          const bf16x8 a = join_tr(lds_read_tr16(kt + tr.at(0, ks, d)),
                                   lds_read_tr16(kt + tr.at(1, ks, d)));
          qacc[d] = mfma32(a, dsb[j], qacc[d]);
        }
      }
    }

    if (has_next) store_tile(en, cur ^ 1);
    if constexpr (kDma) asm volatile("s_waitcnt vmcnt(0)");  // loads into LDS have landed
    lds_barrier();
    e = en;
  };
  if constexpr (D <= 128) {
    // two tiles per trip: each tile's buffer is a constant, its LDS addresses immediates
    // (dQ 1.2-1.4% faster on the 128K workloads, no spills)
    for (int it = 0; it < n_tiles; it += 2) {
      tile(std::integral_constant<int, 0>{}, it);
      if (it + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, it + 1);
    }
  } else {
    for (int it = 0; it < n_tiles; ++it) tile(it & 1, it);
  }

  // D and the log2 LSE go out after the loop: a store before it would keep the compiler
  // from reading the queue through the scalar cache (it cannot tell what a buffer store
  // may overwrite), turning each entry into a vector load waited for in full.  Rows past
  // Nq are dropped by the buffer bounds.
  if (hh == 0) {
    buf_store4(__float_as_uint(lse_row), make_rsrc(p.lse2 + qbase, row_bytes), (uint32_t)row * 4, 0);
    buf_store4(__float_as_uint(d_row), make_rsrc(p.delta + qbase, row_bytes), (uint32_t)row * 4, 0);
  }

  // ---- dQ = scale * acc (bf16); rows past Nq are dropped by the buffer bounds ----
  const rsrc_t dqr = make_rsrc(p.dq + qbase * D, q_bytes);
  const uint32_t ooff = (uint32_t)row * (D * 2) + hh * 8;
#pragma unroll
  for (int d = 0; d < kDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(qacc[d][g * 4 + 0] * p.scale, qacc[d][g * 4 + 1] * p.scale);
      w[1] = pack_bf16x2(qacc[d][g * 4 + 2] * p.scale, qacc[d][g * 4 + 3] * p.scale);
      buf_store8(w, dqr, ooff, (d * 32 + g * 8) * 2);
    }
  }
}

// ---- Reduction of split pairs' partial dK/dV (pairs that store bf16 directly) ----------
struct ReduceParams {
  const int32_t* __restrict__ k_order;
  const int32_t* __restrict__ split_pair;
  const int32_t* __restrict__ split_slot;
  const int32_t* __restrict__ split_counts;
  const float* __restrict__ partials;  // [2][nslots][BK][D]
  bf16* __restrict__ dk;
  bf16* __restrict__ dv;
  HeadMap hm;
  int Hq, Hkv, nKB, Nk, nslots, D;
  int bk;  // keys per dK/dV workgroup (128 or 256)
  float scale;
};

// One workgroup per (split pair, kv head of its set): dK = scale * sum_seg partial_dK and
// dV = sum_seg partial_dV, summed in segment order, stored as bf16 (keys past Nk dropped).
__global__ __launch_bounds__(256) void k_dkdv_reduce(ReduceParams p) {
  const int BK = p.bk;
  const int D = p.D;
  const int per = p.hm.kvpm * p.hm.cpk;
  const int j = blockIdx.x / per, rem = blockIdx.x - j * per;
  if (j >= p.split_counts[1]) return;
  const int sp = p.split_pair[j];
  const int nseg = (int)((unsigned)sp >> 28) + 1, base = p.split_slot[j];
  const DkdvItem wi = dkdv_item(p.hm, p.Hq, p.Hkv, p.nKB, p.k_order[sp & 0xFFFFFF], rem);
  const size_t half = (size_t)p.nslots * BK * D;
  const size_t kvbase = (size_t)(wi.b * p.Hkv + wi.kvh) * p.Nk * D;
  const uint32_t head_bytes = (uint32_t)p.Nk * D * 2;
  const rsrc_t dkr = make_rsrc(p.dk + kvbase, head_bytes);
  const rsrc_t dvr = make_rsrc(p.dv + kvbase, head_bytes);
  for (int t = threadIdx.x; t < BK * D / 4; t += 256) {
    f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < nseg; ++q) {
      const size_t so = (size_t)(base + q * per + rem) * BK * D + (size_t)t * 4;
      sk += *reinterpret_cast<const f32x4*>(p.partials + so);
      sv += *reinterpret_cast<const f32x4*>(p.partials + half + so);
    }
    const uint32_t off = (uint32_t)(wi.kb * BK * D + t * 4) * 2;
    buf_store8(u32x2{pack_bf16x2(sk[0] * p.scale, sk[1] * p.scale),
                     pack_bf16x2(sk[2] * p.scale, sk[3] * p.scale)}, dkr, off, 0);
    buf_store8(u32x2{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])}, dvr, off, 0);
  }
}

unsigned grid_for(size_t n, unsigned cap) {
  size_t g = (n + 255) / 256;
  return (unsigned)(g < cap ? (g ? g : 1) : cap);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s, const BwdEvents& ev) {
  if (a.B == 0 || a.Hq == 0 || (a.Nq == 0 && a.Nk == 0)) return hipSuccess;
  const size_t rows_k = (size_t)a.B * a.Hkv * a.Nk;
  const HeadMap hm = head_map(a.Hq, a.Hkv, a.Hm);
  const bool acc = hm.writers > 1;
  const float c = a.scale * kLog2e;

  // dQ first: it also writes D and the log2 LSE that the dK/dV kernel reads
  DqParams q;
  q.q = static_cast<const bf16*>(a.q);
  q.k = static_cast<const bf16*>(a.k);
  q.v = static_cast<const bf16*>(a.v);
  q.o = static_cast<const bf16*>(a.o);
  q.dout = static_cast<const bf16*>(a.dout);
  q.lse = a.lse;
  q.lse2 = a.lse2;
  q.delta = a.delta;
  q.m = a.m;
  q.dq = static_cast<bf16*>(a.dq);
  q.q_queue = a.q_queue; q.q_count = a.q_count; q.q_order = a.q_order;
  q.B = a.B; q.Hq = a.Hq; q.Hkv = a.Hkv; q.Hm = a.Hm; q.Nq = a.Nq; q.Nk = a.Nk;
  q.nQB = a.nQB_q; q.nKB = a.nKB_q;
  q.pack = a.pack > 1 ? kFwdPack : 1;
  q.c = c;
  q.scale = a.scale;
  const unsigned qgrid = (unsigned)a.B * (unsigned)a.nQB_q * (unsigned)(a.Hq / q.pack);
  if (ev.dq_start) (void)hipEventRecord(ev.dq_start, s);
  const bool multi = a.m.n > 0;
  const bool d64 = a.D == 64;
  if (qgrid > 0) {
    auto kern = d64          ? (multi ? k_attn_bwd_dq<64, true> : k_attn_bwd_dq<64, false>)
                : a.D == 256 ? (multi ? k_attn_bwd_dq<256, true> : k_attn_bwd_dq<256, false>)
                             : (multi ? k_attn_bwd_dq<128, true> : k_attn_bwd_dq<128, false>);
    hipLaunchKernelGGL(kern, dim3(qgrid), dim3(256), 0, s, q);
  }
  if (ev.dq_stop) (void)hipEventRecord(ev.dq_stop, s);

  if (acc && rows_k > 0) {
    hipLaunchKernelGGL(k_zero, dim3(grid_for(rows_k * a.D / 4, 8192)), dim3(256), 0, s,
                       reinterpret_cast<float4*>(a.dk_acc), rows_k * a.D / 4);
    hipLaunchKernelGGL(k_zero, dim3(grid_for(rows_k * a.D / 4, 8192)), dim3(256), 0, s,
                       reinterpret_cast<float4*>(a.dv_acc), rows_k * a.D / 4);
  }

  // work units of the dK/dV kernel: long pairs split along their queues.  wide: 256-key
  // workgroups of 8 waves, one per CU (bk = 256, D = 128 only)
  const bool wide = a.bk == kBwdBlockKWide;
  const int per = hm.kvpm * hm.cpk;
  const int npairs = a.B * a.Hm * a.nKB_k;
  const int nslots = split_slots(per, a.split_extra);
  if (npairs > 0)
    hipLaunchKernelGGL(k_plan_split, dim3(1), dim3(kPlanThreads), 0, s, a.k_count, a.k_order,
                       npairs, per, hm.hc, (wide ? 1 : 2) * device_cu_count(), a.split_extra,
                       acc ? 0 : 1,
                       a.unit_pair, a.unit_slot, a.split_pair, a.split_slot, a.split_counts);

  DkdvParams p;
  p.q = q.q; p.k = q.k; p.v = q.v; p.dout = q.dout;
  p.lse2 = a.lse2;
  p.delta = a.delta;
  p.m = a.m;
  p.k_queue = a.k_queue;
  p.k_count = a.k_count;
  p.k_order = a.k_order;
  p.dk_acc = a.dk_acc;
  p.dv_acc = a.dv_acc;
  p.dk = static_cast<bf16*>(a.dk);
  p.dv = static_cast<bf16*>(a.dv);
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.nQB = a.nQB_k; p.nKB = a.nKB_k;
  p.hm = hm;
  p.unit_pair = a.unit_pair;
  p.unit_slot = a.unit_slot;
  p.split_counts = a.split_counts;
  p.partials = a.partials;
  p.nslots = nslots;
  p.c = c;
  p.scale = a.scale;
  // the largest plan: every pair plus the extra units (those past the plan exit at once)
  const unsigned grid = (unsigned)(npairs + a.split_extra) * (unsigned)per;
  if (ev.dkdv_start) (void)hipEventRecord(ev.dkdv_start, s);
  if (grid > 0) {
    auto kern = d64 ? (multi ? k_attn_bwd_dkdv<64, true, 4> : k_attn_bwd_dkdv<64, false, 4>)
                : a.D == 256
                    ? (multi ? k_attn_bwd_dkdv<256, true, 4> : k_attn_bwd_dkdv<256, false, 4>)
                : wide ? (multi ? k_attn_bwd_dkdv<128, true, 8> : k_attn_bwd_dkdv<128, false, 8>)
                       : (multi ? k_attn_bwd_dkdv<128, true, 4> : k_attn_bwd_dkdv<128, false, 4>);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(wide ? 512 : 256), 0, s, p);
  }
  if (ev.dkdv_stop) (void)hipEventRecord(ev.dkdv_stop, s);

  if (!acc && a.split_extra > 0 && npairs > 0) {
    ReduceParams rp;
    rp.k_order = a.k_order;
    rp.split_pair = a.split_pair;
    rp.split_slot = a.split_slot;
    rp.split_counts = a.split_counts;
    rp.partials = a.partials;
    rp.dk = p.dk;
    rp.dv = p.dv;
    rp.hm = hm;
    rp.Hq = a.Hq; rp.Hkv = a.Hkv; rp.nKB = a.nKB_k; rp.Nk = a.Nk;
    rp.nslots = nslots;
    rp.D = a.D;
    rp.bk = a.bk;
    rp.scale = a.scale;
    hipLaunchKernelGGL(k_dkdv_reduce, dim3((unsigned)a.split_extra * (unsigned)per), dim3(256),
                       0, s, rp);
  }
  if (acc && rows_k > 0) {
    hipLaunchKernelGGL(k_bwd_convert, dim3(grid_for(rows_k * a.D / 8, 16384)), dim3(256), 0, s,
                       a.dk_acc, static_cast<bf16*>(a.dk), a.scale, rows_k * a.D / 8);
    hipLaunchKernelGGL(k_bwd_convert, dim3(grid_for(rows_k * a.D / 8, 16384)), dim3(256), 0, s,
                       a.dv_acc, static_cast<bf16*>(a.dv), 1.0f, rows_k * a.D / 8);
  }
  return hipGetLastError();
}

}  // namespace fm
