// Mask-aware attention forward (gfx950, bf16 MFMA 32x32x16).
//
// One workgroup = one (b, Q-block of 128 rows, query head).  Workgroups are numbered
// in LPT order (Q-blocks by tile cost descending, heads of a Q-block adjacent), so the
// hardware dispatcher performs greedy list scheduling in that order (FlashMask-3 page,
// §3.3; Flash MSA guide, "Optimization Tricks That Actually Matter").  The workgroup
// walks its Q-block's queue of KV blocks (right to left, FlashMask-3 page §3.1): only
// queued blocks are loaded, and the row-interval mask is applied only on tiles tagged
// partial.  Per tile it runs the online softmax of the Flash MSA guide ("The Flash
// Core"): running row max and sum, rescaling of the accumulator, normalisation at the
// end; O and the natural-log LSE are written.
//
// Layout of the work.  4 waves x 32 query rows.  Each wave computes S^T = K Q^T so that
// a lane owns one query row (its 32 scores sit in one lane and its partner lane l^32),
// then O^T += V^T P^T so that the same lane owns that row of the accumulator; the
// softmax statistics therefore never leave the lane pair.  Q stays in registers; K and
// V tiles are double-buffered through LDS (row-major; V is read with the transposing
// ds_read_b64_tr_b16), K one tile ahead of V so that the scores of the next tile are
// computed (MFMA) while the current tile's exponentials run (VALU).  Two row sums are kept: l_f (fp32 sum of p) gives the LSE,
// l_b (sum of the bf16-rounded p that the PV product actually used) normalises O.
#include <type_traits>

#include "fm_device.h"
#include "fm_internal.h"

namespace fm {
namespace {

constexpr int BQ = kFwdBlockQ;  // 128
constexpr int BK = kFwdBlockK;  // 64
// LDS rows per head dimension (LdsRows): K rows are read row-wise only (128-wide: 272 B),
// V rows also by transposing reads (128-wide: 320 B, conflict-free for both).
template <int D>
struct __attribute__((aligned(16))) FwdSmem {
  bf16 k[2][BK * LdsRows<D>::KS];
  bf16 v[2][BK * LdsRows<D>::TS];
  uint32_t mw[2][4][BK];  // hidden-row words: [buffer][wave][key]
};

// A-operand row permutation for S^T = K Q^T: A row a holds key perm(a) so that the
// accumulator rows a lane owns are runs of 8 consecutive keys, which is exactly the
// k-ordering the following PV product wants for its B operand.
__device__ __forceinline__ int perm_rows(int a) {
  return (a & 0x13) | ((a & 4) << 1) | ((a & 8) >> 1);
}

// Lazy offset.  A row's exponent offset m (log2 units) is set from the true row max on
// the row's first visible tile and afterwards only moves when a tile's exponentials
// grow too large: p = 2^(s c - m) is formed against the current m, and only when a
// lane's sum of p over the 32-key half exceeds 2^64 (or is not finite), or the row has
// no offset yet, does the wave take the slow path (row max, rescale of the accumulator
// and sums, recompute), in which only the rows that triggered it move their offset.
// bf16 and fp32 share their exponent range, so p up to 2^64 loses no relative precision,
// and the accumulator stays below 2^(64 + 22 + a few) for any N <= 2^22.  The common
// path therefore needs no per-tile row max at all.
constexpr float kSumLimit = 18446744073709551616.0f;  // 2^64

struct FwdParams {
  const bf16* __restrict__ q;
  const bf16* __restrict__ k;
  const bf16* __restrict__ v;
  MaskArgs m;
  bf16* __restrict__ o;
  float* __restrict__ lse;
  const int32_t* __restrict__ q_queue;
  const int32_t* __restrict__ q_count;
  const int32_t* __restrict__ q_order;
  int B, Hq, Hkv, Hm, Nq, Nk, nQB, nKB;  // Nq query rows, Nk keys, Hm mask sets per batch row
  int pack;  // query heads per workgroup: 1 (128 rows of one head) or 4 (32 rows of four)
  float c;   // softmax scale * log2(e)
};

// D: head dimension (64, 128 or 256).  kMulti: the mask is the multi-interval form (else the
// four-vector form).  D = 256 runs one workgroup per CU (its tiles take 143 KB of LDS), with
// up to 512 registers per lane.
template <int D, bool kMulti>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void k_attn_fwd(FwdParams p) {
  constexpr int KS = LdsRows<D>::KS;  // K row stride in LDS (elements)
  constexpr int VS = LdsRows<D>::TS;  // V row stride in LDS
  constexpr int kS = D / 16;                // k-steps of a 32x32x16 product over D
  constexpr int kDB = D / 32;               // 32-column blocks of O
  constexpr int kCh = D / 8;                // 16-byte chunks per row
  constexpr int kRowsPass = 256 / kCh;      // rows one pass of the tile copy covers
  constexpr int kPasses = BK / kRowsPass;   // passes per 64-row tile
  constexpr int kSteps = 2 * kS;            // score MFMAs per tile
  // the 16 exponential pairs of a tile spread over its kSteps score MFMAs: kExp pairs per
  // step (D <= 128), or one pair every kEvery steps (D = 256)
  constexpr int kExp = kSteps <= 16 ? 16 / kSteps : 1;
  constexpr int kEvery = kSteps <= 16 ? 1 : kSteps / 16;
  __shared__ FwdSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // workgroup L: the (L % gpi)-th group of p.pack query heads of the mask set of LPT item
  // L / gpi.  Packed (p.pack = 4), wave w takes head 4 g + w over the Q-block's 32 rows; else
  // the one head's 128 rows, 32 per wave.  The heads of a group share one kv head.
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
  const int Nq = p.Nq, N = p.Nk;  // N: keys (and mask columns)
  const uint32_t q_bytes = (uint32_t)Nq * D * 2, head_bytes = (uint32_t)N * D * 2;
  const rsrc_t qr_ = make_rsrc(p.q + (size_t)(b * p.Hq + h) * Nq * D, q_bytes);
  const rsrc_t kr_ = make_rsrc(p.k + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const rsrc_t vr_ = make_rsrc(p.v + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const i32x4_t kw_ = rsrc_words(p.k + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const i32x4_t vw_ = rsrc_words(p.v + (size_t)(b * p.Hkv + kvh) * N * D, head_bytes);
  const uint32_t vec_bytes = (uint32_t)N * 4;
  // mask row mr: four vectors of N, or n intervals x N starts and ends (absent intervals
  // m >= n read past the row's bounds and load 0, the empty interval [0, 0))
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
  auto out_rsrc = [&]() { return make_rsrc(p.o + (size_t)(b * p.Hq + h) * Nq * D, q_bytes); };
  auto lse_rsrc = [&]() { return make_rsrc(p.lse + (size_t)(b * p.Hq + h) * Nq, (uint32_t)Nq * 4); };

  // A Q-block that sees no key: O = 0 and LSE = -inf, nothing loaded.  Leaving here keeps
  // every path into the tile loop behind the first tile's score products, so the compiler
  // knows Q's loads have landed there and does not wait on the memory counter in the loop.
  if (n_tiles == 0) {
    const rsrc_t orr = out_rsrc();
    const uint32_t ooff = (uint32_t)row * (D * 2) + hh * 8;
    const u32x2 z = {0u, 0u};
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) buf_store8(z, orr, ooff, (d * 32 + g * 8) * 2);
    if (hh == 0) buf_store4(__float_as_uint(-INFINITY), lse_rsrc(), (uint32_t)row * 4, 0);
    return;
  }

  // Q^T operand: lane holds Q[row][s*16 + hh*8 .. +7] for s = 0..7 (rows past Nq read 0)
  bf16x8 qr[kS];
  {
    const uint32_t off = (uint32_t)row * (D * 2) + hh * 16;
#pragma unroll
    for (int s = 0; s < kS; ++s) qr[s] = __builtin_bit_cast(bf16x8, buf_load16(qr_, off, s * 32));
  }

  f32x16 oacc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) oacc[d] = f32x16{};
  float m_use = -INFINITY, lf = 0.f, lb = 0.f;

  // staging for the tile copy: thread copies rows tid/kCh + kRowsPass*i, chunk tid%kCh
  const int cp_row = tid / kCh, cp_ch = (tid % kCh) * 8;
  const int mk_key = lane, mk_wave = __builtin_amdgcn_readfirstlane(wave);
  constexpr int kVec = kMulti ? 2 * kMaxIntervals : 4;
  // D >= 128: tiles go from memory straight into LDS (buffer loads with the LDS flag), no
  // staging registers.  Each such load writes 64 consecutive 16-byte LDS slots, one per
  // lane, so lane l of load j covers slot 64 j + l of the padded tile (K: 17 slots a row at
  // D = 128, 33 at 256; V: 20, 36) and fetches the 16 bytes that belong there; pad slots
  // take a copy of the row's first chunk.  Wave w issues loads j = w, w + 4, ...
  constexpr bool kDma = D >= 128;
  constexpr int kKSlots = KS * 2 / 16, kVSlots = VS * 2 / 16;
  constexpr int kKLoads = BK * kKSlots / 64, kVLoads = BK * kVSlots / 64;
  constexpr int kDmaPer = (kVLoads + 3) / 4;
  uint32_t koff[kDma ? kDmaPer : 1], voff[kDma ? kDmaPer : 1];
  if constexpr (kDma) {
#pragma unroll
    for (int i = 0; i < kDmaPer; ++i) {
      const int pk = (wave + 4 * i) * 64 + lane, pv = pk;
      const int rk = pk / kKSlots, ck = pk - rk * kKSlots;
      const int rv = pv / kVSlots, cv = pv - rv * kVSlots;
      koff[i] = (uint32_t)(rk * D * 2 + (ck < D / 8 ? ck * 16 : 0));
      voff[i] = (uint32_t)(rv * D * 2 + (cv < D / 8 ? cv * 16 : 0));
    }
  }
  u32x4 kst[kDma ? 1 : kPasses], vst[kDma ? 1 : kPasses];
  uint32_t vec[kVec];
  auto is_partial = [&](int e) {
    return (e < 0) || (ragged && (e & 0x7fffffff) == p.nKB - 1);
  };

  // Software pipeline.  Iteration t computes the scores of tile t+1 (MFMA) in the same
  // block as the softmax of tile t (VALU), then tile t's PV product.  K (with the mask
  // words) therefore runs one tile ahead of V: iteration t reads K/mw buffer (t+1)&1 and
  // V buffer t&1, and refills K/mw buffer t&1 with tile t+2 and V buffer (t+1)&1 with
  // tile t+1; one barrier per iteration separates those reads from those writes.
  // fetch_k / put_k stage through (ks, vv): kst / vec in the loop; the prologue also
  // uses a second set so that both K tiles it needs are requested at once
  auto fetch_k = [&](int e, int buf, u32x4 (&ks)[kDma ? 1 : kPasses], uint32_t (&vec)[kVec]) {
    const int kb = e & 0x7fffffff;
    if constexpr (kDma) {
      // the tile's resource in scalar registers: the per-lane offsets stay constant
      const i32x4_t kt_ = rsrc_advance(kw_, (uint32_t)kb * BK * D * 2);
#pragma unroll
      for (int i = 0; i < kDmaPer; ++i) {
        const int j = mk_wave + 4 * i;
        if (i < kKLoads / 4 || j < kKLoads)
          lds_load16_untracked(kt_, koff[i], lds_addr(&sm.k[buf][j * 512]));
      }
    } else {
      const uint32_t base = (uint32_t)(kb * BK + cp_row) * (D * 2) + cp_ch * 2;
#pragma unroll
      for (int i = 0; i < kPasses; ++i) ks[i] = buf_load16(kr_, base, i * kRowsPass * D * 2);
    }
    if (is_partial(e)) {
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
  auto fetch_v = [&](int e, int buf) {
    const int kb = e & 0x7fffffff;
    if constexpr (kDma) {
      const i32x4_t vt_ = rsrc_advance(vw_, (uint32_t)kb * BK * D * 2);
#pragma unroll
      for (int i = 0; i < kDmaPer; ++i) {
        const int j = mk_wave + 4 * i;
        if (i < kVLoads / 4 || j < kVLoads)
          lds_load16_untracked(vt_, voff[i], lds_addr(&sm.v[buf][j * 512]));
      }
    } else {
      const uint32_t base = (uint32_t)(kb * BK + cp_row) * (D * 2) + cp_ch * 2;
#pragma unroll
      for (int i = 0; i < kPasses; ++i) vst[i] = buf_load16(vr_, base, i * kRowsPass * D * 2);
    }
  };
  auto put_k = [&](int e, int buf, const u32x4 (&ks)[kDma ? 1 : kPasses],
                   const uint32_t (&vec)[kVec]) {
    if constexpr (!kDma) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i)
        *reinterpret_cast<u32x4*>(&sm.k[buf][(cp_row + kRowsPass * i) * KS + cp_ch]) = ks[i];
    }
    if (is_partial(e)) {
      const int key = (e & 0x7fffffff) * BK + mk_key;
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
  auto put_v = [&](int buf) {
    if constexpr (!kDma) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i)
        *reinterpret_cast<u32x4*>(&sm.v[buf][(cp_row + kRowsPass * i) * VS + cp_ch]) = vst[i];
    }
  };
  // the loads into LDS are counted by the memory counter only: wait for them before the
  // barrier that publishes a tile
  auto tiles_landed = [&]() {
    if constexpr (kDma) asm volatile("s_waitcnt vmcnt(0)");
  };

  const int arow = perm_rows(l32);
  // transposing-read coordinates for the V^T operand
  const int tr_row = (lane & 15) >> 2;                         // + key base
  const int tr_col = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);  // + d-block base

  // S^T = K Q^T for one 64-key tile (fp32), from K buffer `buf`
  auto scores = [&](int buf, f32x16 (&acc)[2]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const bf16* kp = &sm.k[buf][(blk * 32 + arow) * KS + hh * 8];
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + s * 16);
        acc[blk] = mfma32(a, qr[s], s == 0 ? f32x16{} : acc[blk]);
      }
    }
  };
  // row-interval mask on a partial tile: hidden scores -> -inf
  auto apply_mask = [&](int buf, f32x16 (&acc)[2]) {
    const uint32_t* mw = sm.mw[buf][wave];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(mw + blk * 32 + j * 16 + hh * 8);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(mw + blk * 32 + j * 16 + hh * 8 + 4);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[blk][j * 8 + t] =
              mask_neg_inf(acc[blk][j * 8 + t], t < 4 ? w0[t] : w1[t - 4], (uint32_t)l32);
      }
    }
  };

  f32x16 sacc[2];
  {
    // tile 0's K and V and tile 1's K in flight together (one memory round trip)
    const int e0 = queue[0];
    const int e1 = n_tiles > 1 ? queue[1] : 0;
    u32x4 kst1[kDma ? 1 : kPasses];
    uint32_t vec1[kVec];
    fetch_k(e0, 0, kst, vec);
    fetch_v(e0, 0);
    if (n_tiles > 1) fetch_k(e1, 1, kst1, vec1);
    put_k(e0, 0, kst, vec);
    put_v(0);
    if (n_tiles > 1) put_k(e1, 1, kst1, vec1);
  }
  tiles_landed();
  lds_barrier();
  {
    scores(0, sacc);
    if (is_partial(queue[0])) apply_mask(0, sacc);
    // The first tile sets each row's offset from its own maximum, so its exponentials are
    // formed once (the lazy test would otherwise send every row through the slow path on
    // its first tile).  Rows that see nothing here keep -inf.
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[blk][i]);
    m_use = max_with_partner32(mx) * p.c;
  }
  // Tile 0's K and mask words (buffer 0) are refilled by the first iteration (tile 2): every
  // wave's reads of them above come first.
  lds_barrier();

  // The loop body for tile `it` (it & 1 == Cur, a compile-time buffer index): sc holds tile
  // it's scores, sn receives tile it+1's.  Two tiles per trip, the score arrays swapping
  // roles: no copy of the scores per tile, and every LDS buffer index is a constant.
  auto step = [&](auto cur_c, int it, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    const bool has1 = it + 1 < n_tiles, has2 = it + 2 < n_tiles;
    const int e1 = has1 ? queue[it + 1] : 0;
    const int e2 = has2 ? queue[it + 2] : 0;
    if (has2) fetch_k(e2, cur, kst, vec);
    if (has1) fetch_v(e1, nxt);

    // ---- scores of tile it+1 (MFMA; stale but unused after the last tile) interleaved
    // with the exponentials of tile it (VALU): step i issues the K fragment read for step
    // i+2, score MFMA i, and the exponentials of score pair i of the current tile.  The
    // scheduling barriers keep that order, so the VALU work runs in the MFMAs' shadow. ----
    bf16x8 pb[2][2];
    float psum[2], pbsum[2];
    // p = 2^(s c - off) for score pair i (half i/8, column group (i%8)/4, rows 2(i%4)+{0,1})
    u32x4 packed[2][2];
    auto exp_pair = [&](int i, float off) {
      const int hb = i / 8, j = (i % 8) / 4, t = (i % 4) * 2;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[hb][j * 8 + t], p.c, -off));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[hb][j * 8 + t + 1], p.c, -off));
      // the first pair of a half starts its sum (an add to 0 cannot be folded: -0 + 0 = +0)
      if (i % 8 == 0) psum[hb] = p0 + p1;
      else psum[hb] += p0 + p1;
      // the packing and the row-sum dot product stay here, among the score MFMAs: left to
      // itself the compiler sinks them past the slow-path branch, where they hold 32 fp32
      // values live and run as a block of their own
      unsigned u = pack_bf16x2(p0, p1);
      asm volatile("" : "+v"(u));
      packed[hb][j][t / 2] = u;
      pbsum[hb] = __builtin_amdgcn_fdot2_f32_bf16(
          __builtin_bit_cast(bf16x2, u), bf16x2{(bf16)1.0f, (bf16)1.0f}, pbsum[hb], false);
      asm volatile("" : "+v"(pbsum[hb]));
    };
    auto exponentiate_all = [&](float off) {
      psum[0] = psum[1] = 0.f;
      pbsum[0] = pbsum[1] = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) exp_pair(i, off);
    };
    // a row without an offset yet uses 0: exact if it saw nothing so far (p = 0)
    const float off0 = m_use == -INFINITY ? 0.f : m_use;
    {
      psum[0] = psum[1] = 0.f;
      pbsum[0] = pbsum[1] = 0.f;
      const bf16* kbase = &sm.k[nxt][arow * KS + hh * 8];
      auto kread = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(kbase + (i / kS) * 32 * KS + (i % kS) * 16);
      };
      bf16x8 kf[3];
      kf[0] = kread(0);
      kf[1] = kread(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        if (i + 2 < kSteps) kf[(i + 2) % 3] = kread(i + 2);
        const int blk = i / kS, st = i % kS;
        sn[blk] = mfma32(kf[i % 3], qr[st], st == 0 ? f32x16{} : sn[blk]);
#pragma unroll
        for (int e = 0; e < kExp; ++e)
          if (i % kEvery == 0) exp_pair((i / kEvery) * kExp + e, off0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    bool slow = !(psum[0] <= kSumLimit) || !(psum[1] <= kSumLimit);
    // A row without an offset (hidden in every earlier tile) takes the slow path as soon as
    // it has any finite score in this tile.  Testing its exponentials instead would miss a
    // row whose visible scores all lie below 2^-126 against offset 0: every p underflows to
    // zero and the row would end with no weight although it sees keys.  Rows without an
    // offset are rare (the rows of a diagonal Q-block above its first queued tile), so
    // the row max is taken only in waves that hold one.
    const bool no_off = m_use == -INFINITY;
    if (__builtin_amdgcn_ballot_w64(no_off)) {
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[blk][i]);
      mx = max_with_partner32(mx);
      slow = slow || (no_off && mx > -INFINITY);
    }
    if (__builtin_amdgcn_ballot_w64(slow)) {
      // row max of the tile (both lanes of the row); offset moved up to it if larger
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[blk][i]);
      mx = max_with_partner32(mx) * p.c;
      // only rows that asked for it move their offset, so a row's result never depends
      // on which rows share its wave
      const unsigned sf = slow ? 1u : 0u;
      const auto sp = __builtin_amdgcn_permlane32_swap(sf, sf, false, false);
      const bool need = (sp[0] | sp[1]) != 0u && mx > m_use;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mx : m_use;
        // 0 when m_use = -inf; lanes that keep their offset keep their sums
        const float alpha = need ? __builtin_amdgcn_exp2f(m_use - m_new) : 1.0f;
        lf *= alpha;
        lb *= alpha;
#pragma unroll
        for (int d = 0; d < kDB; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
        m_use = m_new;
      }
      exponentiate_all(m_use == -INFINITY ? 0.f : m_use);
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 2; ++j) pb[hb][j] = __builtin_bit_cast(bf16x8, packed[hb][j]);
    lf += psum[0] + psum[1];
    lb += pbsum[0] + pbsum[1];

    // ---- O^T += V^T P^T for tile it ----
    const bf16* vb = sm.v[cur];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int key0 = (blk * 2 + j) * 16 + hh * 8 + tr_row;
#pragma unroll
        for (int d = 0; d < kDB; ++d) {
          const bf16* vp = vb + key0 * VS + d * 32 + tr_col;
          const bf16x8 a = join_tr(lds_read_tr16(vp), lds_read_tr16(vp + 4 * VS));
          oacc[d] = mfma32(a, pb[blk][j], oacc[d]);
        }
      }
    }

    if (has1 && is_partial(e1)) apply_mask(nxt, sn);
    if (has2) put_k(e2, cur, kst, vec);
    if (has1) put_v(nxt);
    tiles_landed();
    lds_barrier();
  };
  f32x16 sacc2[2];
  for (int it = 0; it < n_tiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it, sacc, sacc2);
    if (it + 1 < n_tiles) step(std::integral_constant<int, 1>{}, it + 1, sacc2, sacc);
  }

  // ---- epilogue: O = acc / l_b, LSE = ln2 * (m + log2 l_f) ----
  lf = sum_with_partner32(lf);
  lb = sum_with_partner32(lb);
  const float inv = lb > 0.f ? 1.0f / lb : 0.f;
  const rsrc_t orr = out_rsrc();
  const uint32_t ooff = (uint32_t)row * (D * 2) + hh * 8;
#pragma unroll
  for (int d = 0; d < kDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[d][g * 4 + 0] * inv, oacc[d][g * 4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[d][g * 4 + 2] * inv, oacc[d][g * 4 + 3] * inv);
      buf_store8(w, orr, ooff, (d * 32 + g * 8) * 2);
    }
  }
  if (hh == 0) {
    const float l = lf > 0.f ? (m_use + __builtin_amdgcn_logf(lf)) * kLn2 : -INFINITY;
    buf_store4(__float_as_uint(l), lse_rsrc(), (uint32_t)row * 4, 0);
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.B == 0 || a.Nq == 0 || a.Hq == 0) return hipSuccess;
  FwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.m = a.m;
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.q_queue = a.q_queue;
  p.q_count = a.q_count;
  p.q_order = a.q_order;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Hm = a.Hm; p.Nq = a.Nq; p.Nk = a.Nk;
  p.nQB = a.nQB; p.nKB = a.nKB;
  p.pack = a.pack > 1 ? kFwdPack : 1;
  p.c = a.scale * kLog2e;
  const unsigned grid = (unsigned)a.B * (unsigned)a.nQB * (unsigned)(a.Hq / p.pack);
  if (ev0) (void)hipEventRecord(ev0, s);
  if (grid > 0) {
    const bool multi = a.m.n > 0;
    auto kern = a.D == 64    ? (multi ? k_attn_fwd<64, true> : k_attn_fwd<64, false>)
                : a.D == 256 ? (multi ? k_attn_fwd<256, true> : k_attn_fwd<256, false>)
                             : (multi ? k_attn_fwd<128, true> : k_attn_fwd<128, false>);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (ev1) (void)hipEventRecord(ev1, s);
  return e;
}

}  // namespace fm
