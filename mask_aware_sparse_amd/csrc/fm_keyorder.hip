// Key reordering within super-blocks, and the row permutations that go with it (gfx950).
//
// Attention is invariant under a joint permutation of the key columns: K, V and the four
// column vectors permuted alike give the same O, LSE and dQ, and dK, dV permuted back.
// The tile rule (FlashMask-3 page, §3.1) sees blocks of consecutive columns through the
// min/max of their bounds, so a mask whose columns end at scattered rows (the page's
// random-eviction mask, §4) leaves nearly every tile partial.  Per mask row and per
// super-block of kKeyOrderSpan consecutive keys, k_key_order sorts the keys by LTS
// (ties by key index) and keeps that order only where it narrows the tiles: the spread
// (sum over groups of kKeyOrderGroup positions and over the four vectors of max - min,
// bounds clipped to [0, N_q]) must drop strictly, else the natural order stays.
//
// k_permute_rows gathers K and V rows into that order before the attention kernels and
// scatters dK and dV rows back after them.
#include "fm_device.h"
#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kSpan = kKeyOrderSpan;    // 2048 keys per super-block
constexpr int kGroup = kKeyOrderGroup;  // 64 positions per spread group (the forward tile)
constexpr int kThreads = 256;
static_assert(kGroup == 64, "one wave per spread group");
static_assert((kSpan & (kSpan - 1)) == 0, "bitonic sort over a power of two");

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

// one workgroup per (mask row, super-block), numbered row * n_super + super-block; it
// sorts its super-block in LDS
__global__ __launch_bounds__(kThreads) void k_key_order(MaskPtrs m, int Nq, int Nk, int n_super,
                                                        int32_t* __restrict__ perm, MaskOut pv) {
  __shared__ uint64_t keys[kSpan];
  __shared__ int32_t vals[4][kSpan];
  __shared__ long long wsum[2][kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = (int)blockIdx.x / n_super;
  const int s0 = ((int)blockIdx.x - r * n_super) * kSpan;
  const int n = min(kSpan, Nk - s0);
  const size_t row = (size_t)r * Nk + s0;
  const int32_t* src[4] = {m.lts + row, m.lte + row, m.uts + row, m.ute + row};

  for (int i = tid; i < kSpan; i += kThreads) {
    if (i < n) {
#pragma unroll
      for (int x = 0; x < 4; ++x) vals[x][i] = src[x][i];
      // signed order of LTS in the high word (sign bit flipped), key index in the low word:
      // distinct keys, so the sort is stable by construction
      keys[i] = ((uint64_t)((uint32_t)vals[0][i] ^ 0x80000000u) << 32) | (uint32_t)i;
    } else {
      keys[i] = ~0ull;  // padding sorts last
    }
  }
  __syncthreads();

  // spread of an order: wave w takes groups w, w + 4, ...; lane l position g*64 + l
  auto spread = [&](bool sorted, int slot) {
    long long acc = 0;
    for (int g = wave; g * kGroup < n; g += kThreads / 64) {
      const int p = g * kGroup + lane;
      const bool in = p < n;
      const int idx = in ? (sorted ? (int)(uint32_t)keys[p] : p) : 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int v = min(max(vals[x][idx], 0), Nq);
        const int lo = wave_min(in ? v : INT32_MAX), hi = wave_max(in ? v : INT32_MIN);
        acc += (long long)(hi - lo);
      }
    }
    if (lane == 0) wsum[slot][wave] = acc;
  };
  spread(false, 0);

  // bitonic sort, ascending
  for (int k = 2; k <= kSpan; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < kSpan; i += kThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t a = keys[i], b = keys[l];
          if ((a > b) == ((i & k) == 0)) {
            keys[i] = b;
            keys[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }

  spread(true, 1);
  __syncthreads();
  long long nat = 0, srt = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    nat += wsum[0][w];
    srt += wsum[1][w];
  }
  const bool use_sorted = srt < nat;

  int32_t* out[4] = {pv.lts ? pv.lts + row : nullptr, pv.lte ? pv.lte + row : nullptr,
                     pv.uts ? pv.uts + row : nullptr, pv.ute ? pv.ute + row : nullptr};
  for (int p = tid; p < n; p += kThreads) {
    const int idx = use_sorted ? (int)(uint32_t)keys[p] : p;
    perm[row + p] = s0 + idx;
#pragma unroll
    for (int x = 0; x < 4; ++x)
      if (out[x]) out[x][p] = vals[x][idx];
  }
}

// Row permutation of [B][Hkv][Nk][D] bf16 tensors, two at once (K and V, or dK and dV).
// Gather: dst row p = src row perm[p]; scatter: dst row perm[p] = src row p.  kv head h
// uses the permutation of its mask set h / (Hkv / Hm) (Hm divides Hkv).  One thread moves
// 16 bytes.
template <bool kScatter>
__global__ __launch_bounds__(kThreads) void k_permute_rows(const u32x4* __restrict__ src0,
                                                           const u32x4* __restrict__ src1,
                                                           u32x4* __restrict__ dst0,
                                                           u32x4* __restrict__ dst1,
                                                           const int32_t* __restrict__ perm,
                                                           int Hkv, int Hm, int Nk, int chunks,
                                                           size_t total) {
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int c = (int)(t % chunks);
  const size_t rowi = t / chunks;  // (b * Hkv + h) * Nk + p
  const int p = (int)(rowi % Nk);
  const size_t bh = rowi / Nk;
  const int h = (int)(bh % Hkv), b = (int)(bh / Hkv);
  const int set = h / (Hkv / Hm);
  const int q = perm[((size_t)b * Hm + set) * Nk + p];
  const size_t other = (bh * Nk + q) * chunks + c;
  const size_t from = kScatter ? t : other, to = kScatter ? other : t;
  dst0[to] = src0[from];
  dst1[to] = src1[from];
}

}  // namespace

hipError_t launch_key_order(const MaskPtrs& m, int rows, int Nq, int Nk, int32_t* perm,
                            const MaskOut& permuted, hipStream_t s) {
  if (rows == 0 || Nk == 0) return hipSuccess;
  const int n_super = (Nk + kSpan - 1) / kSpan;
  hipLaunchKernelGGL(k_key_order, dim3((unsigned)rows * (unsigned)n_super), dim3(kThreads), 0, s,
                     m, Nq, Nk, n_super, perm, permuted);
  return hipGetLastError();
}

hipError_t launch_permute_rows(bool scatter, const void* src0, const void* src1, void* dst0,
                               void* dst1, const int32_t* perm, int B, int Hkv, int Hm, int Nk,
                               int D, hipStream_t s) {
  const int chunks = D / 8;
  const size_t total = (size_t)B * Hkv * Nk * chunks;
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + kThreads - 1) / kThreads);
  auto kern = scatter ? k_permute_rows<true> : k_permute_rows<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const u32x4*>(src0), static_cast<const u32x4*>(src1),
                     static_cast<u32x4*>(dst0), static_cast<u32x4*>(dst1), perm, Hkv, Hm, Nk,
                     chunks, total);
  return hipGetLastError();
}

}  // namespace fm
