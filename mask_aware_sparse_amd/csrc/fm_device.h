// Device-side helpers shared by the libfm kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fm_internal.h"

namespace fm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// The mask predicate.  Key column j hides query row i iff
//   LTS_j <= i < LTE_j  or  UTS_j <= i < UTE_j
// (column-wise row bounds, FlashMask-3 page, Overview).  Kernels evaluate it 32
// rows at a time: bit r of the word is set iff row r0 + r is hidden.  Every
// consumer of the mask (forward, backward, dense debug expansion) calls this
// function, so they agree bit for bit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t range_bits32(int a, int b, int r0) {
  // bits r in [0, 32) with a <= r0 + r < b
  int lo = min(max(a - r0, 0), 32);
  int hi = min(max(b - r0, 0), 32);
  uint32_t hm = (uint32_t)((1ull << hi) - 1ull);
  uint32_t lm = (uint32_t)((1ull << lo) - 1ull);
  return hm & ~lm;
}

__device__ __forceinline__ uint32_t hidden_rows32(int lts, int lte, int uts, int ute, int r0) {
  return range_bits32(lts, lte, r0) | range_bits32(uts, ute, r0);
}

// Multi-interval form (FlashMask Guide, "Multi-Interval Sparse Masks"): key column j is
// visible to row i iff start_m <= i < end_m for one of its (up to four) intervals; a row
// is hidden when no interval holds it.  Absent intervals are passed as [0, 0).
__device__ __forceinline__ uint32_t hidden_rows32_multi(int4 s, int4 e, int r0) {
  return ~(range_bits32(s.x, e.x, r0) | range_bits32(s.y, e.y, r0) |
           range_bits32(s.z, e.z, r0) | range_bits32(s.w, e.w, r0));
}

// ---------------------------------------------------------------------------
// Tile classification rule (FlashMask-3 page, §3.1, generalized to both row
// intervals).  mm = {minLTS, maxLTS, minLTE, maxLTE, minUTS, maxUTS, minUTE, maxUTE}
// over the KV block's columns; rows [q0, q1).  0 skip, 1 partial, 2 unmasked.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tile_class(const int* mm, int q0, int q1) {
  bool skip = (q0 >= mm[1] && q1 <= mm[2]) || (q0 >= mm[5] && q1 <= mm[6]);
  bool unm = (q1 <= mm[0] || q0 >= mm[3]) && (q1 <= mm[4] || q0 >= mm[7]);
  return skip ? 0 : (unm ? 2 : 1);
}

// The rule for n visible intervals per column, mm = {min start, max start, min end, max
// end} of each interval over the KV block's columns: skipped when every interval lies
// outside rows [q0, q1) in every column, unmasked when one interval holds them in every
// column.
__device__ __forceinline__ int tile_class_multi(const int* mm, int n, int q0, int q1) {
  bool skip = true, unm = false;
#pragma unroll
  for (int m = 0; m < kMaxIntervals; ++m) {
    if (m < n) {
      skip = skip && (q1 <= mm[4 * m] || q0 >= mm[4 * m + 3]);
      unm = unm || (q0 >= mm[4 * m + 1] && q1 <= mm[4 * m + 2]);
    }
  }
  return skip ? 0 : (unm ? 2 : 1);
}

// ---------------------------------------------------------------------------
// Small numeric helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2 v = {(bf16)a, (bf16)b};  // round to nearest even
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ uint16_t bf16_bits(float a) {
  return __builtin_bit_cast(uint16_t, (bf16)a);  // round to nearest even
}

__device__ __forceinline__ float bf16lo_to_f32(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi_to_f32(unsigned u) { return __uint_as_float(u & 0xFFFF0000u); }

// value of lane (l ^ 32) of the same wave, combined with the own value
__device__ __forceinline__ float max_with_partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// XCD-aware workgroup numbering.  The dispatcher hands workgroup p to XCD p % 8 and each
// XCD has its own L2, so consecutive work items (the query heads of one Q-block, which
// read the same K/V tiles, and neighbouring Q-blocks) would land on 8 different L2s.
// xcd_logical() gives each XCD runs of kXcdChunk consecutive logical items while the
// dispatch order still follows the logical (LPT) order band by band; a ragged last band
// keeps the plain numbering.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
#ifndef FM_XCD_CHUNK
#define FM_XCD_CHUNK 16
#endif
constexpr int kXcdChunk = FM_XCD_CHUNK;

__device__ __forceinline__ int xcd_logical(int p, int n) {
  constexpr int band = kXcds * kXcdChunk;
  const int full = n - n % band;
  if (p >= full) return p;
  const int x = p % kXcds, k = p / kXcds;
  return (k / kXcdChunk) * band + x * kXcdChunk + k % kXcdChunk;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS layout for tiles that are read both row-wise (16-byte ds_read_b128 fragments of
// 16 consecutive rows) and column-wise (ds_read_b64_tr_b16 over 4-row groups): rows of
// 320 bytes with the 16-byte chunk index XORed by bits 2..3 of the row.  Both access
// patterns then hit distinct LDS banks (measured with the SQ_LDS_BANK_CONFLICT counter:
// plain 288-byte rows stall row reads, plain 272-byte rows stall transposing reads).
constexpr int kSwzRow = 160;  // elements per row (320 bytes) of the 128-wide layout
// (the 256-wide layout uses rows of 288 elements with the same XOR)
template <int kRow = kSwzRow>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRow + ((chunk ^ ((row >> 2) & 3)) << 3);
}

// Row-read fragments of a swizzled tile: element offset of the 16-byte fragment for
// d-step s (columns s*16 + hh*8 .. +7) of `row`.  The XOR only flips the low two chunk
// bits, so per lane this is one of two bases plus 16*s.
template <int kRow = kSwzRow>
struct SwzRowRead {
  int even, odd;
  __device__ __forceinline__ SwzRowRead(int row, int hh) {
    const int f = (row >> 2) & 3;
    const int base = row * kRow + 8 * (hh ^ (f & 1));
    even = base + 16 * (f >> 1);
    odd = base - 16 * (f >> 1);
  }
  __device__ __forceinline__ int at(int s) const { return ((s & 1) ? odd : even) + 16 * s; }
};
// Transposing-read addresses of a swizzled tile for rows r0 + 4u (r0 = 16*ks + 8*hh +
// (lane&15)/4, u = 0, 1) and the 32-column block d: per lane two bases plus immediates.
template <int kRow = kSwzRow>
struct SwzTrRead {
  int b0, b1;
  __device__ __forceinline__ SwzTrRead(int lane, int hh) {
    const int tr_row = (lane & 15) >> 2;
    const int chunk = ((lane >> 4) & 1) * 2 + ((lane & 3) >> 1);
    const int sub = 4 * (lane & 1);
    b0 = (hh * 8 + tr_row) * kRow + 8 * (chunk ^ (2 * hh)) + sub;
    b1 = (hh * 8 + tr_row + 4) * kRow + 8 * (chunk ^ (2 * hh + 1)) + sub;
  }
  __device__ __forceinline__ int at(int u, int ks, int d) const {
    return (u ? b1 : b0) + ks * 16 * kRow + 32 * d;
  }
};

// LDS row strides (elements) for head dimension D: the 128-wide layouts serve D <= 128 (a
// fragment read's bank pattern depends only on the row stride, so D = 64 uses the first
// half of each row); D = 256 has its own.  KS: rows read only row-wise; TS: rows also read
// by transposing reads (unswizzled); SWZ: swizzled rows.
template <int D>
struct LdsRows {
  static constexpr int W = D > 128 ? D : 128;
  static constexpr int KS = W + 8;
  static constexpr int TS = W + 32;
  static constexpr int SWZ = W + 32;
};

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element i%4 of the 64-bit words fetched by lanes
// 4t + i/4 (t = 0..3).  With lane j of the group pointing at row (r0 + j/4),
// columns (c0 + 4*(j%4)) .. +3 of a row-major 16-bit matrix, lane i receives
// rows r0..r0+3 of column c0 + i.
__device__ __forceinline__ i16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  u32x2 a = __builtin_bit_cast(u32x2, lo);
  u32x2 b = __builtin_bit_cast(u32x2, hi);
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// ---------------------------------------------------------------------------
// Buffer resources (raw, stride 0): loads past `bytes` return 0, stores and atomics
// past it are dropped, so ragged tails need no per-element branches.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store16(u32x4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store8(u32x2 v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store2(uint16_t v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store4(uint32_t v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_atomic_add(float v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, voff, soff, 0);
}

// s if bit `bit` of `word` is clear, -inf if it is set: a sign-extending bit-field
// extract gives an all-ones / all-zeros mask and a three-input bitwise select (LUT 0xCA:
// first ? second : third) picks the bits, two VALU instructions per element.
__device__ __forceinline__ float mask_neg_inf(float s, uint32_t word, uint32_t bit) {
  const unsigned m = (unsigned)__builtin_amdgcn_sbfe((int)word, bit, 1u);
  return __uint_as_float(__builtin_amdgcn_bitop3_b32(m, 0xff800000u, __float_as_uint(s), 0xCA));
}
// p if bit `bit` of `word` is clear, 0 if it is set.
__device__ __forceinline__ float mask_zero(float p, uint32_t word, uint32_t bit) {
  const unsigned m = (unsigned)__builtin_amdgcn_sbfe((int)word, bit, 1u);
  return __uint_as_float(__builtin_amdgcn_bitop3_b32(m, 0u, __float_as_uint(p), 0xCA));
}

// A read-only array seen through the constant address space: loads from it go through the
// scalar cache whatever the kernel stores elsewhere (the compiler cannot tell where a
// buffer store or a buffer-to-LDS load writes, so it would otherwise use vector loads).
// Only for data no kernel in flight writes.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ const_i32_ptr const_view(const int32_t* p) {
  return (const_i32_ptr)p;
}

// The resource of make_rsrc as four dwords, for inline assembly.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4_t{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)bytes, kRsrcWord3};
}
// The resource r moved forward by `off` bytes (wave-uniform, a multiple of 4, below r's
// byte count): offsets past the end of r stay past the end of the result, so the bounds
// check that turns reads past the tensor into zeros is unchanged.  (The scalar offset operand
// of a buffer load would be cheaper still but is not part of that check.)  Scalar arithmetic.
__device__ __forceinline__ i32x4_t rsrc_advance(i32x4_t r, uint32_t off) {
  const uint32_t r0 = __builtin_amdgcn_readfirstlane((uint32_t)r[0]);
  const uint32_t r1 = __builtin_amdgcn_readfirstlane((uint32_t)r[1]);
  const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)r[2]);
  const uint32_t o = __builtin_amdgcn_readfirstlane(off);
  const uint64_t a = ((uint64_t)r0 | ((uint64_t)(r1 & 0xFFFFu) << 32)) + o;
  // callers pass off < records (a tile that starts inside the tensor)
  return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)(n - o), r[3]};
}
// 16 bytes per lane from resource r at byte offset voff into LDS at lds + 16 * lane (lds
// is wave-uniform).  Written in assembly so that the compiler does not track the LDS write:
// it would otherwise wait for every such load before any transposing LDS read (it cannot
// tell their addresses apart).  The caller waits on the memory counter before the data is
// read.  The no-op covers the wait state between writing M0 and the load that reads it.
__device__ __forceinline__ void lds_load16_untracked(i32x4_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "m0");
}

// A workgroup-shared buffer as the LDS-space pointer the buffer-to-LDS loads take.
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) void*)(const_cast<void*>(p));
}

// Its LDS byte address (wave-uniform for a wave-uniform p).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_ptr(p));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, not for
// its outstanding global loads, stores or atomics (waves here exchange data through LDS
// only, so a full __syncthreads would stall every step on in-flight atomics).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace fm
