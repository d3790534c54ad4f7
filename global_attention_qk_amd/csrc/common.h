// Device-side helpers shared by the zgattn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "types.h"

namespace zg {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order: a loop whose
// index is a compile-time constant in every iteration (an MFMA slot stream whose operand
// registers, accumulators and interleaved work are all chosen at compile time).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// cos/sin of the angle p * 2 pi * f, with the phase reduced exactly to [-1/2, 1/2]
// revolutions before the trigonometric evaluation.
__device__ __forceinline__ void rope_cos_sin(int p, float fhi, float flo, float& c, float& s) {
  // No contraction here: fusing (pf * fhi) - n into one FMA would count the product's
  // rounding error twice (it is added back through `lo`).
#pragma clang fp contract(off)
  const float pf = (float)p;                  // exact: |p| < 2^24
  const float a = pf * fhi;
  const float e = __builtin_fmaf(pf, fhi, -a);  // exact rounding error of pf * fhi
  const float lo = __builtin_fmaf(pf, flo, e);
  const float n = __builtin_rintf(a);
  const float fr = (a - n) + lo;              // a - n is exact (Sterbenz)
  sincospif(2.0f * fr, &s, &c);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// sigmoid(x) = 1 / (1 + exp(-x)); +inf -> 1, -inf -> 0, no NaN for infinite x. The
// reciprocal is the hardware one (about 1 ulp), far below the bf16 output rounding.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Packed documents (variable-length prefill): document d covers packed positions
// [cu[d], cu[d+1]). The bounds are clamped into [0, total] and the length to max_len, so a
// malformed table cannot send an access outside the packed tensors.
__device__ __forceinline__ void doc_range(const int32_t* cu, int d, int total, int max_len,
                                          int& start, int& len) {
  const int s0 = min(max(cu[d], 0), total);
  const int s1 = min(max(cu[d + 1], s0), total);
  start = s0;
  len = min(s1 - s0, max_len);
}
// Document holding packed position t: the largest d < n_docs with cu[d] <= t.
__device__ __forceinline__ int doc_of(const int32_t* cu, int n_docs, int t) {
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}
// First V-tile slot of document d in the per-KV-head tile array of a packed batch: the
// slots of document d are [cu[d] / 64 + d, + ceil(len / 64)), which never overlap the next
// document's, and all fit in total / 64 + n_docs slots.
__device__ __forceinline__ int doc_tile_base(int start, int d) { return (start >> 6) + d; }

// Position of 16-byte chunk c within row r of an unpadded LDS tile with CPR (16 or 8)
// chunks per row. The XOR swizzle sends the 16 consecutive rows read by one operand load
// (same chunk) to 16 distinct 16-byte bank groups, and any 8 of them to distinct groups
// of a 128-byte bank row, so the reads are conflict-free with 32 or 64 banks.
template <int CPR>
__device__ __forceinline__ int chunk_pos(int r, int c) {
  return c ^ (CPR == 16 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1)));
}

// LDS DMA of 16 bytes per lane: lane L's bytes from gbase + voff land at LDS byte
// address lds + 16 L. gbase and lds must be wave-uniform (scalar base, M0). Completion is counted by vmcnt
// and left to the caller (vm_wait): the compiler does not see these loads and inserts
// no wait for them. One wait state separates the M0 write from the DMA that reads it.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  // (readfirstlane returns int: each half goes through uint32_t so that it is
  // zero-extended, never sign-extended, into the 64-bit address)
  const uint64_t g = (uint64_t)(uintptr_t)gbase;
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)g);
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
  const uint64_t gu = ((uint64_t)ghi << 32) | (uint64_t)glo;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(voff), "s"(gu) : "memory", "m0");
}
// Wait until at most N vector-memory operations of this wave are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait for every vector-memory load, as an instruction the compiler sees. After register
// operands are loaded ahead of a loop that issues LDS DMA (invisible to the compiler's
// wait counting), this tells the compiler that those loads are complete; otherwise it
// places vmcnt waits for them inside the loop, which the hardware then applies to the
// DMA in flight (waiting for the prefetch of the next tile).
__device__ __forceinline__ void vm_wait_all_known() {
  // gfx9 encoding: vmcnt 0 (bits 3:0 and 15:14), expcnt 7 (6:4), lgkmcnt 15 (11:8)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Sum over each aligned group of N (2, 4, 8 or 16) lanes, the result in every lane of the
// group: cross-lane moves within a row of 16 lanes (DPP), no LDS traffic. The pairings
// (swap neighbours, swap pairs, mirror within 8, mirror within 16) each join two disjoint
// halves of the group summed so far.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2..16 lanes");
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  if (N >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (N >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  if (N >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace zg
