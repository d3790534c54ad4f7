// Standalone QK-RMSNorm + partial RoPE ("ZGCM-1-7B 完全解説" explainer, section
// アーキテクチャ: RMSNorm-based QK normalisation and partial RoPE with rotary ratio 0.33
// on the query and key branches).
//
// 128 rows per workgroup: rows are staged through LDS in fp32 with coalesced 16-byte
// loads, each thread then normalises and rotates one row in place (pairs (k, k + r/2)
// read by LDS index), and the block writes the rows back with coalesced 16-byte stores
// to an arbitrarily strided destination (e.g. straight into a [B, Hkv, S, d] cache).
#include "launch.h"

namespace zg {
namespace {

constexpr int kRowsPerBlock = 128;

template <int D, bool BF16>
__global__ __launch_bounds__(kRowsPerBlock) void qknorm_rope_kernel(const NormRopeArgs p) {
  constexpr int RS = D + 4;  // fp32 row stride in LDS (keeps 16-byte alignment)
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;       // chunks per row
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* rows = (float*)smem;
  float* w = rows + kRowsPerBlock * RS;

  const int t = threadIdx.x;
  const int64_t n_rows = (int64_t)p.B * p.T * p.H;
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock;
  for (int c = t; c < D; c += kRowsPerBlock) w[c] = p.w[c];
  for (int c = t; c < kRowsPerBlock * CPR; c += kRowsPerBlock) {
    const int rr = c / CPR, ch = c % CPR;
    const int64_t row = r0 + rr;
    float* dst = rows + rr * RS + ch * EPC;
    if (row < n_rows) {
      if (BF16) {
        const u32x4 v = *(const u32x4*)((const bf16*)p.x + row * D + ch * 8);
        dst[0] = bf16_lo_to_f32(v.x); dst[1] = bf16_hi_to_f32(v.x);
        dst[2] = bf16_lo_to_f32(v.y); dst[3] = bf16_hi_to_f32(v.y);
        dst[4] = bf16_lo_to_f32(v.z); dst[5] = bf16_hi_to_f32(v.z);
        dst[6] = bf16_lo_to_f32(v.w); dst[7] = bf16_hi_to_f32(v.w);
      } else {
        *(float4*)dst = *(const float4*)((const float*)p.x + row * D + ch * 4);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) dst[e] = 0.f;
    }
  }
  __syncthreads();
  {
    const int64_t row = r0 + t;
    float* x = rows + t * RS;
    if (row < n_rows) {
      const int64_t bt = row / p.H;  // b * T + t
      const int tt = (int)(bt % p.T);
      const int pos = p.pos ? p.pos[bt]
                    : p.cu ? p.pos_offset + tt - p.cu[doc_of(p.cu, p.n_docs, tt)]
                           : p.pos_offset + tt;
      float ss = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) ss = __builtin_fmaf(x[c], x[c], ss);
      const float rn = 1.0f / sqrtf(ss / D + p.eps);
      const int half = p.rdim >> 1;
      for (int j = 0; j < half; ++j) {
        float cs, sn;
        rope_cos_sin(pos, p.fr.hi[j], p.fr.lo[j], cs, sn);
        const float a = x[j] * rn * w[j];
        const float b = x[j + half] * rn * w[j + half];
        x[j] = (a * cs - b * sn) * p.out_scale;
        x[j + half] = (b * cs + a * sn) * p.out_scale;
      }
      for (int c = p.rdim; c < D; ++c) x[c] = x[c] * rn * w[c] * p.out_scale;
    }
  }
  __syncthreads();
  for (int c = t; c < kRowsPerBlock * CPR; c += kRowsPerBlock) {
    const int rr = c / CPR, ch = c % CPR;
    const int64_t row = r0 + rr;
    if (row >= n_rows) continue;
    const int64_t h = row % p.H;
    const int64_t bt = row / p.H;
    const int64_t tt = bt % p.T, bb = bt / p.T;
    const int64_t off = bb * p.ysb + tt * p.yst + h * p.ysh + ch * EPC;
    const float* src = rows + rr * RS + ch * EPC;
    if (BF16) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)src[e];
      *(bf16x8*)((bf16*)p.y + off) = o;
    } else {
      *(float4*)((float*)p.y + off) = *(const float4*)src;
    }
  }
}

template <int D, bool BF16>
hipError_t launch_t(const NormRopeArgs& a, hipStream_t s) {
  const int64_t n_rows = (int64_t)a.B * a.T * a.H;
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks == 0) return hipSuccess;
  const int smem = (kRowsPerBlock * (D + 4) + D) * 4;
  auto kern = qknorm_rope_kernel<D, BF16>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kRowsPerBlock), smem, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qknorm_rope(const NormRopeArgs& a, hipStream_t s) {
  if (a.d == 128) return a.is_bf16 ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
  return a.is_bf16 ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
}

}  // namespace zg
