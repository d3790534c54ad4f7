// Standalone QK-RMSNorm + partial RoPE ("ZGCM-1-7B 完全解説" explainer, section
// アーキテクチャ: RMSNorm-based QK normalisation and partial RoPE with rotary ratio 0.33
// on the query and key branches).
//
// D/8 lanes per row, 8 dims per lane: the row's sum of squares is a reduction over its
// lanes, the lanes share the row's RoPE table (pairs (k, k + r/2), each cos/sin computed
// once) and its normalised values through LDS, so that each lane reads the partners of
// its rotated dims, and every lane stores its 8 results with one 16-byte (bf16) or
// 32-byte (fp32) access to an arbitrarily strided destination (e.g. straight into a
// [B, Hkv, S, d] cache). Packed documents restart positions at each document's first
// token. Row indices are 32-bit (the launcher rejects more than 2^31 - 1 rows).
#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kThreadsNR = 256;

template <int D, bool BF16>
__global__ __launch_bounds__(kThreadsNR) void qknorm_rope_kernel(const NormRopeArgs p) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPB = kThreadsNR / LPR;      // rows per workgroup
  __shared__ float sx[RPB][D + 4];
  __shared__ float2 st[RPB][kMaxHalfRot];
  const int t = threadIdx.x;
  const int rl = t / LPR, sub = t % LPR;
  const uint32_t n_rows = (uint32_t)p.B * p.T * p.H;
  const uint32_t row = blockIdx.x * RPB + rl;
  const bool ok = row < n_rows;
  const uint32_t rc = ok ? row : n_rows - 1;
  float x[8];
  if (BF16) {
    const u32x4 v = *(const u32x4*)((const bf16*)p.x + (size_t)rc * D + sub * 8);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo_to_f32(w4[e]);
      x[2 * e + 1] = bf16_hi_to_f32(w4[e]);
    }
  } else {
    const float4 a = *(const float4*)((const float*)p.x + (size_t)rc * D + sub * 8);
    const float4 b = *(const float4*)((const float*)p.x + (size_t)rc * D + sub * 8 + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  const uint32_t bt = rc / (uint32_t)p.H;    // b * T + t
  const uint32_t h = rc - bt * (uint32_t)p.H;
  const uint32_t bb = bt / (uint32_t)p.T;
  const int tt = (int)(bt - bb * (uint32_t)p.T);
  const int pos = p.pos ? p.pos[bt]
                : p.cu ? p.pos_offset + tt - p.cu[doc_of(p.cu, p.n_docs, tt)]
                       : p.pos_offset + tt;
  const int half = p.rdim >> 1;
  for (int j = sub; j < half; j += LPR) {
    float cs, sn;
    rope_cos_sin(pos, p.fr.hi[j], p.fr.lo[j], cs, sn);
    st[rl][j] = make_float2(cs, sn);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
  ss = group_sum<LPR>(ss);
  const float rn = 1.0f / sqrtf(ss / D + p.eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = x[e] * rn * p.w[sub * 8 + e];
    sx[rl][sub * 8 + e] = x[e];
  }
  __syncthreads();
  // Dims past rotary_dim read partner 0 and pair 0 and discard them (no branches).
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = sub * 8 + e;
    const bool rot = c < p.rdim, lower = c < half;
    const int pc = rot ? (lower ? c + half : c - half) : 0;
    const float2 cs = st[rl][rot ? (lower ? c : c - half) : 0];
    const float partner = sx[rl][pc];
    const float r = lower ? x[e] * cs.x - partner * cs.y : x[e] * cs.x + partner * cs.y;
    y[e] = (rot ? r : x[e]) * p.out_scale;
  }
  if (!ok) return;
  const int64_t off = (int64_t)bb * p.ysb + (int64_t)tt * p.yst + (int64_t)h * p.ysh + sub * 8;
  if (BF16) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)y[e];
    *(bf16x8*)((bf16*)p.y + off) = o;
  } else {
    *(float4*)((float*)p.y + off) = make_float4(y[0], y[1], y[2], y[3]);
    *(float4*)((float*)p.y + off + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
}

template <int D, bool BF16>
hipError_t launch_t(const NormRopeArgs& a, hipStream_t s) {
  constexpr int RPB = kThreadsNR / (D / 8);
  const int64_t n_rows = (int64_t)a.B * a.T * a.H;
  if (n_rows > INT32_MAX) return hipErrorInvalidValue;
  const int64_t blocks = (n_rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((qknorm_rope_kernel<D, BF16>), dim3((unsigned)blocks), dim3(kThreadsNR), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qknorm_rope(const NormRopeArgs& a, hipStream_t s) {
  if (a.d == 128) return a.is_bf16 ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
  return a.is_bf16 ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
}

}  // namespace zg
