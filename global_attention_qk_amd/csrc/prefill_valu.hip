// Prefill attention (both layer kinds) on the vector ALUs, fp32 arithmetic throughout.
//
// Same definition as the bf16 MFMA path (hyper.ai summary of arXiv 2609.13356, section
// 方法; "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ) kept in fp32 end to end:
// the kernel for fp32 tensors, and for bf16 tensors whose shape the MFMA kernels do not
// take (other head groups, rotary dims above 64). One wave64 workgroup owns 64 consecutive
// positions of one query
// head; each lane owns one query row and keeps q~ and its output accumulator in
// registers. K tiles are normalised+rotated once per visit in LDS, V tiles staged in LDS,
// and every lane reads both with broadcast LDS loads. Any head group, rotary_dim <= d.
// Dense batches, or packed documents (one grid slice per document, grid sized by the
// longest).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kT = 64;  // positions per workgroup and keys per tile

struct FArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  void* out;
  const float* wq;
  const float* wk;
  int T, Hq, Hkv, window, rdim, pos_offset, swa, group;
  float eps, scale;
  RopeFreq fr;
  const int32_t* cu;   // packed documents (B == 1, T = total tokens), or nullptr
  int max_len;
};

// RMSNorm + partial RoPE of one LDS row (length D, fp32), written to `dst` (LDS).
template <int D>
__device__ void norm_rope_row_f32(const float* raw, float* dst, const float* w, int pos,
                                  int rdim, float eps, const RopeFreq& fr) {
  float ss = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; ++c) ss = __builtin_fmaf(raw[c], raw[c], ss);
  const float rn = 1.0f / sqrtf(ss / D + eps);
  const int half = rdim >> 1;
  for (int j = 0; j < half; ++j) {
    float cs, sn;
    rope_cos_sin(pos, fr.hi[j], fr.lo[j], cs, sn);
    const float a = raw[j] * rn * w[j];
    const float b = raw[j + half] * rn * w[j + half];
    dst[j] = a * cs - b * sn;
    dst[j + half] = b * cs + a * sn;
  }
  for (int c = rdim; c < D; ++c) dst[c] = raw[c] * rn * w[c];
}

// Four consecutive elements of a row as fp32 (rows start 16-byte aligned).
template <typename T>
__device__ __forceinline__ float4 load4(const T* x) {
  if constexpr (std::is_same<T, float>::value) {
    return *(const float4*)x;
  } else {
    const u32x2 w = *(const u32x2*)x;
    return make_float4(bf16_lo_to_f32(w.x), bf16_hi_to_f32(w.x), bf16_lo_to_f32(w.y),
                       bf16_hi_to_f32(w.y));
  }
}

// E: element type of the tensors (float or bf16)
template <int D, typename E>
__global__ __launch_bounds__(64) void prefill_valu_kernel(const FArgs p) {
  const E* pq = (const E*)p.q;
  const E* pk = (const E*)p.k;
  const E* pv = (const E*)p.v;
  const E* pg = (const E*)p.g;
  E* pout = (E*)p.out;
  constexpr int RS = D + 1;  // padded LDS row
  __shared__ float sRaw[kT * RS];
  __shared__ float sK[kT * RS];
  __shared__ float sV[kT * RS];
  __shared__ float sW[2 * D];
  __shared__ float sS[kT * (kT + 1)];

  const int t = threadIdx.x;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / p.group;
  const int i0 = tile * kT;
  // sequence of this workgroup: tokens [seq0, seq0 + T) of the token order; with packed
  // documents, document b, whose positions restart at pos_offset
  int T = p.T;
  size_t seq0 = (size_t)b * p.T;
  if (p.cu) {
    int start, len;
    doc_range(p.cu, b, p.T, p.max_len, start, len);
    if (i0 >= len) return;   // the whole workgroup, before any barrier
    T = len;
    seq0 = start;
  }
  const int qi = i0 + t;
  for (int c = t; c < D; c += 64) {
    sW[c] = p.wq[c];
    sW[D + c] = p.wk[c];
  }
  __syncthreads();
  // q row -> LDS (thread-per-row), transform into sK (scratch), then to registers.
  {
    const E* src = pq + ((seq0 + qi) * p.Hq + h) * D;
    for (int c = 0; c < D; c += 4) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (qi < T) x = load4(src + c);
      sRaw[t * RS + c] = x.x;
      sRaw[t * RS + c + 1] = x.y;
      sRaw[t * RS + c + 2] = x.z;
      sRaw[t * RS + c + 3] = x.w;
    }
    norm_rope_row_f32<D>(sRaw + t * RS, sK + t * RS, sW, p.pos_offset + qi, p.rdim, p.eps, p.fr);
  }
  float qv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) qv[c] = sK[t * RS + c] * p.scale;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int last = min(i0 + kT, T) - 1;
  int kt_lo = 0;
  if (p.swa) kt_lo = max(0, i0 - p.window + 1) / kT;
  const int kt_hi = last / kT;
  __syncthreads();
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int k0 = kt * kT;
    const int kj = k0 + t;
    {
      const size_t off = ((seq0 + kj) * p.Hkv + kvh) * D;
      for (int c = 0; c < D; c += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kj < T) {
          x = load4(pk + off + c);
          y = load4(pv + off + c);
        }
        sRaw[t * RS + c] = x.x; sRaw[t * RS + c + 1] = x.y;
        sRaw[t * RS + c + 2] = x.z; sRaw[t * RS + c + 3] = x.w;
        sV[t * RS + c] = y.x; sV[t * RS + c + 1] = y.y;
        sV[t * RS + c + 2] = y.z; sV[t * RS + c + 3] = y.w;
      }
      norm_rope_row_f32<D>(sRaw + t * RS, sK + t * RS, sW + D, p.pos_offset + kj, p.rdim,
                           p.eps, p.fr);
    }
    __syncthreads();
    // scores of this lane's query against the tile (LDS, one row per lane)
    float mt = -INFINITY;
    for (int j = 0; j < kT; ++j) {
      const int key = k0 + j;
      bool vis = key <= qi;
      if (p.swa) vis = vis && key > qi - p.window;
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) d = __builtin_fmaf(qv[c], sK[j * RS + c], d);
      d = vis ? d : -INFINITY;
      sS[t * (kT + 1) + j] = d;
      mt = fmaxf(mt, d);
    }
    const float mn = fmaxf(m, mt);
    if (mn != -INFINITY) {
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
      l *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] *= alpha;
      for (int j = 0; j < kT; ++j) {
        const float pj = expf(sS[t * (kT + 1) + j] - mn);
        l += pj;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = __builtin_fmaf(pj, sV[j * RS + c], acc[c]);
      }
      m = mn;
    }
    __syncthreads();
  }
  if (qi < T) {
    const size_t off = ((seq0 + qi) * p.Hq + h) * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float o = acc[c] * inv;
      if (p.swa) o *= 1.0f / (1.0f + expf(-(float)pg[off + c]));
      pout[off + c] = (E)o;
    }
  }
}

}  // namespace

hipError_t launch_prefill_valu(const PrefillArgs& a, bool f32, hipStream_t s) {
  FArgs f;
  f.q = a.q;
  f.k = a.k;
  f.v = a.v;
  f.g = a.g;
  f.out = a.out;
  f.wq = a.wq;
  f.wk = a.wk;
  f.T = a.T;
  f.Hq = a.Hq;
  f.Hkv = a.Hkv;
  f.window = a.window;
  f.rdim = a.rdim;
  f.pos_offset = a.pos_offset;
  f.swa = a.swa;
  f.group = a.Hq / a.Hkv;
  f.eps = a.eps;
  f.scale = a.scale;
  f.fr = a.fr;
  f.cu = a.cu;
  f.max_len = a.max_len;
  const dim3 grid = a.cu ? dim3((a.max_len + kT - 1) / kT, a.Hq, a.n_docs)
                         : dim3((a.T + kT - 1) / kT, a.Hq, a.B);
  if (grid.x == 0) return hipSuccess;
  if (f32) {
    if (a.d == 128) hipLaunchKernelGGL((prefill_valu_kernel<128, float>), grid, dim3(64), 0, s, f);
    else hipLaunchKernelGGL((prefill_valu_kernel<64, float>), grid, dim3(64), 0, s, f);
  } else {
    if (a.d == 128) hipLaunchKernelGGL((prefill_valu_kernel<128, bf16>), grid, dim3(64), 0, s, f);
    else hipLaunchKernelGGL((prefill_valu_kernel<64, bf16>), grid, dim3(64), 0, s, f);
  }
  return hipGetLastError();
}

}  // namespace zg
