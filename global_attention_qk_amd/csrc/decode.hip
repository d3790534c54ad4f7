// Single-token decode for both layer kinds (bf16 caches; fp32 for single-layer calls).
//
// "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ: the 27 gated SWA layers keep a
// fixed 128-token KV cache while the 5 global layers keep the whole sequence, and decode
// is bound by memory bandwidth. The new token (position pos) is normalised and rotated
// like every other q/k row, appended to its cache, and attends to the visible entries.
//
// Global layers (split-K over the cache, three launches on one stream):
//   1. prep:    q~ (scaled by softmax_scale*log2 e) -> workspace, k~_new/v_new -> cache[pos].
//   2. split:   one workgroup per (chunk of cache, kv head, sequence). Scores of all g
//               query heads against 16 cached keys at a time come from one
//               v_mfma_f32_16x16x32_bf16 chain (keys on M, heads on N), straight from
//               global memory; the chunk's softmax statistics are exact (two passes over
//               the chunk's scores in LDS), then P.V streams V once on the vector ALUs.
//               Partial (max, sum, acc) per split go to the workspace.
//   3. combine: log-sum-exp merge of the splits per (sequence, query head).
// SWA layers: one workgroup per (sequence, kv head) does the whole step over the ring
// (MFMA scores with the ring in registers when it holds at most 128 slots, the model's
// window; a per-slot kernel for larger rings).
// fp32 tensors and caches take the same kernels instantiated for float, with the scores on
// the vector ALUs (the per-slot SWA kernel; the global split kernel's fp32 form).
#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "zgattn.h"

namespace zg {

// Scratch of zgattn_global_decode_noalloc: the split-K partials of a global decode step
// for callers that cannot allocate. One copy per GPU, at its own address on each: host
// code must never pass this name to a kernel, only the address that
// hipGetSymbolAddress returns for the current device (decode_noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[ZGATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kThreads = 256;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, or null

__device__ __forceinline__ bool pos_valid(int pos, int limit) { return pos >= 0 && pos < limit; }

// The per-layer tensors of a single-layer call.
__device__ __forceinline__ LayerIO layer_io(const DecodeArgs& p) {
  return LayerIO{p.q, p.k_new, p.v_new, p.g, p.wq, p.wk, p.k_cache, p.v_cache, p.out, p.ws};
}

// Normalise + rotate `nrows` rows of d values held in LDS (fp32, stride D) in place.
// Each wave takes rows wave, wave + 4, ...; all threads must call it.
template <int D>
__device__ void norm_rope_rows_lds(float* buf, const float* wrow[], int nrows, int pos,
                                   int rdim, float eps, const RopeFreq& fr, float* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = rdim >> 1;
  for (int base = 0; base < nrows; base += 4) {
    const int row = base + wave;
    const bool act = row < nrows;
    float x[D / 64];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      x[i] = act ? buf[row * D + lane + 64 * i] : 0.f;
      ss = __builtin_fmaf(x[i], x[i], ss);
    }
    ss = wave_sum(ss);
    const float rn = 1.0f / sqrtf(ss / D + eps);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int c = lane + 64 * i;
      if (act) tmp[row * D + c] = x[i] * rn * wrow[row][c];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int c = lane + 64 * i;
      if (act) {
        float o = tmp[row * D + c];
        if (c < rdim) {
          const int j = c < half ? c : c - half;
          float cs, sn;
          rope_cos_sin(pos, fr.hi[j], fr.lo[j], cs, sn);
          const float pr = tmp[row * D + (c < half ? c + half : c - half)];
          o = c < half ? o * cs - pr * sn : o * cs + pr * sn;
        }
        buf[row * D + c] = o;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// Global decode, step 1: prep.
// ---------------------------------------------------------------------------------------
template <int D, typename T = bf16>
__device__ __forceinline__ void gdec_prep_kernel_body(const DecodeArgs& p, const LayerIO& io, int kvh, int b) {
  const int G = p.Hq / p.Hkv;
  const int pos = p.pos[b];
  if (!pos_valid(pos, p.S)) return;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* buf = (float*)smem;                 // (G + 1) rows
  float* tmp = buf + (G + 1) * D;
  const int t = threadIdx.x;
  const T* q = (const T*)io.q + ((size_t)b * p.Hq + kvh * G) * D;
  const T* kn = (const T*)io.k_new + ((size_t)b * p.Hkv + kvh) * D;
  for (int i = t; i < (G + 1) * D; i += kThreads)
    buf[i] = i < G * D ? (float)q[i] : (float)kn[i - G * D];
  const float* wrow[9];
  for (int r = 0; r < 9; ++r) wrow[r] = r < G ? io.wq : io.wk;
  __syncthreads();
  norm_rope_rows_lds<D>(buf, wrow, G + 1, pos, p.rdim, p.eps, p.fr, tmp);
  const float qs = p.scale * 1.4426950408889634f;
  float* wsq = io.ws + ((size_t)b * p.Hq + kvh * G) * D;
  for (int i = t; i < G * D; i += kThreads) wsq[i] = buf[i] * qs;
  const size_t crow = (((size_t)b * p.Hkv + kvh) * p.S + pos) * D;
  const T* vn = (const T*)io.v_new + ((size_t)b * p.Hkv + kvh) * D;
  for (int c = t; c < D; c += kThreads) {
    ((T*)io.k_cache)[crow + c] = (T)buf[G * D + c];
    ((T*)io.v_cache)[crow + c] = vn[c];
  }
}
template <int D, typename T = bf16>
__global__ __launch_bounds__(kThreads) void gdec_prep_kernel(const DecodeArgs p) {
  gdec_prep_kernel_body<D, T>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y);
}
template <int D>
__global__ __launch_bounds__(kThreads) void gdec_prep_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z;
  gdec_prep_kernel_body<D>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y);
}

// ---------------------------------------------------------------------------------------
// Global decode, step 2: one split of the cache.
// ---------------------------------------------------------------------------------------
template <int D, int G, typename T = bf16>
__device__ __forceinline__ void gdec_split_kernel_body(const DecodeArgs& p, const LayerIO& io, int split, int kvh, int b) {
  constexpr int KS = D / 32;            // k-steps of the 16x16x32 product
  constexpr int DC = D / 8;             // 8-wide d chunks
  constexpr int NKL = kThreads / DC;    // key lanes in the P.V phase
  const int pos = p.pos[b];
  if (!pos_valid(pos, p.S)) return;
  const int c0 = split * p.chunk;
  if (c0 > pos) return;
  const int n = min(p.chunk, pos + 1 - c0);

  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sP = (float*)smem;             // [chunk][G] scores, then probabilities
  float* sRed = (float*)smem;           // [NKL][G][D] after P.V (aliases sP)
  __shared__ float sM[G], sL[G];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const size_t cbase = (((size_t)b * p.Hkv + kvh) * p.S + c0) * D;
  const T* kc = (const T*)io.k_cache + cbase;
  const T* vc = (const T*)io.v_cache + cbase;

  if constexpr (std::is_same<T, float>::value) {
    // fp32 caches: one key per thread at a time, the G dot products on the vector ALUs,
    // q~ from LDS (every lane reads the same word: a broadcast)
    __shared__ float sQ[G * D];
    const float* wsq = io.ws + ((size_t)b * p.Hq + kvh * G) * D;
    for (int i = t; i < G * D; i += kThreads) sQ[i] = wsq[i];
    __syncthreads();
    for (int kl = t; kl < n; kl += kThreads) {
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = 0.f;
      const float* krow = kc + (size_t)kl * D;
#pragma unroll 4
      for (int c = 0; c < D; c += 4) {
        const float4 kv = *(const float4*)(krow + c);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          sc[h] = __builtin_fmaf(sQ[h * D + c], kv.x, sc[h]);
          sc[h] = __builtin_fmaf(sQ[h * D + c + 1], kv.y, sc[h]);
          sc[h] = __builtin_fmaf(sQ[h * D + c + 2], kv.z, sc[h]);
          sc[h] = __builtin_fmaf(sQ[h * D + c + 3], kv.w, sc[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) sP[kl * G + h] = sc[h];
    }
  } else {
  // q~ as the B operand: column = head l16 (zero beyond G), k = d.
  bf16x8 qb[KS];
  {
    const float* wsq = io.ws + ((size_t)b * p.Hq + kvh * G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = (bf16)(l16 < G ? wsq[l16 * D + ks * 32 + q4 * 8 + e] : 0.f);
      qb[ks] = v;
    }
  }
  // Phase A: scores, 16 keys per MFMA chain, two chains in flight per wave.
  const int ngroups = (n + 15) >> 4;
  for (int kg0 = wave * 2; kg0 < ngroups; kg0 += 8) {
    f32x4 acc[2];
    bf16x8 a[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kl = (kg0 + u) * 16 + l16;
      const bool ok = (kg0 + u) < ngroups && kl < n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (ok) raw = *(const u32x4*)(kc + (size_t)kl * D + ks * 32 + q4 * 8);
        a[u][ks] = __builtin_bit_cast(bf16x8, raw);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][ks], qb[ks], acc[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kg = kg0 + u;
      if (kg < ngroups && l16 < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kl = kg * 16 + q4 * 4 + r;
          if (kl < n) sP[kl * G + l16] = acc[u][r];
        }
      }
    }
  }
  }
  __syncthreads();
  // Phase B: exact max / sum per head over the chunk, P in place.
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int kl = lane; kl < n; kl += 64) m = fmaxf(m, sP[kl * G + h]);
    m = wave_max(m);
    float l = 0.f;
    for (int kl = lane; kl < n; kl += 64) {
      const float e = fast_exp2(sP[kl * G + h] - m);
      sP[kl * G + h] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      sM[h] = m;
      sL[h] = l;
    }
  }
  __syncthreads();
  // Phase C: acc[h][:] = sum_k P[k][h] V[k][:] on the vector ALUs.
  const int dc = t % DC, kl0 = t / DC;
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll 4
  for (int kl = kl0; kl < n; kl += NKL) {
    float v[8];
    if constexpr (std::is_same<T, float>::value) {
      const float4 v0 = *(const float4*)(vc + (size_t)kl * D + dc * 8);
      const float4 v1 = *(const float4*)(vc + (size_t)kl * D + dc * 8 + 4);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    } else {
      const u32x4 raw = *(const u32x4*)(vc + (size_t)kl * D + dc * 8);
      v[0] = bf16_lo_to_f32(raw.x); v[1] = bf16_hi_to_f32(raw.x);
      v[2] = bf16_lo_to_f32(raw.y); v[3] = bf16_hi_to_f32(raw.y);
      v[4] = bf16_lo_to_f32(raw.z); v[5] = bf16_hi_to_f32(raw.z);
      v[6] = bf16_lo_to_f32(raw.w); v[7] = bf16_hi_to_f32(raw.w);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pw = sP[kl * G + h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(pw, v[e], acc[h][e]);
    }
  }
  __syncthreads();  // sP is dead; reuse as sRed
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) sRed[(kl0 * G + h) * D + dc * 8 + e] = acc[h][e];
  __syncthreads();
  for (int idx = t; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float s = 0.f;
    for (int k = 0; k < NKL; ++k) s += sRed[(k * G + h) * D + d];
    const size_t hq = (size_t)b * p.Hq + kvh * G + h;
    io.ws[(size_t)p.B * p.Hq * D + (hq * p.nsplit + split) * D + d] = s;
  }
  if (t < G) {
    const size_t hq = (size_t)b * p.Hq + kvh * G + t;
    float* ml = io.ws + (size_t)p.B * p.Hq * D * (1 + (size_t)p.nsplit);
    ml[(hq * p.nsplit + split) * 2 + 0] = sM[t];
    ml[(hq * p.nsplit + split) * 2 + 1] = sL[t];
  }
}
template <int D, int G, typename T = bf16>
__global__ __launch_bounds__(kThreads) void gdec_split_kernel(const DecodeArgs p) {
  gdec_split_kernel_body<D, G, T>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z);
}
template <int D, int G>
__global__ __launch_bounds__(kThreads) void gdec_split_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z / pb.a.B;
  gdec_split_kernel_body<D, G>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z % pb.a.B);
}

// ---------------------------------------------------------------------------------------
// Global decode, step 3: log-sum-exp merge of the splits.
// ---------------------------------------------------------------------------------------
template <int D, typename T = bf16>
__device__ __forceinline__ void gdec_combine_kernel_body(const DecodeArgs& p, const LayerIO& io, int h, int b) {
  const int d = threadIdx.x;
  const int pos = p.pos[b];
  T* out = (T*)io.out + ((size_t)b * p.Hq + h) * D;
  if (!pos_valid(pos, p.S)) {
    out[d] = (T)__builtin_nanf("");
    return;
  }
  const int ns = min(p.nsplit, pos / p.chunk + 1);
  const size_t hq = (size_t)b * p.Hq + h;
  const float* acc = io.ws + (size_t)p.B * p.Hq * D + hq * p.nsplit * D;
  const float* ml = io.ws + (size_t)p.B * p.Hq * D * (1 + (size_t)p.nsplit) + hq * p.nsplit * 2;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = fast_exp2(ml[2 * s] - M);
    L = __builtin_fmaf(ml[2 * s + 1], w, L);
    o = __builtin_fmaf(acc[(size_t)s * D + d], w, o);
  }
  out[d] = (T)(o / L);
}
template <int D, typename T = bf16>
__global__ __launch_bounds__(D) void gdec_combine_kernel(const DecodeArgs p) {
  gdec_combine_kernel_body<D, T>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y);
}
template <int D>
__global__ __launch_bounds__(D) void gdec_combine_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z;
  gdec_combine_kernel_body<D>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y);
}

// ---------------------------------------------------------------------------------------
// SWA decode over the ring: one workgroup per (kv head, sequence).
// ---------------------------------------------------------------------------------------
template <int D, typename T = bf16>
__global__ __launch_bounds__(kThreads) void swa_decode_kernel(const DecodeArgs p) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = p.Hq / p.Hkv;
  const int W = p.window;
  const int pos = p.pos[b];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  T* out = (T*)p.out + ((size_t)b * p.Hq + kvh * G) * D;
  if (!pos_valid(pos, ZGATTN_POS_LIMIT)) {
    for (int i = t; i < G * D; i += kThreads) out[i] = (T)__builtin_nanf("");
    return;
  }
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* buf = (float*)smem;        // G q rows + k_new row
  float* tmp = buf + (G + 1) * D;
  float* sv = tmp + (G + 1) * D;    // v_new
  float* sS = sv + D;               // [G][W]
  const T* q = (const T*)p.q + ((size_t)b * p.Hq + kvh * G) * D;
  const T* kn = (const T*)p.k_new + ((size_t)b * p.Hkv + kvh) * D;
  const T* vn = (const T*)p.v_new + ((size_t)b * p.Hkv + kvh) * D;
  for (int i = t; i < (G + 1) * D; i += kThreads)
    buf[i] = i < G * D ? (float)q[i] : (float)kn[i - G * D];
  for (int c = t; c < D; c += kThreads) sv[c] = (float)vn[c];
  const float* wrow[9];
  for (int r = 0; r < 9; ++r) wrow[r] = r < G ? p.wq : p.wk;
  __syncthreads();
  norm_rope_rows_lds<D>(buf, wrow, G + 1, pos, p.rdim, p.eps, p.fr, tmp);
  const float qs = p.scale * 1.4426950408889634f;
  const int slot = pos % W;
  T* kr = (T*)p.k_cache + ((size_t)b * p.Hkv + kvh) * W * D;
  T* vr = (T*)p.v_cache + ((size_t)b * p.Hkv + kvh) * W * D;
  // the new key as the cache will hold it; the ring slot itself is written last
  for (int c = t; c < D; c += kThreads) buf[G * D + c] = (float)(T)buf[G * D + c];
  __syncthreads();
  // scores
  for (int idx = t; idx < G * W; idx += kThreads) {
    const int h = idx / W, s = idx % W;
    const bool valid = pos >= W - 1 || s <= pos;
    float d = -INFINITY;
    if (valid) {
      d = 0.f;
      if (s == slot) {
        for (int c = 0; c < D; ++c) d = __builtin_fmaf(buf[h * D + c], buf[G * D + c], d);
      } else if constexpr (std::is_same<T, float>::value) {
        const float* kro = kr + (size_t)s * D;
        for (int c = 0; c < D; c += 4) {
          const float4 kv = *(const float4*)(kro + c);
          d = __builtin_fmaf(buf[h * D + c], kv.x, d);
          d = __builtin_fmaf(buf[h * D + c + 1], kv.y, d);
          d = __builtin_fmaf(buf[h * D + c + 2], kv.z, d);
          d = __builtin_fmaf(buf[h * D + c + 3], kv.w, d);
        }
      } else {
        const bf16* kro = kr + (size_t)s * D;
        for (int c = 0; c < D; c += 8) {
          const u32x4 raw = *(const u32x4*)(kro + c);
          const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d = __builtin_fmaf(buf[h * D + c + 2 * e], bf16_lo_to_f32(w4[e]), d);
            d = __builtin_fmaf(buf[h * D + c + 2 * e + 1], bf16_hi_to_f32(w4[e]), d);
          }
        }
      }
      d *= qs;
    }
    sS[h * W + s] = d;
  }
  __syncthreads();
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int s = lane; s < W; s += 64) m = fmaxf(m, sS[h * W + s]);
    m = wave_max(m);
    float l = 0.f;
    for (int s = lane; s < W; s += 64) {
      const float e = fast_exp2(sS[h * W + s] - m);
      sS[h * W + s] = e;
      l += e;
    }
    l = wave_sum(l);
    const float inv = 1.0f / l;
    for (int s = lane; s < W; s += 64) sS[h * W + s] *= inv;
  }
  __syncthreads();
  const T* g = (const T*)p.g + ((size_t)b * p.Hq + kvh * G) * D;
  for (int idx = t; idx < G * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    const int ns = pos >= W - 1 ? W : pos + 1;
    float o = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float vv = s == slot ? sv[c] : (float)vr[(size_t)s * D + c];
      o = __builtin_fmaf(sS[h * W + s], vv, o);
    }
    o *= sigmoidf_((float)g[idx]);
    out[idx] = (T)o;
  }
  __syncthreads();
  for (int c = t; c < D; c += kThreads) {
    kr[(size_t)slot * D + c] = (T)buf[G * D + c];
    vr[(size_t)slot * D + c] = (T)sv[c];
  }
}

constexpr int kRingMax = 128;   // ring slots of the MFMA kernel (the model's window)

// ---------------------------------------------------------------------------------------
// SWA decode, rings of at most 128 slots and at most 8 query heads per KV head (the
// model's shape). One workgroup (4 waves) per (sequence, KV head); wave w owns ring slots
// 32 w .. 32 w + 31. At the start every wave loads its slots' K rows straight into MFMA
// A-operand registers and its V rows into registers (the whole ring is one memory round
// trip and nothing of it goes through LDS), while the workgroup normalises and rotates the
// g query rows and k_new into LDS. Scores of the g heads against the wave's 32 slots come
// from v_mfma_f32_16x16x32_bf16 (slots on M, heads on N); the wave's softmax statistics
// and its partial P.V (vector ALUs: 8 dims and a quarter of the slots per lane) are merged
// across the waves by log-sum-exp, and the gate is applied to the result. The new entry
// replaces its slot's old contents in the registers (scores and P.V see the ring as it is
// after the step) and reaches the ring in HBM at the end.
constexpr int kMfmaDecodeMaxG = 8;

template <int D, int GM>
struct SwaDecSmem {
  static constexpr int kQ = 0;                          // bf16 [16][D]: q~ (rows >= g zero)
  static constexpr int kKn = kQ + 16 * D * 2;           // bf16 [D]: k~_new as the ring holds it
  static constexpr int kVn = kKn + D * 2;               // bf16 [D]
  static constexpr int kTrig = kVn + D * 2;             // float2 [kMaxHalfRot]
  static constexpr int kRaw = kTrig + kMaxHalfRot * 8;  // float [g + 1][D]: normalised rows
  static constexpr int kP = kRaw + (GM + 1) * D * 4;     // float [4][GM][32]
  static constexpr int kO = kP + 4 * GM * 32 * 4;        // float [4][GM][D]
  static constexpr int kML = kO + 4 * GM * D * 4;        // float [4][GM][2]
  static constexpr int kTotal = kML + 4 * GM * 2 * 4;
};

// GM: the most query heads per KV head the instance handles (4, or 8).
template <int D, int GM>
__device__ __forceinline__ void swa_decode_mfma_body(const DecodeArgs& p, const LayerIO& io,
                                                     int kvh, int b) {
  using S = SwaDecSmem<D, GM>;
  constexpr int KS = D / 32;       // k-steps of the score products
  constexpr int DL = D / 8;        // lanes per row (8 dims each) in the P.V layout
  constexpr int KG = 64 / DL;      // slot groups in the P.V layout
  constexpr int KPL = 32 / KG;     // slots per lane in P.V
  const int G = p.Hq / p.Hkv;
  const int W = p.window;
  // An invalid position is not waited for up front: the step runs at position 0 (its loads
  // do not depend on the position), then writes NaN outputs and leaves the ring unchanged.
  const int pos_in = p.pos[b];
  const bool valid = pos_valid(pos_in, ZGATTN_POS_LIMIT);
  const int pos = valid ? pos_in : 0;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  bf16* out = (bf16*)io.out + ((size_t)b * p.Hq + kvh * G) * D;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* sQ = (bf16*)(smem + S::kQ);
  bf16* sKn = (bf16*)(smem + S::kKn);
  bf16* sVn = (bf16*)(smem + S::kVn);
  float2* sTrig = (float2*)(smem + S::kTrig);
  float* sRaw = (float*)(smem + S::kRaw);
  float* sP = (float*)(smem + S::kP);
  float* sO = (float*)(smem + S::kO);
  float* sML = (float*)(smem + S::kML);
  bf16* kr = (bf16*)io.k_cache + ((size_t)b * p.Hkv + kvh) * W * D;
  bf16* vr = (bf16*)io.v_cache + ((size_t)b * p.Hkv + kvh) * W * D;

  // ---- 0. the small inputs first: loads complete in issue order, so the q/k transform
  // below waits only for these, not for the ring behind them --------------------------------
  const int half = p.rdim >> 1;
  const bf16* qg = (const bf16*)io.q + ((size_t)b * p.Hq + kvh * G) * D;
  const bf16* kn = (const bf16*)io.k_new + ((size_t)b * p.Hkv + kvh) * D;
  const bf16* vn = (const bf16*)io.v_new + ((size_t)b * p.Hkv + kvh) * D;
  const bf16* gg = (const bf16*)io.g + ((size_t)b * p.Hq + kvh * G) * D;
  const int sub = t % DL;   // 8 dims of a row per lane
  const int r0 = t / DL;    // the row (q head, or k_new when r0 == G) this lane transforms
  static_assert(kThreads / DL > kMfmaDecodeMaxG, "one pass over the g + 1 rows");
  u32x4 raw0 = {0u, 0u, 0u, 0u}, vn0 = {0u, 0u, 0u, 0u};
  float4 wq0 = {0.f, 0.f, 0.f, 0.f}, wq1 = wq0, wk0 = wq0, wk1 = wq0;
  if (r0 <= G) {
    raw0 = *(const u32x4*)((r0 < G ? qg + r0 * D : kn) + sub * 8);
    // both weight vectors, selected where they are used: a select of the two pointers
    // becomes a per-lane load of the chosen kernel-argument field, and a select of the
    // values here would wait for the loads at once
    wq0 = *(const float4*)(io.wq + sub * 8);
    wq1 = *(const float4*)(io.wq + sub * 8 + 4);
    wk0 = *(const float4*)(io.wk + sub * 8);
    wk1 = *(const float4*)(io.wk + sub * 8 + 4);
  }
  if (t < DL) vn0 = *(const u32x4*)(vn + t * 8);
  float fhi = 0.f, flo = 0.f;
  if (t < half) {
    fhi = p.fr.hi[t];
    flo = p.fr.lo[t];
  }
  constexpr int GIT = (GM * D / 2 + kThreads - 1) / kThreads;
  uint32_t gw[GIT];
#pragma unroll
  for (int i = 0; i < GIT; ++i) {
    const int idx = t + i * kThreads;
    gw[i] = idx < G * D / 2 ? *(const uint32_t*)(gg + 2 * idx) : 0u;
  }

  // ---- 1. the wave's ring slots -> registers (slots past the ring are clamped, masked) ---
  u32x4 ka[2][KS], va[KPL];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int slot = min(32 * wave + 16 * kb + (lane & 15), W - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[kb][ks] = *(const u32x4*)(kr + (size_t)slot * D + 32 * ks + 8 * (lane >> 4));
  }
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int slot = min(32 * wave + lane / DL + KG * i, W - 1);
    va[i] = *(const u32x4*)(vr + (size_t)slot * D + 8 * (lane % DL));
  }

  // ---- 2. q~ (g rows, scaled by softmax_scale * log2 e) and k~_new into LDS ------------
  if (t < half) {
    float cs, sn;
    rope_cos_sin(pos, fhi, flo, cs, sn);
    sTrig[t] = make_float2(cs, sn);
  }
  if (r0 <= G) {
    const int r = r0;
    const float4 w0 = r < G ? wq0 : wk0, w1 = r < G ? wq1 : wk1;
    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint32_t w4[4] = {raw0.x, raw0.y, raw0.z, raw0.w};
    float x[8], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo_to_f32(w4[e]);
      x[2 * e + 1] = bf16_hi_to_f32(w4[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    ss = group_sum<DL>(ss);
    const float rn = 1.0f / sqrtf(ss / D + p.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) sRaw[r * D + sub * 8 + e] = x[e] * rn * w[e];
  }
  for (int c = t; c < (16 - G) * D; c += kThreads) sQ[G * D + c] = (bf16)0.0f;
  if (t < DL) *(u32x4*)(sVn + t * 8) = vn0;
  __syncthreads();
  const float qs = p.scale * 1.4426950408889634f;
  for (int r = t / DL; r <= G; r += kThreads / DL) {
    const float* row = sRaw + r * D;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dims past rotary_dim read pair 0 and partner 0 and keep their value
      const int c = sub * 8 + e;
      const bool rot = c < p.rdim, lower = c < half;
      const float2 cs = sTrig[rot ? (lower ? c : c - half) : 0];
      const float pr = row[rot ? (lower ? c + half : c - half) : 0];
      const float y = lower ? row[c] * cs.x - pr * cs.y : row[c] * cs.x + pr * cs.y;
      const float v = rot ? y : row[c];
      o[e] = (bf16)(r < G ? v * qs : v);
    }
    *(bf16x8*)((r < G ? sQ + r * D : sKn) + sub * 8) = o;
  }
  __syncthreads();

  // ---- 3. the new entry over its slot's old contents ------------------------------------
  const int sn = pos % W;
  if (sn / 32 == wave) {
    const int sl = sn % 32;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (sl / 16 == kb && (lane & 15) == sl % 16) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[kb][ks] = *(const u32x4*)(sKn + 32 * ks + 8 * (lane >> 4));
      }
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (lane / DL == sl % KG && i == sl / KG) va[i] = *(const u32x4*)(sVn + 8 * (lane % DL));
  }

  // ---- 4. scores and the wave's softmax statistics -------------------------------------
  // lane: head n = lane % 16, slots 16 kb + 4 (lane / 16) + r of the wave
  bf16x8 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qb[ks] = *(const bf16x8*)(sQ + (lane & 15) * D + 32 * ks + 8 * (lane >> 4));
  f32x4 sc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sc[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kb][ks]),
                                                       qb[ks], sc[kb], 0, 0, 0);
  }
  const bool full = pos >= W - 1;
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int slot = 32 * wave + 16 * kb + 4 * (lane >> 4) + r;
      const bool ok = slot < W && (full || slot <= pos);
      sc[kb][r] = ok ? sc[kb][r] : -INFINITY;
      m = fmaxf(m, sc[kb][r]);
    }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float mu = m == -INFINITY ? 0.f : m;   // a wave with no visible slot adds nothing
  float l = 0.f;
  const int n = lane & 15;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = fast_exp2(sc[kb][r] - mu);
      l += pr;
      // P stored per (head, slot group, index within the group) for the P.V lanes
      const int sl = 16 * kb + 4 * (lane >> 4) + r;
      if (n < G) sP[(wave * GM + n) * 32 + (sl % KG) * KPL + sl / KG] = pr;
    }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (lane < 16 && n < G) {
    sML[(wave * GM + n) * 2] = mu;
    sML[(wave * GM + n) * 2 + 1] = l;
  }
  __syncthreads();

  // ---- 5. partial P.V of the wave: lane holds dims 8 (lane % DL) .. + 7, slot group lane / DL
  // Slots the query does not see (past the ring, or not yet written while pos < W - 1)
  // carry P = 0, but their V rows may hold anything (a fresh ring is uninitialised
  // memory): they are zeroed so that 0 * NaN or 0 * inf cannot reach the sum.
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int slot = 32 * wave + lane / DL + KG * i;
    if (!(slot < W && (full || slot <= pos))) va[i] = (u32x4){0u, 0u, 0u, 0u};
  }
  float acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  const int kg = lane / DL;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) break;
    float pv[KPL];
    const float* ph = sP + (wave * GM + h) * 32 + kg * KPL;
#pragma unroll
    for (int i = 0; i < KPL; i += 4) {
      const float4 p4 = *(const float4*)(ph + i);
      pv[i] = p4.x; pv[i + 1] = p4.y; pv[i + 2] = p4.z; pv[i + 3] = p4.w;
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint32_t w4[4] = {va[i].x, va[i].y, va[i].z, va[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[h][2 * e] = __builtin_fmaf(pv[i], bf16_lo_to_f32(w4[e]), acc[h][2 * e]);
        acc[h][2 * e + 1] = __builtin_fmaf(pv[i], bf16_hi_to_f32(w4[e]), acc[h][2 * e + 1]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
#pragma unroll
      for (int o = DL; o < 64; o <<= 1) v += __shfl_xor(v, o);
      acc[h][e] = v;
    }
    if (kg == 0) {
      float* dst = sO + (wave * GM + h) * D + 8 * lane;
      *(float4*)dst = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *(float4*)(dst + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  __syncthreads();

  // ---- 6. merge the four waves, gate, store; then the ring slot -------------------------
#pragma unroll
  for (int i = 0; i < GIT; ++i) {
    const int idx = t + i * kThreads;
    if (idx >= G * D / 2) break;
    const int h = idx / (D / 2), c = 2 * (idx - h * (D / 2));
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (sML[(w * GM + h) * 2 + 1] > 0.f) mx = fmaxf(mx, sML[(w * GM + h) * 2]);
    float o0 = 0.f, o1 = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lw = sML[(w * GM + h) * 2 + 1];
      if (lw > 0.f) {
        const float f = fast_exp2(sML[(w * GM + h) * 2] - mx);
        lt = __builtin_fmaf(lw, f, lt);
        o0 = __builtin_fmaf(sO[(w * GM + h) * D + c], f, o0);
        o1 = __builtin_fmaf(sO[(w * GM + h) * D + c + 1], f, o1);
      }
    }
    const float inv = 1.0f / lt;
    const float nan = __builtin_nanf("");
    const bf16x2 ov = {(bf16)(valid ? o0 * inv * sigmoidf_(bf16_lo_to_f32(gw[i])) : nan),
                       (bf16)(valid ? o1 * inv * sigmoidf_(bf16_hi_to_f32(gw[i])) : nan)};
    *(bf16x2*)(out + h * D + c) = ov;
  }
  // every wave's ring loads were consumed before the last barrier
  if (valid && t < DL) {
    *(u32x4*)(kr + (size_t)sn * D + t * 8) = *(const u32x4*)(sKn + t * 8);
    *(u32x4*)(vr + (size_t)sn * D + t * 8) = *(const u32x4*)(sVn + t * 8);
  }
}
template <int D, int GM>
__global__ __launch_bounds__(kThreads) void swa_decode_mfma_kernel(const DecodeArgs p) {
  swa_decode_mfma_body<D, GM>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y);
}
template <int D, int GM>
__global__ __launch_bounds__(kThreads) void swa_decode_mfma_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z;
  swa_decode_mfma_body<D, GM>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y);
}
__host__ __forceinline__ bool swa_decode_mfma_ok(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  return a.window >= 1 && a.window <= kRingMax && G >= 1 && G <= kMfmaDecodeMaxG &&
         (a.d == 64 || a.d == 128) && a.rdim <= a.d;
}

template <typename K>
hipError_t launch_dyn(K kern, dim3 grid, dim3 block, int smem, hipStream_t s,
                      const DecodeArgs& a) {
  if (smem > 64 * 1024) {
    hipError_t e = ensure_dynamic_smem((const void*)kern, smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, smem, s, a);
  return hipGetLastError();
}

template <int D, typename T = bf16>
hipError_t global_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  hipError_t e = launch_dyn(gdec_prep_kernel<D, T>, dim3(a.Hkv, a.B), dim3(kThreads),
                            2 * (G + 1) * D * 4, s, a);
  if (e != hipSuccess) return e;
  constexpr int NKL = kThreads / (D / 8);
  const int smem_split = max(a.chunk * G * 4, NKL * G * D * 4);
  const dim3 g3(a.nsplit, a.Hkv, a.B);
  switch (G) {
    case 1: e = launch_dyn(gdec_split_kernel<D, 1, T>, g3, dim3(kThreads), smem_split, s, a); break;
    case 2: e = launch_dyn(gdec_split_kernel<D, 2, T>, g3, dim3(kThreads), smem_split, s, a); break;
    case 4: e = launch_dyn(gdec_split_kernel<D, 4, T>, g3, dim3(kThreads), smem_split, s, a); break;
    case 8: e = launch_dyn(gdec_split_kernel<D, 8, T>, g3, dim3(kThreads), smem_split, s, a); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gdec_combine_kernel<D, T>), dim3(a.Hq, a.B), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

void global_decode_geometry(int B, int Hq, int d, int capacity, int* nsplit, int* chunk,
                            size_t* ws_bytes) {
  int c = 2048;
  if (capacity <= 65536) {
    c = (capacity + 31) / 32;
    c = ((c + 63) / 64) * 64;
    if (c < 64) c = 64;
  }
  const int ns = (capacity + c - 1) / c;
  *nsplit = ns;
  *chunk = c;
  *ws_bytes = ((size_t)B * Hq * d * (1 + (size_t)ns) + (size_t)B * Hq * ns * 2) * 4;
}

bool global_decode_geometry_capped(int B, int Hq, int Hkv, int d, int capacity,
                                   size_t max_bytes, int* nsplit, int* chunk,
                                   size_t* ws_bytes) {
  global_decode_geometry(B, Hq, d, capacity, nsplit, chunk, ws_bytes);
  const int G = Hq / Hkv;
  const size_t max_lds = 160 * 1024;   // the split kernel keeps chunk x G scores in LDS
  while (*ws_bytes > max_bytes) {
    if (*nsplit == 1) return false;
    const int c = *chunk * 2;
    if ((size_t)c * G * 4 > max_lds) return false;
    *chunk = c;
    *nsplit = (capacity + c - 1) / c;
    *ws_bytes = ((size_t)B * Hq * d * (1 + (size_t)*nsplit) + (size_t)B * Hq * *nsplit * 2) * 4;
  }
  return true;
}

hipError_t decode_noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t launch_global_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.f32) return a.d == 128 ? global_decode_t<128, float>(a, s) : global_decode_t<64, float>(a, s);
  return a.d == 128 ? global_decode_t<128>(a, s) : global_decode_t<64>(a, s);
}

template <typename K>
hipError_t launch_layers(K kern, dim3 grid, dim3 block, int smem, hipStream_t s,
                         const DecodeBatchArgs& pb) {
  if (smem > 64 * 1024) {
    hipError_t e = ensure_dynamic_smem((const void*)kern, smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, smem, s, pb);
  return hipGetLastError();
}

// Launch of the single-layer (LAYERS false) or batched kernel for the call's head dim and
// head group (at most 4 query heads per KV head take the smaller instance).
template <bool LAYERS, typename A>
hipError_t launch_swa_mfma(dim3 grid, hipStream_t s, const DecodeArgs& a, const A& args) {
  const bool g4 = a.Hq / a.Hkv <= 4;
  auto go = [&](auto kern, int smem) -> hipError_t {
    if constexpr (LAYERS) return launch_layers(kern, grid, dim3(kThreads), smem, s, args);
    else return launch_dyn(kern, grid, dim3(kThreads), smem, s, args);
  };
  if constexpr (LAYERS) {
    if (a.d == 128)
      return g4 ? go(swa_decode_mfma_kernel_layers<128, 4>, SwaDecSmem<128, 4>::kTotal)
                : go(swa_decode_mfma_kernel_layers<128, 8>, SwaDecSmem<128, 8>::kTotal);
    return g4 ? go(swa_decode_mfma_kernel_layers<64, 4>, SwaDecSmem<64, 4>::kTotal)
              : go(swa_decode_mfma_kernel_layers<64, 8>, SwaDecSmem<64, 8>::kTotal);
  } else {
    if (a.d == 128)
      return g4 ? go(swa_decode_mfma_kernel<128, 4>, SwaDecSmem<128, 4>::kTotal)
                : go(swa_decode_mfma_kernel<128, 8>, SwaDecSmem<128, 8>::kTotal);
    return g4 ? go(swa_decode_mfma_kernel<64, 4>, SwaDecSmem<64, 4>::kTotal)
              : go(swa_decode_mfma_kernel<64, 8>, SwaDecSmem<64, 8>::kTotal);
  }
}

hipError_t launch_swa_decode_layers(const DecodeArgs& a, const LayerIO* io, int n, hipStream_t s) {
  if (!swa_decode_mfma_ok(a)) return hipErrorInvalidValue;
  DecodeBatchArgs pb;
  pb.a = a;
  for (int l0 = 0; l0 < n; l0 += kMaxDecodeLayers) {
    const int m = min(kMaxDecodeLayers, n - l0);
    for (int i = 0; i < m; ++i) pb.io[i] = io[l0 + i];
    hipError_t e = launch_swa_mfma<true>(dim3(a.Hkv, a.B, m), s, a, pb);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t global_decode_layers_t(const DecodeArgs& a, const LayerIO* io, int n, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  constexpr int NKL = kThreads / (D / 8);
  const int smem_split = max(a.chunk * G * 4, NKL * G * D * 4);
  DecodeBatchArgs pb;
  pb.a = a;
  for (int l0 = 0; l0 < n; l0 += kMaxDecodeLayers) {
    const int m = min(kMaxDecodeLayers, n - l0);
    for (int i = 0; i < m; ++i) pb.io[i] = io[l0 + i];
    hipError_t e = launch_layers(gdec_prep_kernel_layers<D>, dim3(a.Hkv, a.B, m), dim3(kThreads),
                                 2 * (G + 1) * D * 4, s, pb);
    if (e != hipSuccess) return e;
    const dim3 g3(a.nsplit, a.Hkv, a.B * m);
    switch (G) {
      case 1: e = launch_layers(gdec_split_kernel_layers<D, 1>, g3, dim3(kThreads), smem_split, s, pb); break;
      case 2: e = launch_layers(gdec_split_kernel_layers<D, 2>, g3, dim3(kThreads), smem_split, s, pb); break;
      case 4: e = launch_layers(gdec_split_kernel_layers<D, 4>, g3, dim3(kThreads), smem_split, s, pb); break;
      case 8: e = launch_layers(gdec_split_kernel_layers<D, 8>, g3, dim3(kThreads), smem_split, s, pb); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    e = launch_layers(gdec_combine_kernel_layers<D>, dim3(a.Hq, a.B, m), dim3(D), 0, s, pb);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_global_decode_layers(const DecodeArgs& a, const LayerIO* io, int n,
                                       hipStream_t s) {
  return a.d == 128 ? global_decode_layers_t<128>(a, io, n, s)
                    : global_decode_layers_t<64>(a, io, n, s);
}

hipError_t launch_swa_decode(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int smem = (2 * (G + 1) * a.d + a.d + G * a.window) * 4;
  if (a.f32) {   // fp32: the per-slot kernel for every ring size
    if (a.d == 128)
      return launch_dyn(swa_decode_kernel<128, float>, dim3(a.Hkv, a.B), dim3(kThreads), smem, s, a);
    return launch_dyn(swa_decode_kernel<64, float>, dim3(a.Hkv, a.B), dim3(kThreads), smem, s, a);
  }
  if (swa_decode_mfma_ok(a)) return launch_swa_mfma<false>(dim3(a.Hkv, a.B), s, a, a);
  // rings of more than 128 slots: the per-slot kernel
  if (a.d == 128) return launch_dyn(swa_decode_kernel<128>, dim3(a.Hkv, a.B), dim3(kThreads), smem, s, a);
  return launch_dyn(swa_decode_kernel<64>, dim3(a.Hkv, a.B), dim3(kThreads), smem, s, a);
}

}  // namespace zg
