// Single-token decode for both layer kinds (bf16 caches).
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
// (staged in LDS when it holds at most 128 slots).
#include "launch.h"

namespace zg {
namespace {

constexpr int kThreads = 256;

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
template <int D>
__device__ __forceinline__ void gdec_prep_kernel_body(const DecodeArgs& p, const LayerIO& io, int kvh, int b) {
  const int G = p.Hq / p.Hkv;
  const int pos = p.pos[b];
  if (!pos_valid(pos, p.S)) return;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* buf = (float*)smem;                 // (G + 1) rows
  float* tmp = buf + (G + 1) * D;
  const int t = threadIdx.x;
  const bf16* q = (const bf16*)io.q + ((size_t)b * p.Hq + kvh * G) * D;
  const bf16* kn = (const bf16*)io.k_new + ((size_t)b * p.Hkv + kvh) * D;
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
  const bf16* vn = (const bf16*)io.v_new + ((size_t)b * p.Hkv + kvh) * D;
  for (int c = t; c < D; c += kThreads) {
    ((bf16*)io.k_cache)[crow + c] = (bf16)buf[G * D + c];
    ((bf16*)io.v_cache)[crow + c] = vn[c];
  }
}
template <int D>
__global__ __launch_bounds__(kThreads) void gdec_prep_kernel(const DecodeArgs p) {
  gdec_prep_kernel_body<D>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y);
}
template <int D>
__global__ __launch_bounds__(kThreads) void gdec_prep_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z;
  gdec_prep_kernel_body<D>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y);
}

// ---------------------------------------------------------------------------------------
// Global decode, step 2: one split of the cache.
// ---------------------------------------------------------------------------------------
template <int D, int G>
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
  const bf16* kc = (const bf16*)io.k_cache + cbase;
  const bf16* vc = (const bf16*)io.v_cache + cbase;

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
    const u32x4 raw = *(const u32x4*)(vc + (size_t)kl * D + dc * 8);
    float v[8];
    v[0] = bf16_lo_to_f32(raw.x); v[1] = bf16_hi_to_f32(raw.x);
    v[2] = bf16_lo_to_f32(raw.y); v[3] = bf16_hi_to_f32(raw.y);
    v[4] = bf16_lo_to_f32(raw.z); v[5] = bf16_hi_to_f32(raw.z);
    v[6] = bf16_lo_to_f32(raw.w); v[7] = bf16_hi_to_f32(raw.w);
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
template <int D, int G>
__global__ __launch_bounds__(kThreads) void gdec_split_kernel(const DecodeArgs p) {
  gdec_split_kernel_body<D, G>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z);
}
template <int D, int G>
__global__ __launch_bounds__(kThreads) void gdec_split_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z / pb.a.B;
  gdec_split_kernel_body<D, G>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z % pb.a.B);
}

// ---------------------------------------------------------------------------------------
// Global decode, step 3: log-sum-exp merge of the splits.
// ---------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void gdec_combine_kernel_body(const DecodeArgs& p, const LayerIO& io, int h, int b) {
  const int d = threadIdx.x;
  const int pos = p.pos[b];
  bf16* out = (bf16*)io.out + ((size_t)b * p.Hq + h) * D;
  if (!pos_valid(pos, p.S)) {
    out[d] = (bf16)__builtin_nanf("");
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
  out[d] = (bf16)(o / L);
}
template <int D>
__global__ __launch_bounds__(D) void gdec_combine_kernel(const DecodeArgs p) {
  gdec_combine_kernel_body<D>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y);
}
template <int D>
__global__ __launch_bounds__(D) void gdec_combine_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z;
  gdec_combine_kernel_body<D>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y);
}

// ---------------------------------------------------------------------------------------
// SWA decode over the ring: one workgroup per (kv head, sequence).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void swa_decode_kernel(const DecodeArgs p) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = p.Hq / p.Hkv;
  const int W = p.window;
  const int pos = p.pos[b];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  bf16* out = (bf16*)p.out + ((size_t)b * p.Hq + kvh * G) * D;
  if (!pos_valid(pos, ZGATTN_POS_LIMIT)) {
    for (int i = t; i < G * D; i += kThreads) out[i] = (bf16)__builtin_nanf("");
    return;
  }
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* buf = (float*)smem;        // G q rows + k_new row
  float* tmp = buf + (G + 1) * D;
  float* sv = tmp + (G + 1) * D;    // v_new
  float* sS = sv + D;               // [G][W]
  const bf16* q = (const bf16*)p.q + ((size_t)b * p.Hq + kvh * G) * D;
  const bf16* kn = (const bf16*)p.k_new + ((size_t)b * p.Hkv + kvh) * D;
  const bf16* vn = (const bf16*)p.v_new + ((size_t)b * p.Hkv + kvh) * D;
  for (int i = t; i < (G + 1) * D; i += kThreads)
    buf[i] = i < G * D ? (float)q[i] : (float)kn[i - G * D];
  for (int c = t; c < D; c += kThreads) sv[c] = (float)vn[c];
  const float* wrow[9];
  for (int r = 0; r < 9; ++r) wrow[r] = r < G ? p.wq : p.wk;
  __syncthreads();
  norm_rope_rows_lds<D>(buf, wrow, G + 1, pos, p.rdim, p.eps, p.fr, tmp);
  const float qs = p.scale * 1.4426950408889634f;
  const int slot = pos % W;
  bf16* kr = (bf16*)p.k_cache + ((size_t)b * p.Hkv + kvh) * W * D;
  bf16* vr = (bf16*)p.v_cache + ((size_t)b * p.Hkv + kvh) * W * D;
  // the new key as the cache will hold it (bf16); the ring slot itself is written last
  for (int c = t; c < D; c += kThreads) buf[G * D + c] = (float)(bf16)buf[G * D + c];
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
  const bf16* g = (const bf16*)p.g + ((size_t)b * p.Hq + kvh * G) * D;
  for (int idx = t; idx < G * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    const int ns = pos >= W - 1 ? W : pos + 1;
    float o = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float vv = s == slot ? sv[c] : (float)vr[(size_t)s * D + c];
      o = __builtin_fmaf(sS[h * W + s], vv, o);
    }
    o *= sigmoidf_((float)g[idx]);
    out[idx] = (bf16)o;
  }
  __syncthreads();
  for (int c = t; c < D; c += kThreads) {
    kr[(size_t)slot * D + c] = (bf16)buf[G * D + c];
    vr[(size_t)slot * D + c] = (bf16)sv[c];
  }
}

// Ring of at most 128 slots (the model's window): the whole ring is staged in LDS with
// 16-byte loads issued together (one memory round trip instead of one per slot), and the
// scores, softmax and P.V run from LDS. The 16-byte chunks of a K row are XOR-swizzled by
// the row index so that the 64 lanes of a wave, one slot each, read distinct banks while
// the ring stays unpadded (two workgroups fit a CU's LDS).
constexpr int kRingMax = 128;

template <int D>
__device__ __forceinline__ void swa_decode_ring_kernel_body(const DecodeArgs& p, const LayerIO& io, int kvh, int b) {
  constexpr int KRB = D * 2;                       // K row (bytes)
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  // byte offset of chunk ch of K row s
  auto kpos = [](int s, int ch) { return s * KRB + ((ch ^ (s & (CPR - 1))) << 4); };
  constexpr int RIT = kRingMax * CPR / kThreads;   // chunks per thread per ring tensor
  const int G = p.Hq / p.Hkv;
  const int W = p.window;
  const int pos = p.pos[b];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  bf16* out = (bf16*)io.out + ((size_t)b * p.Hq + kvh * G) * D;
  if (!pos_valid(pos, ZGATTN_POS_LIMIT)) {
    for (int i = t; i < G * D; i += kThreads) out[i] = (bf16)__builtin_nanf("");
    return;
  }
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sK = smem;                                  // [W][KRB], swizzled chunks
  bf16* sV = (bf16*)(smem + kRingMax * KRB);        // [W][D]
  float* buf = (float*)(smem + kRingMax * KRB + kRingMax * D * 2);   // G q rows + k_new
  float* tmp = buf + (G + 1) * D;
  float* sv = tmp + (G + 1) * D;                    // v_new
  float* sS = sv + D;                               // [G][W]
  bf16* kr = (bf16*)io.k_cache + ((size_t)b * p.Hkv + kvh) * W * D;
  bf16* vr = (bf16*)io.v_cache + ((size_t)b * p.Hkv + kvh) * W * D;
  // ring -> registers (all loads in flight together), then the new token's rows
  const int nch = W * CPR;
  u32x4 kc[RIT], vc[RIT];
#pragma unroll
  for (int it = 0; it < RIT; ++it) {
    const int c = t + it * kThreads;
    if (c < nch) {
      kc[it] = *(const u32x4*)(kr + (size_t)c * 8);
      vc[it] = *(const u32x4*)(vr + (size_t)c * 8);
    }
  }
  const bf16* q = (const bf16*)io.q + ((size_t)b * p.Hq + kvh * G) * D;
  const bf16* kn = (const bf16*)io.k_new + ((size_t)b * p.Hkv + kvh) * D;
  const bf16* vn = (const bf16*)io.v_new + ((size_t)b * p.Hkv + kvh) * D;
  for (int i = t; i < (G + 1) * D; i += kThreads)
    buf[i] = i < G * D ? (float)q[i] : (float)kn[i - G * D];
  for (int c = t; c < D; c += kThreads) sv[c] = (float)vn[c];
  const float* wrow[9];
  for (int r = 0; r < 9; ++r) wrow[r] = r < G ? io.wq : io.wk;
  __syncthreads();
  norm_rope_rows_lds<D>(buf, wrow, G + 1, pos, p.rdim, p.eps, p.fr, tmp);
  const int slot = pos % W;
#pragma unroll
  for (int it = 0; it < RIT; ++it) {
    const int c = t + it * kThreads;
    if (c < nch) {
      const int row = c / CPR, ch = c % CPR;
      *(u32x4*)(sK + kpos(row, ch)) = kc[it];
      *(u32x4*)(sV + (size_t)c * 8) = vc[it];
    }
  }
  __syncthreads();
  // the new entry as the ring will hold it (bf16), over the slot's old contents
  for (int c = t; c < D; c += kThreads) {
    const bf16 kb = (bf16)buf[G * D + c];
    buf[G * D + c] = (float)kb;
    *(bf16*)(sK + kpos(slot, c >> 3) + (c & 7) * 2) = kb;
    sV[slot * D + c] = (bf16)sv[c];
  }
  __syncthreads();
  // scores: one (head, slot) per thread and pass; four partial sums per dot product
  const float qs = p.scale * 1.4426950408889634f;
  for (int idx = t; idx < G * W; idx += kThreads) {
    const int h = idx / W, s = idx - h * W;
    float d = -INFINITY;
    if (pos >= W - 1 || s <= pos) {
      const float* qh = buf + h * D;
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int ch = 0; ch < CPR; ++ch) {
        const u32x4 raw = *(const u32x4*)(sK + kpos(s, ch));
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a4[e] = __builtin_fmaf(qh[ch * 8 + 2 * e], bf16_lo_to_f32(w4[e]), a4[e]);
          a4[e] = __builtin_fmaf(qh[ch * 8 + 2 * e + 1], bf16_hi_to_f32(w4[e]), a4[e]);
        }
      }
      d = ((a4[0] + a4[1]) + (a4[2] + a4[3])) * qs;
    }
    sS[idx] = d;
  }
  __syncthreads();
  for (int h = wave; h < G; h += kThreads / 64) {
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
  // P.V: two adjacent dims of one head per thread and pass
  const bf16* g = (const bf16*)io.g + ((size_t)b * p.Hq + kvh * G) * D;
  const int ns = pos >= W - 1 ? W : pos + 1;
  for (int idx = t; idx < G * D / 2; idx += kThreads) {
    const int h = idx / (D / 2), c = 2 * (idx - h * (D / 2));
    const float* ph = sS + h * W;
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    int s = 0;
    for (; s + 1 < ns; s += 2) {
      const uint32_t v0 = *(const uint32_t*)(sV + s * D + c);
      const uint32_t v1 = *(const uint32_t*)(sV + (s + 1) * D + c);
      o0 = __builtin_fmaf(ph[s], bf16_lo_to_f32(v0), o0);
      o1 = __builtin_fmaf(ph[s], bf16_hi_to_f32(v0), o1);
      o2 = __builtin_fmaf(ph[s + 1], bf16_lo_to_f32(v1), o2);
      o3 = __builtin_fmaf(ph[s + 1], bf16_hi_to_f32(v1), o3);
    }
    if (s < ns) {
      const uint32_t v0 = *(const uint32_t*)(sV + s * D + c);
      o0 = __builtin_fmaf(ph[s], bf16_lo_to_f32(v0), o0);
      o1 = __builtin_fmaf(ph[s], bf16_hi_to_f32(v0), o1);
    }
    const uint32_t gw = *(const uint32_t*)(g + h * D + c);
    const bf16x2 ov = {(bf16)((o0 + o2) * sigmoidf_(bf16_lo_to_f32(gw))),
                       (bf16)((o1 + o3) * sigmoidf_(bf16_hi_to_f32(gw)))};
    *(bf16x2*)(out + h * D + c) = ov;
  }
  // the ring slot last (every read of the old ring came from the staged copy)
  for (int c = t; c < D; c += kThreads) {
    kr[(size_t)slot * D + c] = (bf16)buf[G * D + c];
    vr[(size_t)slot * D + c] = (bf16)sv[c];
  }
}
template <int D>
__global__ __launch_bounds__(kThreads) void swa_decode_ring_kernel(const DecodeArgs p) {
  swa_decode_ring_kernel_body<D>(p, layer_io(p), (int)blockIdx.x, (int)blockIdx.y);
}
template <int D>
__global__ __launch_bounds__(kThreads) void swa_decode_ring_kernel_layers(const DecodeBatchArgs pb) {
  const int layer = blockIdx.z;
  swa_decode_ring_kernel_body<D>(pb.a, pb.io[layer], (int)blockIdx.x, (int)blockIdx.y);
}

template <typename K>
hipError_t launch_dyn(K kern, dim3 grid, dim3 block, int smem, hipStream_t s,
                      const DecodeArgs& a) {
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, smem, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t global_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  hipError_t e = launch_dyn(gdec_prep_kernel<D>, dim3(a.Hkv, a.B), dim3(kThreads),
                            2 * (G + 1) * D * 4, s, a);
  if (e != hipSuccess) return e;
  constexpr int NKL = kThreads / (D / 8);
  const int smem_split = max(a.chunk * G * 4, NKL * G * D * 4);
  const dim3 g3(a.nsplit, a.Hkv, a.B);
  switch (G) {
    case 1: e = launch_dyn(gdec_split_kernel<D, 1>, g3, dim3(kThreads), smem_split, s, a); break;
    case 2: e = launch_dyn(gdec_split_kernel<D, 2>, g3, dim3(kThreads), smem_split, s, a); break;
    case 4: e = launch_dyn(gdec_split_kernel<D, 4>, g3, dim3(kThreads), smem_split, s, a); break;
    case 8: e = launch_dyn(gdec_split_kernel<D, 8>, g3, dim3(kThreads), smem_split, s, a); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdec_combine_kernel<D>, dim3(a.Hq, a.B), dim3(D), 0, s, a);
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

hipError_t launch_global_decode(const DecodeArgs& a, hipStream_t s) {
  return a.d == 128 ? global_decode_t<128>(a, s) : global_decode_t<64>(a, s);
}

template <typename K>
hipError_t launch_layers(K kern, dim3 grid, dim3 block, int smem, hipStream_t s,
                         const DecodeBatchArgs& pb) {
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, smem, s, pb);
  return hipGetLastError();
}

hipError_t launch_swa_decode_layers(const DecodeArgs& a, const LayerIO* io, int n, hipStream_t s) {
  if (a.window > kRingMax) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  const int smem = 2 * kRingMax * a.d * 2 +
                   (2 * (G + 1) * a.d + a.d + G * a.window) * 4;
  DecodeBatchArgs pb;
  pb.a = a;
  for (int l0 = 0; l0 < n; l0 += kMaxDecodeLayers) {
    const int m = min(kMaxDecodeLayers, n - l0);
    for (int i = 0; i < m; ++i) pb.io[i] = io[l0 + i];
    const dim3 grid(a.Hkv, a.B, m);
    hipError_t e = a.d == 128
        ? launch_layers(swa_decode_ring_kernel_layers<128>, grid, dim3(kThreads), smem, s, pb)
        : launch_layers(swa_decode_ring_kernel_layers<64>, grid, dim3(kThreads), smem, s, pb);
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
  if (a.window <= kRingMax) {
    const int ring = 2 * kRingMax * a.d * 2;
    if (a.d == 128)
      return launch_dyn(swa_decode_ring_kernel<128>, dim3(a.Hkv, a.B), dim3(kThreads),
                        ring + smem, s, a);
    return launch_dyn(swa_decode_ring_kernel<64>, dim3(a.Hkv, a.B), dim3(kThreads), ring + smem,
                      s, a);
  }
  if (a.d == 128) return launch_dyn(swa_decode_kernel<128>, dim3(a.Hkv, a.B), dim3(kThreads), smem, s, a);
  return launch_dyn(swa_decode_kernel<64>, dim3(a.Hkv, a.B), dim3(kThreads), smem, s, a);
}

}  // namespace zg
