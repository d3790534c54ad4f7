// bf16 prefill attention on gfx950 MFMA: gated sliding-window and full-causal GQA.
//
// What is computed (hyper.ai summary of arXiv 2609.13356, section 方法, GatedSWA
// equation; "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ): for every query row,
// RMSNorm + partial RoPE on q and k, softmax(scale * q~ . k~) over the visible keys
// (the last `window` tokens including the query for SWA, the whole prefix for global),
// times V, then the elementwise sigmoid gate for SWA.
//
// Work decomposition (one workgroup = 4 wave64s = 256 query rows):
//   * The rows are all g = Hq/Hkv query heads of one KV head at 256/g consecutive
//     positions, so every K/V tile staged in LDS serves the whole head group.
//   * Each wave owns two 32-row query blocks. Scores are formed transposed,
//     S^T = K~ . Q~^T with v_mfma_f32_32x32x16_bf16 (keys on the M side, queries on N),
//     which leaves one query per lane; the probabilities then already sit in the
//     B-operand layout of O^T += V^T . P^T, so no cross-lane shuffle is needed between
//     the two products and the softmax row statistics are per-lane scalars.
//   * V is transposed into LDS with the keys of each 16-key group permuted so that a
//     lane's eight keys are one 16-byte LDS read.
//   * Q~ is pre-multiplied by scale * log2(e) so that p = exp2(s - m).
//   * The running max is only raised when a tile's max exceeds it by more than 8
//     (factor 256); the result is unchanged (the same m divides out), rescales get rare.
//   * K~: for global layers a separate pass writes normalised+rotated K once into a
//     workspace that the tiles read directly; for SWA layers (each K tile visited by
//     about three query tiles) the transform is fused into the tile load.
#include "launch.h"

namespace zg {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 256;     // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kMaxHalfMfma = 32;  // rotary_dim <= 64 on this path

template <int D>
struct Smem {
  static constexpr int kRowB = D * 2 + 16;           // padded bf16 row (bytes)
  static constexpr int kVtRowB = kBN * 2 + 16;       // padded V^T row (bytes)
  // Phase 1 (Q): raw Q rows, transformed in place; then copied to registers.
  static constexpr int kQ = kRows * kRowB;
  // Main loop: K~ tile, V^T tile, raw K tile (fused), K trig table.
  static constexpr int kK = kBN * kRowB;
  static constexpr int kVt = D * kVtRowB;
  static constexpr int kKraw = kBN * kRowB;
  static constexpr int kKtrig = kBN * kMaxHalfMfma * 8;
  static constexpr int kLoop = kK + kVt + kKraw + kKtrig;
  // Q trig table: up to 256 positions x 32 pairs.
  static constexpr int kQtrig = kRows * kMaxHalfMfma * 8;
  static constexpr int kW = 2 * D * 4;  // wq, wk
  static constexpr int kUnion = (kQ + kQtrig) > kLoop ? (kQ + kQtrig) : kLoop;
  static constexpr int kTotal = kUnion + kW;
};

struct KArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* g;
  bf16* out;
  const float* wq;
  const float* wk;
  const bf16* kt;
  int T, Hq, Hkv, window, rdim, pos_offset;
  int group, bmp, n_qtiles, n_hb;
  float eps, qscale;
  RopeFreq fr;
};

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Swap bits 2 and 3 of a key index within its 16-key group: keys {0-3, 8-11} then
// {4-7, 12-15}, matching which keys a lane holds in the S^T accumulator.
__device__ __forceinline__ int vt_slot(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// In-LDS RMSNorm + partial RoPE of one bf16 row (raw -> dst may alias for the
// thread-owns-the-row case). `tpr` threads cooperate on a row (sub = 0..tpr-1): each
// covers a slice of the pairs and of the pass-through chunks; `rn` is the row's
// 1/rms. The result is multiplied by `oscale` and rounded to bf16.
template <int D>
__device__ __forceinline__ void transform_row(const bf16* raw, bf16* dst, const float* w,
                                              const float2* trig, float rn, float oscale,
                                              int rdim, int sub, int tpr) {
  const int half = rdim >> 1;
  for (int j = sub; j < half; j += tpr) {
    const float a = (float)raw[j] * w[j] * rn;
    const float b = (float)raw[j + half] * w[j + half] * rn;
    const float2 cs = trig[j];
    dst[j] = (bf16)((a * cs.x - b * cs.y) * oscale);
    dst[j + half] = (bf16)((b * cs.x + a * cs.y) * oscale);
  }
  // pass-through dims [rdim, D) in 8-element chunks; the chunk holding rdim is done
  // element-wise so that rotated dims written above are not overwritten.
  const int c0 = rdim >> 3;
  for (int c = c0 + sub; c < D / 8; c += tpr) {
    const u32x4 rv = *(const u32x4*)(raw + c * 8);
    float x[8];
    x[0] = bf16_lo_to_f32(rv.x); x[1] = bf16_hi_to_f32(rv.x);
    x[2] = bf16_lo_to_f32(rv.y); x[3] = bf16_hi_to_f32(rv.y);
    x[4] = bf16_lo_to_f32(rv.z); x[5] = bf16_hi_to_f32(rv.z);
    x[6] = bf16_lo_to_f32(rv.w); x[7] = bf16_hi_to_f32(rv.w);
    if (c * 8 >= rdim) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)(x[e] * w[c * 8 + e] * rn * oscale);
      *(bf16x8*)(dst + c * 8) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c * 8 + e >= rdim) dst[c * 8 + e] = (bf16)(x[e] * w[c * 8 + e] * rn * oscale);
    }
  }
}

template <int D, bool SWA, bool KPRE>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(const KArgs p) {
  using S = Smem<D>;
  constexpr int KS = D / 16;   // k-steps of the QK^T product
  constexpr int DB = D / 32;   // 32-wide d blocks of O
  constexpr int RW = S::kRowB / 2;      // padded row length in bf16 elements
  constexpr int VW = S::kVtRowB / 2;

  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* sQ = (bf16*)smem;
  float2* sQtrig = (float2*)(smem + S::kQ);
  bf16* sK = (bf16*)smem;
  bf16* sVt = (bf16*)(smem + S::kK);
  bf16* sKraw = (bf16*)(smem + S::kK + S::kVt);
  float2* sKtrig = (float2*)(smem + S::kK + S::kVt + S::kKraw);
  float* sWq = (float*)(smem + S::kUnion);
  float* sWk = sWq + D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Heavy query tiles first (global layers); consecutive workgroups cover different
  // (batch, kv-head) pairs so that one pair's tiles share an XCD's L2.
  const int lin = blockIdx.x;
  const int hb = lin % p.n_hb;
  const int tile_rank = lin / p.n_hb;
  const int qt = SWA ? tile_rank : (p.n_qtiles - 1 - tile_rank);
  const int b = hb / p.Hkv;
  const int kvh = hb % p.Hkv;
  const int i0 = qt * p.bmp;
  const int T = p.T;
  const int half = p.rdim >> 1;
  const int bpp = p.bmp >> 5;  // 32-row blocks per head in the tile

  for (int i = tid; i < D; i += kThreads) {
    sWq[i] = p.wq[i];
    sWk[i] = p.wk[i];
  }

  // ---- Phase 1: Q tile -> LDS (coalesced), trig table for its positions -------------
  {
    const int g = p.group;
    const int chunks_per_pos = g * (D / 8);
    const int n_chunks = p.bmp * chunks_per_pos;
    const bf16* qbase = p.q + ((size_t)b * T * p.Hq + (size_t)kvh * g) * D;
    for (int c = tid; c < n_chunks; c += kThreads) {
      const int pi = c / chunks_per_pos;
      const int rem = c - pi * chunks_per_pos;
      const int hg = rem / (D / 8);
      const int dc = rem - hg * (D / 8);
      const int pos = i0 + pi;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (pos < T) val = *(const u32x4*)(qbase + (size_t)pos * p.Hq * D + hg * D + dc * 8);
      *(u32x4*)(sQ + (hg * p.bmp + pi) * RW + dc * 8) = val;
    }
    for (int e = tid; e < p.bmp * half; e += kThreads) {
      const int pi = e / half, j = e - pi * half;
      float c, s;
      rope_cos_sin(p.pos_offset + i0 + pi, p.fr.hi[j], p.fr.lo[j], c, s);
      sQtrig[pi * kMaxHalfMfma + j] = make_float2(c, s);
    }
  }
  __syncthreads();
  // Thread-per-row RMSNorm + RoPE + scale, in place.
  {
    const int row = tid;
    const int pi = row % p.bmp;
    bf16* r = sQ + row * RW;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 v = *(const u32x4*)(r + c * 8);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_lo_to_f32(w4[e]), bb = bf16_hi_to_f32(w4[e]);
        ss = __builtin_fmaf(a, a, ss);
        ss = __builtin_fmaf(bb, bb, ss);
      }
    }
    const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
    transform_row<D>(r, r, sWq, sQtrig + pi * kMaxHalfMfma, rn, p.qscale, p.rdim, 0, 1);
  }
  __syncthreads();
  // Q~ into registers as the B operand: lane holds query row l32 of its block and the
  // eight d values 16*ks + 8*hi .. +7 for each k-step.
  bf16x8 qreg[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = (wave * 2 + qb) * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[qb][ks] = *(const bf16x8*)(sQ + row * RW + ks * 16 + hi * 8);
  }
  // Absolute positions of this lane's two query rows (for masking).
  int qpos[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int blk = wave * 2 + qb;
    qpos[qb] = i0 + (blk % bpp) * 32 + l32;
  }
  __syncthreads();  // Q region is reused by the K/V tiles below

  // ---- Key-tile range -----------------------------------------------------------------
  const int q_last = min(i0 + p.bmp, T) - 1;   // last valid query position of the tile
  int kt_lo = 0;
  if (SWA) kt_lo = max(0, i0 - p.window + 1) / kBN;
  const int kt_hi = q_last / kBN;              // inclusive

  f32x16 oacc[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const bf16* kbase = p.k + ((size_t)b * T * p.Hkv + kvh) * D;
  const bf16* vbase = p.v + ((size_t)b * T * p.Hkv + kvh) * D;
  const size_t kvstride = (size_t)p.Hkv * D;

  // Tiles from the diagonal backwards: every row sees itself in the first tile it meets
  // when bmp <= kBN, and the -inf guard below covers the other shapes.
  for (int kt = kt_hi; kt >= kt_lo; --kt) {
    const int k0 = kt * kBN;
    // -- K tile --
    if (KPRE) {
      const bf16* src = p.kt + (((size_t)b * p.Hkv + kvh) * T) * D;
#pragma unroll
      for (int it = 0; it < (kBN * D / 8) / kThreads; ++it) {
        const int c = tid + it * kThreads;
        const int kr = c / (D / 8), dc = c % (D / 8);
        const int pos = k0 + kr;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (pos < T) val = *(const u32x4*)(src + (size_t)pos * D + dc * 8);
        *(u32x4*)(sK + kr * RW + dc * 8) = val;
      }
    } else {
#pragma unroll
      for (int it = 0; it < (kBN * D / 8) / kThreads; ++it) {
        const int c = tid + it * kThreads;
        const int kr = c / (D / 8), dc = c % (D / 8);
        const int pos = k0 + kr;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (pos < T) val = *(const u32x4*)(kbase + (size_t)pos * kvstride + dc * 8);
        *(u32x4*)(sKraw + kr * RW + dc * 8) = val;
      }
      for (int e = tid; e < kBN * half; e += kThreads) {
        const int kr = e / half, j = e - kr * half;
        float c, s;
        rope_cos_sin(p.pos_offset + k0 + kr, p.fr.hi[j], p.fr.lo[j], c, s);
        sKtrig[kr * kMaxHalfMfma + j] = make_float2(c, s);
      }
    }
    // -- V tile, transposed: thread loads 4 keys x 8 dims and writes 8 rows of 4 keys --
    {
      constexpr int DC = D / 8;  // 8-dim chunks per row
      for (int c = tid; c < (kBN / 4) * DC; c += kThreads) {
        const int kg = c / DC;       // group of 4 keys
        const int dc = c % DC;
        u32x4 vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = k0 + kg * 4 + e;
          vv[e] = (u32x4){0u, 0u, 0u, 0u};
          if (pos < T) vv[e] = *(const u32x4*)(vbase + (size_t)pos * kvstride + dc * 8);
        }
        const int slot = vt_slot(kg * 4);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          // element dd of each key's chunk
          const int wsel = dd >> 1;
          const bool hiw = dd & 1;
          const uint32_t e0 = vv[0][wsel], e1 = vv[1][wsel];
          const uint32_t e2 = vv[2][wsel], e3 = vv[3][wsel];
          uint32_t lo01, lo23;
          if (hiw) {
            lo01 = (e0 >> 16) | (e1 & 0xffff0000u);
            lo23 = (e2 >> 16) | (e3 & 0xffff0000u);
          } else {
            lo01 = (e0 & 0xffffu) | (e1 << 16);
            lo23 = (e2 & 0xffffu) | (e3 << 16);
          }
          *(u32x2*)(sVt + (dc * 8 + dd) * VW + slot) = (u32x2){lo01, lo23};
        }
      }
    }
    __syncthreads();
    if (!KPRE) {
      // Fused K transform: 4 threads per key row.
      const int kr = tid >> 2, sub = tid & 3;
      const bf16* r = sKraw + kr * RW;
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 v = *(const u32x4*)(r + (sub * (D / 32) + c) * 8);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16_lo_to_f32(w4[e]), bb = bf16_hi_to_f32(w4[e]);
          ss = __builtin_fmaf(a, a, ss);
          ss = __builtin_fmaf(bb, bb, ss);
        }
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
      transform_row<D>(r, sK + kr * RW, sWk, sKtrig + kr * kMaxHalfMfma, rn, 1.0f, p.rdim,
                       sub, 4);
      __syncthreads();
    }

    // -- S^T = K~ Q~^T for both query blocks and both 32-key blocks --
    f32x16 sacc[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *(const bf16x8*)(sK + (kb * 32 + l32) * RW + ks * 16 + hi * 8);
        sacc[0][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[0][ks], sacc[0][kb], 0, 0, 0);
        sacc[1][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[1][ks], sacc[1][kb], 0, 0, 0);
      }
    }

    // -- mask, online softmax, P to bf16 --
    const bool need_mask = (k0 + kBN - 1 > i0) || (SWA && k0 <= q_last - p.window) ||
                           (k0 + kBN > T);
    bf16x8 pb[2][2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (need_mask) {
        const int qi = qpos[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = k0 + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            bool vis = kj <= qi;
            if (SWA) vis = vis && (kj > qi - p.window);
            if (!vis) sacc[qb][kb][r] = -INFINITY;
          }
      }
      float mt = sacc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[qb][kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_old = m_run[qb];
      const bool raise = mt > m_old + 8.0f;
      if (__ballot(raise)) {
        const float m_new = raise ? mt : m_old;
        const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        m_run[qb] = m_new;
      }
      const float mu = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int jh = 0; jh < 2; ++jh) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pe = fast_exp2(sacc[qb][kb][jh * 8 + e] - mu);
            ls += pe;
            v[e] = (bf16)pe;
          }
          pb[qb][kb][jh] = v;
        }
      }
      l_run[qb] += ls;
    }

    // -- O^T += V^T P^T --
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int jh = 0; jh < 2; ++jh) {
          const bf16x8 a = *(const bf16x8*)(sVt + (db * 32 + l32) * VW + kb * 32 + jh * 16 + hi * 8);
          oacc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[0][kb][jh], oacc[0][db], 0, 0, 0);
          oacc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[1][kb][jh], oacc[1][db], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next tile overwrites sK / sVt
  }

  // ---- Epilogue: O = acc / l (* sigmoid(G)), bf16 store ------------------------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const int pos = qpos[qb];
    if (pos >= T) continue;
    const float inv = 1.0f / lt;
    const int blk = wave * 2 + qb;
    const int hg = blk / bpp;
    const int h = kvh * p.group + hg;
    const size_t rowoff = (((size_t)b * T + pos) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int d0 = db * 32 + t4 * 8 + hi * 4;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = oacc[qb][db][t4 * 4 + e] * inv;
        if (SWA) {
          const u32x2 gw = *(const u32x2*)(p.g + rowoff + d0);
          o[0] *= sigmoidf_(bf16_lo_to_f32(gw.x));
          o[1] *= sigmoidf_(bf16_hi_to_f32(gw.x));
          o[2] *= sigmoidf_(bf16_lo_to_f32(gw.y));
          o[3] *= sigmoidf_(bf16_hi_to_f32(gw.y));
        }
        bf16x4 ov = {(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
        *(bf16x4*)(p.out + rowoff + d0) = ov;
      }
    }
  }
}

template <int D, bool SWA, bool KPRE>
hipError_t launch_t(const KArgs& ka, int n_blocks, hipStream_t s) {
  constexpr int smem = Smem<D>::kTotal;
  auto kern = prefill_bf16_kernel<D, SWA, KPRE>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(n_blocks), dim3(kThreads), smem, s, ka);
  return hipGetLastError();
}

}  // namespace

bool prefill_bf16_supported(int d, int group, int rdim) {
  if (d != 64 && d != 128) return false;
  if (group < 1 || kRows % group != 0 || (kRows / group) % 32 != 0) return false;
  if (rdim > 2 * kMaxHalfMfma) return false;
  return true;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  KArgs ka;
  ka.q = (const bf16*)a.q;
  ka.k = (const bf16*)a.k;
  ka.v = (const bf16*)a.v;
  ka.g = (const bf16*)a.g;
  ka.out = (bf16*)a.out;
  ka.wq = a.wq;
  ka.wk = a.wk;
  ka.kt = a.kt;
  ka.T = a.T;
  ka.Hq = a.Hq;
  ka.Hkv = a.Hkv;
  ka.window = a.window;
  ka.rdim = a.rdim;
  ka.pos_offset = a.pos_offset;
  ka.group = a.Hq / a.Hkv;
  ka.bmp = kRows / ka.group;
  ka.n_qtiles = (a.T + ka.bmp - 1) / ka.bmp;
  ka.n_hb = a.B * a.Hkv;
  ka.eps = a.eps;
  ka.qscale = a.scale * 1.4426950408889634f;
  ka.fr = a.fr;
  const int n_blocks = ka.n_qtiles * ka.n_hb;
  if (n_blocks == 0) return hipSuccess;
  const bool kpre = (a.kt != nullptr);
  if (a.d == 128) {
    if (a.swa) return launch_t<128, true, false>(ka, n_blocks, s);
    return kpre ? launch_t<128, false, true>(ka, n_blocks, s)
                : launch_t<128, false, false>(ka, n_blocks, s);
  }
  if (a.swa) return launch_t<64, true, false>(ka, n_blocks, s);
  return kpre ? launch_t<64, false, true>(ka, n_blocks, s)
              : launch_t<64, false, false>(ka, n_blocks, s);
}

}  // namespace zg
