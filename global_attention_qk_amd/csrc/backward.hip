// Backward pass of both layer kinds (bf16, head_dim 64 or 128).
//
// The layer (hyper.ai summary of arXiv 2609.13356, section 方法, GatedSWA equation; the
// "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ) is
//   q~ = RoPE(RMSNorm(q) * w_q), k~ likewise, s = scale * q~ . k~ over the visible keys,
//   A = softmax(s) V, O = A * sigmoid(G) (SWA) or O = A (global),
// and the pages train it end to end (explainer, training sections) without printing a
// backward formula: these kernels compute the gradient of that forward.
//
// With P = softmax(s) and dA = dO * sigmoid(G):
//   dV = P^T dA,  dP = dA V^T,  dS = P * (dP - D) with D_i = sum_c dA_ic A_ic = sum_c dO_ic O_ic
//   (the gate cancels), dq~ = scale dS k~, dk~ = scale dS^T q~, dG = dO * O * (1 - sigmoid(G)),
// then the RMSNorm + RoPE Jacobians take dq~ / dk~ back to dq / dk and the norm weights.
//
// Launch sequence (one stream): Q~ and K~ (the forward's transform, into the workspace),
// prep (dA, D, dG), dQ (per query tile: a pass for the row log-sum-exp, then S, dP, dS and
// dQ~ += dS K~ on MFMA), dK/dV (per key tile: S, dP, dS, dV^T += dA^T P, dK~^T += Q~^T dS on
// MFMA, keys on the lanes so that P and dS are B operands as they come out of the
// accumulators), the norm/RoPE backward for q and k rows with per-block weight partials,
// and the reduction of those partials.
#include "launch.h"

namespace zg {
namespace {

constexpr int kT = 256;         // threads per workgroup (4 waves)
constexpr int kKB = 64;         // keys per tile (dQ) / per workgroup (dK, dV)
constexpr int kQB = 64;         // queries per tile (dK, dV)
constexpr int kRowsDQ = 128;    // query rows per dQ workgroup (4 waves x 32)
constexpr int kNormRows = 64;   // rows per norm/RoPE backward workgroup

// Swap bits 2 and 3 of an index within its 16-group: the order in which a lane-half holds
// rows of a 32x32 accumulator (rows 8 (r/4) + 4 hi + r%4), used as the k-slot order of the
// operand that multiplies an accumulator taken as a B operand.
__device__ __forceinline__ int slot_row(int s) {
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int j) {
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)x[8 * j + e];
  return o;
}

struct BArgs {
  const bf16* k;      // raw inputs
  const bf16* v;
  const bf16* g;      // gate pre-activation (SWA) or nullptr
  const bf16* out;    // forward output O
  const bf16* dout;
  const bf16* qt;     // Q~ [B][Hq][T][D] (workspace)
  const bf16* kt;     // K~ [B][Hkv][T][D] (workspace)
  bf16* da;           // dA [B][T][Hq][D] (workspace; dout itself for the global layer)
  float* dsum;        // D [B][Hq][T]
  float* lse;         // row log-sum-exp, log2 units [B][Hq][T]
  float* dqt;         // dq~ [B][T][Hq][D] fp32
  float* dkt;         // dk~ [B][T][Hkv][D] fp32
  bf16* dv;           // dV [B][T][Hkv][D]
  bf16* dg;           // dG [B][T][Hq][D] or nullptr
  int B, T, Hq, Hkv, window, group;
  float qscale;       // softmax scale * log2(e)
  float scale;        // softmax scale
};

// ---- prep: dA = dO sigmoid(G), D = sum dO O, dG = dO O (1 - sigmoid(G)) ---------------
template <int D>
__global__ __launch_bounds__(kT) void bwd_prep_kernel(const BArgs p) {
  constexpr int CPR = D / 8;                    // 8-element chunks per row
  const int64_t n_rows = (int64_t)p.B * p.T * p.Hq;
  const int64_t c = (int64_t)blockIdx.x * kT + threadIdx.x;
  const int64_t row = c / CPR;
  const int ch = (int)(c % CPR);
  float dot = 0.f;
  if (row < n_rows) {
    const size_t off = (size_t)row * D + ch * 8;
    const u32x4 dw = *(const u32x4*)(p.dout + off);
    const u32x4 ow = *(const u32x4*)(p.out + off);
    const uint32_t d4[4] = {dw.x, dw.y, dw.z, dw.w}, o4[4] = {ow.x, ow.y, ow.z, ow.w};
    float dox[8], ox[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dox[2 * e] = bf16_lo_to_f32(d4[e]);
      dox[2 * e + 1] = bf16_hi_to_f32(d4[e]);
      ox[2 * e] = bf16_lo_to_f32(o4[e]);
      ox[2 * e + 1] = bf16_hi_to_f32(o4[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(dox[e], ox[e], dot);
    if (p.g) {
      const u32x4 gw = *(const u32x4*)(p.g + off);
      const uint32_t g4[4] = {gw.x, gw.y, gw.z, gw.w};
      bf16x8 da, dg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = (e & 1) ? bf16_hi_to_f32(g4[e >> 1]) : bf16_lo_to_f32(g4[e >> 1]);
        const float sg = sigmoidf_(gv);
        da[e] = (bf16)(dox[e] * sg);
        dg[e] = (bf16)(dox[e] * ox[e] * (1.0f - sg));
      }
      *(bf16x8*)(p.da + off) = da;
      *(bf16x8*)(p.dg + off) = dg;
    }
  }
  // the CPR lanes of a row are adjacent: reduce over them
#pragma unroll
  for (int o = 1; o < CPR; o <<= 1) dot += __shfl_xor(dot, o);
  if (row < n_rows && ch == 0) {
    const int h = (int)(row % p.Hq);
    const int64_t bt = row / p.Hq;
    const int t = (int)(bt % p.T), b = (int)(bt / p.T);
    p.dsum[((size_t)b * p.Hq + h) * p.T + t] = dot;
  }
}

// ---- dQ: one workgroup per (batch, KV head, 128 query rows of the group's heads) --------
template <int D, bool SWA>
__global__ __launch_bounds__(kT) void bwd_dq_kernel(const BArgs p) {
  constexpr int KS = D / 16;             // k-steps over d
  constexpr int DB = D / 32;             // 32-row d blocks
  constexpr int RW = D + 8;              // padded row (elements)
  constexpr int TW = kKB + 8;            // padded transposed row (elements)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* sK = (bf16*)smem;                        // [64][RW] K~ rows
  bf16* sV = sK + kKB * RW;                      // [64][RW] V rows
  bf16* sKT = sV + kKB * RW;                     // [D][TW] K~^T, keys in slot order

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int G = p.group, bmp = kRowsDQ / G, T = p.T;
  const int n_qt = (T + bmp - 1) / bmp;
  const int qt = blockIdx.x % n_qt;
  const int hb = blockIdx.x / n_qt;
  const int b = hb / p.Hkv, kvh = hb % p.Hkv;
  const int i0 = qt * bmp;
  const int row = wave * 32 + l32;                // this lane's query row in the tile
  const int hg = row / bmp, pi = row % bmp;
  const int h = kvh * G + hg;
  const int qpos = i0 + pi;
  const bool qvalid = qpos < T;
  const int qc = min(qpos, T - 1);

  // Q~ and dA of this lane's query as B operands (k = d)
  bf16x8 qreg[KS], dreg[KS];
  {
    const bf16* qrow = p.qt + (((size_t)b * p.Hq + h) * T + qc) * D;
    const bf16* drow = p.da + (((size_t)b * T + qc) * p.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = *(const bf16x8*)(qrow + ks * 16 + hi * 8);
      dreg[ks] = *(const bf16x8*)(drow + ks * 16 + hi * 8);
    }
  }
  const float drow_sum = p.dsum[((size_t)b * p.Hq + h) * T + qc];

  const int q_last = min(i0 + bmp, T) - 1;
  const int k_lo = SWA ? max(0, i0 - p.window + 1) : 0;
  const int kt_lo = k_lo / kKB, kt_hi = q_last / kKB;
  const bf16* kbase = p.kt + ((size_t)b * p.Hkv + kvh) * T * D;
  const bf16* vbase = p.v + ((size_t)b * T * p.Hkv + kvh) * D;

  auto stage = [&](int kt, bool with_v) {
    const int k0 = kt * kKB;
    for (int c = tid; c < kKB * (D / 8); c += kT) {
      const int r = c / (D / 8), dc = c % (D / 8);
      const int key = min(k0 + r, T - 1);
      *(u32x4*)(sK + r * RW + dc * 8) = *(const u32x4*)(kbase + (size_t)key * D + dc * 8);
      if (with_v)
        *(u32x4*)(sV + r * RW + dc * 8) =
            *(const u32x4*)(vbase + (size_t)key * p.Hkv * D + dc * 8);
    }
    __syncthreads();
    if (with_v) {
      for (int c = tid; c < D * kKB; c += kT) {
        const int dd = c / kKB, s = c % kKB;
        sKT[dd * TW + s] = sK[slot_row(s) * RW + dd];
      }
      __syncthreads();
    }
  };
  auto visible = [&](int key) {
    return qvalid && key <= qpos && (!SWA || key > qpos - p.window);
  };
  auto scores = [&](int kb, f32x16& acc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mfma32(*(const bf16x8*)(sK + (kb * 32 + l32) * RW + ks * 16 + hi * 8), qreg[ks], acc);
  };

  // pass 1: row log-sum-exp (log2 units), online over the key tiles
  float m = -INFINITY, l = 0.f;
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    stage(kt, false);
    const int k0 = kt * kKB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s;
      scores(kb, s);
      float tm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = visible(key) ? s[r] * p.qscale : -INFINITY;
        tm = fmaxf(tm, s[r]);
      }
      const float mn = fmaxf(m, tm);
      if (mn != -INFINITY) {
        float add = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) add += fast_exp2(s[r] - mn);
        l = l * fast_exp2(m - mn) + add;
        m = mn;
      }
    }
    __syncthreads();
  }
  {
    const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
    const float ma = fmaxf(m, mo);
    const float la = (m == -INFINITY ? 0.f : l * fast_exp2(m - ma)) +
                     (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - ma));
    m = ma == -INFINITY ? 0.f : ma + __log2f(la);   // m now holds the row's log2 LSE
  }
  const float lse2 = m;

  // pass 2: P, dP, dS and dQ~^T += K~^T dS^T
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    stage(kt, true);
    const int k0 = kt * kKB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
      scores(kb, s);
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        dp = mfma32(*(const bf16x8*)(sV + (kb * 32 + l32) * RW + ks * 16 + hi * 8), dreg[ks], dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float pr = visible(key) ? fast_exp2(s[r] * p.qscale - lse2) : 0.f;
        s[r] = pr * (dp[r] - drow_sum);               // dS^T
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 bo = pack8(s, j);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(*(const bf16x8*)(sKT + (db * 32 + l32) * TW + kb * 32 + 16 * j + hi * 8),
                           bo, acc[db]);
      }
    }
    __syncthreads();
  }
  if (qvalid) {
    float* dst = p.dqt + (((size_t)b * T + qpos) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = acc[db][4 * r4] * p.scale;
        v.y = acc[db][4 * r4 + 1] * p.scale;
        v.z = acc[db][4 * r4 + 2] * p.scale;
        v.w = acc[db][4 * r4 + 3] * p.scale;
        *(float4*)(dst + db * 32 + 8 * r4 + 4 * hi) = v;
      }
    if (hi == 0) p.lse[((size_t)b * p.Hq + h) * T + qpos] = lse2;
  }
}

// ---- dK, dV: one workgroup per (batch, KV head, 64 keys) --------------------------------
template <int D, bool SWA>
__global__ __launch_bounds__(kT) void bwd_dkdv_kernel(const BArgs p) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RW = D + 8;
  constexpr int TW = kQB + 8;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* sQ = (bf16*)smem;                  // [64][RW] Q~ rows
  bf16* sA = sQ + kQB * RW;                // [64][RW] dA rows
  bf16* sQT = sA + kQB * RW;               // [D][TW] Q~^T, queries in slot order
  bf16* sAT = sQT + D * TW;                // [D][TW] dA^T
  float* sL = (float*)(sAT + D * TW);      // [64] log2 LSE
  float* sD = sL + kQB;                    // [64] D

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int kb = wave & 1, qh = wave >> 1;
  const int T = p.T, G = p.group;
  const int n_kt = (T + kKB - 1) / kKB;
  const int kt = blockIdx.x % n_kt;
  const int hb = blockIdx.x / n_kt;
  const int b = hb / p.Hkv, kvh = hb % p.Hkv;
  const int k0 = kt * kKB;
  const int key = k0 + kb * 32 + l32;      // this lane's key (column of S, dP)
  const int kc = min(key, T - 1);

  bf16x8 kreg[KS], vreg[KS];
  {
    const bf16* krow = p.kt + (((size_t)b * p.Hkv + kvh) * T + kc) * D;
    const bf16* vrow = p.v + (((size_t)b * T + kc) * p.Hkv + kvh) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = *(const bf16x8*)(krow + ks * 16 + hi * 8);
      vreg[ks] = *(const bf16x8*)(vrow + ks * 16 + hi * 8);
    }
  }
  f32x16 dvt[DB], dkt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvt[db][r] = 0.f;
      dkt[db][r] = 0.f;
    }

  const int k_last = min(k0 + kKB, T) - 1;
  const int q_hi = SWA ? min(T - 1, k_last + p.window - 1) : T - 1;
  const int qt_lo = k0 / kQB, qt_hi = q_hi / kQB;
  for (int hg = 0; hg < G; ++hg) {
    const int h = kvh * G + hg;
    const bf16* qbase = p.qt + ((size_t)b * p.Hq + h) * T * D;
    const bf16* abase = p.da + ((size_t)b * T * p.Hq + h) * D;
    for (int qt = qt_lo; qt <= qt_hi; ++qt) {
      const int i0 = qt * kQB;
      for (int c = tid; c < kQB * (D / 8); c += kT) {
        const int r = c / (D / 8), dc = c % (D / 8);
        const int qi = min(i0 + r, T - 1);
        *(u32x4*)(sQ + r * RW + dc * 8) = *(const u32x4*)(qbase + (size_t)qi * D + dc * 8);
        *(u32x4*)(sA + r * RW + dc * 8) =
            *(const u32x4*)(abase + (size_t)qi * p.Hq * D + dc * 8);
      }
      if (tid < kQB) {
        const int qi = min(i0 + tid, T - 1);
        sL[tid] = p.lse[((size_t)b * p.Hq + h) * T + qi];
        sD[tid] = p.dsum[((size_t)b * p.Hq + h) * T + qi];
      }
      __syncthreads();
      for (int c = tid; c < D * kQB; c += kT) {
        const int dd = c / kQB, s = c % kQB;
        sQT[dd * TW + s] = sQ[slot_row(s) * RW + dd];
        sAT[dd * TW + s] = sA[slot_row(s) * RW + dd];
      }
      __syncthreads();
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(*(const bf16x8*)(sQ + (qh * 32 + l32) * RW + ks * 16 + hi * 8), kreg[ks], s);
        dp = mfma32(*(const bf16x8*)(sA + (qh * 32 + l32) * RW + ks * 16 + hi * 8), vreg[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = qh * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int qi = i0 + qr;
        const bool vis = key < T && qi < T && key <= qi && (!SWA || key > qi - p.window);
        const float pr = vis ? fast_exp2(s[r] * p.qscale - sL[qr]) : 0.f;
        s[r] = pr;
        dp[r] = pr * (dp[r] - sD[qr]);              // dS
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 pp = pack8(s, j), dd = pack8(dp, j);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = (db * 32 + l32) * TW + qh * 32 + 16 * j + hi * 8;
          dvt[db] = mfma32(*(const bf16x8*)(sAT + off), pp, dvt[db]);
          dkt[db] = mfma32(*(const bf16x8*)(sQT + off), dd, dkt[db]);
        }
      }
      __syncthreads();
    }
  }
  // the two query halves of each key block: qh 1 hands its sums to qh 0 through LDS
  float* red = (float*)smem;               // [2 kb][DB][2][16][64]
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[(((kb * DB + db) * 2 + 0) * 16 + r) * 64 + lane] = dvt[db][r];
        red[(((kb * DB + db) * 2 + 1) * 16 + r) * 64 + lane] = dkt[db][r];
      }
  }
  __syncthreads();
  if (qh == 0 && key < T) {
    bf16* vdst = p.dv + (((size_t)b * T + key) * p.Hkv + kvh) * D;
    float* kdst = p.dkt + (((size_t)b * T + key) * p.Hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float vv[4], kk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          vv[e] = dvt[db][r] + red[(((kb * DB + db) * 2 + 0) * 16 + r) * 64 + lane];
          kk[e] = (dkt[db][r] + red[(((kb * DB + db) * 2 + 1) * 16 + r) * 64 + lane]) * p.scale;
        }
        const int d0 = db * 32 + 8 * r4 + 4 * hi;
        *(bf16x4*)(vdst + d0) = (bf16x4){(bf16)vv[0], (bf16)vv[1], (bf16)vv[2], (bf16)vv[3]};
        *(float4*)(kdst + d0) = make_float4(kk[0], kk[1], kk[2], kk[3]);
      }
  }
}

// ---- norm/RoPE backward: dx~ -> dx and per-block weight partials ------------------------
struct NArgs {
  const bf16* x;       // raw q or k [B][T][H][D]
  const float* w;
  const float* dxt;    // dx~ [B][T][H][D] fp32
  bf16* dx;            // [B][T][H][D]
  float* part;         // [n_blocks][D] sum over the block's rows of u * x^
  int B, T, H, rdim, pos_offset;
  float eps;
  RopeFreq fr;
};

template <int D>
__global__ __launch_bounds__(kNormRows) void bwd_norm_rope_kernel(const NArgs p) {
  constexpr int RS = D + 1;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* xs = (float*)smem;                 // [rows][RS]
  float* us = xs + kNormRows * RS;          // [rows][RS]
  const int t = threadIdx.x;
  const int64_t n_rows = (int64_t)p.B * p.T * p.H;
  const int64_t r0 = (int64_t)blockIdx.x * kNormRows;
  for (int c = t; c < kNormRows * D; c += kNormRows) {
    const int rr = c / D, cc = c % D;
    const int64_t row = r0 + rr;
    xs[rr * RS + cc] = row < n_rows ? (float)p.x[row * D + cc] : 0.f;
    us[rr * RS + cc] = row < n_rows ? p.dxt[row * D + cc] : 0.f;
  }
  __syncthreads();
  {
    const int64_t row = r0 + t;
    float* x = xs + t * RS;
    float* u = us + t * RS;
    if (row < n_rows) {
      const int pos = p.pos_offset + (int)((row / p.H) % p.T);
      float ss = 0.f;
      for (int c = 0; c < D; ++c) ss = __builtin_fmaf(x[c], x[c], ss);
      const float rn = 1.0f / sqrtf(ss / D + p.eps);
      // u = R^T dx~ (rotate each pair back)
      const int half = p.rdim >> 1;
      for (int j = 0; j < half; ++j) {
        float cs, sn;
        rope_cos_sin(pos, p.fr.hi[j], p.fr.lo[j], cs, sn);
        const float ga = u[j], gb = u[j + half];
        u[j] = ga * cs + gb * sn;
        u[j + half] = gb * cs - ga * sn;
      }
      float dot = 0.f;
      for (int c = 0; c < D; ++c) {
        const float xh = x[c] * rn;
        const float dxh = u[c] * p.w[c];
        dot = __builtin_fmaf(dxh, xh, dot);
        u[c] = u[c] * xh;                  // weight-gradient contribution of this row
        x[c] = dxh;                        // keep dx^ (x^ is recomputed below)
      }
      dot *= 1.0f / D;
      for (int c = 0; c < D; ++c) {
        const float xh = (float)p.x[row * D + c] * rn;
        x[c] = rn * (x[c] - xh * dot);     // dx
      }
    } else {
      for (int c = 0; c < D; ++c) {
        x[c] = 0.f;
        u[c] = 0.f;
      }
    }
  }
  __syncthreads();
  for (int c = t; c < kNormRows * D; c += kNormRows) {
    const int rr = c / D, cc = c % D;
    const int64_t row = r0 + rr;
    if (row < n_rows) p.dx[row * D + cc] = (bf16)xs[rr * RS + cc];
  }
  for (int c = t; c < D; c += kNormRows) {
    float s = 0.f;
    for (int rr = 0; rr < kNormRows; ++rr) s += us[rr * RS + c];
    p.part[(size_t)blockIdx.x * D + c] = s;
  }
}

template <int D>
__global__ __launch_bounds__(D) void bwd_dw_reduce_kernel(const float* part, int n, float* dw) {
  const int c = threadIdx.x;
  float s = 0.f;
  for (int i = 0; i < n; ++i) s += part[(size_t)i * D + c];
  dw[c] = s;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qt, kt, da, dsum, lse, dqt, dkt, part, total;
  int nq_blk, nk_blk;
};

WsLayout ws_layout(int B, int T, int Hq, int Hkv, int d) {
  WsLayout L;
  size_t o = 0;
  const size_t nq = (size_t)B * T * Hq, nk = (size_t)B * T * Hkv;
  L.qt = o;   o += align256(nq * d * 2);
  L.kt = o;   o += align256(nk * d * 2);
  L.da = o;   o += align256(nq * d * 2);
  L.dsum = o; o += align256(nq * 4);
  L.lse = o;  o += align256(nq * 4);
  L.dqt = o;  o += align256(nq * d * 4);
  L.dkt = o;  o += align256(nk * d * 4);
  L.nq_blk = (int)((nq + kNormRows - 1) / kNormRows);
  L.nk_blk = (int)((nk + kNormRows - 1) / kNormRows);
  L.part = o; o += align256((size_t)(L.nq_blk + L.nk_blk) * d * 4);
  L.total = o;
  return L;
}

template <typename K, typename A>
hipError_t launch_big(K kern, dim3 grid, dim3 block, int smem, hipStream_t s, const A& a) {
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, smem, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t backward_t(const BackwardArgs& a, hipStream_t s) {
  const WsLayout L = ws_layout(a.B, a.T, a.Hq, a.Hkv, D);
  char* ws = (char*)a.ws;
  // Q~ [B][Hq][T][D] and K~ [B][Hkv][T][D], as the forward's operands
  NormRopeArgs n;
  n.pos = nullptr;
  n.B = a.B;
  n.T = a.T;
  n.d = D;
  n.rdim = a.rdim;
  n.pos_offset = a.pos_offset;
  n.is_bf16 = 1;
  n.eps = a.eps;
  n.out_scale = 1.0f;
  n.fr = a.fr;
  n.x = a.q;
  n.w = a.wq;
  n.y = ws + L.qt;
  n.H = a.Hq;
  n.ysb = (int64_t)a.Hq * a.T * D;
  n.yst = D;
  n.ysh = (int64_t)a.T * D;
  hipError_t e = launch_qknorm_rope(n, s);
  if (e != hipSuccess) return e;
  n.x = a.k;
  n.w = a.wk;
  n.y = ws + L.kt;
  n.H = a.Hkv;
  n.ysb = (int64_t)a.Hkv * a.T * D;
  n.ysh = (int64_t)a.T * D;
  e = launch_qknorm_rope(n, s);
  if (e != hipSuccess) return e;

  BArgs p;
  p.k = (const bf16*)a.k;
  p.v = (const bf16*)a.v;
  p.g = (const bf16*)a.g;
  p.out = (const bf16*)a.out;
  p.dout = (const bf16*)a.dout;
  p.qt = (const bf16*)(ws + L.qt);
  p.kt = (const bf16*)(ws + L.kt);
  p.da = a.g ? (bf16*)(ws + L.da) : (bf16*)a.dout;
  p.dsum = (float*)(ws + L.dsum);
  p.lse = (float*)(ws + L.lse);
  p.dqt = (float*)(ws + L.dqt);
  p.dkt = (float*)(ws + L.dkt);
  p.dv = (bf16*)a.dv;
  p.dg = (bf16*)a.dg;
  p.B = a.B;
  p.T = a.T;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.window = a.window;
  p.group = a.Hq / a.Hkv;
  p.scale = a.scale;
  p.qscale = a.scale * 1.4426950408889634f;

  const int64_t prep_threads = (int64_t)a.B * a.T * a.Hq * (D / 8);
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((prep_threads + kT - 1) / kT)),
                     dim3(kT), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int bmp = kRowsDQ / p.group;
  const int n_qt = (a.T + bmp - 1) / bmp;
  const int dq_smem = (2 * kKB * (D + 8) + D * (kKB + 8)) * 2;
  const dim3 gq((unsigned)(n_qt * a.B * a.Hkv));
  e = a.swa ? launch_big(bwd_dq_kernel<D, true>, gq, dim3(kT), dq_smem, s, p)
            : launch_big(bwd_dq_kernel<D, false>, gq, dim3(kT), dq_smem, s, p);
  if (e != hipSuccess) return e;

  const int n_kt = (a.T + kKB - 1) / kKB;
  const int stage = (2 * kQB * (D + 8) + 2 * D * (kQB + 8)) * 2 + 2 * kQB * 4;
  const int red = 2 * (D / 32) * 2 * 16 * 64 * 4;
  const int kv_smem = stage > red ? stage : red;
  const dim3 gk((unsigned)(n_kt * a.B * a.Hkv));
  e = a.swa ? launch_big(bwd_dkdv_kernel<D, true>, gk, dim3(kT), kv_smem, s, p)
            : launch_big(bwd_dkdv_kernel<D, false>, gk, dim3(kT), kv_smem, s, p);
  if (e != hipSuccess) return e;

  NArgs nb;
  nb.B = a.B;
  nb.T = a.T;
  nb.rdim = a.rdim;
  nb.pos_offset = a.pos_offset;
  nb.eps = a.eps;
  nb.fr = a.fr;
  const int nsm = 2 * kNormRows * (D + 1) * 4;
  float* part = (float*)(ws + L.part);
  nb.x = (const bf16*)a.q;
  nb.w = a.wq;
  nb.dxt = p.dqt;
  nb.dx = (bf16*)a.dq;
  nb.part = part;
  nb.H = a.Hq;
  e = launch_big(bwd_norm_rope_kernel<D>, dim3(L.nq_blk), dim3(kNormRows), nsm, s, nb);
  if (e != hipSuccess) return e;
  nb.x = (const bf16*)a.k;
  nb.w = a.wk;
  nb.dxt = p.dkt;
  nb.dx = (bf16*)a.dk;
  nb.part = part + (size_t)L.nq_blk * D;
  nb.H = a.Hkv;
  e = launch_big(bwd_norm_rope_kernel<D>, dim3(L.nk_blk), dim3(kNormRows), nsm, s, nb);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dw_reduce_kernel<D>, dim3(1), dim3(D), 0, s, (const float*)part,
                     L.nq_blk, a.dwq);
  hipLaunchKernelGGL(bwd_dw_reduce_kernel<D>, dim3(1), dim3(D), 0, s,
                     (const float*)(part + (size_t)L.nq_blk * D), L.nk_blk, a.dwk);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int B, int T, int Hq, int Hkv, int d) {
  return ws_layout(B, T, Hq, Hkv, d).total;
}

hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t s) {
  return a.d == 128 ? backward_t<128>(a, s) : backward_t<64>(a, s);
}

}  // namespace zg
