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
constexpr int kRowsDQ = 256;    // query rows per dQ workgroup (8 waves x 32)
constexpr int kTDQ = 512;       // its threads

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
  const bf16* ktT;    // K~^T tiles [B][Hkv][n64][D][64], keys in slot order (workspace)
  const bf16* qtT;    // Q~^T tiles [B][Hq][n64][D][64]
  const bf16* daT;    // dA^T tiles [B][Hq][n64][D][64]
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

// ---- transposed 64-position tiles --------------------------------------------------------
// src row (b, h, pos) at src + b * sb + h * sh + pos * sp (elements); dst tile
// ((b * H + h) * n_tiles + tile) is [D][64] with column s holding position 64 tile +
// slot_row(s) (positions past T are zero).
template <int D>
__global__ __launch_bounds__(kT) void bwd_tiles_kernel(const bf16* src, int64_t sb, int64_t sh,
                                                       int64_t sp, int H, int T, int n_tiles,
                                                       bf16* dst) {
  __shared__ __attribute__((aligned(16))) bf16 t[64][D + 8];
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const bf16* base = src + b * sb + h * sh;
  for (int c = threadIdx.x; c < 64 * (D / 8); c += kT) {
    const int r = c / (D / 8), dc = c % (D / 8);
    const int pos = tile * 64 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (pos < T) val = *(const u32x4*)(base + pos * sp + dc * 8);
    *(u32x4*)&t[r][dc * 8] = val;
  }
  __syncthreads();
  bf16* out = dst + ((size_t)bh * n_tiles + tile) * (64 * D);
  for (int c = threadIdx.x; c < D * 8; c += kT) {
    const int d = c / 8, sc = c % 8;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = t[slot_row(sc * 8 + e)][d];
    *(bf16x8*)(out + d * 64 + sc * 8) = o;
  }
}

// ---- dQ: one workgroup per (batch, KV head, 256 query rows of the group's heads) --------
// LDS tiles are unpadded and filled by LDS DMA, their 16-byte chunks XOR-swizzled as in
// the forward kernel (chunk_pos): a key-tile buffer holds K~ rows [64][D], V rows [64][D]
// and K~^T [D][64]; tiles are fetched kDQAhead tiles ahead into kDQAhead + 1 buffers.
constexpr int kDQAhead = 2;

template <int D, bool SWA>
__global__ __launch_bounds__(kTDQ) void bwd_dq_kernel(const BArgs p) {
  constexpr int KS = D / 16;             // k-steps over d
  constexpr int DB = D / 32;             // 32-row d blocks
  constexpr int RB = D * 2;              // row bytes
  constexpr int TILE = kKB * RB;         // bytes of one [64][D] (or [D][64]) tile
  constexpr int BUF = 3 * TILE;
  constexpr int NB = kDQAhead + 1;
  constexpr int KPW = D / 64;            // 1 KiB DMA blocks per wave per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int G = p.group, bmp = kRowsDQ / G, T = p.T;
  const int n_qt = (T + bmp - 1) / bmp;
  const int n_kt = (T + kKB - 1) / kKB;
  const int qt = blockIdx.x % n_qt;
  const int hb = blockIdx.x / n_qt;
  const int b = hb / p.Hkv, kvh = hb % p.Hkv;
  const int i0 = qt * bmp;
  const int row = wave * 32 + l32;
  const int hg = row / bmp, pi = row % bmp;
  const int h = kvh * G + hg;
  const int qpos = i0 + pi;
  const bool qvalid = qpos < T;
  const int qc = min(qpos, T - 1);

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
  const int n_tiles = kt_hi - kt_lo + 1;
  const bf16* kbase = p.kt + ((size_t)b * p.Hkv + kvh) * T * D;
  const bf16* vbase = p.v + ((size_t)b * T * p.Hkv + kvh) * D;
  const bf16* tbase = p.ktT + ((size_t)b * p.Hkv + kvh) * n_kt * (size_t)(kKB * D);

  // DMA piece j of tile kt (with_v: K rows, V rows, K^T; else K rows only)
  auto dma = [&](int kt, int buf, bool with_v) {
    const uint32_t dst = lds0 + buf * BUF;
    const int k0 = kt * kKB;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      constexpr int CPR = D / 8, RPB = 1024 / RB;
      const int blk = wave * KPW + j;
      const int r = blk * RPB + lane / CPR;
      const int c = chunk_pos<CPR>(r, lane % CPR);
      const int rr = min(r, T - 1 - k0);
      dma16(kbase + (size_t)k0 * D, (uint32_t)(rr * RB + c * 16), dst + blk * 1024);
      if (with_v)
        dma16(vbase + (size_t)k0 * p.Hkv * D, (uint32_t)(rr * p.Hkv * RB + c * 16),
              dst + TILE + blk * 1024);
    }
    if (with_v) {
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const int blk = wave * KPW + j;
        const int d = blk * 8 + (lane >> 3);
        const int c = chunk_pos<8>(d, lane & 7);
        dma16(tbase + (size_t)kt * (kKB * D), (uint32_t)(d * 128 + c * 16),
              dst + 2 * TILE + blk * 1024);
      }
    }
  };
  // per-lane operand offsets within a buffer (row swizzle depends on l32 & 15 only)
  int roff[KS], toff[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = l32 * RB + chunk_pos<D / 8>(l32, 2 * ks + hi) * 16;
#pragma unroll
  for (int x = 0; x < 4; ++x) toff[x] = 2 * TILE + l32 * 128 + chunk_pos<8>(l32, 2 * x + hi) * 16;

  auto visible = [&](int key) {
    return qvalid && key <= qpos && (!SWA || key > qpos - p.window);
  };
  auto run = [&](bool second, auto&& body) {
    const int nd = second ? 3 * KPW : KPW;   // DMA instructions per wave per tile
#pragma unroll
    for (int a = 0; a < kDQAhead; ++a) dma(kt_lo + min(a, n_tiles - 1), a, second);
    if (second) vm_wait<(kDQAhead - 1) * 3 * KPW>(); else vm_wait<(kDQAhead - 1) * KPW>();
    __syncthreads();
    int cur = 0;
    for (int i = 0; i < n_tiles; ++i) {
      const int ahead = (cur + kDQAhead) % NB;
      dma(kt_lo + min(i + kDQAhead, n_tiles - 1), ahead, second);
      body(kt_lo + i, smem + cur * BUF);
      if (second) vm_wait<(kDQAhead - 1) * 3 * KPW>(); else vm_wait<(kDQAhead - 1) * KPW>();
      __syncthreads();
      cur = cur == NB - 1 ? 0 : cur + 1;
    }
    vm_wait<0>();
    __syncthreads();
    (void)nd;
  };
  auto scores = [&](const char* tb, int kb, f32x16& acc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mfma32(*(const bf16x8*)(tb + roff[ks] + kb * 32 * RB), qreg[ks], acc);
  };

  // pass 1: row log-sum-exp (log2 units)
  float m = -INFINITY, l = 0.f;
  run(false, [&](int kt, const char* tb) {
    const int k0 = kt * kKB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s;
      scores(tb, kb, s);
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
  });
  {
    const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
    const float ma = fmaxf(m, mo);
    const float la = (m == -INFINITY ? 0.f : l * fast_exp2(m - ma)) +
                     (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - ma));
    m = ma == -INFINITY ? 0.f : ma + __log2f(la);
  }
  const float lse2 = m;

  // pass 2: P, dP, dS and dQ~^T += K~^T dS^T
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  run(true, [&](int kt, const char* tb) {
    const int k0 = kt * kKB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
      scores(tb, kb, s);
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        dp = mfma32(*(const bf16x8*)(tb + TILE + roff[ks] + kb * 32 * RB), dreg[ks], dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float pr = visible(key) ? fast_exp2(s[r] * p.qscale - lse2) : 0.f;
        s[r] = pr * (dp[r] - drow_sum);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 bo = pack8(s, j);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(*(const bf16x8*)(tb + toff[2 * kb + j] + db * 32 * 128), bo, acc[db]);
      }
    }
  });
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

// ---- dK, dV: one workgroup per (batch, KV head, 128 keys) -------------------------------
// Eight waves: wave w owns keys 32 (w % 4) .. of the workgroup and half of the head dims
// (w / 4) of their dK / dV. Every query tile streamed through LDS (Q~ rows, dA rows,
// Q~^T and dA^T tiles, unpadded and swizzled, fetched by LDS DMA one tile ahead, and the
// tile's log-sum-exp and D) thus serves 128 keys; the two waves of a key block both form
// S and dP (over all head dims), which costs a third more MFMA work than splitting the
// queries but halves the bytes streamed per key, the bound of this kernel.
constexpr int kKV = 128;           // keys per dK/dV workgroup
constexpr int kTKV = 512;          // its threads

template <int D, bool SWA>
__global__ __launch_bounds__(kTKV) void bwd_dkdv_kernel(const BArgs p) {
  constexpr int KS = D / 16;
  constexpr int DBH = D / 64;              // 32-row d blocks per wave (half the dims)
  constexpr int RB = D * 2;
  constexpr int TILE = kQB * RB;
  constexpr int BUF = 4 * TILE + 2 * kQB * 4;
  constexpr int DPW = TILE / 1024 / 8;     // DMA blocks per wave per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int kb = wave & 3, dh = wave >> 2;
  const int T = p.T, G = p.group;
  const int n64 = (T + 63) / 64;
  const int nkt = (T + kKV - 1) / kKV;
  const int kt = blockIdx.x % nkt;
  const int hb = blockIdx.x / nkt;
  const int b = hb / p.Hkv, kvh = hb % p.Hkv;
  const int k0 = kt * kKV;
  const int key = k0 + kb * 32 + l32;
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
  f32x16 dvt[DBH], dkt[DBH];
#pragma unroll
  for (int db = 0; db < DBH; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvt[db][r] = 0.f;
      dkt[db][r] = 0.f;
    }

  const int k_last = min(k0 + kKV, T) - 1;
  const int q_hi = SWA ? min(T - 1, k_last + p.window - 1) : T - 1;
  const int qt_lo = k0 / kQB, qt_hi = q_hi / kQB;
  const int n_q = qt_hi - qt_lo + 1;
  const int n_it = G * n_q;             // (head of the group, query tile) steps

  int roff[KS], toff[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = l32 * RB + chunk_pos<D / 8>(l32, 2 * ks + hi) * 16;
#pragma unroll
  for (int x = 0; x < 4; ++x) toff[x] = l32 * 128 + chunk_pos<8>(l32, 2 * x + hi) * 16;

  // step `it` into buffer `buf`: DMA of the four tiles; the row statistics go through
  // registers (lsr, dsr), written into the buffer by put_stats at the end of the step
  float lsr = 0.f, dsr = 0.f;
  auto fetch = [&](int it, int buf) {
    const int hg = it / n_q, qt = qt_lo + it % n_q;
    const int h = kvh * G + hg, i0 = qt * kQB;
    const uint32_t dst = lds0 + buf * BUF;
    const bf16* qbase = p.qt + (((size_t)b * p.Hq + h) * T + i0) * D;
    const bf16* abase = p.da + (((size_t)b * T + i0) * p.Hq + h) * D;
    const size_t tb = (((size_t)b * p.Hq + h) * n64 + qt) * (size_t)(kQB * D);
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      constexpr int CPR = D / 8, RPB = 1024 / RB;
      const int blk = wave * DPW + j;
      const int r = blk * RPB + lane / CPR;
      const int c = chunk_pos<CPR>(r, lane % CPR);
      const int rr = min(r, T - 1 - i0);
      dma16(qbase, (uint32_t)(rr * RB + c * 16), dst + blk * 1024);
      dma16(abase, (uint32_t)(rr * p.Hq * RB + c * 16), dst + TILE + blk * 1024);
      const int d = blk * 8 + (lane >> 3);
      const int c8 = chunk_pos<8>(d, lane & 7);
      dma16(p.qtT + tb, (uint32_t)(d * 128 + c8 * 16), dst + 2 * TILE + blk * 1024);
      dma16(p.daT + tb, (uint32_t)(d * 128 + c8 * 16), dst + 3 * TILE + blk * 1024);
    }
    if (tid < kQB) {
      const size_t si = ((size_t)b * p.Hq + h) * T + min(i0 + tid, T - 1);
      lsr = p.lse[si];
      dsr = p.dsum[si];
    }
  };
  auto put_stats = [&](int buf) {
    if (tid < kQB) {
      float* st = (float*)(smem + buf * BUF + 4 * TILE);
      st[tid] = lsr;
      st[kQB + tid] = dsr;
    }
  };

  fetch(0, 0);
  put_stats(0);
  vm_wait<0>();
  __syncthreads();
  int cur = 0;
  for (int it = 0; it < n_it; ++it) {
    const int nxt = cur ^ 1;
    fetch(min(it + 1, n_it - 1), nxt);
    const char* tb = smem + cur * BUF;
    const float* sL = (const float*)(tb + 4 * TILE);
    const float* sD = sL + kQB;
    const int i0 = (qt_lo + it % n_q) * kQB;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(*(const bf16x8*)(tb + roff[ks] + qb * 32 * RB), kreg[ks], s);
        dp = mfma32(*(const bf16x8*)(tb + TILE + roff[ks] + qb * 32 * RB), vreg[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int qi = i0 + qr;
        const bool vis = key < T && qi < T && key <= qi && (!SWA || key > qi - p.window);
        const float pr = vis ? fast_exp2(s[r] * p.qscale - sL[qr]) : 0.f;
        s[r] = pr;
        dp[r] = pr * (dp[r] - sD[qr]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 pp = pack8(s, j), dd = pack8(dp, j);
#pragma unroll
        for (int db = 0; db < DBH; ++db) {
          const int off = toff[2 * qb + j] + (dh * DBH + db) * 32 * 128;
          dvt[db] = mfma32(*(const bf16x8*)(tb + 3 * TILE + off), pp, dvt[db]);
          dkt[db] = mfma32(*(const bf16x8*)(tb + 2 * TILE + off), dd, dkt[db]);
        }
      }
    }
    put_stats(nxt);
    vm_wait<0>();
    __syncthreads();
    cur = nxt;
  }
  if (key < T) {
    bf16* vdst = p.dv + (((size_t)b * T + key) * p.Hkv + kvh) * D;
    float* kdst = p.dkt + (((size_t)b * T + key) * p.Hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < DBH; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = (dh * DBH + db) * 32 + 8 * r4 + 4 * hi;
        const int r = 4 * r4;
        *(bf16x4*)(vdst + d0) = (bf16x4){(bf16)dvt[db][r], (bf16)dvt[db][r + 1],
                                         (bf16)dvt[db][r + 2], (bf16)dvt[db][r + 3]};
        *(float4*)(kdst + d0) = make_float4(dkt[db][r] * p.scale, dkt[db][r + 1] * p.scale,
                                            dkt[db][r + 2] * p.scale, dkt[db][r + 3] * p.scale);
      }
  }
}

// ---- norm/RoPE backward: dx~ -> dx and per-block weight partials ------------------------
// 16 lanes per row (8 dims each), 16 rows per pass, grid-stride over the rows; the rotated
// pair partners are exchanged through LDS. Each workgroup leaves one partial of the
// weight gradient (sum over its rows of u * x^, u = R^T dx~).
struct NArgs {
  const bf16* x;       // raw q or k [B][T][H][D]
  const float* w;
  const float* dxt;    // dx~ [B][T][H][D] fp32
  bf16* dx;            // [B][T][H][D]
  float* part;         // [gridDim.x][D]
  int B, T, H, rdim, pos_offset;
  float eps;
  RopeFreq fr;
};
constexpr int kNormBlocks = 1024;

template <int D>
__global__ __launch_bounds__(kT) void bwd_norm_rope_kernel(const NArgs p) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPP = kT / LPR;              // rows per pass
  __shared__ float su[RPP][D + 4];
  __shared__ float sw[RPP][D];               // column partials at the end
  const int t = threadIdx.x;
  const int rl = t / LPR, sub = t % LPR;     // row slot, lane in the row
  const int half = p.rdim >> 1;
  const int64_t n_rows = (int64_t)p.B * p.T * p.H;
  float wv[8], acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wv[e] = p.w[sub * 8 + e];
    acc[e] = 0.f;
  }
  for (int64_t r0 = (int64_t)blockIdx.x * RPP; r0 < n_rows; r0 += (int64_t)gridDim.x * RPP) {
    const int64_t row = r0 + rl;
    const bool ok = row < n_rows;
    const int64_t rc = ok ? row : n_rows - 1;
    float x[8], g[8];
    {
      const u32x4 xw = *(const u32x4*)(p.x + rc * D + sub * 8);
      const uint32_t x4[4] = {xw.x, xw.y, xw.z, xw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo_to_f32(x4[e]);
        x[2 * e + 1] = bf16_hi_to_f32(x4[e]);
      }
      const float4 g0 = *(const float4*)(p.dxt + rc * D + sub * 8);
      const float4 g1 = *(const float4*)(p.dxt + rc * D + sub * 8 + 4);
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
      g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o);
    const float rn = 1.0f / sqrtf(ss / D + p.eps);
    // u = R^T dx~: pair (j, j + half) for j < half
    __syncthreads();   // su free (previous pass done)
#pragma unroll
    for (int e = 0; e < 8; ++e) su[rl][sub * 8 + e] = g[e];
    __syncthreads();
    const int pos = p.pos_offset + (int)((rc / p.H) % p.T);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = sub * 8 + e;
      if (c < p.rdim) {
        const int j = c < half ? c : c - half;
        float cs, sn;
        rope_cos_sin(pos, p.fr.hi[j], p.fr.lo[j], cs, sn);
        const float partner = su[rl][c < half ? c + half : c - half];
        g[e] = c < half ? g[e] * cs + partner * sn : g[e] * cs - partner * sn;
      }
    }
    float dot = 0.f, xh[8], dxh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xh[e] = x[e] * rn;
      dxh[e] = g[e] * wv[e];
      dot = __builtin_fmaf(dxh[e], xh[e], dot);
      if (ok) acc[e] = __builtin_fmaf(g[e], xh[e], acc[e]);
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o);
    dot *= 1.0f / D;
    if (ok) {
      bf16x8 o8;
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = (bf16)(rn * (dxh[e] - xh[e] * dot));
      *(bf16x8*)(p.dx + row * D + sub * 8) = o8;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sw[rl][sub * 8 + e] = acc[e];
  __syncthreads();
  for (int c = t; c < D; c += kT) {
    float sacc = 0.f;
    for (int r = 0; r < RPP; ++r) sacc += sw[r][c];
    p.part[(size_t)blockIdx.x * D + c] = sacc;
  }
}

// dw[c] = sum over the n partials: one workgroup per column
template <int D>
__global__ __launch_bounds__(kT) void bwd_dw_reduce_kernel(const float* part, int n, float* dw) {
  __shared__ float red[kT / 64];
  const int c = blockIdx.x;
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += kT) s += part[(size_t)i * D + c];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int i = 0; i < kT / 64; ++i) tot += red[i];
    dw[c] = tot;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qt, kt, da, dsum, lse, dqt, dkt, part, qtT, daT, ktT, total;
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
  L.nq_blk = kNormBlocks;
  L.nk_blk = kNormBlocks;
  L.part = o; o += align256((size_t)(L.nq_blk + L.nk_blk) * d * 4);
  const size_t n64 = (size_t)(T + 63) / 64;
  L.qtT = o;  o += align256((size_t)B * Hq * n64 * 64 * d * 2);
  L.daT = o;  o += align256((size_t)B * Hq * n64 * 64 * d * 2);
  L.ktT = o;  o += align256((size_t)B * Hkv * n64 * 64 * d * 2);
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

  // transposed tiles of K~, Q~ and dA (slot order) for the operands taken along positions
  const int n64 = (a.T + 63) / 64;
  p.ktT = (const bf16*)(ws + L.ktT);
  p.qtT = (const bf16*)(ws + L.qtT);
  p.daT = (const bf16*)(ws + L.daT);
  hipLaunchKernelGGL(bwd_tiles_kernel<D>, dim3(n64, a.B * a.Hkv), dim3(kT), 0, s, p.kt,
                     (int64_t)a.Hkv * a.T * D, (int64_t)a.T * D, (int64_t)D, a.Hkv, a.T, n64,
                     (bf16*)(ws + L.ktT));
  hipLaunchKernelGGL(bwd_tiles_kernel<D>, dim3(n64, a.B * a.Hq), dim3(kT), 0, s, p.qt,
                     (int64_t)a.Hq * a.T * D, (int64_t)a.T * D, (int64_t)D, a.Hq, a.T, n64,
                     (bf16*)(ws + L.qtT));
  hipLaunchKernelGGL(bwd_tiles_kernel<D>, dim3(n64, a.B * a.Hq), dim3(kT), 0, s,
                     (const bf16*)p.da, (int64_t)a.T * a.Hq * D, (int64_t)D,
                     (int64_t)a.Hq * D, a.Hq, a.T, n64, (bf16*)(ws + L.daT));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int bmp = kRowsDQ / p.group;
  const int n_qt = (a.T + bmp - 1) / bmp;
  const int dq_smem = (kDQAhead + 1) * 3 * kKB * D * 2;
  const dim3 gq((unsigned)(n_qt * a.B * a.Hkv));
  e = a.swa ? launch_big(bwd_dq_kernel<D, true>, gq, dim3(kTDQ), dq_smem, s, p)
            : launch_big(bwd_dq_kernel<D, false>, gq, dim3(kTDQ), dq_smem, s, p);
  if (e != hipSuccess) return e;

  const int n_kt = (a.T + kKV - 1) / kKV;
  const int kv_smem = 2 * (4 * kQB * D * 2 + 2 * kQB * 4);
  const dim3 gk((unsigned)(n_kt * a.B * a.Hkv));
  e = a.swa ? launch_big(bwd_dkdv_kernel<D, true>, gk, dim3(kTKV), kv_smem, s, p)
            : launch_big(bwd_dkdv_kernel<D, false>, gk, dim3(kTKV), kv_smem, s, p);
  if (e != hipSuccess) return e;

  NArgs nb;
  nb.B = a.B;
  nb.T = a.T;
  nb.rdim = a.rdim;
  nb.pos_offset = a.pos_offset;
  nb.eps = a.eps;
  nb.fr = a.fr;
  float* part = (float*)(ws + L.part);
  nb.x = (const bf16*)a.q;
  nb.w = a.wq;
  nb.dxt = p.dqt;
  nb.dx = (bf16*)a.dq;
  nb.part = part;
  nb.H = a.Hq;
  hipLaunchKernelGGL(bwd_norm_rope_kernel<D>, dim3(L.nq_blk), dim3(kT), 0, s, nb);
  nb.x = (const bf16*)a.k;
  nb.w = a.wk;
  nb.dxt = p.dkt;
  nb.dx = (bf16*)a.dk;
  nb.part = part + (size_t)L.nq_blk * D;
  nb.H = a.Hkv;
  hipLaunchKernelGGL(bwd_norm_rope_kernel<D>, dim3(L.nk_blk), dim3(kT), 0, s, nb);
  hipLaunchKernelGGL(bwd_dw_reduce_kernel<D>, dim3(D), dim3(kT), 0, s, (const float*)part,
                     L.nq_blk, a.dwq);
  hipLaunchKernelGGL(bwd_dw_reduce_kernel<D>, dim3(D), dim3(kT), 0, s,
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
