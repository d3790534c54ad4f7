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
#include <type_traits>
#include <utility>

#include "common.h"
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
  const bf16* qt;     // Q~ * scale * log2(e), [B][Hq][T][D] (workspace)
  const bf16* kt;     // K~ [B][Hkv][T][D] (workspace)
  bf16* da;           // dA [B][T][Hq][D] (workspace; dout itself for the global layer)
  float* dsum;        // D [B][Hq][T]
  float* lse;         // row log-sum-exp, log2 units [B][Hq][T]
  const float* lse_in;  // the forward's row log-sum-exp, natural log [B][Hq][T], or nullptr
  const bf16* ktT;    // K~^T tiles [B][Hkv][n64][D][64], keys in slot order (workspace)
  const bf16* qtT;    // the same as Q~^T tiles [B][Hq][n64][D][64]
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
  const float lse_given = p.lse_in ? p.lse_in[((size_t)b * p.Hq + h) * T + qc] : 0.f;
  vm_wait_all_known();

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
  // Key tiles below every row of the workgroup (all their keys before its first query,
  // global layers) need no mask; they come first, then the masked ones (the diagonal, and
  // every tile of a windowed layer). Two loops, so that the two kinds of step do not meet
  // at a join.
  const int n_full = SWA ? 0 : max(0, min(n_tiles, (i0 + 1) / kKB - kt_lo));
  auto run = [&](bool second, auto&& body) {
#pragma unroll
    for (int a = 0; a < kDQAhead; ++a) dma(kt_lo + min(a, n_tiles - 1), a, second);
    if (second) vm_wait<(kDQAhead - 1) * 3 * KPW>(); else vm_wait<(kDQAhead - 1) * KPW>();
    __syncthreads();
    int cur = 0;
    auto one = [&](int i, auto masked_tag) {
      const int ahead = (cur + kDQAhead) % NB;
      dma(kt_lo + min(i + kDQAhead, n_tiles - 1), ahead, second);
      body(kt_lo + i, smem + cur * BUF, masked_tag);
      if (second) vm_wait<(kDQAhead - 1) * 3 * KPW>(); else vm_wait<(kDQAhead - 1) * KPW>();
      __syncthreads();
      cur = cur == NB - 1 ? 0 : cur + 1;
    };
    int i = 0;
    for (; i < n_full; ++i) one(i, std::integral_constant<bool, false>{});
    for (; i < n_tiles; ++i) one(i, std::integral_constant<bool, true>{});
    vm_wait<0>();
    __syncthreads();
  };
  // S^T of one 32-key block, the accumulator starting at `init`
  auto scores = [&](const char* tb, int kb, const f32x16& init, f32x16& acc) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mfma32(*(const bf16x8*)(tb + roff[ks] + kb * 32 * RB), qreg[ks], ks == 0 ? init : acc);
  };
  f32x16 zero16;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero16[r] = 0.f;

  // pass 1: row log-sum-exp (log2 units), unless the forward's is given (the branch is
  // uniform over the grid)
  float m = -INFINITY, l = 0.f;
  if (p.lse_in == nullptr) run(false, [&](int kt, const char* tb, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = kt * kKB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s;
      scores(tb, kb, zero16, s);
      float tm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (MASKED) s[r] = visible(key) ? s[r] : -INFINITY;
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
  if (p.lse_in == nullptr) {
    const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
    const float ma = fmaxf(m, mo);
    const float la = (m == -INFINITY ? 0.f : l * fast_exp2(m - ma)) +
                     (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - ma));
    m = ma == -INFINITY ? 0.f : ma + __log2f(la);
  } else {
    m = lse_given * 1.4426950408889634f;
  }
  const float lse2 = m;

  // pass 2: P, dP, dS and dQ~^T += K~^T dS^T. The S and dP accumulators start at -L and
  // -D (the lane's row), so that P = exp2(S acc) and dS = P * (dP acc).
  f32x16 negl, negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    negl[r] = -lse2;
    negd[r] = -drow_sum;
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  run(true, [&](int kt, const char* tb, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = kt * kKB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
      scores(tb, kb, negl, s);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        dp = mfma32(*(const bf16x8*)(tb + TILE + roff[ks] + kb * 32 * RB), dreg[ks],
                    ks == 0 ? negd : dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(s[r]);
        if (MASKED) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          pr = visible(key) ? pr : 0.f;
        }
        s[r] = pr * dp[r];
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

// ---- dK, dV: one workgroup per (batch, KV head, 256 keys) -------------------------------
// Four waves, one per SIMD: wave w owns keys 64 w .. 64 w + 63 of the workgroup (two 32-key
// blocks) and all head dims of their dK and dV, whose accumulators (4 D / 32 x 16 values
// per lane and block) stay in AGPRs, the products that feed them being issued as inline
// assembly. Every query tile streamed through LDS (Q~ rows, dA rows, Q~^T and dA^T tiles,
// unpadded and swizzled, fetched by LDS DMA one step ahead, and the tile's log-sum-exp and
// D) serves the 256 keys, and every operand read from it feeds the products of both key
// blocks of a wave. Per query block of 32 rows: S and dP of both key blocks (keys on the
// lanes), then P = exp2(S - L), dS = P (dP - D), then dV^T += dA^T P^T and
// dK~^T += Q~^T dS^T with P and dS as B operands straight from the score registers.
constexpr int kKV = 256;           // keys per dK/dV workgroup
constexpr int kTKV = 256;          // its threads
// Order of a dK/dV workgroup's (head, query tile) steps: 1 = query tiles from the last one
// down, the group's heads inside (every workgroup of a KV head starts on the same tile and
// they advance together, so an XCD's L2 serves a tile to all of them); 0 = per head, query
// tiles upwards from the diagonal.
#ifndef ZG_BWD_DESC
#define ZG_BWD_DESC 1
#endif

// Accumulate into an AGPR-pinned accumulator. The s_nop covers the wait states an operand
// written by a vector instruction needs before an MFMA reads it.
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The same without wait states, for operands written at least one product earlier.
__device__ __forceinline__ void mfma_agpr_late(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void pin_agpr(f32x16& v) { asm volatile("" : "+a"(v)); }

template <int D, bool SWA>
__global__ __launch_bounds__(kTKV, 1) void bwd_dkdv_kernel(const BArgs p) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;               // 32-row d blocks of dK^T / dV^T
  constexpr int RB = D * 2;
  constexpr int TILE = kQB * RB;
  constexpr int BUF = 4 * TILE + 2 * kQB * 4;
  constexpr int DPW = TILE / 1024 / 4;     // 1 KiB DMA blocks per wave per tile
  static_assert(DPW >= 1, "every wave takes part in each tile's DMA");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int T = p.T, G = p.group;
  const int n64 = (T + 63) / 64;
  const int nkt = (T + kKV - 1) / kKV;
  const int kt = blockIdx.x % nkt;
  const int hb = blockIdx.x / nkt;
  const int b = hb / p.Hkv, kvh = hb % p.Hkv;
  const int k0 = kt * kKV;
  const int wk0 = k0 + 64 * wave;          // the wave's first key

  // the wave's K~ and V rows as B operands: lane l32 holds key wk0 + 32 kb + l32
  bf16x8 kreg[2][KS], vreg[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kc = min(wk0 + 32 * kb + l32, T - 1);
    const bf16* krow = p.kt + (((size_t)b * p.Hkv + kvh) * T + kc) * D;
    const bf16* vrow = p.v + (((size_t)b * T + kc) * p.Hkv + kvh) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[kb][ks] = *(const bf16x8*)(krow + ks * 16 + hi * 8);
      vreg[kb][ks] = *(const bf16x8*)(vrow + ks * 16 + hi * 8);
    }
  }
  vm_wait_all_known();
  f32x16 dvt[2][DB], dkt[2][DB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dvt[kb][db][r] = 0.f;
        dkt[kb][db][r] = 0.f;
      }
      pin_agpr(dvt[kb][db]);
      pin_agpr(dkt[kb][db]);
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
  auto coords = [&](int it, int& hg, int& qt) {
    if (ZG_BWD_DESC) {
      hg = it % G;
      qt = qt_hi - it / G;
    } else {
      hg = it / n_q;
      qt = qt_lo + it % n_q;
    }
  };
  auto fetch = [&](int it, int buf) {
    int hg, qt;
    coords(it, hg, qt);
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
      st[tid] = -lsr;
      st[kQB + tid] = -dsr;
    }
  };

  // One step over query tile i0 from buffer tb. MASKED: some (query, key) pair of the
  // step is not visible (diagonal tiles, the window's edges, rows or keys past T).
  // The step is a stream of slots, each one LDS operand read and the two products (key
  // blocks 0 and 1) that use it: per 32-query block qb, KS dP slots (dA rows), KS S slots
  // (Q~ rows), then 4 DB dV / dK slots (dA^T, then Q~^T, per (j, db)). Operands are read
  // kAhead slots before their products, across the phase boundaries, so that the LDS
  // latency stays hidden behind the products; the P and dS vector work of a block sits
  // between its S and its dV / dK slots. The dP and S accumulators start at -D and -L
  // (the C operand of the first product, from the step's statistics, which hold the
  // negated values): Q~ is stored times scale * log2(e), so P = exp2(S acc) and
  // dS = P * (dP acc). The lane's rows are qb * 32 + 8 (r / 4) + 4 hi + r % 4, the
  // accumulator layout of four 4-row groups.
  constexpr int NSQ = 2 * KS + 4 * DB;   // slots per 32-query block
  constexpr int NS = 2 * NSQ;            // slots per step
  constexpr int kAhead = 2;
  auto step = [&](const char* tb, int i0, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const float* sL = (const float*)(tb + 4 * TILE);
    const float* sD = sL + kQB;
    auto read_op = [&](int u) -> bf16x8 {
      const int qb = u / NSQ, w = u % NSQ;
      if (w < KS) return *(const bf16x8*)(tb + TILE + roff[w] + qb * 32 * RB);
      if (w < 2 * KS) return *(const bf16x8*)(tb + roff[w - KS] + qb * 32 * RB);
      const int t = (w - 2 * KS) >> 1, j = t / DB, db = t % DB;
      const int off = toff[2 * qb + j] + db * 32 * 128;
      return *(const bf16x8*)(tb + ((w & 1) ? 2 : 3) * TILE + off);
    };
    auto read_stats = [&](const float* src, int qb) {
      f32x16 x;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 v = *(const float4*)(src + qb * 32 + 8 * g4 + 4 * hi);
        x[4 * g4] = v.x; x[4 * g4 + 1] = v.y; x[4 * g4 + 2] = v.z; x[4 * g4 + 3] = v.w;
      }
      return x;
    };
    bf16x8 ops[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ops[i] = read_op(i);
    f32x16 negc = read_stats(sD, 0);
    f32x16 dp[2], sc[2];
    bf16x8 pp[2][2], dd[2][2];
    static_for<NS>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int qb = u / NSQ, w = u % NSQ;
      const bf16x8 a = ops[0];
#pragma unroll
      for (int i = 0; i + 1 < kAhead; ++i) ops[i] = ops[i + 1];
      if constexpr (u + kAhead < NS) ops[kAhead - 1] = read_op(u + kAhead);
      if constexpr (w < KS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dp[kb] = mfma32(a, vreg[kb][w], w == 0 ? negc : dp[kb]);
        if constexpr (w == KS - 2) negc = read_stats(sL, qb);
      } else if constexpr (w < 2 * KS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sc[kb] = mfma32(a, kreg[kb][w - KS], w == KS ? negc : sc[kb]);
        if constexpr (w == 2 * KS - 1) {
          // P and dS, rounded to bf16 in pairs: the B operands of the dV and dK products
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int key = wk0 + 32 * kb + l32;
            u32x4 pw[2], dw[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              float pr[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                pr[e] = fast_exp2(sc[kb][r + e]);
                if (MASKED) {
                  const int qi = i0 + qb * 32 + 8 * ((r + e) >> 2) + 4 * hi + ((r + e) & 3);
                  const bool vis =
                      key < T && qi < T && key <= qi && (!SWA || key > qi - p.window);
                  pr[e] = vis ? pr[e] : 0.f;
                }
              }
              const bf16x2 pb = {(bf16)pr[0], (bf16)pr[1]};
              const bf16x2 db2 = {(bf16)(pr[0] * dp[kb][r]), (bf16)(pr[1] * dp[kb][r + 1])};
              pw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pb);
              dw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, db2);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              pp[kb][j] = __builtin_bit_cast(bf16x8, pw[j]);
              dd[kb][j] = __builtin_bit_cast(bf16x8, dw[j]);
            }
          }
        }
      } else {
        constexpr int t = (w - 2 * KS) >> 1, j = t / DB, db = t % DB;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // the first products after the vector block wait for its last writes
          if constexpr (w & 1) {
            if constexpr (db == 0) mfma_agpr(dkt[kb][db], a, dd[kb][j]);
            else mfma_agpr_late(dkt[kb][db], a, dd[kb][j]);
          } else {
            if constexpr (db == 0) mfma_agpr(dvt[kb][db], a, pp[kb][j]);
            else mfma_agpr_late(dvt[kb][db], a, pp[kb][j]);
          }
        }
        if constexpr (qb == 0 && w == NSQ - 2) negc = read_stats(sD, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  fetch(0, 0);
  put_stats(0);
  vm_wait<0>();
  __syncthreads();
  int cur = 0;
  auto advance = [&](int it, auto masked_tag) {
    const int nxt = cur ^ 1;
    fetch(min(it + 1, n_it - 1), nxt);
    int hg, qt;
    coords(it, hg, qt);
    step(smem + cur * BUF, qt * kQB, masked_tag);
    put_stats(nxt);
    vm_wait<0>();
    __syncthreads();
    cur = nxt;
  };
  if (SWA) {
    for (int it = 0; it < n_it; ++it) advance(it, std::integral_constant<bool, true>{});
  } else {
    // The query tiles that see every key of the workgroup (all their queries after its
    // last key, inside the sequence) are one run [f_lo, f_hi] between the diagonal tiles
    // below it and a ragged last tile above it. The steps over them and over the masked
    // tiles go in separate loops, so that masked and unmasked steps never meet at a join
    // (where the compiler would copy the accumulators between registers).
    const bool any = k0 + kKV <= T;
    const int f_lo = any ? (k0 + kKV - 1 + kQB - 1) / kQB : qt_hi + 1;
    const int f_hi = any ? min(qt_hi, T / kQB - 1) : qt_hi;   // empty when f_lo > f_hi
    auto run = [&](int it0, int it1, auto masked_tag) {
      for (int it = it0; it < it1; ++it) advance(it, masked_tag);
    };
    const std::integral_constant<bool, true> masked{};
    const std::integral_constant<bool, false> unmasked{};
    const bool none = f_lo > f_hi;   // then the first masked run takes every step
    if (ZG_BWD_DESC) {
      // tiles qt_hi .. f_hi + 1 (ragged top), f_hi .. f_lo, f_lo - 1 .. qt_lo (diagonal)
      const int a = none ? n_it : (qt_hi - f_hi) * G;
      const int c = none ? n_it : (qt_hi - f_lo + 1) * G;
      run(0, a, masked);
      run(a, c, unmasked);
      run(c, n_it, masked);
    } else {
      const int a = none ? n_q : f_lo - qt_lo;
      const int c = none ? n_q : f_hi - qt_lo + 1;
      for (int hg = 0; hg < G; ++hg) {
        run(hg * n_q, hg * n_q + a, masked);
        run(hg * n_q + a, hg * n_q + c, unmasked);
        run(hg * n_q + c, (hg + 1) * n_q, masked);
      }
    }
  }
  // 18 wait states at least between the last product and the reads of its accumulators
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      pin_agpr(dvt[kb][db]);
      pin_agpr(dkt[kb][db]);
    }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = wk0 + 32 * kb + l32;
    if (key >= T) continue;
    bf16* vdst = p.dv + (((size_t)b * T + key) * p.Hkv + kvh) * D;
    float* kdst = p.dkt + (((size_t)b * T + key) * p.Hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hi;
        const int r = 4 * r4;
        *(bf16x4*)(vdst + d0) = (bf16x4){(bf16)dvt[kb][db][r], (bf16)dvt[kb][db][r + 1],
                                         (bf16)dvt[kb][db][r + 2], (bf16)dvt[kb][db][r + 3]};
        // dk~ = scale * dS^T q~ and the Q~^T tiles hold q~ * scale * log2(e)
        const float ks = p.scale / p.qscale;
        *(float4*)(kdst + d0) =
            make_float4(dkt[kb][db][r] * ks, dkt[kb][db][r + 1] * ks, dkt[kb][db][r + 2] * ks,
                        dkt[kb][db][r + 3] * ks);
      }
  }
}

// ---- norm/RoPE backward: dx~ -> dx and per-block weight partials ------------------------
// 16 lanes per row (8 dims each), 16 rows per pass, grid-stride over the rows; the rotated
// pair partners are exchanged through LDS. Each workgroup leaves one partial of the
// weight gradient (sum over its rows of u * x^, u = R^T dx~).
struct NArgs {
  const void* x;       // raw q or k [B][T][H][D] (element type E of the kernel)
  const float* w;
  const float* dxt;    // dx~ [B][T][H][D] fp32
  void* dx;            // [B][T][H][D] (E)
  float* part;         // [gridDim.x][D]
  int B, T, H, rdim, pos_offset;
  float eps;
  RopeFreq fr;
};
constexpr int kNormBlocks = 1024;

template <int D, typename E = bf16>
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
      if constexpr (std::is_same<E, float>::value) {
        const float4 x0 = *(const float4*)((const float*)p.x + rc * D + sub * 8);
        const float4 x1 = *(const float4*)((const float*)p.x + rc * D + sub * 8 + 4);
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
        x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
      } else {
        const u32x4 xw = *(const u32x4*)((const bf16*)p.x + rc * D + sub * 8);
        const uint32_t x4[4] = {xw.x, xw.y, xw.z, xw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_lo_to_f32(x4[e]);
          x[2 * e + 1] = bf16_hi_to_f32(x4[e]);
        }
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
      if constexpr (std::is_same<E, float>::value) {
        float* o = (float*)p.dx + row * D + sub * 8;
        *(float4*)o = make_float4(rn * (dxh[0] - xh[0] * dot), rn * (dxh[1] - xh[1] * dot),
                                  rn * (dxh[2] - xh[2] * dot), rn * (dxh[3] - xh[3] * dot));
        *(float4*)(o + 4) = make_float4(rn * (dxh[4] - xh[4] * dot), rn * (dxh[5] - xh[5] * dot),
                                        rn * (dxh[6] - xh[6] * dot), rn * (dxh[7] - xh[7] * dot));
      } else {
        bf16x8 o8;
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = (bf16)(rn * (dxh[e] - xh[e] * dot));
        *(bf16x8*)((bf16*)p.dx + row * D + sub * 8) = o8;
      }
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
    hipError_t e = ensure_dynamic_smem((const void*)kern, smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, smem, s, a);
  return hipGetLastError();
}

// ---- vector-ALU backward: fp32 tensors, or head groups the MFMA kernels do not take ------
// The same gradient in fp32 arithmetic throughout (element type E of the tensors): Q~ (times
// the softmax scale) and K~ from the forward's transform, then
//   prep:  dA = dO sigmoid(G) (SWA; dO itself for the global layer), D = sum dO O, dG,
//   dq:    per query (one lane, 64 per workgroup): the row log-sum-exp unless the forward
//          gave it, then dq~ = scale sum_j P (dP - D) k~_j over the visible keys,
//   dk/dv: per key (one lane): dv = sum_i P dA_i, dk~ = sum_i dS q~_i (scale included in
//          Q~) over the visible queries of every head of the group,
// and the norm/RoPE backward and weight reductions of the MFMA path.
constexpr int kVT = 64;   // rows (queries or keys) per workgroup of the vector-ALU kernels

struct VArgs {
  const void* out;     // forward output O [B][T][Hq][D]
  const void* dout;
  const void* g;       // gate pre-activation (SWA) or nullptr
  const void* v;       // [B][T][Hkv][D]
  const void* qt;      // Q~ * scale [B][Hq][T][D]
  const void* kt;      // K~ [B][Hkv][T][D]
  void* da;            // dA [B][T][Hq][D] (dout itself for the global layer)
  float* dsum;         // D [B][Hq][T]
  float* lse;          // row log-sum-exp, natural log [B][Hq][T]
  const float* lse_in; // the forward's, or nullptr
  float* dqt;          // dq~ [B][T][Hq][D] fp32
  float* dkt;          // dk~ [B][T][Hkv][D] fp32
  void* dv;            // [B][T][Hkv][D]
  void* dg;            // [B][T][Hq][D] or nullptr
  int B, T, Hq, Hkv, window, swa, group;
  float scale;
};

template <typename E>
__device__ __forceinline__ float ld(const E* x, size_t i) { return (float)x[i]; }

// one thread per (b, t, head) row
template <int D, typename E>
__global__ __launch_bounds__(kT) void valu_bwd_prep_kernel(const VArgs p) {
  const int64_t row = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (row >= (int64_t)p.B * p.T * p.Hq) return;
  const int h = (int)(row % p.Hq);
  const int64_t bt = row / p.Hq;
  const int b = (int)(bt / p.T), t = (int)(bt % p.T);
  const E* dO = (const E*)p.dout + row * D;
  const E* O = (const E*)p.out + row * D;
  float dsum = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; ++c) dsum = __builtin_fmaf(ld(dO, c), ld(O, c), dsum);
  if (p.g) {
    const E* G = (const E*)p.g + row * D;
    E* dA = (E*)p.da + row * D;
    E* dG = (E*)p.dg + row * D;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      const float sg = sigmoidf_(ld(G, c));
      dA[c] = (E)(ld(dO, c) * sg);
      dG[c] = (E)(ld(dO, c) * ld(O, c) * (1.0f - sg));
    }
  }
  p.dsum[((size_t)b * p.Hq + h) * p.T + t] = dsum;
}

__device__ __forceinline__ bool valu_visible(int key, int q, int T, int swa, int window) {
  return key < T && q < T && key <= q && (!swa || key > q - window);
}

// grid (query tiles, Hq, B), kVT threads; dynamic LDS: K~, V and dA rows (padded)
template <int D, typename E>
__global__ __launch_bounds__(kVT) void valu_bwd_dq_kernel(const VArgs p) {
  constexpr int RS = D + 1;
  extern __shared__ float vsm[];
  float* sK = vsm;
  float* sV = sK + kVT * RS;
  float* sA = sV + kVT * RS;
  const int t = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / p.group;
  const int i0 = blockIdx.x * kVT, i = i0 + t;
  const bool valid = i < p.T;
  const int ic = valid ? i : p.T - 1;
  const E* qrow = (const E*)p.qt + (((size_t)b * p.Hq + h) * p.T + ic) * D;
  const E* arow = (const E*)p.da + (((size_t)b * p.T + ic) * p.Hq + h) * D;
  float qv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = ld(qrow, c);
    sA[t * RS + c] = ld(arow, c);
  }
  const size_t st = ((size_t)b * p.Hq + h) * p.T + ic;
  const float dsum = p.dsum[st];
  const int kt_lo = p.swa ? max(0, i0 - p.window + 1) / kVT : 0;
  const int kt_hi = (min(i0 + kVT, p.T) - 1) / kVT;
  auto stage = [&](int kt, bool with_v) {
    const int j = min(kt * kVT + t, p.T - 1);
    const E* krow = (const E*)p.kt + (((size_t)b * p.Hkv + kvh) * p.T + j) * D;
    const E* vrow = (const E*)p.v + (((size_t)b * p.T + j) * p.Hkv + kvh) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      sK[t * RS + c] = ld(krow, c);
      if (with_v) sV[t * RS + c] = ld(vrow, c);
    }
  };
  float lse;
  if (p.lse_in) {
    lse = p.lse_in[st];
  } else {
    float m = -INFINITY, l = 0.f;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      __syncthreads();
      stage(kt, false);
      __syncthreads();
      for (int jj = 0; jj < kVT; ++jj) {
        const int key = kt * kVT + jj;
        if (!valu_visible(key, i, p.T, p.swa, p.window)) continue;
        float sc = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) sc = __builtin_fmaf(qv[c], sK[jj * RS + c], sc);
        const float mn = fmaxf(m, sc);
        l = l * expf(m - mn) + expf(sc - mn);
        m = mn;
      }
    }
    lse = m + logf(l);
  }
  if (valid) p.lse[st] = lse;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    __syncthreads();
    stage(kt, true);
    __syncthreads();
    for (int jj = 0; jj < kVT; ++jj) {
      const int key = kt * kVT + jj;
      if (!valu_visible(key, i, p.T, p.swa, p.window)) continue;
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        sc = __builtin_fmaf(qv[c], sK[jj * RS + c], sc);
        dp = __builtin_fmaf(sA[t * RS + c], sV[jj * RS + c], dp);
      }
      const float ds = expf(sc - lse) * (dp - dsum);
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = __builtin_fmaf(ds, sK[jj * RS + c], acc[c]);
    }
  }
  if (valid) {
    float* dst = p.dqt + (((size_t)b * p.T + i) * p.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) dst[c] = acc[c] * p.scale;
  }
}

// grid (key tiles, Hkv, B), kVT threads; dynamic LDS: Q~ and dA rows of a query tile, the
// lane's own K~ and V rows (padded), the tile's lse and D
template <int D, typename E>
__global__ __launch_bounds__(kVT) void valu_bwd_dkdv_kernel(const VArgs p) {
  constexpr int RS = D + 1;
  extern __shared__ float vsm[];
  float* sQ = vsm;
  float* sA = sQ + kVT * RS;
  float* sK = sA + kVT * RS;
  float* sV = sK + kVT * RS;
  float* sL = sV + kVT * RS;
  float* sD = sL + kVT;
  const int t = threadIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int k0 = blockIdx.x * kVT, j = k0 + t;
  const int jc = min(j, p.T - 1);
  {
    const E* krow = (const E*)p.kt + (((size_t)b * p.Hkv + kvh) * p.T + jc) * D;
    const E* vrow = (const E*)p.v + (((size_t)b * p.T + jc) * p.Hkv + kvh) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      sK[t * RS + c] = ld(krow, c);
      sV[t * RS + c] = ld(vrow, c);
    }
  }
  float dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const int q_last = p.swa ? min(p.T - 1, k0 + kVT - 1 + p.window - 1) : p.T - 1;
  for (int hh = 0; hh < p.group; ++hh) {
    const int h = kvh * p.group + hh;
    for (int qt = k0 / kVT; qt * kVT <= q_last; ++qt) {
      const int ic = min(qt * kVT + t, p.T - 1);
      const E* qrow = (const E*)p.qt + (((size_t)b * p.Hq + h) * p.T + ic) * D;
      const E* arow = (const E*)p.da + (((size_t)b * p.T + ic) * p.Hq + h) * D;
      __syncthreads();
#pragma unroll
      for (int c = 0; c < D; ++c) {
        sQ[t * RS + c] = ld(qrow, c);
        sA[t * RS + c] = ld(arow, c);
      }
      sL[t] = p.lse[((size_t)b * p.Hq + h) * p.T + ic];
      sD[t] = p.dsum[((size_t)b * p.Hq + h) * p.T + ic];
      __syncthreads();
      for (int r = 0; r < kVT; ++r) {
        const int i = qt * kVT + r;
        if (!valu_visible(j, i, p.T, p.swa, p.window)) continue;
        float sc = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          sc = __builtin_fmaf(sQ[r * RS + c], sK[t * RS + c], sc);
          dp = __builtin_fmaf(sA[r * RS + c], sV[t * RS + c], dp);
        }
        const float pr = expf(sc - sL[r]);
        const float ds = pr * (dp - sD[r]);
#pragma unroll
        for (int c = 0; c < D; ++c) {
          dv[c] = __builtin_fmaf(pr, sA[r * RS + c], dv[c]);
          dk[c] = __builtin_fmaf(ds, sQ[r * RS + c], dk[c]);
        }
      }
    }
  }
  if (j < p.T) {
    const size_t o = (((size_t)b * p.T + j) * p.Hkv + kvh) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      ((E*)p.dv)[o + c] = (E)dv[c];
      p.dkt[o + c] = dk[c];
    }
  }
}

// Workspace of the vector-ALU path (Q~, K~ and dA in the tensors' element type), within
// the bytes backward_workspace_bytes gives for the MFMA path of the same shape.
WsLayout valu_ws_layout(int B, int T, int Hq, int Hkv, int d, int esz) {
  WsLayout L{};
  size_t o = 0;
  const size_t nq = (size_t)B * T * Hq, nk = (size_t)B * T * Hkv;
  L.qt = o;   o += align256(nq * d * esz);
  L.kt = o;   o += align256(nk * d * esz);
  L.da = o;   o += align256(nq * d * esz);
  L.dsum = o; o += align256(nq * 4);
  L.lse = o;  o += align256(nq * 4);
  L.dqt = o;  o += align256(nq * d * 4);
  L.dkt = o;  o += align256(nk * d * 4);
  L.nq_blk = kNormBlocks;
  L.nk_blk = kNormBlocks;
  L.part = o; o += align256((size_t)(L.nq_blk + L.nk_blk) * d * 4);
  L.total = o;
  return L;
}

template <int D, typename E>
hipError_t valu_backward_t(const BackwardArgs& a, hipStream_t s) {
  const WsLayout L = valu_ws_layout(a.B, a.T, a.Hq, a.Hkv, D, (int)sizeof(E));
  char* ws = (char*)a.ws;
  NormRopeArgs n;
  n.pos = nullptr;
  n.B = a.B;
  n.T = a.T;
  n.d = D;
  n.rdim = a.rdim;
  n.pos_offset = a.pos_offset;
  n.is_bf16 = std::is_same<E, bf16>::value;
  n.eps = a.eps;
  n.fr = a.fr;
  n.x = a.q;
  n.w = a.wq;
  n.y = ws + L.qt;
  n.out_scale = a.scale;   // Q~ carries the (natural-log) softmax scale
  n.H = a.Hq;
  n.ysb = (int64_t)a.Hq * a.T * D;
  n.yst = D;
  n.ysh = (int64_t)a.T * D;
  hipError_t e = launch_qknorm_rope(n, s);
  if (e != hipSuccess) return e;
  n.x = a.k;
  n.w = a.wk;
  n.y = ws + L.kt;
  n.out_scale = 1.0f;
  n.H = a.Hkv;
  n.ysb = (int64_t)a.Hkv * a.T * D;
  n.ysh = (int64_t)a.T * D;
  e = launch_qknorm_rope(n, s);
  if (e != hipSuccess) return e;

  VArgs p;
  p.out = a.out;
  p.dout = a.dout;
  p.g = a.g;
  p.v = a.v;
  p.qt = ws + L.qt;
  p.kt = ws + L.kt;
  p.da = a.g ? (void*)(ws + L.da) : const_cast<void*>(a.dout);
  p.dsum = (float*)(ws + L.dsum);
  p.lse = (float*)(ws + L.lse);
  p.lse_in = a.lse;
  p.dqt = (float*)(ws + L.dqt);
  p.dkt = (float*)(ws + L.dkt);
  p.dv = a.dv;
  p.dg = a.dg;
  p.B = a.B;
  p.T = a.T;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.window = a.window;
  p.swa = a.swa;
  p.group = a.Hq / a.Hkv;
  p.scale = a.scale;
  const int64_t rows = (int64_t)a.B * a.T * a.Hq;
  hipLaunchKernelGGL((valu_bwd_prep_kernel<D, E>), dim3((unsigned)((rows + kT - 1) / kT)),
                     dim3(kT), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned n_t = (unsigned)((a.T + kVT - 1) / kVT);
  e = launch_big(valu_bwd_dq_kernel<D, E>, dim3(n_t, a.Hq, a.B), dim3(kVT),
                 3 * kVT * (D + 1) * 4, s, p);
  if (e != hipSuccess) return e;
  e = launch_big(valu_bwd_dkdv_kernel<D, E>, dim3(n_t, a.Hkv, a.B), dim3(kVT),
                 (4 * kVT * (D + 1) + 2 * kVT) * 4, s, p);
  if (e != hipSuccess) return e;

  NArgs nb;
  nb.B = a.B;
  nb.T = a.T;
  nb.rdim = a.rdim;
  nb.pos_offset = a.pos_offset;
  nb.eps = a.eps;
  nb.fr = a.fr;
  float* part = (float*)(ws + L.part);
  nb.x = a.q;
  nb.w = a.wq;
  nb.dxt = p.dqt;
  nb.dx = a.dq;
  nb.part = part;
  nb.H = a.Hq;
  hipLaunchKernelGGL((bwd_norm_rope_kernel<D, E>), dim3(L.nq_blk), dim3(kT), 0, s, nb);
  nb.x = a.k;
  nb.w = a.wk;
  nb.dxt = p.dkt;
  nb.dx = a.dk;
  nb.part = part + (size_t)L.nq_blk * D;
  nb.H = a.Hkv;
  hipLaunchKernelGGL((bwd_norm_rope_kernel<D, E>), dim3(L.nk_blk), dim3(kT), 0, s, nb);
  hipLaunchKernelGGL(bwd_dw_reduce_kernel<D>, dim3(D), dim3(kT), 0, s, (const float*)part,
                     L.nq_blk, a.dwq);
  hipLaunchKernelGGL(bwd_dw_reduce_kernel<D>, dim3(D), dim3(kT), 0, s,
                     (const float*)(part + (size_t)L.nq_blk * D), L.nk_blk, a.dwk);
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
  n.out_scale = a.scale * 1.4426950408889634f;   // Q~ carries the log2-domain score scale
  n.H = a.Hq;
  n.ysb = (int64_t)a.Hq * a.T * D;
  n.yst = D;
  n.ysh = (int64_t)a.T * D;
  hipError_t e = launch_qknorm_rope(n, s);
  if (e != hipSuccess) return e;
  n.x = a.k;
  n.w = a.wk;
  n.y = ws + L.kt;
  n.out_scale = 1.0f;
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
  p.lse_in = a.swa ? nullptr : a.lse;
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
  nb.x = a.q;
  nb.w = a.wq;
  nb.dxt = p.dqt;
  nb.dx = a.dq;
  nb.part = part;
  nb.H = a.Hq;
  hipLaunchKernelGGL(bwd_norm_rope_kernel<D>, dim3(L.nq_blk), dim3(kT), 0, s, nb);
  nb.x = a.k;
  nb.w = a.wk;
  nb.dxt = p.dkt;
  nb.dx = a.dk;
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
  // the MFMA path's layout, or the vector-ALU path's with fp32 rows if that is larger
  const size_t m = ws_layout(B, T, Hq, Hkv, d).total;
  const size_t v = valu_ws_layout(B, T, Hq, Hkv, d, 4).total;
  return m > v ? m : v;
}

bool backward_mfma_supported(int group) { return group == 1 || group == 2 || group == 4 || group == 8; }

hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t s) {
  if (a.f32)
    return a.d == 128 ? valu_backward_t<128, float>(a, s) : valu_backward_t<64, float>(a, s);
  if (!backward_mfma_supported(a.Hq / a.Hkv))
    return a.d == 128 ? valu_backward_t<128, bf16>(a, s) : valu_backward_t<64, bf16>(a, s);
  return a.d == 128 ? backward_t<128>(a, s) : backward_t<64>(a, s);
}

}  // namespace zg
