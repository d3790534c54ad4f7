// bf16 prefill attention on gfx950 MFMA: gated sliding-window and full-causal GQA.
//
// What is computed (hyper.ai summary of arXiv 2609.13356, section 方法, GatedSWA
// equation; "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ): for every query row,
// RMSNorm + partial RoPE on q and k, softmax(scale * q~ . k~) over the visible keys
// (the last `window` tokens including the query for SWA, the whole prefix for global),
// times V, then the elementwise sigmoid gate for SWA.
//
// Work decomposition (one workgroup = 256 query rows at a time; global layers of dense
// batches launch one workgroup per CU, each walking several query tiles in turn):
//   * The rows are all g = Hq/Hkv query heads of one KV head at 256/g consecutive
//     positions, so every K/V tile staged in LDS serves the whole head group.
//   * Global layers with K~ / V tiles from the workspace: 4 wave64s, one per SIMD, each
//     owning two 32-row query blocks (each LDS operand read feeds two products); the
//     other forms: 8 wave64s of one block each. Scores are formed transposed,
//     S^T = K~ . Q~^T with v_mfma_f32_32x32x16_bf16 (keys on the M side, queries on N),
//     which leaves one query per lane; the probabilities then already sit in the
//     B-operand layout of O^T += V^T . P^T, so no cross-lane shuffle is needed between
//     the two products and the softmax row statistics are per-lane scalars.
//   * V is transposed with the keys of each 16-key group permuted so that a lane's eight
//     keys are one 16-byte LDS read. Global layers: a pre-pass writes V as such tiles and
//     the kernel moves K~ / V^T tiles from the workspace straight into three rotating LDS
//     buffers by LDS DMA, two tiles ahead. The other forms stage the next tile through
//     registers into two LDS buffers while the current one is computed.
//   * Q~ is pre-multiplied by scale * log2(e) so that p = exp2(s - m).
//   * Static shift: after RMSNorm every score obeys |s| <= B = qscale * d * max|wq| *
//     max|wk| (RoPE keeps norms). When B is moderate, p = exp2(s - B) with the constant
//     shift B in place of the running max is exact (softmax is shift-invariant): the
//     score accumulators start at -B (the MFMA C operand, so the shift costs nothing),
//     every p lies in [2^-2B, 1], so neither the row sum nor the fp32 P.V accumulator can
//     overflow (at most T * max|v|), and with B <= 48 the largest p of a row is at least
//     2^-96, far above the fp32 normal range's end. The running max, its reduction and
//     the accumulator rescale disappear. An online-max form of the tile handles larger
//     bounds; one launch carries both, and the bound (the same for every workgroup) picks
//     one.
//   * The O accumulators stay in AGPRs for the whole kernel (the P.V product is issued
//     through a constrained MFMA), leaving the VGPRs to the scores and operands.
//   * K~: for global layers a separate pass writes normalised+rotated K once into a
//     workspace that the tiles read directly; for SWA layers (each K tile visited by
//     about three query tiles) the transform is fused into the tile load.
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kRows = 256;        // query rows per workgroup
// Waves per workgroup: 8 waves of 32 query rows keep two waves on every SIMD, so one
// wave's softmax (exp, convert, row sums) overlaps the other's MFMAs.
#ifndef ZG_PREFILL_WAVES
#define ZG_PREFILL_WAVES 8
#endif
constexpr int kWavesPerBlock = ZG_PREFILL_WAVES;
// Global layers with K~ / V tiles from the workspace: 4 waves of 64 query rows (one wave
// per SIMD, half the LDS operand traffic per product of 32-row waves) with the fenced
// software pipeline of compute_pipe.
#ifndef ZG_GLOBAL_WAVES
#define ZG_GLOBAL_WAVES 4
#endif
// LDS DMA buffers of the pipelined global path: tiles are fetched kDmaBufs - 1 ahead.
#ifndef ZG_DMA_BUFS
#define ZG_DMA_BUFS 3
#endif
constexpr int kDmaBufs = ZG_DMA_BUFS;
// Phase of the pipelined tile (0 A .. 3 D) whose slots issue the DMA pieces.
#ifndef ZG_DMA_PHASE
#define ZG_DMA_PHASE 3
#endif
constexpr int kDmaPhase = ZG_DMA_PHASE;
// Persistent global launches (one workgroup per CU walking several query tiles).
#ifndef ZG_PERSISTENT
#define ZG_PERSISTENT 1
#endif
constexpr int kBN = 64;           // keys per tile
constexpr int kXcds = 8;          // accelerator complex dies (one L2 each)
constexpr int kMaxHalfMfma = 32;  // rotary_dim <= 64 on this path
constexpr int kQTrigStride = kMaxHalfMfma + 1;  // float2 per Q position: rows 8 banks apart
// Rotated pairs of the model's partial RoPE, rotary_dim = 2 * floor(0.33 * d / 2).
template <int D>
constexpr int kModelHalf = D == 128 ? 21 : 10;
constexpr float kStaticShiftMax = 48.0f;  // largest score bound (log2 units) without a max

template <int D>
struct Smem {
  static constexpr int kRowB = D * 2 + 16;      // padded bf16 row (bytes)
  static constexpr int kVtRowB = kBN * 2 + 16;  // padded V^T row (bytes)
  // Phase 1 (Q): raw Q rows, transformed in place; then copied to registers.
  static constexpr int kQ = kRows * kRowB;
  static constexpr int kQtrig = kRows * kQTrigStride * 8;
  // Main loop: two K~ / V^T buffers, raw K tile and its trig table (fused path).
  static constexpr int kK = kBN * kRowB;
  static constexpr int kVt = D * kVtRowB;
  static constexpr int kBuf = kK + kVt;
  static constexpr int kKraw = kBN * kRowB;
  static constexpr int kKtrig = kBN * kMaxHalfMfma * 8;
  static constexpr int kLoop = 2 * kBuf + kKraw + kKtrig;
  // Pipelined global path: kDmaBufs buffers filled by LDS DMA, each K~ as 64 unpadded
  // rows of 2*D bytes and V^T as D unpadded rows of 128 bytes (16-byte chunks swizzled).
  static constexpr int kDK = kBN * D * 2;
  static constexpr int kDBuf = kDK + D * kBN * 2;
  static constexpr int kDLoop = kDmaBufs * kDBuf;
  static constexpr int kW = 2 * D * 4;  // wq, wk
  static constexpr int kFr = 2 * kMaxHalfMfma * 4;  // RoPE phase steps (head, tail)
  static constexpr int kMain = kLoop > kDLoop ? kLoop : kDLoop;
  static constexpr int kUnion = (kQ + kQtrig) > kMain ? (kQ + kQtrig) : kMain;
  // Persistent global path: RoPE of the in-tile offsets 0 .. kBN-1 (one table per
  // workgroup) and of each tile's first position, combined by angle addition.
  static constexpr int kOffT = kBN * kMaxHalfMfma * 8;
  static constexpr int kBaseT = kMaxHalfMfma * 8;
  static constexpr int kTotal = kUnion + kW + kFr + kOffT + kBaseT;
  static_assert(kTotal <= 160 * 1024, "LDS budget of a CU");
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
  const bf16* vt;     // tile-transposed V (with kt), see kv_prepass_kernel
  int T, Hq, Hkv, window, rdim, pos_offset;
  int group, bmp, n_qtiles, n_hb;
  float eps, qscale;
  RopeFreq fr;
  // packed documents (B == 1, T = total tokens): cu [n_docs + 1], n_hb = n_docs * Hkv,
  // n_qtiles sized by max_len; nullptr for dense batches
  const int32_t* cu;
  int max_len, vt_slots;
  int n_blocks;       // query tiles in all: n_qtiles * n_hb
  float* lse;         // row log-sum-exp [B][Hq][T] (natural log), dense global only; or nullptr
};

// Swap bits 2 and 3 of a key index within its 16-key group: keys {0-3, 8-11} then
// {4-7, 12-15}, matching which keys a lane holds in the S^T accumulator.
__device__ __forceinline__ int vt_slot(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// O^T += V^T P^T on an accumulator pinned to AGPRs. The leading s_nop covers the two
// wait states a VALU-written operand (P) needs before an MFMA may read it.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The same product without the wait states, for schedules where P was written at least
// one MFMA slot earlier (slots are fenced by scheduling barriers).
__device__ __forceinline__ void mfma_acc_late(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

#ifndef ZG_PREFILL_PIPE
#define ZG_PREFILL_PIPE 1
#endif
#ifndef ZG_PREFILL_SETPRIO
#define ZG_PREFILL_SETPRIO 0
#endif
template <int P>
__device__ __forceinline__ void set_prio() {
  if (ZG_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(P);
}

// A barrier for LDS reuse: the workgroup's LDS accesses before it complete before any
// after it, while global loads and stores stay in flight (__syncthreads also waits for
// every store the wave has issued).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Keep a value in AGPRs from here on (so that loop-carried accumulators never take a
// mixed register class).
__device__ __forceinline__ void pin_agpr(f32x16& v) { asm volatile("" : "+a"(v)); }

// Wait states between the last MFMA that wrote the accumulators and any other access.
template <int QB, int DB>
__device__ __forceinline__ void acc_fence(f32x16 (&o)[QB][DB]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(o[qb][db]));
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

// One query tile (blockIdx-independent: `lin` names the tile). Below, `sinit` starts every
// score accumulator: -B (the static shift) or 0 (online variant).
template <int D, bool SWA, bool KPRE, int NW>
__device__ __forceinline__ void prefill_tile(const KArgs& p) {
  using S = Smem<D>;
  constexpr int kThreads = NW * 64;
  constexpr int QB = kRows / 32 / NW;  // 32-row query blocks per wave
  constexpr int TPR = kThreads / kBN;  // threads per key row in the fused K transform
  constexpr int KS = D / 16;   // k-steps of the QK^T product
  constexpr int DB = D / 32;   // 32-wide d blocks of O
  constexpr int RW = S::kRowB / 2;      // padded row length in bf16 elements
  constexpr int VW = S::kVtRowB / 2;
  constexpr int DC = D / 8;                     // 16-byte chunks per row
  constexpr int KIT = (kBN * DC) / kThreads;    // K chunks per thread per tile
  constexpr int KG = (kBN * DC) / kThreads;     // keys per thread in the V transpose
  static_assert(KG == 1 || KG == 2 || KG == 4, "V staging expects 1, 2 or 4 keys per thread");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* sQ = (bf16*)smem;
  float2* sQtrig = (float2*)(smem + S::kQ);
  bf16* sKraw = (bf16*)(smem + 2 * S::kBuf);
  float2* sKtrig = (float2*)(smem + 2 * S::kBuf + S::kKraw);
  float* sWq = (float*)(smem + S::kUnion);
  float* sWk = sWq + D;
  float* sFr = sWk + D;   // [0, 32): phase step heads, [32, 64): tails
  float2* sOffT = (float2*)(smem + S::kUnion + S::kW + S::kFr);  // [offset][pair]
  float2* sBaseT = (float2*)((char*)sOffT + S::kOffT);           // [pair]

  // Global layers with K~ from the workspace may walk several query tiles (persistent
  // launch); the other forms always take one.
  constexpr bool PERSIST = KPRE && !SWA;
  const int tid0 = threadIdx.x;
  const int lane0 = tid0 & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);

  // The norm weights and RoPE steps are loaded first and stored to LDS only after the Q
  // tile's loads are issued below, so that both travel in one memory round trip (loads
  // complete in issue order: storing the weights waits for them alone).
  static_assert(kThreads >= D && kThreads >= kMaxHalfMfma, "one weight per thread");
  float wq_l = 0.f, wk_l = 0.f, fr_hi = 0.f, fr_lo = 0.f;
  if (tid0 < D) {
    wq_l = p.wq[tid0];
    wk_l = p.wk[tid0];
  }
  // (a lane-dependent index into the kernel arguments would be a memory load per use)
  if (tid0 < kMaxHalfMfma) {
    fr_hi = p.fr.hi[tid0];
    fr_lo = p.fr.lo[tid0];
  }

  // Query tiles of the workgroup, heaviest first (global layers). A launch of n_blocks
  // workgroups gives each one tile; a persistent launch (fewer workgroups, dense batches)
  // deals the tiles out in snake order: round k hands the next gridDim.x tiles of the
  // list to the workgroups forwards on even rounds and backwards on odd ones, so that a
  // heavy tile is paired with a light one and every workgroup gets about the same number
  // of key tiles. Workgroup i runs on XCD i % 8 (round-robin dispatch); when the
  // (batch, kv-head) pairs divide by 8, each XCD takes its pairs one after another, so
  // that its L2 holds the K~ / V tiles of one or two pairs at a time.
  auto item_lin = [&](int k) -> int {
    const int G = gridDim.x, j = blockIdx.x;
    if (p.n_hb % kXcds == 0) {
      const int per = G / kXcds, x = j % kXcds, w = j / kXcds;
      return (k * per + ((k & 1) ? per - 1 - w : w)) * kXcds + x;
    }
    return k * G + ((k & 1) ? G - 1 - j : j);
  };
  // One query tile: sequence `seq0` (its first row in the [B*T] or packed token order) of
  // length T, KV head kvh, first position i0; K~ rows and V tiles start at kt_row0 /
  // vt_tile0 of the workspace. `skip`: past the end of a shorter packed document.
  struct Item {
    int b, kvh, T, i0;
    size_t seq0, kt_row0, vt_tile0;
    bool skip;
  };
  auto decode = [&](int lin) -> Item {
    int hb, tile_rank;
    if (p.n_hb % kXcds == 0) {
      const int x = lin % kXcds, slot = lin / kXcds;
      hb = (slot / p.n_qtiles) * kXcds + x;
      tile_rank = slot % p.n_qtiles;
    } else {
      hb = lin % p.n_hb;
      tile_rank = lin / p.n_hb;
    }
    Item it;
    it.b = hb / p.Hkv;        // batch element, or document of a packed batch
    it.kvh = hb % p.Hkv;
    it.T = p.T;
    int n_qtiles = p.n_qtiles;
    it.seq0 = (size_t)it.b * p.T;
    it.kt_row0 = ((size_t)it.b * p.Hkv + it.kvh) * p.T;
    it.vt_tile0 = ((size_t)it.b * p.Hkv + it.kvh) * ((p.T + kBN - 1) / kBN);
    it.skip = false;
    if (p.cu) {
      int start, len;
      doc_range(p.cu, it.b, p.T, p.max_len, start, len);
      it.T = len;
      n_qtiles = (len + p.bmp - 1) / p.bmp;
      it.skip = tile_rank >= n_qtiles;
      it.seq0 = start;
      it.kt_row0 = (size_t)it.kvh * p.T + start;
      it.vt_tile0 = (size_t)it.kvh * p.vt_slots + doc_tile_base(start, it.b);
    }
    const int qt = SWA ? tile_rank : (n_qtiles - 1 - tile_rank);
    it.i0 = qt * p.bmp;
    return it;
  };
  const int half = p.rdim >> 1;
  const int bpp = p.bmp >> 5;  // 32-row blocks per head in the tile

  // ---- Phase 1: Q tile -> LDS, QK-norm + RoPE + scale in place ----------------------
  // The tile is bmp * group = kRows rows of DC 16-byte chunks. Thread t always holds chunk
  // dc = t % DC (kThreads is a multiple of DC) of rows q_row(i), so its 8 weights and the
  // RoPE partners of its 8 dims are fixed; the DC lanes holding one row sum its squares
  // with shuffles. All loads are issued before the first LDS write.
  constexpr int QIT = kRows * DC / kThreads;
  static_assert(QIT * kThreads == kRows * DC && kThreads % DC == 0, "Q chunks per thread");
  auto q_pi = [&](int i, int t) { return (t + i * kThreads) / (p.group * DC); };
  auto q_row = [&](int i, int t) {
    const int c = t + i * kThreads, cpp = p.group * DC, pi = c / cpp;
    return (c - pi * cpp) / DC * p.bmp + pi;
  };
  u32x4 qv[QIT];
  auto load_q = [&](const Item& it, const int tid) {
    const int dc = tid % DC;
    const bf16* qbase = p.q + (it.seq0 * p.Hq + (size_t)it.kvh * p.group) * D;
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
      const int c = tid + i * kThreads, cpp = p.group * DC;
      const int pi = c / cpp, hg = (c - pi * cpp) / DC;
      const int pos = min(it.i0 + pi, it.T - 1);   // rows past the end read a valid row, then zero
      qv[i] = *(const u32x4*)(qbase + (size_t)pos * p.Hq * D + hg * D + dc * 8);
    }
  };
  int k_item = 0, cur_lin = item_lin(0);
  Item cur = decode(cur_lin);
  if (cur.skip) return;   // the whole workgroup, before any barrier
  load_q(cur, tid0);
  if (tid0 < D) {
    sWq[tid0] = wq_l;
    sWk[tid0] = wk_l;
  }
  if (tid0 < kMaxHalfMfma) {
    sFr[tid0] = fr_hi;
    sFr[kMaxHalfMfma + tid0] = fr_lo;
  }
  __syncthreads();   // weights and RoPE steps are in LDS
  // Softmax form: after RMSNorm every score obeys |s| <= B = |qscale| d max|wq| max|wk|
  // (2 % margin for the bf16 operands). The bound is the same for every workgroup, so they
  // all take the same form: the static shift (score accumulators start at -B, p <= 1)
  // while B <= kStaticShiftMax, else the online max.
  float bound;
  {
    float wqm = 0.f, wkm = 0.f;
    for (int c = lane0; c < D; c += 64) {
      wqm = fmaxf(wqm, fabsf(sWq[c]));
      wkm = fmaxf(wkm, fabsf(sWk[c]));
    }
    bound = fabsf(p.qscale) * (float)D * wave_max(wqm) * wave_max(wkm) * 1.02f;
  }
  // Persistent launches with at most 64 positions per tile build each tile's RoPE table
  // by angle addition: cos/sin(b + o) from the exact angles of the tile's first position
  // b and of the offsets o = 0 .. 63 (the offsets once per workgroup), 4 FMAs per entry
  // in place of a reduced sine and cosine.
  const bool trig_add = PERSIST && p.bmp <= kBN;
  if (trig_add) {
    for (int e = tid0; e < p.bmp * half; e += kThreads) {
      const int o = e / half, j = e - o * half;
      float c, s;
      rope_cos_sin(o, sFr[j], sFr[kMaxHalfMfma + j], c, s);
      sOffT[o * kMaxHalfMfma + j] = make_float2(c, s);
    }
  }
  auto rest = [&](auto static_tag, const float sinit) {
  constexpr bool STATIC = decltype(static_tag)::value;
  int tid_c = tid0;
  for (;;) {
  // Persistent: the thread index passes through an empty assembly statement at the top
  // of every tile, so that the compiler cannot hoist what it derives from it (offsets,
  // row indices) out of this loop and hold it in registers across the key loop.
  if constexpr (PERSIST) asm volatile("" : "+v"(tid_c));
  const int tid = tid_c, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int b = cur.b, kvh = cur.kvh, T = cur.T, i0 = cur.i0;
  const size_t seq0 = cur.seq0, kt_row0 = cur.kt_row0, vt_tile0 = cur.vt_tile0;
  if (trig_add) {
    if (tid < half) {
      float c, s;
      rope_cos_sin(p.pos_offset + i0, sFr[tid], sFr[kMaxHalfMfma + tid], c, s);
      sBaseT[tid] = make_float2(c, s);
    }
    lds_barrier();   // the angle tables are in LDS; the output rows have left the Q region
  } else if (k_item > 0) {
    lds_barrier();   // every wave's output rows have left the Q region
  }
  {
    const int dc = tid % DC;
    for (int e = tid; e < p.bmp * half; e += kThreads) {
      const int pi = e / half, j = e - pi * half;
      float c, s;
      if (trig_add) {
        const float2 b = sBaseT[j], o = sOffT[pi * kMaxHalfMfma + j];
        c = __builtin_fmaf(b.x, o.x, -b.y * o.y);
        s = __builtin_fmaf(b.y, o.x, b.x * o.y);
      } else {
        rope_cos_sin(p.pos_offset + i0 + pi, sFr[j], sFr[kMaxHalfMfma + j], c, s);
      }
      sQtrig[pi * kQTrigStride + j] = make_float2(c, s);
    }
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      if (i0 + q_pi(it, tid) >= T) qv[it] = zero;
      *(u32x4*)(sQ + q_row(it, tid) * RW + dc * 8) = qv[it];
    }
    if (p.rdim == 2 * kModelHalf<D>) {
      // The model's rotary dim: one thread per tile row. The row comes from LDS into
      // registers whole, so the sum of squares needs no cross-lane reduction and each
      // rotated pair meets its partner in registers; the transformed row goes back in
      // place (no other thread reads it before the barrier below).
      constexpr int H = kModelHalf<D>;
      __syncthreads();   // raw rows and the trig table are in LDS
      for (int r = tid; r < kRows; r += kThreads) {
        bf16* row = sQ + r * RW;
        const float2* trig = sQtrig + (r % p.bmp) * kQTrigStride;
        uint32_t xw[D / 2];
#pragma unroll
        for (int k = 0; k < DC; ++k) {
          const u32x4 v = *(const u32x4*)(row + k * 8);
          xw[4 * k] = v.x;
          xw[4 * k + 1] = v.y;
          xw[4 * k + 2] = v.z;
          xw[4 * k + 3] = v.w;
        }
        float2 cs[H];
#pragma unroll
        for (int j = 0; j < H; ++j) cs[j] = trig[j];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < D / 2; ++i) {
          const bf16x2 t = __builtin_bit_cast(bf16x2, xw[i]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(t, t, ss, false);
        }
        const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps) * p.qscale;
        auto xv = [&](int c) -> float {
          return (c & 1) ? bf16_hi_to_f32(xw[c >> 1]) : bf16_lo_to_f32(xw[c >> 1]);
        };
#pragma unroll
        for (int k = 0; k < DC; ++k) {
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int c = 8 * k + e + u;
              const float a = xv(c) * sWq[c];
              float rv = a;
              if (c < H) {
                rv = __builtin_fmaf(a, cs[c].x, -(xv(c + H) * sWq[c + H]) * cs[c].y);
              } else if (c < 2 * H) {
                rv = __builtin_fmaf(a, cs[c - H].x, (xv(c - H) * sWq[c - H]) * cs[c - H].y);
              }
              y[u] = rv * rs;
            }
            const bf16x2 pr = {(bf16)y[0], (bf16)y[1]};
            o[e / 2] = __builtin_bit_cast(uint32_t, pr);
          }
          *(u32x4*)(row + k * 8) = (u32x4){o[0], o[1], o[2], o[3]};
        }
      }
    } else {
      // Per-dim constants of this thread's chunk: weight, RoPE partner (dim k pairs with
      // k + r/2), the partner's weight with the sign of its term (minus in the lower half),
      // and the pair index. Dims past rotary_dim take partner 0 and pair 0 (read, then
      // discarded): the loop below has no branches, so its LDS reads overlap.
      float wv[8], wp[8];
      int part[8], tj[8];
      bool rot[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = dc * 8 + e;
        const bool lower = c < half;
        rot[e] = c < p.rdim;
        part[e] = rot[e] ? (lower ? c + half : c - half) : 0;
        tj[e] = rot[e] ? (lower ? c : c - half) : 0;
        wv[e] = sWq[c];
        wp[e] = lower ? -sWq[part[e]] : sWq[part[e]];
      }
      __syncthreads();   // raw rows and the trig table are in LDS
      u32x4 res[QIT];
#pragma unroll
      for (int it = 0; it < QIT; ++it) {
        const uint32_t w4[4] = {qv[it].x, qv[it].y, qv[it].z, qv[it].w};
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_lo_to_f32(w4[e]);
          x[2 * e + 1] = bf16_hi_to_f32(w4[e]);
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
        ss = group_sum<DC>(ss);
        const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps) * p.qscale;
        const bf16* row = sQ + q_row(it, tid) * RW;
        const float2* trig = sQtrig + q_pi(it, tid) * kQTrigStride;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = x[e] * wv[e];
          const float b = (float)row[part[e]] * wp[e];
          const float2 cs = trig[tj[e]];
          const float r = __builtin_fmaf(a, cs.x, b * cs.y);
          y[e] = (rot[e] ? r : a) * rs;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = {(bf16)y[2 * e], (bf16)y[2 * e + 1]};
          res[it][e] = __builtin_bit_cast(uint32_t, pr);
        }
      }
      __syncthreads();   // every partner read of the raw rows is done
#pragma unroll
      for (int it = 0; it < QIT; ++it) *(u32x4*)(sQ + q_row(it, tid) * RW + dc * 8) = res[it];

    }
  }
  __syncthreads();
  // Q~ into registers as the B operand: lane holds query row l32 of its block and the
  // eight d values 16*ks + 8*hi .. +7 for each k-step.
  bf16x8 qreg[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = (wave * QB + qb) * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[qb][ks] = *(const bf16x8*)(sQ + row * RW + ks * 16 + hi * 8);
  }
  // Absolute positions of this lane's two query rows (for masking).
  int qpos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qpos[qb] = i0 + ((wave * QB + qb) % bpp) * 32 + l32;
  __syncthreads();  // the Q region is reused by the K/V tiles below

  // ---- Key-tile schedule ----------------------------------------------------------------
  // Tiles [kt_lo, kt_hi] meet the band. Unmasked tiles are those entirely below every
  // query of the tile (k0 + 63 <= i0) and, for SWA, entirely inside every query's window
  // (k0 > q_last - W). They run first, as one branch-free stretch in ascending key order
  // (the workgroups of one KV head, which share an XCD, then stream the same K/V tiles
  // at about the same time and hit in L2); the masked tiles (diagonal, band edge)
  // follow. Unmasked tiles are fully visible to every row, so the first tile always
  // gives the online variant a finite running max.
  const int q_last = min(i0 + p.bmp, T) - 1;
  const int kt_lo = SWA ? max(0, i0 - p.window + 1) / kBN : 0;
  const int kt_hi = q_last / kBN;
  const int kt_cm = i0 >= kBN - 1 ? (i0 - (kBN - 1)) / kBN + 1 : 0;   // first causal-masked
  const int kt_bm = (SWA && q_last - p.window >= 0) ? (q_last - p.window) / kBN : -1;
  int u_lo = max(kt_lo, kt_bm + 1), u_hi = min(kt_hi, kt_cm - 1);
  if (u_lo > u_hi) {
    u_lo = kt_lo;
    u_hi = kt_lo - 1;
  }
  const int n_unm = u_hi - u_lo + 1;
  const int n_hi_m = kt_hi - u_hi;
  const int n_tiles = kt_hi - kt_lo + 1;
  auto tile_of = [&](int i) -> int {
    if (i < n_unm) return u_lo + i;
    i -= n_unm;
    if (i < n_hi_m) return u_hi + 1 + i;
    return kt_lo + (i - n_hi_m);
  };

  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) pin_agpr(oacc[qb][db]);
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const bf16* kbase = p.k + (seq0 * p.Hkv + kvh) * D;
  const bf16* vbase = p.v + (seq0 * p.Hkv + kvh) * D;
  const bf16* ktsrc = KPRE ? p.kt + kt_row0 * D : nullptr;
  const bf16* vtsrc = KPRE ? p.vt + vt_tile0 * (size_t)(kBN * D) : nullptr;
  const size_t kvstride = (size_t)p.Hkv * D;

  // Global -> registers for tile kt (issued one tile ahead of its use). Rows past the
  // end are clamped to the last row: such keys are always masked out, and clamped
  // values keep the products finite.
  u32x4 kreg[KIT];
  u32x4 vreg[KG];
  auto fetch = [&](int kt) {
    const int k0 = kt * kBN;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int c = tid + it * kThreads;
      const int kr = c / DC, dc = c % DC;
      const int pos = min(k0 + kr, T - 1);
      kreg[it] = KPRE ? *(const u32x4*)(ktsrc + (size_t)pos * D + dc * 8)
                      : *(const u32x4*)(kbase + (size_t)pos * kvstride + dc * 8);
    }
    if constexpr (KPRE) {
      // pre-transposed tile: [D][64 keys] rows of 8 chunks, copied as they are
      const bf16* src = vtsrc + (size_t)kt * (kBN * D);
#pragma unroll
      for (int it = 0; it < KG; ++it) vreg[it] = *(const u32x4*)(src + (tid + it * kThreads) * 8);
    } else {
      // every thread carries KG keys x 8 dims of V; the key group is the fastest index
      // so that the transposed LDS writes of one instruction cover all banks
      const int kg = tid % (kBN / KG), dc = tid / (kBN / KG);
#pragma unroll
      for (int e = 0; e < KG; ++e) {
        const int pos = min(k0 + kg * KG + e, T - 1);
        vreg[e] = *(const u32x4*)(vbase + (size_t)pos * kvstride + dc * 8);
      }
    }
  };
  // Registers -> LDS buffer `buf`: K rows as they are (or raw, for the fused transform),
  // V transposed with the per-16-key slot permutation; fused path: the tile's RoPE table.
  auto stage = [&](int kt, int buf) {
    const int k0 = kt * kBN;
    bf16* sK = (bf16*)(smem + buf * S::kBuf);
    bf16* sVt = (bf16*)(smem + buf * S::kBuf + S::kK);
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int c = tid + it * kThreads;
      const int kr = c / DC, dc = c % DC;
      *(u32x4*)((KPRE ? sK : sKraw) + kr * RW + dc * 8) = kreg[it];
    }
    if constexpr (KPRE) {
#pragma unroll
      for (int it = 0; it < KG; ++it) {
        const int c = tid + it * kThreads;   // chunk c: row d = c / 8, 8 slots (c % 8)*8..
        *(u32x4*)(sVt + (c >> 3) * VW + (c & 7) * 8) = vreg[it];
      }
    } else {
      const int kg = tid % (kBN / KG), dc = tid / (kBN / KG);
      const int slot = vt_slot(kg * KG);   // KG consecutive keys keep consecutive slots
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wsel = dd >> 1;
        uint32_t h[KG];   // element dd of each key, in the low 16 bits
#pragma unroll
        for (int e = 0; e < KG; ++e)
          h[e] = (dd & 1) ? (vreg[e][wsel] >> 16) : (vreg[e][wsel] & 0xffffu);
        bf16* dst = sVt + (dc * 8 + dd) * VW + slot;
        if constexpr (KG == 4) {
          *(u32x2*)dst = (u32x2){h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        } else if constexpr (KG == 2) {
          *(uint32_t*)dst = h[0] | (h[1] << 16);
        } else {
          *(uint16_t*)dst = (uint16_t)h[0];
        }
      }
    }
    if (!KPRE) {
      for (int e = tid; e < kBN * half; e += kThreads) {
        const int kr = e / half, j = e - kr * half;
        float c, s;
        rope_cos_sin(p.pos_offset + k0 + kr, sFr[j], sFr[kMaxHalfMfma + j], c, s);
        sKtrig[kr * kMaxHalfMfma + j] = make_float2(c, s);
      }
    }
  };

  // LDS DMA of tile kt into buffer buf of the pipelined path. Piece j (0 .. NPW-1) is one
  // 1 KiB block per wave, its 64 lanes landing in consecutive 16-byte slots: the first
  // KPW pieces cover K~ (512 / D rows per block), the rest V^T (8 rows per block).
  // Each lane fetches the chunk that the swizzle puts in its slot; K~ rows past the end
  // are clamped to the last row (masked keys).
  constexpr int KPW = D / 8 / NW;   // K~ (and V^T) pieces per wave and tile
  constexpr int NPW = 2 * KPW;
  const uint32_t lds_smem = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  // Per-lane source offsets of the K~ pieces within a tile (row r of the tile, chunk c),
  // the same for every tile. A tile past the sequence end reads on into the next head's
  // rows or the workspace's kKtSlackRows rows of slack: always inside the workspace, and
  // such keys are always masked (their scores are replaced, not used), so no row is
  // clamped.
  constexpr int CPR = D / 8, RPB = 1024 / (2 * D);
  static_assert(kKtSlackRows >= kBN, "a whole tile of slack past the last K~ row");
  uint32_t kdma_off[KPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int r = (wave * KPW + j) * RPB + lane / CPR;
    kdma_off[j] = (uint32_t)(r * (2 * D) + chunk_pos<CPR>(r, lane % CPR) * 16);
  }
  auto dma_piece = [&](int kt, int buf, int j) {
    const uint32_t dst = lds_smem + buf * S::kDBuf;
    const int k0 = kt * kBN;
    if (j < KPW) {
      dma16(ktsrc + (size_t)k0 * D, kdma_off[j], dst + (wave * KPW + j) * 1024);
    } else {
      const int blk = wave * KPW + (j - KPW);
      const int d = blk * 8 + (lane >> 3);
      const int c = chunk_pos<8>(d, lane & 7);
      dma16(vtsrc + (size_t)kt * (kBN * D), (uint32_t)(d * 128 + c * 16),
            dst + S::kDK + blk * 1024);
    }
  };

  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};

  // Scores of one 32-key block (rows kb*32.. of the K~ tile) for every query block.
  auto qk = [&](const bf16* sK, int kb, f32x16 (&sacc)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[qb][r] = sinit;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *(const bf16x8*)(sK + (kb * 32 + l32) * RW + ks * 16 + hi * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], sacc[qb], 0, 0, 0);
    }
  };
  // Mask (edge tiles): scores of keys the row does not see become -inf.
  auto mask_block = [&](f32x16 (&sacc)[QB], int kb, const int (&rel)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = kb * 32 + (r >> 2) * 8 + (r & 3);  // key - k0 - 4*hi
        bool vis = off <= rel[qb];
        if (SWA) vis = vis && (off > rel[qb] - p.window);
        if (!vis) sacc[qb][r] = -INFINITY;
      }
  };
  // Online variant: this lane's largest (masked) score per query block.
  auto lane_max = [&](const f32x16 (&sacc)[QB], float (&mt)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = sacc[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, sacc[qb][r]);
      mt[qb] = fmaxf(mt[qb], m);
    }
  };
  // Online variant: raise the running max to the row's max over scores not yet
  // exponentiated (lazily: only when it grows by more than 8, so p <= 2^8), rescaling the
  // row sum and every P.V product accumulated so far. Every block whose P is formed after
  // this call must have its scores in `mt`, so that no P is formed against an older max.
  auto raise_max = [&](const float (&mt_lane)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mt = fmaxf(mt_lane[qb], __shfl_xor(mt_lane[qb], 32));
      const float m_old = m_run[qb];
      const bool raise = mt > m_old + 8.0f;
      if (__ballot(raise)) {
        const float m_new = raise ? mt : m_old;
        const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
        l_run[qb] *= alpha;
        acc_fence<QB, DB>(oacc);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) pin_agpr(oacc[qb][db]);
        m_run[qb] = m_new;
      }
    }
  };
  // Exponentiate against the running max (static variant: the accumulators already hold
  // s - B), round to bf16 (the P operand) and add the rounded values to the row sums.
  auto expo = [&](const f32x16 (&sacc)[QB], bf16x8 (&pb)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mu = (STATIC || m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float ls = l_run[qb];
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)fast_exp2(sacc[qb][jh * 8 + e] - mu);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {v[e], v[e + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
        }
        pb[qb][jh] = v;
      }
      l_run[qb] = ls;
    }
  };
  // One 32-key block: mask, (online) raise the max, exponentiate. The block's P.V must be
  // accumulated before the next block's probs() can raise the max again.
  auto probs = [&](f32x16 (&sacc)[QB], int kb, const int (&rel)[QB], bf16x8 (&pb)[QB][2],
                   auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if (MASKED) mask_block(sacc, kb, rel);
    if (!STATIC) {
      float mt[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mt[qb] = -INFINITY;
      lane_max(sacc, mt);
      raise_max(mt);
    }
    expo(sacc, pb);
  };
  // O^T += V^T P^T for one 32-key block.
  auto pv = [&](const bf16* sVt, int kb, bf16x8 (&pb)[QB][2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const bf16x8 a =
            *(const bf16x8*)(sVt + (db * 32 + l32) * VW + kb * 32 + jh * 16 + hi * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) mfma_acc(oacc[qb][db], a, pb[qb][jh]);
      }
    }
  };
  // One 64-key tile from LDS buffer `buf`. With two query blocks per wave the two 32-key
  // halves go one after the other (32 score registers live per block); with one query
  // block the halves form two independent MFMA chains. `mid` runs between the score
  // work and the P.V products (the global path stages the next tile there).
  auto compute = [&](int kt, int buf, auto masked_tag, auto&& mid) {
    const bf16* sK = (const bf16*)(smem + buf * S::kBuf);
    const bf16* sVt = (const bf16*)(smem + buf * S::kBuf + S::kK);
    const int k0 = kt * kBN;
    int rel[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) rel[qb] = qpos[qb] - k0 - 4 * hi;
    if constexpr (QB == 1) {
      f32x16 s0[1], s1[1];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[0][r] = sinit;
        s1[0][r] = sinit;
      }
      // The two waves sharing a SIMD run the same phases; raising the priority in the
      // MFMA phases lets the MFMA issuer win arbitration while the other wave's
      // softmax fills the gaps.
      set_prio<1>();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a0 = *(const bf16x8*)(sK + l32 * RW + ks * 16 + hi * 8);
        const bf16x8 a1 = *(const bf16x8*)(sK + (32 + l32) * RW + ks * 16 + hi * 8);
        s0[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[0][ks], s0[0], 0, 0, 0);
        s1[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[0][ks], s1[0], 0, 0, 0);
      }
      set_prio<0>();
      // Both blocks' P are formed before either P.V: the online max is raised once over
      // the whole tile, so that P of block 0 and block 1 share one max.
      bf16x8 p0[1][2], p1[1][2];
      if (decltype(masked_tag)::value) {
        mask_block(s0, 0, rel);
        mask_block(s1, 1, rel);
      }
      if (!STATIC) {
        float mt[1] = {-INFINITY};
        lane_max(s0, mt);
        lane_max(s1, mt);
        raise_max(mt);
      }
      expo(s0, p0);
      expo(s1, p1);
      mid();
      set_prio<1>();
      pv(sVt, 0, p0);
      pv(sVt, 1, p1);
      set_prio<0>();
    } else if constexpr (ZG_PREFILL_PIPE) {
      // Software pipeline within the tile, one wave per SIMD:
      //   QK(0) | QK(1) with softmax(0) | P.V(0) with softmax(1) | P.V(1)
      // so that each softmax phase runs under a stretch of independent MFMAs.
      f32x16 s0[QB], s1[QB];
      bf16x8 p0[QB][2], p1[QB][2];
      qk(sK, 0, s0);
      qk(sK, 1, s1);
      probs(s0, 0, rel, p0, masked_tag);
      mid();
      pv(sVt, 0, p0);
      probs(s1, 1, rel, p1, masked_tag);
      pv(sVt, 1, p1);
      constexpr int kQK = QB * KS;       // MFMAs of one 32-key score block
      constexpr int kPV = QB * DB * 2;   // MFMAs of one 32-key P.V block
      constexpr int kSM = QB * 32;       // VALU ops of one softmax block (exp, cvt, dot)
      // mask bits: 0x8 MFMA, 0x2 VALU, 0x400 transcendental, 0x100 LDS read
#pragma unroll
      for (int j = 0; j < kQK; ++j) __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
#pragma unroll
      for (int j = 0; j < kQK; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, kSM / kQK, 0);
      }
#pragma unroll
      for (int j = 0; j < kPV; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, kSM / kPV, 0);
      }
#pragma unroll
      for (int j = 0; j < kPV; ++j) __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sacc[QB];
        qk(sK, kb, sacc);
        bf16x8 pb[QB][2];
        probs(sacc, kb, rel, pb, masked_tag);
        if (kb == 0) mid();
        pv(sVt, kb, pb);
      }
    }
  };
  // Static shift, K~ / V tiles from the workspace: a fenced software pipeline over the
  // tile's two 32-key blocks,
  //   A: QK(0) | B: QK(1) + softmax(0) | C: P.V(0) + softmax(1) + DMA | D: P.V(1)
  // with the vector work cut into pieces placed between the MFMAs so that it issues in
  // their shadow (the P.V products are inline assembly, so the order is pinned with
  // scheduling barriers rather than left to the scheduler). Two query blocks per wave and
  // one wave per SIMD by default (ZG_GLOBAL_WAVES=4); one block per wave and two waves per
  // SIMD with ZG_GLOBAL_WAVES=8 (twice the LDS operand reads per product: 3 % slower at
  // T = 262,144, level at B = 4, T = 4096).
  // Per-lane byte offsets of the operand reads within a buffer: the K~ row of a lane is
  // kb*32 + l32 and its chunk 2*ks + hi; the V^T row is db*32 + l32 and its chunk
  // 4*kb + 2*jh + hi. Both swizzles depend on the row only through l32 & 15, so the
  // block indices kb / db become immediate offsets.
  int koff[KS], voff[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    koff[ks] = l32 * (2 * D) + chunk_pos<D / 8>(l32, 2 * ks + hi) * 16;
#pragma unroll
  for (int x = 0; x < 4; ++x) voff[x] = S::kDK + l32 * 128 + chunk_pos<8>(l32, 2 * x + hi) * 16;
  auto compute_pipe = [&](int kt, int buf, auto masked_tag, int dma_kt, int dma_buf) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int PV_STEPS = 2 * DB;
    constexpr int NP = 4 * QB;   // softmax pieces per 32-key block
    static_assert(PV_STEPS == KS && KS % NPW == 0, "DMA pieces spread evenly over a phase");
    const char* tb = smem + buf * S::kDBuf;
    const int k0 = kt * kBN;
    int rel[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) rel[qb] = qpos[qb] - k0 - 4 * hi;
    f32x16 sc[2][QB];
    u32x4 pw[2][QB][2];   // P as packed bf16 pairs: [block][qb][jh]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][qb][r] = sinit;
    // softmax piece j (0 .. NP-1) of block kb: query block j / 4, half j / 2 % 2 of the 16
    // scores, four of them (j % 2)
    auto sm_piece = [&](int kb, int j) {
      const int qb = j >> 2, jh = (j >> 1) & 1, eh = j & 1;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = jh * 8 + eh * 4 + e;
        float x = sc[kb][qb][r];
        if (MASKED) {
          const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
          if (off > rel[qb]) x = -INFINITY;
        }
        v[e] = fast_exp2(x);
      }
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const bf16x2 pr = {(bf16)v[e], (bf16)v[e + 1]};
        pw[kb][qb][jh][eh * 2 + (e >> 1)] = __builtin_bit_cast(uint32_t, pr);
        l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_run[qb], false);
      }
    };
    // The tile as one stream of MFMA slots (each: one A operand from LDS, one product
    // per query block): A = K~ block 0 by k-step, B = K~ block 1, C = V^T block 0 by
    // (d block, key half), D = V^T block 1.
    constexpr int NSLOT = 2 * KS + 2 * PV_STEPS;
    auto read_op = [&](int u) -> bf16x8 {
      if (u < 2 * KS) {
        const int kb = u / KS, ks = u % KS;
        return *(const bf16x8*)(tb + koff[ks] + kb * 32 * (2 * D));
      }
      // key half outer, d block inner: an accumulator recurs every DB slots
      const int t = (u - 2 * KS) % PV_STEPS, kb = (u - 2 * KS) / PV_STEPS;
      const int db = t % DB, jh = t / DB;
      return *(const bf16x8*)(tb + voff[2 * kb + jh] + db * 32 * 128);
    };
    // Operand o is read at slot rd_slot(o). With two query blocks per wave (one wave per
    // SIMD) the operands of phases A, B and C are read during phase A, three per slot, so
    // that the softmax phases issue no LDS reads (at T = 262,144 0.7 % faster than every
    // operand two slots ahead, at B = 4, T = 4096 3 %), and phase D's two slots ahead; with
    // one query block per wave (two waves per SIMD, half the registers) every operand two
    // slots ahead.
    auto rd_slot = [](int o) { return (QB == 2 && o < 3 * KS) ? o / 3 : (o < 2 ? 0 : o - 2); };
    bf16x8 ops[NSLOT];
    static_for<NSLOT>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
#pragma unroll
      for (int o = 0; o < NSLOT; ++o)
        if (rd_slot(o) == u) ops[o] = read_op(o);
      const bf16x8 a = ops[u];
      if constexpr (u < 2 * KS) {
        constexpr int kb = u / KS, ks = u % KS;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], sc[kb][qb], 0, 0, 0);
        if constexpr (kb == 1) {
          // B: softmax of block 0 under the block-1 score products
#pragma unroll
          for (int w = ks * NP / KS; w < (ks + 1) * NP / KS; ++w) sm_piece(0, w);
        }
      } else {
        constexpr int t = (u - 2 * KS) % PV_STEPS, kb = (u - 2 * KS) / PV_STEPS;
        constexpr int db = t % DB, jh = t / DB;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          mfma_acc_late(oacc[qb][db], a, __builtin_bit_cast(bf16x8, pw[kb][qb][jh]));
        if constexpr (kb == 0) {
          // C: softmax of block 1 under the block-0 P.V products
#pragma unroll
          for (int w = t * NP / PV_STEPS; w < (t + 1) * NP / PV_STEPS; ++w) sm_piece(1, w);
        }
      }
      // a later tile goes to its buffer, its NPW pieces spread over phase kDmaPhase
      if constexpr (u / KS == kDmaPhase && (u % KS) % (KS / NPW) == 0)
        dma_piece(dma_kt, dma_buf, (u % KS) / (KS / NPW));
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto nothing = [] {};

  int i = 0;
  if constexpr (KPRE && STATIC) {
    // K~ / V^T tiles go from the workspace straight into LDS (DMA), kDmaBufs - 1 tiles
    // ahead of their use, through kDmaBufs rotating buffers: one barrier per tile. Past
    // the end the last tile is fetched again into an idle buffer (in bounds, never read).
    constexpr int AHEAD = kDmaBufs - 1;
    static_assert(AHEAD >= 1 && S::kDLoop <= S::kUnion, "DMA buffers");
    const int last = n_tiles - 1;
#pragma unroll
    for (int a = 0; a < AHEAD; ++a)
#pragma unroll
      for (int j = 0; j < NPW; ++j) dma_piece(tile_of(min(a, last)), a, j);
    vm_wait<(AHEAD - 1) * NPW>();
    __syncthreads();
    int cur = 0;
    auto step = [&](int i, auto masked_tag) {
      const int ahead = (cur + AHEAD) % kDmaBufs;
      compute_pipe(tile_of(i), cur, masked_tag, tile_of(min(i + AHEAD, last)), ahead);
      vm_wait<(AHEAD - 1) * NPW>();   // this wave's DMA of tile i + 1 has landed ...
      __syncthreads();  // ... and every wave's; tile i's buffer may be overwritten
      cur = cur == kDmaBufs - 1 ? 0 : cur + 1;
    };
    for (; i < n_unm; ++i) step(i, std::integral_constant<bool, false>{});
    for (; i < n_tiles; ++i) step(i, std::integral_constant<bool, true>{});
    vm_wait<0>();   // no DMA may still be writing LDS when the workgroup ends
  } else if constexpr (KPRE) {
    // K~ comes ready-made: tile i + 1 is written to the other LDS buffer and tile i + 2
    // is fetched while tile i is computed, leaving one barrier per tile.
    fetch(tile_of(0));
    stage(tile_of(0), 0);
    if (n_tiles > 1) fetch(tile_of(1));
    __syncthreads();
    auto step = [&](int i, auto masked_tag) {
      // Branch-free: past the end, the last tile is re-staged into the idle buffer and
      // re-fetched (in-bounds and never read), so the loop body is one basic block.
      compute(tile_of(i), i & 1, masked_tag, [&] {
        stage(tile_of(min(i + 1, n_tiles - 1)), (i + 1) & 1);
        fetch(tile_of(min(i + 2, n_tiles - 1)));
      });
      __syncthreads();  // tile i + 1 is in LDS; tile i's buffer may be overwritten
    };
    for (; i < n_unm; ++i) step(i, std::integral_constant<bool, false>{});
    for (; i < n_tiles; ++i) step(i, std::integral_constant<bool, true>{});
  } else {
    // Fused K transform: stage the raw tile, transform it into the K~ buffer, compute.
    auto step = [&](int i, auto masked_tag) {
      const int kt = tile_of(i);
      const int buf = i & 1;
      stage(kt, buf);
      __syncthreads();  // tile i is in LDS; every wave is done with tile i - 2's buffer
      bf16* sK = (bf16*)(smem + buf * S::kBuf);
      const int kr = tid / TPR, sub = tid % TPR;
      const bf16* r = sKraw + kr * RW;
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < DC / TPR; ++c) {
        const u32x4 v = *(const u32x4*)(r + (sub * (DC / TPR) + c) * 8);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16_lo_to_f32(w4[e]), bb = bf16_hi_to_f32(w4[e]);
          ss = __builtin_fmaf(a, a, ss);
          ss = __builtin_fmaf(bb, bb, ss);
        }
      }
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o);
      const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
      transform_row<D>(r, sK + kr * RW, sWk, sKtrig + kr * kMaxHalfMfma, rn, 1.0f, p.rdim,
                       sub, TPR);
      __syncthreads();  // K~ ready; sKraw / sKtrig free for the next stage()
      if (i + 1 < n_tiles) fetch(tile_of(i + 1));  // in flight during this tile's math
      compute(kt, buf, masked_tag, nothing);
    };
    fetch(tile_of(0));
    for (; i < n_unm; ++i) step(i, std::integral_constant<bool, false>{});
    for (; i < n_tiles; ++i) step(i, std::integral_constant<bool, true>{});
  }

  // The next query tile's Q rows load under this tile's epilogue (persistent launch).
  const int nlin = item_lin(k_item + 1);
  const bool more = PERSIST && nlin < p.n_blocks;
  const Item nxt = decode(more ? nlin : cur_lin);
  if (more) load_q(nxt, tid);

  // ---- Epilogue: O = acc / l (* sigmoid(G)), bf16 store ------------------------------
  // Each wave stages its QB * 32 rows in its own slice of the (now idle) Q region, then
  // stores whole 16-byte chunks of contiguous rows (a lane of the accumulator layout
  // holds 4 consecutive dims of a row; stored as they are, every store instruction
  // would touch 32 rows).
  acc_fence<QB, DB>(oacc);
  __syncthreads();   // every wave is done reading the tile buffers
  bf16* sO = sQ + wave * (QB * 32) * RW;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = 1.0f / lt;
    const int pos = min(qpos[qb], T - 1);   // rows past the end are staged, never stored
    const int hg = (wave * QB + qb) / bpp;
    if (p.lse != nullptr && hi == 0 && qpos[qb] < T) {
      // the probabilities were exp2(s - shift) with s in log2 units: the row's log-sum-exp
      // is log2(l) + shift, returned in natural-log units
      const float shift = STATIC ? -sinit : m_run[qb];
      p.lse[((size_t)b * p.Hq + kvh * p.group + hg) * T + qpos[qb]] =
          (__log2f(lt) + shift) * 0.6931471805599453f;
    }
    const size_t rowoff = ((seq0 + pos) * p.Hq + kvh * p.group + hg) * D;
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
        const bf16x4 ov = {(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
        *(bf16x4*)(sO + (qb * 32 + l32) * RW + d0) = ov;
      }
    }
  }
  // The slice is this wave's own: its LDS operations complete in order, so a wait for
  // its writes is all the reads below need.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int OIT = QB * 32 * DC / 64;
#pragma unroll
  for (int it = 0; it < OIT; ++it) {
    const int c = lane + it * 64;
    const int r = c / DC, dc = c % DC;
    const int blk = wave * QB + r / 32;
    const int pos = i0 + (blk % bpp) * 32 + r % 32;
    const u32x4 v = *(const u32x4*)(sO + r * RW + dc * 8);
    if (pos < T) {
      const int h = kvh * p.group + blk / bpp;
      *(u32x4*)(p.out + ((seq0 + pos) * p.Hq + h) * D + dc * 8) = v;
    }
  }
  if (!more) break;
  cur = nxt;
  cur_lin = nlin;
  ++k_item;
  }
  };
  if (bound <= kStaticShiftMax)
    rest(std::true_type{}, -bound);
  else
    rest(std::false_type{}, 0.f);

}

// Score bound (uniform over the grid): after RMSNorm, ||q^|| <= sqrt(d) max|wq| and
// ||k^|| <= sqrt(d) max|wk|, so every log2-domain score obeys
// |s| <= qscale * d * max|wq| * max|wk| (2% margin for the bf16 rounding of q~ and k~).
// One launch: a query tile per workgroup, or several per workgroup when the grid is
// smaller than the tile count (the softmax form is chosen inside).
template <int D, bool SWA, bool KPRE, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(const KArgs p) {
  prefill_tile<D, SWA, KPRE, NW>(p);
}

template <int D, bool SWA, bool KPRE, int NW = kWavesPerBlock>
hipError_t launch_t(const KArgs& ka, int grid, hipStream_t s) {
  constexpr int smem = Smem<D>::kTotal;
  constexpr int kThreads = NW * 64;
  auto kern = prefill_bf16_kernel<D, SWA, KPRE, NW>;
  hipError_t e = ensure_dynamic_smem((const void*)kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), smem, s, ka);
  return hipGetLastError();
}


// The global path's pre-pass, one 64-key tile per workgroup:
//   * K~ rows (RMSNorm * wk, then partial RoPE at the row's position within its sequence)
//     into the workspace's row layout [B][Hkv][T][D] (packed: [Hkv][T][D]). Rows are written
//     only for positions inside the sequence (in the dense layout the rows after a head's
//     last one belong to the next head). D / 8 lanes per row, 8 dims each; rotated partners
//     go through LDS.
//   * V transposed into tiles [B][Hkv][ceil(T/64)][D][64] with the 64 keys of each row in
//     the slot order of the attention kernel's LDS V^T tile (keys past the end are 0), so
//     that the attention kernel stages V^T tiles with plain 16-byte copies. Packed
//     documents (cu != nullptr, B == 1): blockIdx.z is the document, its tiles start at its
//     own first token and go to slots doc_tile_base(start, doc) .. of each KV head's
//     vt_slots.
// Every K and V load of a thread is issued before the first is used.
template <int D>
__global__ __launch_bounds__(256) void kv_prepass_kernel(const bf16* k, const bf16* v,
                                                         const float* wk, bf16* kt, bf16* vt,
                                                         int T, int Hkv, int n_kt,
                                                         const int32_t* cu, int max_len,
                                                         int vt_slots, int rdim, int pos_offset,
                                                         float eps, RopeFreq fr) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;              // rows per pass (16 lanes per row at d 128)
  constexpr int NP = kBN / RPP;               // passes over the tile's 64 rows
  __shared__ __attribute__((aligned(16))) bf16 sv[kBN][D + 8];
  __shared__ float sx[RPP][D + 4];
  __shared__ float2 st[RPP][kMaxHalfRot / 2 + 1];
  const int tile = blockIdx.x, hb = blockIdx.y;
  const int b = hb / Hkv, kvh = hb % Hkv;
  const int tid = threadIdx.x, sub = tid % CPR, r0 = tid / CPR;
  size_t seq0 = (size_t)b * T, kt_row0 = ((size_t)b * Hkv + kvh) * T;
  int len = T;
  size_t out_tile = (size_t)hb * n_kt + tile;
  if (cu) {
    const int doc = blockIdx.z;
    int start;
    doc_range(cu, doc, T, max_len, start, len);
    if (tile * kBN >= len) return;
    seq0 = start;
    kt_row0 = (size_t)kvh * T + start;
    out_tile = (size_t)kvh * vt_slots + doc_tile_base(start, doc) + tile;
  }
  // all loads first: pass i covers rows r0 + RPP i
  u32x4 kv4[NP], vv4[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pos = tile * kBN + r0 + RPP * i;
    kv4[i] = vv4[i] = (u32x4){0u, 0u, 0u, 0u};
    if (pos < len) {
      const size_t off = ((seq0 + pos) * Hkv + kvh) * D + sub * 8;
      kv4[i] = *(const u32x4*)(k + off);
      vv4[i] = *(const u32x4*)(v + off);
    }
  }
  float w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = wk[sub * 8 + e];
  const int half = rdim >> 1;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = r0 + RPP * i;          // tile row of this lane in pass i
    const int pos = tile * kBN + r;
    *(u32x4*)&sv[r][sub * 8] = vv4[i];
    // RoPE table of the pass's rows (rows past the end are computed and unused)
    for (int e = tid; e < RPP * half; e += 256) {
      const int rr = e / half, j = e - rr * half;
      float c, sn;
      rope_cos_sin(pos_offset + tile * kBN + rr + RPP * i, fr.hi[j], fr.lo[j], c, sn);
      st[rr][j] = make_float2(c, sn);
    }
    // normalise (sum of squares over the row's lanes) and stage for the partner reads
    const uint32_t w4[4] = {kv4[i].x, kv4[i].y, kv4[i].z, kv4[i].w};
    float x[8], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo_to_f32(w4[e]);
      x[2 * e + 1] = bf16_hi_to_f32(w4[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    ss = group_sum<CPR>(ss);
    const float rn = 1.0f / sqrtf(ss / D + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = x[e] * rn * w[e];
      sx[r0][sub * 8 + e] = x[e];
    }
    __syncthreads();
    // rotate and store the K~ rows inside the sequence
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dims past rotary_dim read pair 0 and partner 0 and keep their value
      const int c = sub * 8 + e;
      const bool rot = c < rdim, lower = c < half;
      const float2 cs = st[r0][rot ? (lower ? c : c - half) : 0];
      const float pr = sx[r0][rot ? (lower ? c + half : c - half) : 0];
      const float y = lower ? x[e] * cs.x - pr * cs.y : x[e] * cs.x + pr * cs.y;
      o[e] = (bf16)(rot ? y : x[e]);
    }
    if (pos < len) *(bf16x8*)(kt + (kt_row0 + pos) * D + sub * 8) = o;
    __syncthreads();   // sx / st free for the next pass; sv complete after the last
  }
  // V^T tile, keys in slot order (rows past the end were staged as zeros)
  bf16* out = vt + out_tile * (kBN * D);
  for (int c = tid; c < D * (kBN / 8); c += 256) {
    const int d = c / (kBN / 8), sc = c % (kBN / 8);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = sv[vt_slot(sc * 8 + e)][d];  // the slot map is an involution
    *(bf16x8*)(out + d * kBN + sc * 8) = o;
  }
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
  ka.kt = (const bf16*)a.kt;
  ka.vt = (const bf16*)a.vt;
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
  ka.cu = a.cu;
  ka.max_len = a.max_len;
  ka.vt_slots = a.cu ? varlen_vtile_slots(a.T, a.n_docs) : 0;
  if (a.cu) {   // one (document, KV head) per sequence slot, tiles sized by the longest
    ka.n_hb = a.n_docs * a.Hkv;
    ka.n_qtiles = (a.max_len + ka.bmp - 1) / ka.bmp;
  }
  const int n_blocks = ka.n_qtiles * ka.n_hb;
  if (n_blocks == 0) return hipSuccess;
  ka.n_blocks = n_blocks;
  ka.lse = (a.swa || a.cu) ? nullptr : a.lse;
  if (swa_stream_supported(a)) return launch_swa_stream(a, s);
  const bool kpre = (a.kt != nullptr);
  // Global layers of dense batches with K~ / V tiles from the workspace run persistent:
  // one workgroup per CU (a multiple of 8 when the tiles are dealt out per XCD), each
  // walking its share of the query tiles, so that a tile's Q load overlaps the previous
  // tile's epilogue. Everything else: one workgroup per query tile.
  int grid = n_blocks;
  if (ZG_PERSISTENT && kpre && !a.swa && a.cu == nullptr) {
    int cus = 0;
    hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    if (ka.n_hb % kXcds == 0) cus -= cus % kXcds;
    if (cus > 0 && cus < n_blocks) grid = cus;
  }
  if (a.d == 128) {
    if (a.swa) return launch_t<128, true, false>(ka, grid, s);
    return kpre ? launch_t<128, false, true, ZG_GLOBAL_WAVES>(ka, grid, s)
                : launch_t<128, false, false>(ka, grid, s);
  }
  if (a.swa) return launch_t<64, true, false>(ka, grid, s);
  return kpre ? launch_t<64, false, true, ZG_GLOBAL_WAVES>(ka, grid, s)
              : launch_t<64, false, false>(ka, grid, s);
}

}  // namespace zg

namespace zg {

size_t prefill_vtiles_bytes(int B, int Hkv, int T, int d) {
  return (size_t)B * Hkv * ((T + kBN - 1) / kBN) * kBN * d * 2;
}

size_t prefill_vtiles_bytes_varlen(int Hkv, int T, int n_docs, int d) {
  return (size_t)Hkv * varlen_vtile_slots(T, n_docs) * kBN * d * 2;
}

hipError_t launch_kv_prepass(const PrefillArgs& a, hipStream_t s) {
  const bool packed = a.cu != nullptr;
  const int n_kt = ((packed ? a.max_len : a.T) + kBN - 1) / kBN;
  const dim3 grid(n_kt, packed ? a.Hkv : a.B * a.Hkv, packed ? a.n_docs : 1);
  const int slots = packed ? varlen_vtile_slots(a.T, a.n_docs) : 0;
  if (n_kt == 0) return hipSuccess;
  if (a.d == 128)
    hipLaunchKernelGGL(kv_prepass_kernel<128>, grid, dim3(256), 0, s, (const bf16*)a.k,
                       (const bf16*)a.v, a.wk, (bf16*)a.kt, (bf16*)a.vt, a.T, a.Hkv, n_kt, a.cu,
                       a.max_len, slots, a.rdim, a.pos_offset, a.eps, a.fr);
  else
    hipLaunchKernelGGL(kv_prepass_kernel<64>, grid, dim3(256), 0, s, (const bf16*)a.k,
                       (const bf16*)a.v, a.wk, (bf16*)a.kt, (bf16*)a.vt, a.T, a.Hkv, n_kt, a.cu,
                       a.max_len, slots, a.rdim, a.pos_offset, a.eps, a.fr);
  return hipGetLastError();
}


}  // namespace zg
