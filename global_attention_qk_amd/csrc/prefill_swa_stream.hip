// Gated sliding-window prefill as a stream along the sequence (bf16, head_dim 128, four
// query heads per KV head, rotary_dim 42, window <= 128: the model's layer shape).
//
// What is computed (hyper.ai summary of arXiv 2609.13356, section 方法, GatedSWA equation;
// "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ): every query row attends, after
// RMSNorm + partial RoPE of q and k, to the `window` most recent keys including itself,
// and the result is multiplied elementwise by sigmoid(G).
//
// Such a layer reads Q, K, V and G once and writes O once (28 KiB per position at 32
// query / 8 KV heads), while its MFMA work is small: it is bound by HBM bandwidth, and the
// design aims at keeping loads in flight rather than at MFMA throughput.
//
//   * A workgroup (8 wave64s) owns one (batch, KV head) and a contiguous segment of the
//     sequence, which it walks 64 positions per step. The 256 query rows of a step are the
//     4 heads x 64 positions; wave w takes head w % 4 and the 32 positions 32 * (w / 4) ..
//     of the step, one query per lane (scores are formed transposed, S^T = K~ Q~^T, so P
//     lands in the B-operand layout of O^T += V^T P^T).
//   * K~ (normalised, rotated) and V^T live in LDS as a ring of six 32-key blocks: each
//     key block is loaded from HBM, transformed and transposed once per segment, and each
//     wave reads the five blocks its window touches (one band-edge block, three full
//     blocks, the diagonal block).
//   * Loads run ahead of use: the next step's Q goes straight into registers in the MFMA
//     operand layout, the next key tile into registers and then LDS, and the gate of the
//     current step is issued at the step's start so that it has landed by the epilogue.
//   * Head dims are permuted inside the products (the same permutation on both operands
//     of each product): in Q~ . K~ a lane's two halves hold dims [0, 64) and [64, 128),
//     so the rotated pairs (j, j + 21) never cross lanes; in O^T the V^T rows are ordered
//     so that a lane's sixteen accumulator registers of a 32-dim block are sixteen
//     consecutive dims, which makes the G loads and O stores 16-byte accesses.
//   * Static softmax shift as in the other prefill kernel: when the score bound implied
//     by the norm weights is moderate, p = exp2(s) with no running max; otherwise an
//     online-max variant runs (both are launched; each returns unless selected).
#include <type_traits>

#include "launch.h"

namespace zg {
namespace {

constexpr int kD = 128;
constexpr int kG = 4;              // query heads per KV head
constexpr int kRH = 21;            // rotated pairs (rotary_dim 42)
constexpr int kRHP = 22;           // trig table row stride (16-byte aligned rows)
constexpr int kStep = 64;          // positions per step
constexpr int kBK = 32;            // keys per ring block
constexpr int kRing = 6;           // ring blocks
constexpr int kNB = 5;             // blocks a 32-row wave visits per step (window <= 128)
constexpr int kThreads = 512;
constexpr int kMaxWindow = 128;
constexpr int kMinSegSteps = 4;
constexpr float kStaticShiftMax = 96.0f;

constexpr int kKRowB = kD * 2 + 16;        // padded K~ row
constexpr int kKBlkB = kBK * kKRowB;       // K~ block: 32 rows
constexpr int kVBlkB = kD * kBK * 2;       // V^T block: 128 rows x 64 B
constexpr int kRawRowB = kD * 2 + 16;      // padded raw K row
constexpr int kRawB = kStep * kRawRowB;
constexpr int kTrigB = kStep * kRHP * 8;
constexpr int kOffK = 0;
constexpr int kOffV = kOffK + kRing * kKBlkB;
constexpr int kOffRaw = kOffV + kRing * kVBlkB;   // two raw K buffers
constexpr int kOffTrig = kOffRaw + 2 * kRawB;     // two trig tables
constexpr int kOffW = kOffTrig + 2 * kTrigB;      // wq * qscale, wk
constexpr int kSmem = kOffW + 2 * kD * 4;
static_assert(kSmem <= 160 * 1024, "LDS budget");

struct SArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* g;
  bf16* out;
  const float* wq;
  const float* wk;
  int T, Hq, Hkv, window, pos_offset;
  int n_hb, seg_steps, n_steps;
  float eps, qscale;
  RopeFreq fr;
};

__device__ __forceinline__ int ring_slot(int kb) { return (kb + 4 * kRing) % kRing; }  // kb >= -4

// K~ block: rows padded by 16 bytes, so one 16-byte chunk read across 16 consecutive keys
// touches every bank once, and a lane's chunks are one base plus immediate offsets.
__device__ __forceinline__ int kblk_off(int row, int chunk) { return row * kKRowB + (chunk << 4); }
// V^T block: row m (0..127) holds 32 key slots (64 B); chunk c at c ^ ((m >> 2) & 3).
__device__ __forceinline__ int vblk_off(int m, int chunk) {
  return m * (kBK * 2) + ((chunk ^ ((m >> 2) & 3)) << 4);
}
// Row of a 32-dim block that holds dim dd: rows are ordered so that accumulator register
// r of lane half h is dim 16 h + r.
__device__ __forceinline__ int vt_row_of_dim(int dd) {
  return 8 * ((dd >> 2) & 3) + 4 * (dd >> 4) + (dd & 3);
}
// Swap bits 2 and 3 of a key index within its 16-key group (which keys a lane holds in
// the S^T accumulator, in B-operand order).
__device__ __forceinline__ int key_slot(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// All accumulators are VGPRs (no AGPRs are used, so the compiler may give the whole
// 256-register budget of two waves per SIMD to VGPRs).
__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A value the optimiser must treat as recomputed here: keeps lane-derived indices from
// being hoisted out of the step loop and held in registers for its whole length.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Sum over the 8 lanes of an aligned lane octet (DPP: xor 1, xor 2, then mirror within 8).
__device__ __forceinline__ float octet_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float bf16_elem(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? bf16_hi_to_f32(w) : bf16_lo_to_f32(w);
}

template <bool STATIC>
__global__ __launch_bounds__(kThreads, 1) void swa_stream_kernel(const SArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sWq = (float*)(smem + kOffW);
  float* sWk = sWq + kD;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;     // query column of this lane
  const int hi = lane >> 5;
  const int hg = wave & 3;     // head within the group
  const int ph = wave >> 2;    // which 32 positions of the step

  for (int i = tid; i < kD; i += kThreads) {
    sWq[i] = p.wq[i] * p.qscale;
    sWk[i] = p.wk[i];
  }
  __syncthreads();
  {
    // |s| <= d * max|wq * qscale| * max|wk| after RMSNorm (2% margin for bf16 operands).
    float wqm = 0.f, wkm = 0.f;
    for (int c = lane; c < kD; c += 64) {
      wqm = fmaxf(wqm, fabsf(sWq[c]));
      wkm = fmaxf(wkm, fabsf(sWk[c]));
    }
    wqm = wave_max(wqm);
    wkm = wave_max(wkm);
    const bool use_static = (float)kD * wqm * wkm * 1.02f <= kStaticShiftMax;
    if (use_static != STATIC) return;
  }

  const int lin = blockIdx.x;
  const int hb = lin % p.n_hb;
  const int seg = lin / p.n_hb;
  const int b = hb / p.Hkv;
  const int kvh = hb % p.Hkv;
  const int s_begin = seg * p.seg_steps;
  const int s_end = min(s_begin + p.seg_steps, p.n_steps);
  if (s_begin >= s_end) return;
  const int T = p.T;
  const int W = p.window;
  const int h = kvh * kG + hg;
  const size_t qstride = (size_t)p.Hq * kD;
  const size_t qoff = ((size_t)b * T * p.Hq + h) * kD;
  const size_t kvstride = (size_t)p.Hkv * kD;
  const bf16* kbase = p.k + ((size_t)b * T * p.Hkv + kvh) * kD;
  const bf16* vbase = p.v + ((size_t)b * T * p.Hkv + kvh) * kD;

  // ---- loads -----------------------------------------------------------------------
  // Q of step s in the B-operand layout: this lane's query, dims 64 hi + 8 ks .. + 7.
  auto load_q = [&](int s, u32x4 (&dst)[8]) {
    const int pos = min(s * kStep + 32 * ph + n, T - 1);
    const bf16* src = p.q + qoff + (size_t)pos * qstride + hi * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) dst[ks] = *(const u32x4*)(src + ks * 8);
  };
  // G of step s in the O^T accumulator layout: dims 32 db + 16 hi .. + 15.
  auto load_g = [&](int s, u32x4 (&dst)[4][2]) {
    const int pos = min(s * kStep + 32 * ph + n, T - 1);
    const bf16* src = p.g + qoff + (size_t)pos * qstride + hi * 16;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) dst[db][e] = *(const u32x4*)(src + db * 32 + e * 8);
  };
  // K and V rows of tile t (positions 64 t .., clamped into [0, T); such rows are never
  // visible and keep every product finite). K: chunks (tid & 7) and (tid & 7) + 8 of row
  // tid >> 3. V: rows 2 (tid & 31) and + 1, chunk tid >> 5.
  auto load_kv = [&](int t, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
    const int k0 = t * kStep;
    const int tl = opaque(tid);
    const int krow = tl >> 3, kc = tl & 7;
    const bf16* ks = kbase + (size_t)min(max(k0 + krow, 0), T - 1) * kvstride;
    kr[0] = *(const u32x4*)(ks + kc * 8);
    kr[1] = *(const u32x4*)(ks + (kc + 8) * 8);
    const int kp = tl & 31, vc = tl >> 5;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int pos = min(max(k0 + 2 * kp + e, 0), T - 1);
      vr[e] = *(const u32x4*)(vbase + (size_t)pos * kvstride + vc * 8);
    }
  };

  // ---- LDS producers -----------------------------------------------------------------
  // RoPE cos/sin of the 64 positions of tile t.
  auto make_trig = [&](int t, int buf) {
    float2* tr = (float2*)(smem + kOffTrig + buf * kTrigB);
    for (int e = tid; e < kStep * kRH; e += kThreads) {
      const int pl = e / kRH, j = e - pl * kRH;
      float c, s;
      rope_cos_sin(p.pos_offset + max(t * kStep + pl, 0), p.fr.hi[j], p.fr.lo[j], c, s);
      tr[pl * kRHP + j] = make_float2(c, s);
    }
  };
  auto stage_k = [&](const u32x4 (&kr)[2], int buf) {
    char* raw = smem + kOffRaw + buf * kRawB;
    const int t8 = opaque(tid);
    const int krow = t8 >> 3, kc = t8 & 7;
    *(u32x4*)(raw + krow * kRawRowB + kc * 16) = kr[0];
    *(u32x4*)(raw + krow * kRawRowB + (kc + 8) * 16) = kr[1];
  };
  // RMSNorm + partial RoPE of the staged tile t into its two ring blocks. Eight lanes per
  // key; a lane writes dims 8 kc .. + 7 (rotated where < 42, partner read from the raw
  // row) and 64 + 8 kc .. + 7 (never rotated).
  auto transform_k = [&](const u32x4 (&kr)[2], int t, int buf) {
    const char* raw = smem + kOffRaw + buf * kRawB;
    const float2* tr = (const float2*)(smem + kOffTrig + buf * kTrigB);
    const int t8 = opaque(tid);
    const int krow = t8 >> 3, kc = t8 & 7;
    float x0[8], x1[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x0[e] = bf16_elem(kr[0], e);
      x1[e] = bf16_elem(kr[1], e);
      ss = __builtin_fmaf(x0[e], x0[e], ss);
      ss = __builtin_fmaf(x1[e], x1[e], ss);
    }
    ss = octet_sum(ss);
    const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + p.eps);
    const bf16* rrow = (const bf16*)(raw + krow * kRawRowB);
    bf16x8 o0, o1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = kc * 8 + e;
      const bool rot = d < 2 * kRH;
      const bool first = d < kRH;
      const int j = first ? d : d - kRH;
      const int pd = rot ? (first ? d + kRH : d - kRH) : d;
      const float xp = (float)rrow[pd] * sWk[pd];
      float c = 1.f, s = 0.f;
      if (rot) {
        const float2 cs = tr[krow * kRHP + j];
        c = cs.x;
        s = first ? -cs.y : cs.y;
      }
      o0[e] = (bf16)((x0[e] * sWk[d] * c + xp * s) * rn);
      o1[e] = (bf16)(x1[e] * sWk[64 + d] * rn);
    }
    const int kb = 2 * t + (krow >> 5);
    char* blk = smem + kOffK + ring_slot(kb) * kKBlkB;
    const int row = krow & 31;
    *(bf16x8*)(blk + kblk_off(row, kc)) = o0;
    *(bf16x8*)(blk + kblk_off(row, kc + 8)) = o1;
  };
  // V of tile t, transposed into its two ring blocks (keys 2 kp, 2 kp + 1 of the tile are
  // adjacent slots, so each store is one 32-bit word).
  auto stage_v = [&](const u32x4 (&vr)[2], int t) {
    const int tv = opaque(tid);
    const int kp = tv & 31, vc = tv >> 5;
    const int key = 2 * kp;
    char* blk = smem + kOffV + ring_slot(2 * t + (key >> 5)) * kVBlkB;
    const int sl = key_slot(key & 31);
    const int chunk = sl >> 3, within = sl & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = vc * 8 + e;
      const int m = (d & ~31) + vt_row_of_dim(d & 31);
      const uint32_t w0 = vr[0][e >> 1], w1 = vr[1][e >> 1];
      const uint32_t word = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                    : ((w0 & 0xffffu) | (w1 << 16));
      *(uint32_t*)(blk + vblk_off(m, chunk) + within * 2) = word;
    }
  };
  // RMSNorm + RoPE + scale of this lane's query row (64 dims per lane half; the rotated
  // dims [0, 42) all sit in the lower half), as the B operand.
  auto q_transform = [&](const u32x4 (&raw)[8], int buf, bf16x8 (&qreg)[8]) {
    // values are unpacked where used, so that no 64-float copy of the row is live
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float xv = bf16_elem(raw[i >> 3], i & 7);
      ss = __builtin_fmaf(xv, xv, ss);
    }
    ss += __shfl_xor(ss, 32);
    const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + p.eps);
    const float* w = sWq + hi * 64;
    const float2* tr = (const float2*)(smem + kOffTrig + buf * kTrigB) + (32 * ph + n) * kRHP;
#pragma unroll
    for (int j = 0; j < kRH; ++j) {
      const float2 cs = tr[j];
      const float c = hi ? 1.f : cs.x;
      const float sn = hi ? 0.f : cs.y;
      const float a = bf16_elem(raw[j >> 3], j & 7) * w[j];
      const float bb = bf16_elem(raw[(j + kRH) >> 3], (j + kRH) & 7) * w[j + kRH];
      qreg[j >> 3][j & 7] = (bf16)((a * c - bb * sn) * rn);
      qreg[(j + kRH) >> 3][(j + kRH) & 7] = (bf16)((bb * c + a * sn) * rn);
    }
#pragma unroll
    for (int i = 2 * kRH; i < 64; ++i) qreg[i >> 3][i & 7] = (bf16)(bf16_elem(raw[i >> 3], i & 7) * w[i] * rn);
  };

  // ---- attention state -----------------------------------------------------------------
  f32x16 oacc[4];
  float l_run = 0.f, m_run = -INFINITY;
  auto reset_acc = [&] {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    }
    l_run = 0.f;
    m_run = -INFINITY;
  };
  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};

  // One 32-key ring block for this wave's 32 queries of step s.
  auto do_block = [&](int s, int jb, const bf16x8 (&qreg)[8], auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int kb = 2 * s - 4 + ph + jb;
    const int ln = opaque(lane);
    const int n = ln & 31, hi = ln >> 5;
    const char* sK = smem + kOffK + ring_slot(kb) * kKBlkB;
    const char* sV = smem + kOffV + ring_slot(kb) * kVBlkB;
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = *(const bf16x8*)(sK + kblk_off(n, 8 * hi + ks));
      sacc = mfma(a, qreg[ks], sacc);
    }
    if (MASKED) {
      // key - query for register r: 32 kb + 8 (r / 4) + 4 hi + r % 4 - q
      const int rel = 32 * kb + 4 * hi - (s * kStep + 32 * ph + n);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dk = rel + (r >> 2) * 8 + (r & 3);
        if (dk > 0 || dk <= -W) sacc[r] = -INFINITY;
      }
    }
    float mu = 0.f;
    if (!STATIC) {
      float mt = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_old = m_run;
      const bool raise = mt > m_old + 8.0f;
      if (__ballot(raise)) {
        const float m_new = raise ? mt : m_old;
        const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
      }
      mu = (m_run == -INFINITY) ? 0.f : m_run;
    }
    bf16x8 pb[2];
    float ls = l_run;
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = (bf16)fast_exp2(STATIC ? sacc[jh * 8 + e] : sacc[jh * 8 + e] - mu);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {v[e], v[e + 1]};
        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
      }
      pb[jh] = v;
    }
    l_run = ls;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const bf16x8 a = *(const bf16x8*)(sV + vblk_off(db * 32 + n, 2 * jh + hi));
        oacc[db] = mfma(a, pb[jh], oacc[db]);
      }
  };
  // Blocks [j0, j1) of step s. The band-edge block (0) and the diagonal block (4) are
  // masked, and every block when the window is shorter than 128; blocks wholly before
  // position 0 or wholly outside the window are skipped (uniform per wave).
  auto blocks = [&](int s, int j0, int j1, const bf16x8 (&qreg)[8]) {
    const int q_lo = s * kStep + 32 * ph;
    for (int jb = j0; jb < j1; ++jb) {
      const int kb = 2 * s - 4 + ph + jb;
      if (kb < 0 || 32 * kb + 31 <= q_lo - W) continue;
      if (jb == 0 || jb == kNB - 1 || W < kMaxWindow)
        do_block(s, jb, qreg, std::integral_constant<bool, true>{});
      else
        do_block(s, jb, qreg, std::integral_constant<bool, false>{});
    }
  };
  auto epilogue = [&](int s, const u32x4 (&graw)[4][2]) {
    const float lt = l_run + __shfl_xor(l_run, 32);
    const int pos = s * kStep + 32 * ph + n;
    if (pos < T) {
      const float inv = 1.0f / lt;
      bf16* dst = p.out + qoff + (size_t)pos * qstride + hi * 16;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            o[e] = (bf16)(oacc[db][e2 * 8 + e] * inv * sigmoidf_(bf16_elem(graw[db][e2], e)));
          *(bf16x8*)(dst + db * 32 + e2 * 8) = o;
        }
    }
  };

  // ---- prologue: ring <- tiles s_begin - 2 .. s_begin, trig of s_begin ---------------
  u32x4 qraw[8];
  load_q(s_begin, qraw);
  for (int t = max(s_begin - 2, 0); t <= s_begin; ++t) {
    u32x4 kr[2], vr[2];
    load_kv(t, kr, vr);
    make_trig(t, t & 1);
    stage_k(kr, t & 1);
    __syncthreads();
    transform_k(kr, t, t & 1);
    stage_v(vr, t);
    __syncthreads();
  }
  u32x4 kr[2], vr[2];
  if (s_begin + 1 < s_end) load_kv(s_begin + 1, kr, vr);
  reset_acc();

  // ---- steady state -------------------------------------------------------------------
  for (int s = s_begin; s < s_end; ++s) {
    const bool more = s + 1 < s_end;
    bf16x8 qreg[8];
    q_transform(qraw, s & 1, qreg);
    u32x4 graw[4][2];
    load_g(s, graw);
    if (more) load_q(s + 1, qraw);
    blocks(s, 0, 2, qreg);
    if (more) {
      stage_k(kr, (s + 1) & 1);
      make_trig(s + 1, (s + 1) & 1);
    }
    // Every wave is done with the two oldest blocks; tile s + 1's raw K and trig are in
    // LDS. (The raw/trig buffers alternate, so the next writes to these ones come after
    // the next barrier.)
    __syncthreads();
    if (more) {
      transform_k(kr, s + 1, (s + 1) & 1);
      stage_v(vr, s + 1);
      if (s + 2 < s_end) load_kv(s + 2, kr, vr);
    }
    blocks(s, 2, kNB, qreg);
    epilogue(s, graw);
    reset_acc();
  }
}

template <bool STATIC>
hipError_t set_smem() {
  return hipFuncSetAttribute((const void*)swa_stream_kernel<STATIC>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, kSmem);
}

}  // namespace

bool swa_stream_supported(const PrefillArgs& a) {
  return a.swa && a.d == kD && a.Hq == kG * a.Hkv && a.rdim == 2 * kRH && a.window >= 1 &&
         a.window <= kMaxWindow;
}

hipError_t launch_swa_stream(const PrefillArgs& a, hipStream_t s) {
  SArgs ka;
  ka.q = (const bf16*)a.q;
  ka.k = (const bf16*)a.k;
  ka.v = (const bf16*)a.v;
  ka.g = (const bf16*)a.g;
  ka.out = (bf16*)a.out;
  ka.wq = a.wq;
  ka.wk = a.wk;
  ka.T = a.T;
  ka.Hq = a.Hq;
  ka.Hkv = a.Hkv;
  ka.window = a.window;
  ka.pos_offset = a.pos_offset;
  ka.eps = a.eps;
  ka.qscale = a.scale * 1.4426950408889634f;
  ka.fr = a.fr;
  ka.n_hb = a.B * a.Hkv;
  ka.n_steps = (a.T + kStep - 1) / kStep;
  if (ka.n_steps == 0 || ka.n_hb == 0) return hipSuccess;
  // One resident workgroup per CU (the LDS ring takes most of a CU): split every
  // (batch, KV head) stream into segments so that the grid covers the CUs once.
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // Segments of at least kMinSegSteps steps keep the three-tile prologue of a segment
  // (and its serial load latency) small against the segment's work.
  const int n_seg_target = max(1, (cus + ka.n_hb - 1) / ka.n_hb);
  ka.seg_steps = max(kMinSegSteps, (ka.n_steps + n_seg_target - 1) / n_seg_target);
  const int n_seg = (ka.n_steps + ka.seg_steps - 1) / ka.seg_steps;
  const int n_blocks = ka.n_hb * n_seg;
  e = set_smem<true>();
  if (e != hipSuccess) return e;
  e = set_smem<false>();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(swa_stream_kernel<true>, dim3(n_blocks), dim3(kThreads), kSmem, s, ka);
  hipLaunchKernelGGL(swa_stream_kernel<false>, dim3(n_blocks), dim3(kThreads), kSmem, s, ka);
  return hipGetLastError();
}

}  // namespace zg
