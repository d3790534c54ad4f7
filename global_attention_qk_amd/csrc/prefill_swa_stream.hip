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
// design aims at keeping loads in flight and the vector ALUs' latency hidden.
//
//   * A workgroup (8 wave64s, two per SIMD) owns one (batch, KV head) and a contiguous
//     segment of the sequence, which it walks 32 positions per step. Wave w takes query
//     head w % 4 at the 16 positions 16 * (w / 4) .. of the step. Products run on
//     v_mfma_f32_16x16x32_bf16 with scores formed transposed (S^T = K~ Q~^T: keys on M,
//     queries on N), so each lane holds one query and P lands in the B-operand layout of
//     O^T += V^T P^T.
//   * K~ (normalised, rotated) and V^T live in LDS as a ring of six 32-key blocks: each key
//     block is loaded from HBM, transformed and transposed once per segment, and each wave
//     reads the five blocks its window touches (one band-edge block, three full blocks,
//     the diagonal block). Step s writes block s + 1 into the slot of block s - 5, so a
//     single barrier per step orders the ring, the raw-K staging and the RoPE tables.
//   * Loads run one step ahead: Q and G of the next step go straight into registers in
//     the MFMA operand / accumulator layouts, the next K and V tiles into registers, and
//     every load of a step is consumed at the top of the next step, before that step's
//     own loads are issued; a step's outputs are stored as soon as its epilogue is done.
//   * Head dims are permuted inside the products (the same permutation on both operands
//     of each product): lane group g (lanes 16 g .. 16 g + 15) holds dims [32 g, 32 g + 32)
//     of its query in Q~ and in O^T, so Q and G are loaded and O stored with 16-byte
//     accesses, and of the rotated pairs (j, j + 21) only j = 11 .. 20 cross lane groups
//     (exchanged with one swizzle).
//   * Static softmax shift as in the other prefill kernel: when the score bound B implied
//     by the norm weights is moderate (B <= 48 log2 units), the score accumulators start
//     at -B and p = exp2(s - B) lies in [2^-2B, 1] with no running max; otherwise the
//     online-max form runs (one launch carries both; the bound picks one).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kD = 128;
constexpr int kG = 4;              // query heads per KV head
constexpr int kRH = 21;            // rotated pairs (rotary_dim 42)
constexpr int kRHP = 22;           // trig table row stride (16-byte aligned rows)
constexpr int kStep = 32;          // positions per step (= keys per ring block)
constexpr int kRing = 6;           // ring blocks
constexpr int kNB = 5;             // blocks a wave visits per step (window <= 128)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxWindow = 128;
constexpr int kMinSegSteps = 8;
constexpr int kTrigBufs = 3;
constexpr float kStaticShiftMax = 48.0f;   // largest score bound (log2 units) without a max

constexpr int kKRowB = kD * 2 + 16;        // padded K~ / raw K row
constexpr int kKBlkB = kStep * kKRowB;     // K~ block: 32 rows
constexpr int kVBlkB = kD * kStep * 2;     // V^T block: 128 rows x 64 B
constexpr int kRawB = kStep * kKRowB;
constexpr int kTrigB = kStep * kRHP * 8;
constexpr int kOffK = 0;
constexpr int kOffV = kOffK + kRing * kKBlkB;
constexpr int kOffRaw = kOffV + kRing * kVBlkB;       // two raw K buffers
constexpr int kOffTrig = kOffRaw + 2 * kRawB;         // three trig tables
constexpr int kOffW = kOffTrig + kTrigBufs * kTrigB;  // wq * qscale, wk
constexpr int kOffFr = kOffW + 2 * kD * 4;            // RoPE frequencies (hi, lo)
constexpr int kOffRn = kOffFr + 2 * 32 * 4;           // 1/rms of the tile's key rows
constexpr int kOffRot = kOffRn + kStep * 4;           // cos/sin of the 32 in-step offsets
constexpr int kOffBase = kOffRot + kTrigB;            // cos/sin at two steps' first positions
constexpr int kSmem = kOffBase + 2 * 32 * 8;
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
  const int32_t* cu;   // packed documents (B == 1, T = total tokens), or nullptr
  int max_len;
};

__device__ __forceinline__ int ring_slot(int kb) { return (kb + 4 * kRing) % kRing; }  // kb >= -24

// Padded rows: one 16-byte chunk read across 16 consecutive keys touches every 16-byte
// bank group once, and a lane's chunks are one base plus immediate offsets. (Measured on
// gfx950 with the LDS bank-conflict counter: the 16x16x32 operand read, where lanes l,
// l + 16, l + 32 and l + 48 read other chunks of the same 16 rows, still takes two passes
// instead of one with this layout and with an XOR-swizzled one alike; a layout in which
// every 16 lanes read one contiguous 256 bytes takes one. Making both operand reads of
// the blocks conflict-free that way shortened the whole kernel by about 2 %.)
__device__ __forceinline__ int krow_off(int row, int chunk) { return row * kKRowB + (chunk << 4); }
// V^T block: row m (0..127) holds 32 key slots (64 B); chunk c sits at
// c ^ ((m >> 2) & 3) ^ (m & 2), so that one chunk read across 8 consecutive rows covers
// 128 distinct bytes and across 16 rows 256 distinct bytes (the operand read still takes
// two passes on gfx950, as for K~ above).
__device__ __forceinline__ int vblk_off(int m, int chunk) {
  return m * (kStep * 2) + ((chunk ^ ((m >> 2) & 3) ^ (m & 2)) << 4);
}
// V^T row holding dim d: accumulator register r of 16-row block db in lane group g is
// dim 32 g + 4 db + r.
__device__ __forceinline__ int vt_row_of_dim(int d) {
  return 16 * ((d >> 2) & 7) + 4 * (d >> 5) + (d & 3);
}
// V^T slot of key k (0..31): slot 8 g + e holds the key that lane group g's P value e
// stands for, 16 (e / 4) + 4 g + e % 4.
__device__ __forceinline__ int key_slot(int k) {
  return (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A value the optimiser must treat as recomputed here: keeps lane-derived indices from
// being hoisted out of the step loop and held in registers for its whole length (used
// where the registers matter more than the few instructions; the block products' indices
// are left hoistable).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row: xor 1, xor 2, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
// Lane l <-> lane l ^ 16 (within each half of the wave).
__device__ __forceinline__ uint32_t swap16(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);
}
__device__ __forceinline__ float swap16f(float x) { return __uint_as_float(swap16(__float_as_uint(x))); }
// Sum over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float group_sum(float x) {
  x += swap16f(x);
  return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, swap16f(x));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float bf16_elem(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? bf16_hi_to_f32(w) : bf16_lo_to_f32(w);
}
__device__ __forceinline__ float bf16_word(uint32_t w, int half) {
  return half ? bf16_hi_to_f32(w) : bf16_lo_to_f32(w);
}

// Slot stream of the fast path's five blocks for the waves holding positions 16 PH .. of
// a step: one MFMA per slot, phases S(b) (scores of block b, 4 slots per 16-key half
// computed) and PV(b) (8 slots) in the order S0 S1 PV0 S2 PV1 S3 PV2 S4 PV3 PV4; the
// softmax of block b runs under phase kSmPhase[b] (after S(b), before PV(b)).
template <int PH>
struct FullSched {
  static constexpr int h0(int b) { return (b == 0 && PH == 1) ? 1 : 0; }          // band edge
  static constexpr int h1(int b) { return (b == kNB - 1 && PH == 0) ? 0 : 1; }    // diagonal
  static constexpr int kPhases = 2 * kNB;
  static constexpr int kind(int ph) { return (ph == 0 || ph == 1 || ph == 3 || ph == 5 || ph == 7) ? 0 : 1; }
  static constexpr int blk(int ph) {
    constexpr int b[kPhases] = {0, 1, 0, 2, 1, 3, 2, 4, 3, 4};
    return b[ph];
  }
  static constexpr int sm_phase(int b) {
    constexpr int q[kNB] = {1, 3, 5, 7, 8};
    return q[b];
  }
  static constexpr int len(int ph) { return kind(ph) ? 8 : 4 * (h1(blk(ph)) - h0(blk(ph)) + 1); }
  static constexpr int first(int ph) { return ph == 0 ? 0 : first(ph - 1) + len(ph - 1); }
  static constexpr int kSlots = first(kPhases - 1) + len(kPhases - 1);
  static constexpr int phase_of(int u) {
    int ph = 0;
    while (ph + 1 < kPhases && first(ph + 1) <= u) ++ph;
    return ph;
  }
};

// The stream of one workgroup; `sinit` starts every score accumulator: -B for the static
// shift (so p <= 1), 0 for the online max. The norm weights and RoPE frequencies are in
// LDS already.
template <bool STATIC>
__device__ __forceinline__ void swa_stream_body(const SArgs& p, const float sinit) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sWq = (float*)(smem + kOffW);
  float* sWk = sWq + kD;
  float* sFr = (float*)(smem + kOffFr);   // [0, 32): hi, [32, 64): lo

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3;     // head within the group
  const int ph = wave >> 2;    // which 16 positions of the step
  const int n = lane & 15;     // query column of this lane
  const int grp = lane >> 4;   // lane group: dims [32 grp, 32 grp + 32)

  const int lin = blockIdx.x;
  const int hb = lin % p.n_hb;
  const int seg = lin / p.n_hb;
  const int b = hb / p.Hkv;        // batch element, or document of a packed batch
  const int kvh = hb % p.Hkv;
  int T = p.T, n_steps = p.n_steps;
  size_t seq0 = (size_t)b * p.T;   // first token of the sequence in token order
  if (p.cu) {
    int start, len;
    doc_range(p.cu, b, p.T, p.max_len, start, len);
    T = len;
    n_steps = (len + kStep - 1) / kStep;
    seq0 = start;
  }
  const int s_begin = seg * p.seg_steps;
  const int s_end = min(s_begin + p.seg_steps, n_steps);
  if (s_begin >= s_end) return;
  const int W = p.window;
  const int h = kvh * kG + hg;
  // Wave-uniform bases with 32-bit per-lane byte offsets (one sequence of one tensor is
  // below 4 GiB, checked on the host).
  const uint32_t qrow_b = (uint32_t)p.Hq * kD * 2;    // bytes between positions in Q/G/O
  const uint32_t kvrow_b = (uint32_t)p.Hkv * kD * 2;  // bytes between positions in K/V
  const size_t qoff = (seq0 * p.Hq + h) * kD;
  const char* qbase = (const char*)(p.q + qoff);
  const char* gbase = (const char*)(p.g + qoff);
  char* obase = (char*)(p.out + qoff);
  const char* kbase = (const char*)(p.k + (seq0 * p.Hkv + kvh) * kD);
  const char* vbase = (const char*)(p.v + (seq0 * p.Hkv + kvh) * kD);

  // ---- loads -----------------------------------------------------------------------
  // Q (or G) row of this lane's query at step s: dims 32 grp .. + 31, as four chunks.
  auto load_row = [&](const char* base, int s, u32x4 (&dst)[4]) {
    const int pos = min(s * kStep + 16 * ph + n, T - 1);
    const uint32_t off = (uint32_t)pos * qrow_b + grp * 64;
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = *(const u32x4*)(base + off + c * 16);
  };
  // K rows of tile t (positions 32 t .., clamped into [0, T); such rows are never visible
  // and keep every product finite): chunk tid & 15 of row tid >> 4.
  auto load_k = [&](int t, u32x4& kr) {
    const int tl = opaque(tid);
    const int krow = tl >> 4, kc = tl & 15;
    kr = *(const u32x4*)(kbase + (uint32_t)min(max(t * kStep + krow, 0), T - 1) * kvrow_b + kc * 16);
  };
  // V rows 2 (tid & 15) and + 1 of tile t, dims 4 (tid >> 4) .. + 3.
  auto load_v = [&](int t, u32x2 (&vr)[2]) {
    const int tl = opaque(tid);
    const int kp = tl & 15, dq = tl >> 4;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int pos = min(max(t * kStep + 2 * kp + e, 0), T - 1);
      vr[e] = *(const u32x2*)(vbase + (uint32_t)pos * kvrow_b + dq * 8);
    }
  };

  // ---- LDS producers -----------------------------------------------------------------
  auto trig_buf = [&](int t) { return (float2*)(smem + kOffTrig + ((t + 3 * kTrigBufs) % kTrigBufs) * kTrigB); };
  auto raw_buf = [&](int t) { return smem + kOffRaw + (t & 1) * kRawB; };
  // RoPE cos/sin of the 32 positions of tile t, each evaluated from its position (the
  // prologue's tiles).
  auto make_trig_direct = [&](int t) {
    float2* tr = trig_buf(t);
    for (int e = tid; e < kStep * kRH; e += kThreads) {
      const int pl = e / kRH, j = e - pl * kRH;
      float c, s;
      // frequencies from LDS: indexing the kernel arguments at run time would be a global
      // load, and waiting for it would also wait for every prefetch issued before it
      rope_cos_sin(p.pos_offset + max(t * kStep + pl, 0), sFr[j], sFr[32 + j], c, s);
      tr[pl * kRHP + j] = make_float2(c, s);
    }
  };
  // cos/sin at the first position of tile t (t >= 0), for the steady state's tables: the
  // last wave, which builds the fewest table entries.
  auto make_base = [&](int t) {
    if (wave == kWaves - 1 && lane < kRH) {
      float c, s;
      rope_cos_sin(p.pos_offset + t * kStep, sFr[lane], sFr[32 + lane], c, s);
      ((float2*)(smem + kOffBase))[(t & 1) * 32 + lane] = make_float2(c, s);
    }
  };
  // The same table in the steady state (t >= 0) by angle addition: the rotation at
  // position p0 + i is the one at p0 (make_base, a step earlier) times the one at i
  // (the kernel's constant table of in-step offsets); both factors are evaluated from
  // their positions, so the product is within a few ulp at any position.
  auto make_trig = [&](int t) {
    float2* tr = trig_buf(t);
    const float2* base = (const float2*)(smem + kOffBase) + (t & 1) * 32;
    const float2* rot = (const float2*)(smem + kOffRot);
    for (int e = tid; e < kStep * kRH; e += kThreads) {
      const int pl = e / kRH, j = e - pl * kRH;
      const float2 b0 = base[j], r0 = rot[pl * kRHP + j];
      tr[pl * kRHP + j] = make_float2(__builtin_fmaf(b0.x, r0.x, -b0.y * r0.y),
                                      __builtin_fmaf(b0.y, r0.x, b0.x * r0.y));
    }
  };
  auto stage_k = [&](const u32x4& kr, int t) {
    const int tl = opaque(tid);
    *(u32x4*)(raw_buf(t) + krow_off(tl >> 4, tl & 15)) = kr;
  };
  // RMSNorm + partial RoPE of staged tile t into its ring block, in two branch-free passes
  // over the four key rows of this wave (rows 4 w .. 4 w + 3 in both passes, so the
  // second pass sees the first one's LDS writes in order, with no barrier):
  //   1. 16 lanes per key, lane kc: dims 8 kc .. + 7 normalised and weighted,
  //      x w / rms, the row's 1/rms kept in LDS;
  //   2. one lane per rotated pair (4 keys x 21 pairs = 84 jobs, two rounds): both
  //      members of the pair from the raw row, rotated, overwriting what pass 1 wrote.
  auto transform_k = [&](int t) {
    const char* raw = raw_buf(t);
    const float2* tr = trig_buf(t);
    char* blk = smem + kOffK + ring_slot(t) * kKBlkB;
    float* sRn = (float*)(smem + kOffRn);
    {
      const int tl = opaque(tid);
      const int krow = tl >> 4, kc = tl & 15;
      const u32x4 r0 = *(const u32x4*)(raw + krow_off(krow, kc));
      const float4 w0 = *(const float4*)(sWk + 8 * kc);
      const float4 w1 = *(const float4*)(sWk + 8 * kc + 4);
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float x[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = bf16_elem(r0, e);
        ss = __builtin_fmaf(x[e], x[e], ss);
      }
      ss = row16_sum(ss);
      const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + p.eps);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)(x[e] * w[e] * rn);
      *(bf16x8*)(blk + krow_off(krow, kc)) = o;
      if (kc == 0) sRn[krow] = rn;
    }
    const int ln = opaque(lane);
    const int row0 = 4 * wave;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int job = ln + 64 * it;
      if (job < 4 * kRH) {
        const int kr = row0 + job / kRH;   // key row of the tile
        const int j = job - (job / kRH) * kRH;
        const bf16* rrow = (const bf16*)(raw + kr * kKRowB);
        const float a = (float)rrow[j] * sWk[j];
        const float b2 = (float)rrow[j + kRH] * sWk[j + kRH];
        const float2 cs = tr[kr * kRHP + j];
        const float rn = sRn[kr];
        bf16* orow = (bf16*)(blk + kr * kKRowB);
        orow[j] = (bf16)(__builtin_fmaf(a, cs.x, -b2 * cs.y) * rn);
        orow[j + kRH] = (bf16)(__builtin_fmaf(b2, cs.x, a * cs.y) * rn);
      }
    }
  };
  // V of tile t, transposed into its ring block (keys 2 kp, 2 kp + 1 are adjacent slots,
  // so each store is one 32-bit word).
  auto stage_v = [&](const u32x2 (&vr)[2], int t) {
    const int tl = opaque(tid);
    const int kp = tl & 15, dq = tl >> 4;
    char* blk = smem + kOffV + ring_slot(t) * kVBlkB;
    const int sl = key_slot(2 * kp);
    const int chunk = sl >> 3, within = sl & 7;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = vt_row_of_dim(dq * 4 + e);
      const uint32_t w0 = vr[0][e >> 1], w1 = vr[1][e >> 1];
      const uint32_t word = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                    : ((w0 & 0xffffu) | (w1 << 16));
      *(uint32_t*)(blk + vblk_off(m, chunk) + within * 2) = word;
    }
  };
  // RMSNorm + RoPE + scale of this lane's 32 dims of its query row, as the B operand.
  // Rotated pairs (j, j + 21): group 0 holds both members for j <= 10 and j's member for
  // j = 11 .. 20, whose partners (dims 32 .. 41) sit in group 1; those ten values cross
  // between groups 0 and 1 (and meaningless ones between groups 2 and 3).
  auto q_transform = [&](const u32x4 (&raw)[4], int s, bf16x8 (&qreg)[4]) {
    uint32_t dw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) dw[i] = raw[i >> 2][i & 3];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float xv = bf16_word(dw[i >> 1], i & 1);
      ss = __builtin_fmaf(xv, xv, ss);
    }
    ss = group_sum(ss);
    const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + p.eps);
    // group 0 sends its dims 10 .. 21 (words 5 .. 10), group 1 its dims 32 .. 43 (words 0 .. 5)
    const bool odd = grp & 1;
    uint32_t rc[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) rc[k] = swap16(odd ? dw[k] : dw[5 + k]);
    const float* w = sWq + grp * 32;
    const float2* tr = trig_buf(s) + (16 * ph + n) * kRHP;
    float2 cs[kRH];
#pragma unroll
    for (int j = 0; j < kRH; ++j) cs[j] = tr[j];
    const bool g0 = grp == 0, g1 = grp == 1;
    auto outv = [&](int i) -> float {
      const float xi = bf16_word(dw[i >> 1], i & 1) * w[i];
      float c = 1.f, sn = 0.f, pv = 0.f;
      if (i <= 9) {
        // group 0: partner i + 21 (own), pair j = i; group 1: dim 32 + i, partner 11 + i
        const float p0 = bf16_word(dw[(i + kRH) >> 1], (i + kRH) & 1) * sWq[i + kRH];
        const float p1 = bf16_word(rc[(i + 1) >> 1], (i + 1) & 1) * sWq[11 + i];
        c = g0 ? cs[i].x : (g1 ? cs[11 + i].x : 1.f);
        sn = g0 ? -cs[i].y : (g1 ? cs[11 + i].y : 0.f);
        pv = g0 ? p0 : p1;
      } else if (i == 10) {
        const float p0 = bf16_word(dw[(i + kRH) >> 1], (i + kRH) & 1) * sWq[i + kRH];
        c = g0 ? cs[i].x : 1.f;
        sn = g0 ? -cs[i].y : 0.f;
        pv = p0;
      } else if (i <= 20) {
        // partner dim i + 21 = 32 + (i - 11) from group 1
        const float p0 = bf16_word(rc[(i - 11) >> 1], (i - 11) & 1) * sWq[i + kRH];
        c = g0 ? cs[i].x : 1.f;
        sn = g0 ? -cs[i].y : 0.f;
        pv = p0;
      } else {
        // group 0: second member of pair j = i - 21 (partner own)
        const float p0 = bf16_word(dw[(i - kRH) >> 1], (i - kRH) & 1) * sWq[i - kRH];
        c = g0 ? cs[i - kRH].x : 1.f;
        sn = g0 ? cs[i - kRH].y : 0.f;
        pv = p0;
      }
      return (xi * c + pv * sn) * rn;
    };
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (bf16)outv(ks * 8 + e);
      qreg[ks] = v;
    }
  };

  // ---- attention state -----------------------------------------------------------------
  f32x4 oacc[8];
  float l_run = 0.f, m_run = -INFINITY;
  auto reset_acc = [&] {
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    m_run = -INFINITY;
  };
  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};

  // Scores of ring block kb for this wave's 16 queries: two 16-key halves; lane group g
  // holds keys 16 kh + 4 g + r.
  // Halves outside [KH0, KH1] are not computed.
  auto scores = [&](int kb, const bf16x8 (&qreg)[4], f32x4 (&sacc)[2], auto kh0_tag,
                    auto kh1_tag) {
    constexpr int KH0 = decltype(kh0_tag)::value, KH1 = decltype(kh1_tag)::value;
    const int ln = lane;
    const int nn = ln & 15, gg = ln >> 4;
    const char* sK = smem + kOffK + ring_slot(kb) * kKBlkB;
#pragma unroll
    for (int kh = KH0; kh <= KH1; ++kh) {
      sacc[kh] = (f32x4){sinit, sinit, sinit, sinit};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = *(const bf16x8*)(sK + krow_off(16 * kh + nn, 4 * gg + ks));
        sacc[kh] = mfma16(a, qreg[ks], sacc[kh]);
      }
    }
  };
  auto pv_block = [&](int kb, const bf16x8& pb, bool first) {
    const int ln = lane;
    const int nn = ln & 15, gg = ln >> 4;
    const char* sV = smem + kOffV + ring_slot(kb) * kVBlkB;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 a = *(const bf16x8*)(sV + vblk_off(16 * db + nn, gg));
      oacc[db] = mfma16(a, pb, first ? (f32x4){0.f, 0.f, 0.f, 0.f} : oacc[db]);
    }
  };
  // P (bf16, B-operand order) from scores, with the row-sum update.
  auto to_p = [&](const float (&pf)[8], float& ls) -> bf16x8 {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)pf[e];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 pr = {v[e], v[e + 1]};
      ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
    }
    return v;
  };

  // Fast path (128-key window, static shift, away from position 0): the five blocks as
  // one compile-time stream of MFMA slots (FullSched), specialised on which 16 positions
  // of the step the wave holds (PH). Each slot issues one product, reads the LDS operand
  // of the slot two ahead, and carries a piece of the softmax of the block before, so
  // that neither the operand reads nor the products' results are waited for right away.
  // Masks only on the band-edge block (visible: keys above the query's offset in its
  // block) and the diagonal block (keys at or below it), whose 16-key half on the far
  // side of the wave's queries is not computed at all; the first block starts the
  // accumulators from zero.
  auto blocks_full = [&](int s, const bf16x8 (&qreg)[4], auto ph_tag) {
    constexpr int PH = decltype(ph_tag)::value;
    using FS = FullSched<PH>;
    constexpr int NS = FS::kSlots;
    const int ln = lane;
    const int nn = ln & 15, gg = ln >> 4;
    const int qo = 16 * PH + nn;   // query offset within the step's 32 positions
    // per-lane operand offsets of a block (ring-slot base added per block)
    const char* kbase0 = smem + kOffK;
    const char* vbase0 = smem + kOffV;
    int kslot[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) kslot[b] = ring_slot(s - (kNB - 1) + b);
    auto read_op = [&](auto uc) -> bf16x8 {
      constexpr int u = decltype(uc)::value;
      constexpr int ph = FS::phase_of(u), i = u - FS::first(ph), b = FS::blk(ph);
      if constexpr (FS::kind(ph) == 0) {
        constexpr int kh = FS::h0(b) + i / 4, ks = i % 4;
        return *(const bf16x8*)(kbase0 + kslot[b] * kKBlkB + krow_off(16 * kh + nn, 4 * gg + ks));
      } else {
        return *(const bf16x8*)(vbase0 + kslot[b] * kVBlkB + vblk_off(16 * i + nn, gg));
      }
    };
    f32x4 sacc[kNB][2];
    float pf[kNB][8];
    bf16x8 pb[kNB];
    bf16x8 ops[NS];
    float ls = 0.f;
    ops[0] = read_op(std::integral_constant<int, 0>{});
    if constexpr (NS > 1) ops[1] = read_op(std::integral_constant<int, 1>{});
    static_for<NS>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int ph = FS::phase_of(u), i = u - FS::first(ph), b = FS::blk(ph);
      if constexpr (u + 2 < NS) ops[u + 2] = read_op(std::integral_constant<int, u + 2>{});
      if constexpr (FS::kind(ph) == 0) {
        constexpr int kh = FS::h0(b) + i / 4, ks = i % 4;
        if constexpr (ks == 0) sacc[b][kh] = (f32x4){sinit, sinit, sinit, sinit};
        sacc[b][kh] = mfma16(ops[u], qreg[ks], sacc[b][kh]);
      } else {
        oacc[i] = mfma16(ops[u], pb[b], b == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : oacc[i]);
      }
      // softmax piece of block sb under this phase: its computed values spread evenly
      // over the phase's slots, each pair converted (and summed) after its second value
      static_for<kNB>([&](auto sbc) {
        constexpr int sb = decltype(sbc)::value;
        if constexpr (FS::sm_phase(sb) == ph) {
          constexpr int e0 = 4 * FS::h0(sb), nv = 4 * (FS::h1(sb) - FS::h0(sb) + 1);
          constexpr int L = FS::len(ph);
          static_for<nv>([&](auto vc) {
            constexpr int v = decltype(vc)::value;
            if constexpr (v * L / nv == i) {
              constexpr int e = e0 + v, kh = e >> 2, r = e & 3;
              float x = fast_exp2(sacc[sb][kh][r]);
              const bool below = 16 * kh + 4 * gg + r <= qo;
              if constexpr (sb == 0 && kh == PH) x = below ? 0.f : x;
              if constexpr (sb == kNB - 1 && kh == PH) x = below ? x : 0.f;
              pf[sb][e] = x;
              if constexpr (e & 1) {
                const bf16x2 pr = {(bf16)pf[sb][e - 1], (bf16)x};
                pb[sb][e - 1] = pr[0];
                pb[sb][e] = pr[1];
                ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
              }
              if constexpr (v == 0) {
                // values of skipped halves
#pragma unroll
                for (int z = 0; z < 8; ++z)
                  if (z < e0 || z >= e0 + nv) pb[sb][z] = (bf16)0.f;
              }
            }
          });
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    l_run = ls;
  };
  // General path: any window <= 128, blocks before position 0, and the online variant.
  auto blocks = [&](int s, const bf16x8 (&qreg)[4]) {
    const int q_lo = s * kStep + 16 * ph;
    for (int jb = 0; jb < kNB; ++jb) {
      const int kb = s - (kNB - 1) + jb;
      if (kb < 0 || kStep * kb + kStep - 1 <= q_lo - W) continue;
      const int ln = opaque(lane);
      const int nn = ln & 15, gg = ln >> 4;
      f32x4 sacc[2];
      scores(kb, qreg, sacc, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      // key - query for value e: 32 kb + 16 (e / 4) + 4 g + e % 4 - q
      const int rel = kStep * kb + 4 * gg - (q_lo + nn);
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dk = rel + 16 * (e >> 2) + (e & 3);
        sv[e] = (dk > 0 || dk <= -W) ? -INFINITY : sacc[e >> 2][e & 3];
      }
      float mu = 0.f;
      if (!STATIC) {
        float mt = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
        mt = group_max(mt);
        const float m_old = m_run;
        const bool raise = mt > m_old + 8.0f;
        if (__ballot(raise)) {
          const float m_new = raise ? mt : m_old;
          const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
          m_run = m_new;
        }
        mu = (m_run == -INFINITY) ? 0.f : m_run;
      }
      float pf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = fast_exp2(sv[e] - mu);
      float ls = l_run;
      const bf16x8 pb = to_p(pf, ls);
      l_run = ls;
      pv_block(kb, pb, false);
    }
  };
  // O = acc / l * sigmoid(G) of one step as bf16 (dims 32 g + 8 c .. + 7 in ob[c]):
  // o / l * sigmoid(g) = o * rcp(l + l * exp(-g)).
  auto epilogue = [&](const u32x4 (&graw)[4], bf16x8 (&ob)[4]) {
    const float lt = group_sum(l_run);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float eg = __expf(-bf16_elem(graw[c], e));
        o[e] = (bf16)(oacc[2 * c + (e >> 2)][e & 3] * __builtin_amdgcn_rcpf(__builtin_fmaf(lt, eg, lt)));
      }
      ob[c] = o;
    }
  };
  auto store_out = [&](int s, const bf16x8 (&ob)[4]) {
    const int pos = s * kStep + 16 * ph + n;
    if (pos < T) {
      char* dst = obase + (uint32_t)pos * qrow_b + grp * 64;
#pragma unroll
      for (int c = 0; c < 4; ++c) *(bf16x8*)(dst + c * 16) = ob[c];
    }
  };

  // ---- prologue --------------------------------------------------------------------------
  // Ring <- blocks s_begin - 4 .. s_begin; raw K and trig of block s_begin + 1 staged;
  // trig of s_begin ready; registers: Q and G of s_begin, V of s_begin + 1, K of
  // s_begin + 2.
  for (int t = max(s_begin - (kNB - 1), 0); t <= s_begin; ++t) {
    u32x4 kr;
    u32x2 vr[2];
    load_k(t, kr);
    load_v(t, vr);
    make_trig_direct(t);
    stage_k(kr, t);
    __syncthreads();
    transform_k(t);
    stage_v(vr, t);
    __syncthreads();
  }
  u32x4 kr;
  u32x2 vr[2];
  load_k(s_begin + 1, kr);
  make_trig_direct(s_begin + 1);
  make_base(s_begin + 2);
  stage_k(kr, s_begin + 1);
  // the loads the first step consumes, issued in the order the steady state issues them
  // (Q, V, K, then G), so that the waits at the loop head are the same on both entries
  u32x4 qraw[4], graw[4];
  load_row(qbase, s_begin, qraw);
  load_v(s_begin + 1, vr);
  load_k(s_begin + 2, kr);
  load_row(gbase, s_begin, graw);
  __syncthreads();

  // ---- steady state -------------------------------------------------------------------
  // Loads run one step ahead. At the top of step s the loads issued at the top of step
  // s - 1 are consumed (Q of s, V of s + 1, K of s + 2) and the next loads issued; G of s,
  // issued after the previous epilogue, is consumed by this step's epilogue, whose
  // outputs are stored right away (before the next G load, so that waiting for that load
  // a step later also finds the stores done). Loads past the segment are clamped and
  // unused.
  for (int s = s_begin; s < s_end; ++s) {
    bf16x8 qreg[4];
    q_transform(qraw, s, qreg);
    // V of block s + 1 into the slot of block s - 5 (last read in step s - 1), raw K of
    // s + 2; then the registers take the next loads
    stage_v(vr, s + 1);
    stage_k(kr, s + 2);
    load_row(qbase, s + 1, qraw);
    load_v(s + 2, vr);
    load_k(s + 3, kr);
    transform_k(s + 1);
    make_trig(s + 2);
    make_base(s + 3);
    if (STATIC && W == kMaxWindow && s >= kNB - 1) {
      if (ph)
        blocks_full(s, qreg, std::integral_constant<int, 1>{});
      else
        blocks_full(s, qreg, std::integral_constant<int, 0>{});
    } else {
      reset_acc();
      blocks(s, qreg);
    }
    bf16x8 ob[4];
    epilogue(graw, ob);
    store_out(s, ob);
    // G of the next step, consumed by the next epilogue
    load_row(gbase, s + 1, graw);
    // Block s + 1, raw K of s + 2 and trig of s + 2 are visible to every wave; every wave
    // is done with block s - 4 (its slot takes block s + 2 next).
    __syncthreads();
  }
}

// One launch: the score bound is the same for every workgroup, so they all take the same
// form (static shift when the bound allows it, else the online max).
__global__ __launch_bounds__(kThreads, 1) void swa_stream_kernel(const SArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sWq = (float*)(smem + kOffW);
  float* sWk = sWq + kD;
  float* sFr = (float*)(smem + kOffFr);
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kD; i += kThreads) {
    sWq[i] = p.wq[i] * p.qscale;
    sWk[i] = p.wk[i];
  }
  if (tid < kRH) {
    sFr[tid] = p.fr.hi[tid];
    sFr[32 + tid] = p.fr.lo[tid];
  }
  __syncthreads();
  for (int e = tid; e < kStep * kRH; e += kThreads) {
    const int pl = e / kRH, j = e - pl * kRH;
    float c, s;
    rope_cos_sin(pl, sFr[j], sFr[32 + j], c, s);
    ((float2*)(smem + kOffRot))[pl * kRHP + j] = make_float2(c, s);
  }
  // |s| <= d * max|wq * qscale| * max|wk| after RMSNorm (2% margin for bf16 operands).
  float wqm = 0.f, wkm = 0.f;
  for (int c = lane; c < kD; c += 64) {
    wqm = fmaxf(wqm, fabsf(sWq[c]));
    wkm = fmaxf(wkm, fabsf(sWk[c]));
  }
  wqm = wave_max(wqm);
  wkm = wave_max(wkm);
  const float bound = (float)kD * wqm * wkm * 1.02f;
  if (bound <= kStaticShiftMax)
    swa_stream_body<true>(p, -bound);
  else
    swa_stream_body<false>(p, 0.f);
}

hipError_t set_smem() { return ensure_dynamic_smem((const void*)swa_stream_kernel, kSmem); }

}  // namespace

bool swa_stream_supported(const PrefillArgs& a) {
  // per-lane offsets are 32-bit byte offsets within one sequence of Q / G / O
  const bool fits = (size_t)(a.cu ? a.max_len : a.T) * a.Hq * kD * 2 <= (size_t)UINT32_MAX;
  return a.swa && a.d == kD && a.Hq == kG * a.Hkv && a.rdim == 2 * kRH && a.window >= 1 &&
         a.window <= kMaxWindow && fits;
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
  ka.cu = a.cu;
  ka.max_len = a.max_len;
  ka.n_hb = (a.cu ? a.n_docs : a.B) * a.Hkv;
  ka.n_steps = ((a.cu ? a.max_len : a.T) + kStep - 1) / kStep;
  if (ka.n_steps == 0 || ka.n_hb == 0) return hipSuccess;
  // One resident workgroup per CU (the LDS ring takes most of a CU): split every
  // (batch, KV head) stream into segments so that the grid covers the CUs once.
  int cus = 0;
  hipError_t e = device_cu_count(&cus);
  if (e != hipSuccess) return e;
  // Segments of at least kMinSegSteps steps keep the three-tile prologue of a segment
  // (and its serial load latency) small against the segment's work.
  const int n_seg_target = max(1, (cus + ka.n_hb - 1) / ka.n_hb);
  ka.seg_steps = max(kMinSegSteps, (ka.n_steps + n_seg_target - 1) / n_seg_target);
  if (a.cu) {
    // Packed documents differ in length: segments sized from the total work (about two
    // per CU) rather than from the longest document keep the CUs evenly loaded; the
    // segments past a short document's end exit at once.
    const int64_t units = ((int64_t)a.T / kStep + a.n_docs) * a.Hkv;
    ka.seg_steps = max(kMinSegSteps, (int)((units + 2 * cus - 1) / (2 * cus)));
  }
  const int n_seg = (ka.n_steps + ka.seg_steps - 1) / ka.seg_steps;
  const int n_blocks = ka.n_hb * n_seg;
  e = set_smem();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(swa_stream_kernel, dim3(n_blocks), dim3(kThreads), kSmem, s, ka);
  return hipGetLastError();
}

}  // namespace zg
