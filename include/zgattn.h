/*
 * zgattn -- hybrid gated sliding-window / global causal GQA attention on MI355X (gfx950).
 *
 * The layer these entry points compute is the one the ZGCM-1 pages state:
 *   GatedSWA(h) = o_proj( A_SWA(q, k, v) (*) sigmoid(g_proj(h)) )
 * with q, k, v, g projected in parallel from the normalised hidden state, RMSNorm ("QK
 * normalisation") and partial RoPE (rotary ratio 0.33) on the q and k branches, a
 * 128-token sliding window for A_SWA, and ungated full-causal attention in the global
 * layers (hyper.ai summary of arXiv 2609.13356, section 方法, display equation; the
 * "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ). The projections and o_proj are
 * outside this library: the calls take post-projection Q, K, V and the gate
 * pre-activation G and return the pre-o_proj output.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *    allocates, frees or synchronises; every call is asynchronous on `stream`
 *    (a hipStream_t; NULL = the default stream). Inputs are never modified. Only `out`,
 *    the caches (decode appends the new token) and `workspace` are written.
 *  - Layouts are dense and contiguous, d fastest: Q, G, O are [B, T, Hq, d]; K, V are
 *    [B, T, Hkv, d]; decode caches are [B, Hkv, S, d]. Q, K, V, G, O and caches share
 *    one element type (`dtype`); RMSNorm weights are always fp32 [d].
 *  - Query head h reads KV head h / (Hq / Hkv).
 *  - Key j is visible to query i iff j <= i (global) and additionally i - window < j
 *    (SWA): the window counts the query itself (the jaehun.me review's worked example,
 *    section 게이트형 SWA의 동작: with window 4 the 4th token sees 4 tokens).
 *  - RMSNorm is per head over d: x / sqrt(mean(x^2) + rms_eps) * w. RoPE then rotates
 *    the leading rotary_dim dims in pairs (k, k + rotary_dim/2) by the angle
 *    pos * rope_base^(-2k/rotary_dim); dims [rotary_dim, d) pass through.
 *  - Scores are softmax_scale * q~ . k~ (softmax_scale <= 0 selects 1/sqrt(d)).
 *  - The gate is elementwise: O = A * 1/(1 + exp(-G)), G with O's shape.
 *  - Errors: every call returns a zgattn_status. Arguments are checked on the host
 *    before anything is launched; on error nothing is launched and the outputs are
 *    untouched. A failed launch returns ZGATTN_EHIP. No call prints or aborts.
 *  - Thread-safe: no mutable global state except a per-device property cache.
 */
#ifndef ZGATTN_H
#define ZGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZGATTN_ABI_VERSION 2

typedef enum {
  ZGATTN_OK = 0,
  ZGATTN_EINVAL = -1,       /* a size or parameter is out of range                     */
  ZGATTN_ENULL = -2,        /* a required pointer is NULL                              */
  ZGATTN_EDTYPE = -3,       /* unknown dtype                                           */
  ZGATTN_EUNSUPPORTED = -4, /* valid but not implemented (e.g. d not in {64, 128})     */
  ZGATTN_EWORKSPACE = -5,   /* workspace missing or smaller than the queried size      */
  ZGATTN_ERANGE = -6,       /* a position or capacity is out of range                  */
  ZGATTN_EHIP = -7          /* the HIP runtime reported an error at launch             */
} zgattn_status;

typedef enum { ZGATTN_F32 = 0, ZGATTN_BF16 = 1 } zgattn_dtype;

typedef struct {
  int32_t batch;        /* B >= 1                                                       */
  int32_t seq_len;      /* T >= 0 (prefill); ignored by decode                          */
  int32_t n_q_heads;    /* Hq >= 1                                                      */
  int32_t n_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0                                       */
  int32_t head_dim;     /* d in {64, 128}                                               */
  int32_t window;       /* SWA window W >= 1 (128 in the model); ignored by global calls */
  int32_t rotary_dim;   /* even, 0 <= r <= d (2*floor(0.33*d/2) in the model: 42 or 20) */
  int32_t pos_offset;   /* absolute position of prefill row 0 (>= 0)                    */
  float rope_base;      /* > 0 (10000 in the workloads)                                 */
  float rms_eps;        /* >= 0 (1e-6 in the workloads)                                 */
  float softmax_scale;  /* <= 0 selects 1/sqrt(d)                                       */
  int32_t dtype;        /* zgattn_dtype                                                 */
} zgattn_desc;

/* Positions (pos_offset + T - 1, decode pos) must stay below 2^24 so that they are exact
 * in fp32; larger values return ZGATTN_ERANGE. */
#define ZGATTN_MAX_POSITION ((1 << 24) - 1)

int zgattn_abi_version(void);
const char* zgattn_strerror(int status);

/*
 * Gated SWA prefill (hyper.ai summary, section 方法: GatedSWA equation without o_proj).
 *   q, g, out: [B, T, Hq, d];  k, v: [B, T, Hkv, d];  wq, wk: fp32 [d].
 *   out = softmax over the window of (q~ . k~) applied to v, times sigmoid(g).
 * QK-RMSNorm and partial RoPE are applied on the fly as Q and K tiles are loaded.
 * bf16 on the MFMA kernels for head groups 1, 2, 4, 8 and rotary_dim <= 64, any other
 * bf16 shape and fp32 on a vector-ALU kernel (fp32 arithmetic).
 * T == 0 is a no-op. out must not alias any input.
 */
int zgattn_swa_prefill(const zgattn_desc* desc, const void* q, const void* k, const void* v,
                       const void* g, const float* wq, const float* wk, void* out,
                       void* stream);

/*
 * Global (full-causal, ungated) prefill (explainer, section アーキテクチャ: the global
 * layers attend to the whole context and carry no gate).
 *   q, out: [B, T, Hq, d];  k, v: [B, T, Hkv, d];  wq, wk: fp32 [d].
 * `workspace` (device, >= zgattn_global_prefill_workspace_bytes(desc) bytes, 256-byte
 * aligned) receives normalised+rotated K once before the attention kernel reads it; with
 * workspace == NULL the K transform is instead fused into every K-tile load (slower for
 * long sequences, where each K tile is visited by many query tiles).
 * `lse` (optional, device fp32 [B, Hq, T], 4-byte aligned; NULL to skip) receives each
 * row's log-sum-exp of its scaled scores, ln sum_j exp(softmax_scale * q~_i . k~_j) over
 * the visible keys, for zgattn_global_prefill_backward; bf16 only (ZGATTN_EUNSUPPORTED
 * for fp32 and for the bf16 shapes that run on the vector-ALU kernel, as for
 * zgattn_swa_prefill, when lse is not NULL).
 */
int zgattn_global_prefill(const zgattn_desc* desc, const void* q, const void* k,
                          const void* v, const float* wq, const float* wk, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream);
size_t zgattn_global_prefill_workspace_bytes(const zgattn_desc* desc);

/*
 * Packed variable-length prefill (the 256K fine-tuning variant trains on packed tokens:
 * "ZGCM-1-7B 完全解説" explainer, section 事後訓練 — SFTと混合RL、think/no-thinkの共存;
 * that documents do not attend across their boundaries and restart their positions is this
 * library's reading, the pages do not say). The batch is
 * one packed sequence of desc->seq_len tokens: q, g, out [seq_len, Hq, d]; k, v
 * [seq_len, Hkv, d] (desc->batch must be 1). cu_seqlens: DEVICE int32 [n_docs + 1],
 * non-decreasing, cu_seqlens[0] = 0 and cu_seqlens[n_docs] = seq_len; document i is
 * tokens [cu_seqlens[i], cu_seqlens[i+1]) and is attended as an independent sequence:
 * keys of other documents are never visible, and positions restart at pos_offset at each
 * document's first token (RoPE). max_seqlen (host) bounds every document's length and sizes
 * the grid. The table lives on the device and is not validated on the host: out-of-range
 * entries are clamped (no access leaves the tensors) and give unspecified outputs.
 * bf16 on the MFMA paths (their head-group and rotary limits; ZGATTN_EUNSUPPORTED
 * otherwise), or fp32 on the vector-ALU kernel (any head group and rotary dim). The bf16
 * global form takes the same optional workspace as zgattn_global_prefill, sized by
 * zgattn_global_prefill_varlen_workspace_bytes(desc, n_docs) (0 for fp32, which uses none).
 */
int zgattn_swa_prefill_varlen(const zgattn_desc* desc, const int32_t* cu_seqlens,
                              int32_t n_docs, int32_t max_seqlen, const void* q,
                              const void* k, const void* v, const void* g, const float* wq,
                              const float* wk, void* out, void* stream);
int zgattn_global_prefill_varlen(const zgattn_desc* desc, const int32_t* cu_seqlens,
                                 int32_t n_docs, int32_t max_seqlen, const void* q,
                                 const void* k, const void* v, const float* wq,
                                 const float* wk, void* workspace, size_t workspace_bytes,
                                 void* out, void* stream);
size_t zgattn_global_prefill_varlen_workspace_bytes(const zgattn_desc* desc, int32_t n_docs);

/*
 * Backward pass of a prefill call: the gradients of sum(dout * out) with respect to q, k,
 * v, g (SWA), w_q and w_k, where out is the layer of zgattn_swa_prefill /
 * zgattn_global_prefill on the same inputs (the pages train the model end to end, explainer
 * training sections, but print no backward formula: this is the gradient of the forward
 * stated above). out is the forward's output. The global form takes the forward's `lse`
 * (as written by zgattn_global_prefill; device fp32 [B, Hq, T]) or NULL, in which case the
 * log-sum-exp is recomputed by an extra pass over the keys; the SWA form always recomputes
 * it (its rows see at most `window` keys). dq, dg: [B, T, Hq, d]; dk, dv: [B, T, Hkv, d]
 * (the tensors' dtype, written, not accumulated); dwq, dwk: fp32 [d] (written). workspace
 * (device, >= zgattn_prefill_backward_workspace_bytes(desc) bytes, the same for bf16 and
 * fp32) holds the transformed q~/k~, the row statistics and the fp32 gradients of q~ and
 * k~. bf16 with head groups 1, 2, 4, 8 runs on MFMA kernels; fp32 tensors and other head
 * groups run on vector-ALU kernels (fp32 arithmetic), which also take the forward's `lse`.
 */
size_t zgattn_prefill_backward_workspace_bytes(const zgattn_desc* desc);
int zgattn_swa_prefill_backward(const zgattn_desc* desc, const void* q, const void* k,
                                const void* v, const void* g, const float* wq, const float* wk,
                                const void* out, const void* dout, void* dq, void* dk,
                                void* dv, void* dg, float* dwq, float* dwk, void* workspace,
                                size_t workspace_bytes, void* stream);
int zgattn_global_prefill_backward(const zgattn_desc* desc, const void* q, const void* k,
                                   const void* v, const float* wq, const float* wk,
                                   const void* out, const float* lse, const void* dout,
                                   void* dq, void* dk, void* dv, float* dwq, float* dwk,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gated SWA decode: one new token per sequence against a ring of `window` entries
 * (explainer, section アーキテクチャ: the SWA layers keep only a fixed 128 tokens).
 *   q, g, out: [B, Hq, d];  k_new, v_new: [B, Hkv, d] (raw, before norm/RoPE);
 *   k_ring, v_ring: [B, Hkv, window, d] holding post-norm, post-RoPE K and raw V;
 *   pos: device int32 [B], absolute position of the new token.
 * Position p lives in ring slot p % window. The call writes k~_new and v_new into slot
 * pos % window, then attends over positions max(0, pos-window+1) .. pos. A sequence
 * whose pos is negative or above ZGATTN_MAX_POSITION gets NaN outputs and an untouched
 * ring (checked on the device, since pos lives there). Tensors and ring are bf16 or fp32
 * (desc->dtype).
 */
int zgattn_swa_decode(const zgattn_desc* desc, const void* q, const void* k_new,
                      const void* v_new, const void* g, const float* wq, const float* wk,
                      void* k_ring, void* v_ring, const int32_t* pos, void* out,
                      void* stream);

/*
 * Global decode with split-K over the cache (explainer, section アーキテクチャ: decode is
 * memory-bandwidth-bound and the global layers keep the whole sequence).
 *   q, out: [B, Hq, d];  k_new, v_new: [B, Hkv, d];  caches [B, Hkv, capacity, d]
 *   (post-norm, post-RoPE K; raw V) valid for indices < pos[b];  pos: device int32 [B].
 * The call writes k~_new, v_new at cache index pos[b], then attends over 0 .. pos[b].
 * `workspace` (device, >= zgattn_global_decode_workspace_bytes(desc, capacity) bytes)
 * holds per-split partial results. A sequence with pos outside [0, capacity) gets NaN
 * outputs and an untouched cache. Tensors and caches are bf16 or fp32 (desc->dtype).
 */
int zgattn_global_decode(const zgattn_desc* desc, const void* q, const void* k_new,
                         const void* v_new, const float* wq, const float* wk,
                         void* k_cache, void* v_cache, int32_t capacity,
                         const int32_t* pos, void* workspace, size_t workspace_bytes,
                         void* out, void* stream);
size_t zgattn_global_decode_workspace_bytes(const zgattn_desc* desc, int32_t capacity);

/*
 * zgattn_global_decode without a caller workspace and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Arguments, outputs and cache update are those of
 * zgattn_global_decode. The split-K partials go to a scratch array of
 * ZGATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on, until the
 * process ends. The same kernels run; when zgattn_global_decode's split geometry would need
 * more scratch than that, this call takes longer cache chunks (fewer splits), which
 * changes only the rounding. If the partials cannot fit even so (roughly
 * B * Hq * head_dim * 8 bytes above the limit) the call returns ZGATTN_EWORKSPACE before
 * anything is launched. All calls on one GPU share its scratch: calls that overlap on one
 * GPU (other streams, or threads without ordering between them) race and give undefined
 * outputs; calls ordered on one stream are safe. Nothing in the scratch needs clearing
 * between calls: every value a step reads was written earlier in the same step.
 */
#define ZGATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int zgattn_global_decode_noalloc(const zgattn_desc* desc, const void* q, const void* k_new,
                                 const void* v_new, const float* wq, const float* wk,
                                 void* k_cache, void* v_cache, int32_t capacity,
                                 const int32_t* pos, void* out, void* stream);

/*
 * One decode step of a whole layer stack (explainer, section アーキテクチャ: 27 gated SWA
 * layers with a fixed 128-token cache and 5 global layers with the full sequence; the
 * jaehun.me review, section "KV 캐시가 6.4배 줄어드는 이유": 20 KiB of KV per token for the
 * stack). Each layer is exactly zgattn_swa_decode or zgattn_global_decode on its own
 * tensors; the layers are independent (post-projection inputs are given per layer), so
 * the call runs all SWA layers in one launch and all global layers in three (per 32
 * layers), instead of one to three launches per layer.
 *   layers: host array [n_layers]; is_global: host int32 [n_layers] (0 = gated SWA).
 *   Per layer: q, g, out [B, Hq, d]; k_new, v_new [B, Hkv, d]; wq, wk fp32 [d];
 *   k_cache, v_cache: SWA ring [B, Hkv, window, d] (window <= 128 here) or global cache
 *   [B, Hkv, capacity, d]. g is ignored (may be NULL) for global layers.
 *   pos: device int32 [B], shared by every layer. workspace (device, >=
 *   zgattn_model_decode_workspace_bytes(...) bytes) holds the global layers' partials.
 * Shapes and parameters come from desc (one desc for the stack). Errors as for the
 * single-layer calls; any invalid layer fails the whole call before anything launches.
 * bf16: SWA rings of at most 128 slots (ZGATTN_EUNSUPPORTED above). fp32 tensors and
 * caches run the layers one after another through the single-layer kernels.
 */
typedef struct {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* g;
  const float* wq;
  const float* wk;
  void* k_cache;
  void* v_cache;
  void* out;
} zgattn_decode_layer;

int zgattn_model_decode(const zgattn_desc* desc, int32_t n_layers, const int32_t* is_global,
                        const zgattn_decode_layer* layers, int32_t capacity,
                        const int32_t* pos, void* workspace, size_t workspace_bytes,
                        void* stream);
size_t zgattn_model_decode_workspace_bytes(const zgattn_desc* desc, int32_t n_layers,
                                           const int32_t* is_global, int32_t capacity);

/*
 * Standalone QK-RMSNorm + partial RoPE: the transform the q and k branches of both layer
 * kinds go through before attention ("ZGCM-1-7B 完全解説" explainer, section アーキテクチャ:
 * QK normalisation by RMSNorm and partial RoPE with rotary ratio 0.33; the jaehun.me
 * review, section "1) 구조·시스템 공동 설계", states both model-wide). Per row of d values:
 * y = RoPE(x / sqrt(mean(x^2) + rms_eps) * w, position), rotating the leading rotary_dim
 * dims as described at the top of this header. Its use here is building decode caches
 * (which hold post-norm, post-RoPE K) from a prefill's K.
 *   x: [B, T, n_heads, d] contiguous (desc->dtype);  w: fp32 [d];
 *   pos: device int32 [B*T] absolute positions, or NULL for pos_offset + t;
 *   y: same dtype, element (b, t, h, c) stored at
 *      y + b*y_stride_b + t*y_stride_t + h*y_stride_h + c   (strides in elements),
 *   so it can write straight into a [B, Hkv, S, d] cache. y must not overlap x.
 */
/* Errors: ZGATTN_ENULL for a NULL x, w or y (seq_len > 0); ZGATTN_EINVAL for unaligned
 * pointers or strides that are not multiples of 16 bytes or are negative; ZGATTN_ERANGE
 * when pos is NULL and pos_offset + seq_len - 1 exceeds ZGATTN_MAX_POSITION. Positions
 * given through pos are not checked on the host. */
int zgattn_qknorm_rope(const zgattn_desc* desc, int32_t n_heads, const void* x,
                       const float* w, const int32_t* pos, void* y, int64_t y_stride_b,
                       int64_t y_stride_t, int64_t y_stride_h, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZGATTN_H */
