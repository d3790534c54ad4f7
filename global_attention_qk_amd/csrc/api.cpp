// C ABI of libzgattn: host-side argument checks, RoPE frequency tables and launches.
// Every check happens before anything is launched; see include/zgattn.h for the contract.
#include "zgattn.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace zg {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // 0 = not queried yet
struct SmemAttr {
  const void* kernel;
  int dev;
  int bytes;
};
constexpr int kMaxSmemAttrs = 512;
SmemAttr g_smem[kMaxSmemAttrs];
int g_n_smem = 0;
std::mutex g_smem_mu;
}  // namespace

hipError_t device_cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (c < 1) c = 1;
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return hipSuccess;
}

hipError_t ensure_dynamic_smem(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_smem_mu);
  for (int i = 0; i < g_n_smem; ++i)
    if (g_smem[i].kernel == kernel && g_smem[i].dev == dev && g_smem[i].bytes >= bytes)
      return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  for (int i = 0; i < g_n_smem; ++i)
    if (g_smem[i].kernel == kernel && g_smem[i].dev == dev) {
      g_smem[i].bytes = bytes;
      return hipSuccess;
    }
  if (g_n_smem < kMaxSmemAttrs) g_smem[g_n_smem++] = SmemAttr{kernel, dev, bytes};
  return hipSuccess;
}

}  // namespace zg

using namespace zg;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_desc(const zgattn_desc* d) {
  if (!d) return ZGATTN_ENULL;
  if (d->dtype != ZGATTN_F32 && d->dtype != ZGATTN_BF16) return ZGATTN_EDTYPE;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return ZGATTN_EINVAL;
  if (d->n_q_heads % d->n_kv_heads != 0) return ZGATTN_EINVAL;
  if (d->head_dim != 64 && d->head_dim != 128) return ZGATTN_EUNSUPPORTED;
  if (d->rotary_dim < 0 || d->rotary_dim > d->head_dim || (d->rotary_dim & 1)) return ZGATTN_EINVAL;
  if (!(d->rope_base > 0.0f) || !isfinite(d->rope_base)) return ZGATTN_EINVAL;
  if (!(d->rms_eps >= 0.0f) || !isfinite(d->rms_eps)) return ZGATTN_EINVAL;
  if (!isfinite(d->softmax_scale)) return ZGATTN_EINVAL;
  if (d->pos_offset < 0 || d->pos_offset > ZGATTN_MAX_POSITION) return ZGATTN_ERANGE;
  return ZGATTN_OK;
}

float scale_of(const zgattn_desc* d) {
  return d->softmax_scale > 0.0f ? d->softmax_scale : (float)(1.0 / sqrt((double)d->head_dim));
}

// f_k = base^(-2k/r) / (2 pi) revolutions per position, as an fp32 head + tail pair.
RopeFreq rope_freq(int rdim, float base) {
  RopeFreq f;
  for (int k = 0; k < kMaxHalfRot; ++k) {
    f.hi[k] = 0.0f;
    f.lo[k] = 0.0f;
  }
  const int half = rdim / 2;
  const long double two_pi = 6.283185307179586476925286766559L;
  for (int k = 0; k < half; ++k) {
    const long double v = powl((long double)base, -2.0L * k / rdim) / two_pi;
    const float h = (float)v;
    f.hi[k] = h;
    f.lo[k] = (float)(v - (long double)h);
  }
  return f;
}

int prefill_common(const zgattn_desc* d, const void* q, const void* k, const void* v,
                   const float* wq, const float* wk, void* out) {
  int st = check_desc(d);
  if (st) return st;
  if (d->seq_len < 0) return ZGATTN_EINVAL;
  if (d->seq_len > 0 && (int64_t)d->pos_offset + d->seq_len - 1 > ZGATTN_MAX_POSITION)
    return ZGATTN_ERANGE;
  if (d->seq_len == 0) return ZGATTN_OK;
  if (!q || !k || !v || !wq || !wk || !out) return ZGATTN_ENULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ZGATTN_EINVAL;
  return ZGATTN_OK;
}

PrefillArgs make_prefill(const zgattn_desc* d, const void* q, const void* k, const void* v,
                         const void* g, const float* wq, const float* wk, void* out, int swa) {
  PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.out = out;
  a.wq = wq;
  a.wk = wk;
  a.kt = nullptr;
  a.vt = nullptr;
  a.B = d->batch;
  a.T = d->seq_len;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.window = d->window;
  a.rdim = d->rotary_dim;
  a.pos_offset = d->pos_offset;
  a.swa = swa;
  a.eps = d->rms_eps;
  a.scale = scale_of(d);
  a.fr = rope_freq(d->rotary_dim, d->rope_base);
  return a;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ZGATTN_OK : ZGATTN_EHIP; }

int decode_common(const zgattn_desc* d, const void* q, const void* k_new, const void* v_new,
                  const float* wq, const float* wk, void* kc, void* vc, const int32_t* pos,
                  void* out, bool allow_f32 = true) {
  int st = check_desc(d);
  if (st) return st;
  if (!q || !k_new || !v_new || !wq || !wk || !kc || !vc || !pos || !out) return ZGATTN_ENULL;
  if (d->dtype != ZGATTN_BF16 && !(allow_f32 && d->dtype == ZGATTN_F32))
    return ZGATTN_EUNSUPPORTED;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ZGATTN_EUNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(kc) ||
      !aligned16(vc) || !aligned16(out))
    return ZGATTN_EINVAL;
  return ZGATTN_OK;
}

DecodeArgs make_decode(const zgattn_desc* d, const void* q, const void* k_new,
                       const void* v_new, const void* g, const float* wq, const float* wk,
                       void* kc, void* vc, const int32_t* pos, void* out) {
  DecodeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.g = g;
  a.wq = wq;
  a.wk = wk;
  a.k_cache = kc;
  a.v_cache = vc;
  a.pos = pos;
  a.out = out;
  a.ws = nullptr;
  a.B = d->batch;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.S = 0;
  a.rdim = d->rotary_dim;
  a.window = d->window;
  a.nsplit = 0;
  a.chunk = 0;
  a.f32 = d->dtype == ZGATTN_F32;
  a.eps = d->rms_eps;
  a.scale = scale_of(d);
  a.fr = rope_freq(d->rotary_dim, d->rope_base);
  return a;
}

}  // namespace

extern "C" {

int zgattn_abi_version(void) { return ZGATTN_ABI_VERSION; }

const char* zgattn_strerror(int status) {
  switch (status) {
    case ZGATTN_OK: return "ok";
    case ZGATTN_EINVAL: return "invalid argument (size, parameter or alignment)";
    case ZGATTN_ENULL: return "required pointer is NULL";
    case ZGATTN_EDTYPE: return "unknown dtype";
    case ZGATTN_EUNSUPPORTED: return "unsupported configuration";
    case ZGATTN_EWORKSPACE: return "workspace missing or too small";
    case ZGATTN_ERANGE: return "position or capacity out of range";
    case ZGATTN_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int zgattn_swa_prefill(const zgattn_desc* d, const void* q, const void* k, const void* v,
                       const void* g, const float* wq, const float* wk, void* out,
                       void* stream) {
  int st = prefill_common(d, q, k, v, wq, wk, out);
  if (st) return st;
  if (d->window < 1) return ZGATTN_EINVAL;
  if (d->seq_len == 0) return ZGATTN_OK;
  if (!g) return ZGATTN_ENULL;
  if (!aligned16(g)) return ZGATTN_EINVAL;
  PrefillArgs a = make_prefill(d, q, k, v, g, wq, wk, out, 1);
  hipStream_t s = (hipStream_t)stream;
  if (d->dtype == ZGATTN_F32 || !prefill_bf16_supported(a.d, a.Hq / a.Hkv, a.rdim))
    return hip_status(launch_prefill_valu(a, d->dtype == ZGATTN_F32, s));
  return hip_status(launch_prefill_bf16(a, s));
}

size_t zgattn_global_prefill_workspace_bytes(const zgattn_desc* d) {
  if (check_desc(d) || d->seq_len < 0) return 0;
  if (d->dtype != ZGATTN_BF16) return 0;
  // normalised+rotated K (plus a tile of slack), then V as transposed 64-key tiles
  return prefill_kt_bytes((size_t)d->batch * d->n_kv_heads * (size_t)d->seq_len, d->head_dim) +
         prefill_vtiles_bytes(d->batch, d->n_kv_heads, d->seq_len, d->head_dim);
}

int zgattn_global_prefill(const zgattn_desc* d, const void* q, const void* k, const void* v,
                          const float* wq, const float* wk, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream) {
  int st = prefill_common(d, q, k, v, wq, wk, out);
  if (st) return st;
  if (lse && ((uintptr_t)lse & 3)) return ZGATTN_EINVAL;
  // fp32, or a bf16 shape the MFMA kernels do not take: the vector-ALU kernel (no
  // workspace used, no log-sum-exp output)
  const bool valu = d->dtype == ZGATTN_F32 ||
                    !prefill_bf16_supported(d->head_dim, d->n_q_heads / d->n_kv_heads,
                                            d->rotary_dim);
  if (lse && valu) return ZGATTN_EUNSUPPORTED;
  if (d->seq_len == 0) return ZGATTN_OK;
  PrefillArgs a = make_prefill(d, q, k, v, nullptr, wq, wk, out, 0);
  a.lse = lse;
  hipStream_t s = (hipStream_t)stream;
  if (valu) return hip_status(launch_prefill_valu(a, d->dtype == ZGATTN_F32, s));
  if (workspace) {
    if (workspace_bytes < zgattn_global_prefill_workspace_bytes(d) || !aligned16(workspace))
      return ZGATTN_EWORKSPACE;
    // K~ rows [B][Hkv][T][d] and V tiles, one pre-pass
    a.kt = workspace;
    a.vt = (void*)((char*)workspace + prefill_kt_bytes((size_t)a.B * a.Hkv * a.T, a.d));
    if (launch_kv_prepass(a, s) != hipSuccess) return ZGATTN_EHIP;
  }
  return hip_status(launch_prefill_bf16(a, s));
}

int zgattn_swa_decode(const zgattn_desc* d, const void* q, const void* k_new, const void* v_new,
                      const void* g, const float* wq, const float* wk, void* k_ring,
                      void* v_ring, const int32_t* pos, void* out, void* stream) {
  int st = decode_common(d, q, k_new, v_new, wq, wk, k_ring, v_ring, pos, out);
  if (st) return st;
  if (!g) return ZGATTN_ENULL;
  if (!aligned16(g)) return ZGATTN_EINVAL;
  if (d->window < 1 || d->window > 4096) return ZGATTN_EINVAL;
  DecodeArgs a = make_decode(d, q, k_new, v_new, g, wq, wk, k_ring, v_ring, pos, out);
  return hip_status(launch_swa_decode(a, (hipStream_t)stream));
}

size_t zgattn_global_decode_workspace_bytes(const zgattn_desc* d, int32_t capacity) {
  if (check_desc(d) || capacity < 1) return 0;
  int ns, chunk;
  size_t bytes;
  global_decode_geometry(d->batch, d->n_q_heads, d->head_dim, capacity, &ns, &chunk, &bytes);
  return bytes;
}

int zgattn_global_decode(const zgattn_desc* d, const void* q, const void* k_new,
                         const void* v_new, const float* wq, const float* wk, void* k_cache,
                         void* v_cache, int32_t capacity, const int32_t* pos, void* workspace,
                         size_t workspace_bytes, void* out, void* stream) {
  int st = decode_common(d, q, k_new, v_new, wq, wk, k_cache, v_cache, pos, out);
  if (st) return st;
  if (capacity < 1 || capacity > ZGATTN_MAX_POSITION + 1) return ZGATTN_ERANGE;
  if (!workspace || !aligned16(workspace)) return ZGATTN_EWORKSPACE;
  DecodeArgs a = make_decode(d, q, k_new, v_new, nullptr, wq, wk, k_cache, v_cache, pos, out);
  size_t need;
  global_decode_geometry(a.B, a.Hq, a.d, capacity, &a.nsplit, &a.chunk, &need);
  if (workspace_bytes < need) return ZGATTN_EWORKSPACE;
  a.S = capacity;
  a.ws = (float*)workspace;
  return hip_status(launch_global_decode(a, (hipStream_t)stream));
}

int zgattn_global_decode_noalloc(const zgattn_desc* d, const void* q, const void* k_new,
                                 const void* v_new, const float* wq, const float* wk,
                                 void* k_cache, void* v_cache, int32_t capacity,
                                 const int32_t* pos, void* out, void* stream) {
  int st = decode_common(d, q, k_new, v_new, wq, wk, k_cache, v_cache, pos, out);
  if (st) return st;
  if (capacity < 1 || capacity > ZGATTN_MAX_POSITION + 1) return ZGATTN_ERANGE;
  DecodeArgs a = make_decode(d, q, k_new, v_new, nullptr, wq, wk, k_cache, v_cache, pos, out);
  size_t need;
  if (!global_decode_geometry_capped(a.B, a.Hq, a.Hkv, a.d, capacity,
                                     ZGATTN_NOALLOC_SCRATCH_BYTES, &a.nsplit, &a.chunk, &need))
    return ZGATTN_EWORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (decode_noalloc_scratch(&ws, &ws_bytes) != hipSuccess) return ZGATTN_EHIP;
  if (need > ws_bytes) return ZGATTN_EWORKSPACE;
  a.S = capacity;
  a.ws = (float*)ws;
  return hip_status(launch_global_decode(a, (hipStream_t)stream));
}

size_t zgattn_model_decode_workspace_bytes(const zgattn_desc* d, int32_t n_layers,
                                           const int32_t* is_global, int32_t capacity) {
  if (check_desc(d) || n_layers < 0 || (n_layers > 0 && !is_global)) return 0;
  int n_glob = 0;
  for (int i = 0; i < n_layers; ++i) n_glob += is_global[i] != 0;
  if (n_glob == 0) return 0;
  const size_t per = zgattn_global_decode_workspace_bytes(d, capacity);
  return per ? n_glob * ((per + 255) & ~(size_t)255) : 0;
}

// Packed documents: B == 1, T = total tokens, cu [n_docs + 1] on the device.
int varlen_common(const zgattn_desc* d, const int32_t* cu, int32_t n_docs, int32_t max_len,
                  const void* q, const void* k, const void* v, const float* wq,
                  const float* wk, void* out) {
  int st = check_desc(d);
  if (st) return st;
  if (d->batch != 1 || d->seq_len < 0) return ZGATTN_EINVAL;
  if (n_docs < 1 || n_docs > 65535 || max_len < 0 || max_len > d->seq_len) return ZGATTN_EINVAL;
  if (max_len > 0 && (int64_t)d->pos_offset + max_len - 1 > ZGATTN_MAX_POSITION)
    return ZGATTN_ERANGE;
  if (d->seq_len == 0 || max_len == 0) return ZGATTN_OK;
  if (!cu || !q || !k || !v || !wq || !wk || !out) return ZGATTN_ENULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ZGATTN_EINVAL;
  return ZGATTN_OK;
}

// fp32 tensors, or bf16 shapes the MFMA kernels do not take: the vector-ALU kernel.
bool prefill_takes_valu(const zgattn_desc* d) {
  return d->dtype == ZGATTN_F32 ||
         !prefill_bf16_supported(d->head_dim, d->n_q_heads / d->n_kv_heads, d->rotary_dim);
}

int zgattn_swa_prefill_varlen(const zgattn_desc* d, const int32_t* cu_seqlens, int32_t n_docs,
                              int32_t max_seqlen, const void* q, const void* k, const void* v,
                              const void* g, const float* wq, const float* wk, void* out,
                              void* stream) {
  int st = varlen_common(d, cu_seqlens, n_docs, max_seqlen, q, k, v, wq, wk, out);
  if (st) return st;
  if (d->window < 1) return ZGATTN_EINVAL;
  if (d->seq_len == 0 || max_seqlen == 0) return ZGATTN_OK;
  if (!g) return ZGATTN_ENULL;
  if (!aligned16(g)) return ZGATTN_EINVAL;
  PrefillArgs a = make_prefill(d, q, k, v, g, wq, wk, out, 1);
  a.cu = cu_seqlens;
  a.n_docs = n_docs;
  a.max_len = max_seqlen;
  if (prefill_takes_valu(d))
    return hip_status(launch_prefill_valu(a, d->dtype == ZGATTN_F32, (hipStream_t)stream));
  return hip_status(launch_prefill_bf16(a, (hipStream_t)stream));
}

size_t zgattn_global_prefill_varlen_workspace_bytes(const zgattn_desc* d, int32_t n_docs) {
  if (check_desc(d) || d->seq_len < 0 || d->batch != 1 || n_docs < 1) return 0;
  if (d->dtype != ZGATTN_BF16) return 0;
  return prefill_kt_bytes((size_t)d->n_kv_heads * d->seq_len, d->head_dim) +
         prefill_vtiles_bytes_varlen(d->n_kv_heads, d->seq_len, n_docs, d->head_dim);
}

int zgattn_global_prefill_varlen(const zgattn_desc* d, const int32_t* cu_seqlens,
                                 int32_t n_docs, int32_t max_seqlen, const void* q,
                                 const void* k, const void* v, const float* wq,
                                 const float* wk, void* workspace, size_t workspace_bytes,
                                 void* out, void* stream) {
  int st = varlen_common(d, cu_seqlens, n_docs, max_seqlen, q, k, v, wq, wk, out);
  if (st) return st;
  if (d->seq_len == 0 || max_seqlen == 0) return ZGATTN_OK;
  PrefillArgs a = make_prefill(d, q, k, v, nullptr, wq, wk, out, 0);
  a.cu = cu_seqlens;
  a.n_docs = n_docs;
  a.max_len = max_seqlen;
  hipStream_t s = (hipStream_t)stream;
  // the vector-ALU kernel takes no workspace (a given one is not used)
  if (prefill_takes_valu(d)) return hip_status(launch_prefill_valu(a, d->dtype == ZGATTN_F32, s));
  if (workspace) {
    if (workspace_bytes < zgattn_global_prefill_varlen_workspace_bytes(d, n_docs) ||
        !aligned16(workspace))
      return ZGATTN_EWORKSPACE;
    // K~ rows [Hkv][T][d] (positions restart at each document) and per-document V tiles
    a.kt = workspace;
    a.vt = (void*)((char*)workspace + prefill_kt_bytes((size_t)a.Hkv * a.T, a.d));
    if (launch_kv_prepass(a, s) != hipSuccess) return ZGATTN_EHIP;
  }
  return hip_status(launch_prefill_bf16(a, s));
}

size_t zgattn_prefill_backward_workspace_bytes(const zgattn_desc* d) {
  if (check_desc(d) || d->seq_len < 0) return 0;
  return backward_workspace_bytes(d->batch, d->seq_len, d->n_q_heads, d->n_kv_heads,
                                  d->head_dim);
}

int backward_common(const zgattn_desc* d, int swa, const void* q, const void* k, const void* v,
                    const void* g, const float* wq, const float* wk, const void* out,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dg,
                    float* dwq, float* dwk, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int st = prefill_common(d, q, k, v, wq, wk, const_cast<void*>(out));
  if (st) return st;
  if (lse && ((uintptr_t)lse & 3)) return ZGATTN_EINVAL;
  if (swa && d->window < 1) return ZGATTN_EINVAL;
  if (d->seq_len == 0) return ZGATTN_OK;
  if (!dout || !dq || !dk || !dv || !dwq || !dwk || (swa && (!g || !dg))) return ZGATTN_ENULL;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (swa && (!aligned16(g) || !aligned16(dg))))
    return ZGATTN_EINVAL;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < zgattn_prefill_backward_workspace_bytes(d))
    return ZGATTN_EWORKSPACE;
  BackwardArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = swa ? g : nullptr;
  a.out = out;
  a.dout = dout;
  a.wq = wq;
  a.wk = wk;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = swa ? dg : nullptr;
  a.dwq = dwq;
  a.dwk = dwk;
  a.lse = lse;
  a.ws = workspace;
  a.B = d->batch;
  a.T = d->seq_len;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.window = d->window;
  a.rdim = d->rotary_dim;
  a.pos_offset = d->pos_offset;
  a.swa = swa;
  a.eps = d->rms_eps;
  a.scale = scale_of(d);
  a.fr = rope_freq(d->rotary_dim, d->rope_base);
  a.f32 = d->dtype == ZGATTN_F32;
  return hip_status(launch_prefill_backward(a, (hipStream_t)stream));
}

int zgattn_swa_prefill_backward(const zgattn_desc* d, const void* q, const void* k,
                                const void* v, const void* g, const float* wq, const float* wk,
                                const void* out, const void* dout, void* dq, void* dk,
                                void* dv, void* dg, float* dwq, float* dwk, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!g && d && d->seq_len > 0) return check_desc(d) ? check_desc(d) : ZGATTN_ENULL;
  return backward_common(d, 1, q, k, v, g, wq, wk, out, nullptr, dout, dq, dk, dv, dg, dwq,
                         dwk, workspace, workspace_bytes, stream);
}

int zgattn_global_prefill_backward(const zgattn_desc* d, const void* q, const void* k,
                                   const void* v, const float* wq, const float* wk,
                                   const void* out, const float* lse, const void* dout,
                                   void* dq, void* dk, void* dv, float* dwq, float* dwk,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return backward_common(d, 0, q, k, v, nullptr, wq, wk, out, lse, dout, dq, dk, dv, nullptr,
                         dwq, dwk, workspace, workspace_bytes, stream);
}

int zgattn_model_decode(const zgattn_desc* d, int32_t n_layers, const int32_t* is_global,
                        const zgattn_decode_layer* layers, int32_t capacity,
                        const int32_t* pos, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_desc(d);
  if (st) return st;
  if (n_layers < 0 || n_layers > 1024) return ZGATTN_EINVAL;
  if (n_layers == 0) return ZGATTN_OK;
  if (!is_global || !layers || !pos) return ZGATTN_ENULL;
  // every layer is checked before anything is launched
  int n_glob = 0, n_swa = 0;
  for (int i = 0; i < n_layers; ++i) {
    const zgattn_decode_layer& L = layers[i];
    st = decode_common(d, L.q, L.k_new, L.v_new, L.wq, L.wk, L.k_cache, L.v_cache, pos, L.out);
    if (st) return st;
    if (is_global[i]) {
      ++n_glob;
    } else {
      if (!L.g) return ZGATTN_ENULL;
      if (!aligned16(L.g)) return ZGATTN_EINVAL;
      ++n_swa;
    }
  }
  const bool f32 = d->dtype == ZGATTN_F32;
  if (n_swa && d->window < 1) return ZGATTN_EINVAL;
  if (n_swa && !f32 && d->window > kSwaDecodeLayersMaxWindow) return ZGATTN_EUNSUPPORTED;
  DecodeArgs a = make_decode(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, pos, nullptr);
  size_t stride = 0;
  if (n_glob) {
    if (capacity < 1 || capacity > ZGATTN_MAX_POSITION + 1) return ZGATTN_ERANGE;
    if (!workspace || !aligned16(workspace)) return ZGATTN_EWORKSPACE;
    size_t per;
    global_decode_geometry(a.B, a.Hq, a.d, capacity, &a.nsplit, &a.chunk, &per);
    stride = (per + 255) & ~(size_t)255;
    if (workspace_bytes < n_glob * stride) return ZGATTN_EWORKSPACE;
    a.S = capacity;
  }
  const hipStream_t s = (hipStream_t)stream;
  if (f32) {
    // fp32: the single-layer kernels, one layer after another
    int gi = 0;
    for (int i = 0; i < n_layers; ++i) {
      const zgattn_decode_layer& L = layers[i];
      DecodeArgs la = a;
      la.q = L.q;
      la.k_new = L.k_new;
      la.v_new = L.v_new;
      la.wq = L.wq;
      la.wk = L.wk;
      la.k_cache = L.k_cache;
      la.v_cache = L.v_cache;
      la.out = L.out;
      if (is_global[i]) {
        la.g = nullptr;
        la.ws = (float*)((char*)workspace + (gi++) * stride);
        st = hip_status(launch_global_decode(la, s));
      } else {
        la.g = L.g;
        la.ws = nullptr;
        st = hip_status(launch_swa_decode(la, s));
      }
      if (st) return st;
    }
    return ZGATTN_OK;
  }
  // launches per kind, kMaxDecodeLayers layers at a time (all SWA layers first)
  LayerIO io[kMaxDecodeLayers];
  for (int kind = 0; kind < 2; ++kind) {
    int m = 0, gi = 0;
    for (int i = 0; i <= n_layers; ++i) {
      const bool take = i < n_layers && (is_global[i] != 0) == (kind == 1);
      if (take) {
        const zgattn_decode_layer& L = layers[i];
        io[m++] = LayerIO{L.q, L.k_new, L.v_new, L.g, L.wq, L.wk, L.k_cache, L.v_cache, L.out,
                          kind ? (float*)((char*)workspace + (gi++) * stride) : nullptr};
      }
      if (m == kMaxDecodeLayers || (i == n_layers && m > 0)) {
        st = hip_status(kind ? launch_global_decode_layers(a, io, m, s)
                             : launch_swa_decode_layers(a, io, m, s));
        if (st) return st;
        m = 0;
      }
    }
  }
  return ZGATTN_OK;
}

int zgattn_qknorm_rope(const zgattn_desc* d, int32_t n_heads, const void* x, const float* w,
                       const int32_t* pos, void* y, int64_t y_stride_b, int64_t y_stride_t,
                       int64_t y_stride_h, void* stream) {
  int st = check_desc(d);
  if (st) return st;
  if (d->seq_len < 0 || n_heads < 1) return ZGATTN_EINVAL;
  if (!pos && d->seq_len > 0 && (int64_t)d->pos_offset + d->seq_len - 1 > ZGATTN_MAX_POSITION)
    return ZGATTN_ERANGE;
  if (d->seq_len == 0) return ZGATTN_OK;
  if (!x || !w || !y) return ZGATTN_ENULL;
  const int esz = d->dtype == ZGATTN_BF16 ? 2 : 4;
  if (!aligned16(x) || !aligned16(y)) return ZGATTN_EINVAL;
  if ((y_stride_b * esz) % 16 || (y_stride_t * esz) % 16 || (y_stride_h * esz) % 16)
    return ZGATTN_EINVAL;
  if (y_stride_b < 0 || y_stride_t < 0 || y_stride_h < 0) return ZGATTN_EINVAL;
  NormRopeArgs n;
  n.x = x;
  n.w = w;
  n.pos = pos;
  n.y = y;
  n.ysb = y_stride_b;
  n.yst = y_stride_t;
  n.ysh = y_stride_h;
  n.B = d->batch;
  n.T = d->seq_len;
  n.H = n_heads;
  n.d = d->head_dim;
  n.rdim = d->rotary_dim;
  n.pos_offset = d->pos_offset;
  n.is_bf16 = d->dtype == ZGATTN_BF16;
  n.eps = d->rms_eps;
  n.out_scale = 1.0f;
  n.fr = rope_freq(d->rotary_dim, d->rope_base);
  return hip_status(launch_qknorm_rope(n, (hipStream_t)stream));
}

}  // extern "C"
