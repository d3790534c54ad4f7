// Internal launch interface between the C ABI (api.cpp) and the kernel translation units.
#pragma once

// Host-side only: it includes the HIP runtime API, not the device headers, so the C ABI
// (api.cpp) builds with an ordinary C++ compiler too (the host-check test does so).
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "types.h"

namespace zg {

// Per-device facts queried once per device and process (the only global state of the
// library): the compute-unit count of the current device, and the dynamic-LDS limit of
// a kernel raised once per (device, kernel). Thread-safe.
hipError_t device_cu_count(int* cus);
hipError_t ensure_dynamic_smem(const void* kernel, int bytes);

// One prefill call (either layer kind), already validated on the host.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;      // gate pre-activation (SWA) or nullptr (global)
  void* out;
  const float* wq;
  const float* wk;
  void* kt;           // bf16 normalised+rotated K, [B][Hkv][T][d] (global with workspace) or nullptr
  void* vt;           // bf16 V as transposed 64-key tiles (with kt), see launch_kv_prepass
  int B, T, Hq, Hkv, d, window, rdim, pos_offset;
  int swa;            // 1: gated sliding window; 0: ungated full causal
  float eps;
  float scale;        // softmax scale (natural-log units)
  RopeFreq fr;
  // Packed documents (B == 1, T = total tokens): cu [n_docs + 1] on the device, each
  // document an independent sequence of at most max_len tokens; nullptr for dense batches.
  const int32_t* cu = nullptr;
  int n_docs = 0;
  int max_len = 0;
  // Optional row log-sum-exp, natural log, fp32 [B][Hq][T] (dense bf16 global layers).
  float* lse = nullptr;
};
// Rows of slack after the last K~ row of the global-prefill workspace: a 64-key tile that
// starts at the last row stays inside the workspace without clamping its row indices.
constexpr int kKtSlackRows = 64;
// Bytes of the K~ part of the global-prefill workspace (rows of all heads + slack), and
// where the V tiles start (256-byte aligned).
inline size_t prefill_kt_bytes(size_t rows, int d) {
  return ((rows + kKtSlackRows) * d * 2 + 255) & ~(size_t)255;
}
// V-tile slots per KV head of a packed batch (see doc_tile_base).
inline int varlen_vtile_slots(int T, int n_docs) { return T / 64 + n_docs; }
size_t prefill_vtiles_bytes_varlen(int Hkv, int T, int n_docs, int d);

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
// The vector-ALU prefill (fp32 arithmetic): fp32 tensors (f32), or bf16 tensors of shapes
// the MFMA kernels do not take (prefill_bf16_supported false). Dense or packed documents.
hipError_t launch_prefill_valu(const PrefillArgs& a, bool f32, hipStream_t s);
bool prefill_bf16_supported(int d, int group, int rdim);
// Tile-transposed V for the global path: [B][Hkv][ceil(T/64)][d][64] bf16.
size_t prefill_vtiles_bytes(int B, int Hkv, int T, int d);
// The global path's pre-pass: K~ rows into a.kt and V tiles into a.vt (dense or packed).
hipError_t launch_kv_prepass(const PrefillArgs& a, hipStream_t s);
// Streaming sliding-window kernel for the model's layer shape (d 128, 4 query heads per KV
// head, rotary_dim 42, window <= 128); launch_prefill_bf16 routes such calls to it.
bool swa_stream_supported(const PrefillArgs& a);
hipError_t launch_swa_stream(const PrefillArgs& a, hipStream_t s);

// Standalone QK-RMSNorm + partial RoPE with strided output.
struct NormRopeArgs {
  const void* x;
  const float* w;
  const int32_t* pos;  // [B*T] or nullptr
  void* y;
  int64_t ysb, yst, ysh;  // output strides in elements
  int B, T, H, d, rdim, pos_offset, is_bf16;
  float eps;
  float out_scale;        // multiplies the result (1 for the public entry point)
  RopeFreq fr;
  const int32_t* cu = nullptr;   // packed documents (B == 1): positions restart per document
  int n_docs = 0;
};
hipError_t launch_qknorm_rope(const NormRopeArgs& a, hipStream_t s);

// Backward pass of a prefill call (d 64 or 128): gradients of sum(dout * out). bf16 with
// head groups 1, 2, 4, 8 on the MFMA kernels; fp32 and other head groups on vector-ALU
// kernels.
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;       // gate pre-activation (SWA) or nullptr
  const void* out;     // the forward's output
  const void* dout;
  const float* wq;
  const float* wk;
  void* dq;
  void* dk;
  void* dv;
  void* dg;            // SWA only
  float* dwq;
  float* dwk;
  const float* lse;    // the forward's row log-sum-exp [B][Hq][T] (natural log) or nullptr
  void* ws;            // workspace of backward_workspace_bytes()
  int B, T, Hq, Hkv, d, window, rdim, pos_offset, swa;
  float eps, scale;
  RopeFreq fr;
  int f32;             // fp32 tensors (the vector-ALU kernels), else bf16
};
size_t backward_workspace_bytes(int B, int T, int Hq, int Hkv, int d);
hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t s);

// One decode step (either layer kind), bf16.
struct DecodeArgs {
  const void* q;       // [B][Hq][d]
  const void* k_new;   // [B][Hkv][d]
  const void* v_new;
  const void* g;       // [B][Hq][d] (SWA) or nullptr
  const float* wq;
  const float* wk;
  void* k_cache;       // [B][Hkv][S][d]
  void* v_cache;
  const int32_t* pos;  // [B]
  void* out;           // [B][Hq][d]
  float* ws;           // global: workspace; SWA: unused
  int B, Hq, Hkv, d, S, rdim, window, nsplit, chunk;
  float eps, scale;
  RopeFreq fr;
  int f32;             // tensors and caches fp32 (single-layer calls), else bf16
};
hipError_t launch_swa_decode(const DecodeArgs& a, hipStream_t s);

// The tensors of one layer in a batched (several layers, one launch per kernel) decode
// step; the scalar fields (shapes, positions, RoPE table) come from the DecodeArgs.
struct LayerIO {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* g;
  const float* wq;
  const float* wk;
  void* k_cache;
  void* v_cache;
  void* out;
  float* ws;
};
constexpr int kMaxDecodeLayers = 32;   // layers per launch (kernel-argument table)
struct DecodeBatchArgs {
  DecodeArgs a;
  LayerIO io[kMaxDecodeLayers];
};
static_assert(sizeof(DecodeBatchArgs) <= 4096, "kernel arguments");
// One decode step of many layers: SWA layers (rings of a.window <= 128 slots) in one
// launch per kMaxDecodeLayers, global layers (caches of a.S positions, split-K geometry
// in a.nsplit / a.chunk, workspace per layer in io.ws) in three.
hipError_t launch_swa_decode_layers(const DecodeArgs& a, const LayerIO* io, int n, hipStream_t s);
hipError_t launch_global_decode_layers(const DecodeArgs& a, const LayerIO* io, int n,
                                       hipStream_t s);
constexpr int kSwaDecodeLayersMaxWindow = 128;
hipError_t launch_global_decode(const DecodeArgs& a, hipStream_t s);
// Split-K geometry and workspace bytes for a global decode call.
void global_decode_geometry(int B, int Hq, int d, int capacity, int* nsplit, int* chunk,
                            size_t* ws_bytes);
// The same geometry with chunks lengthened (doubled) until the workspace fits max_bytes
// and the split kernel's LDS stays within a CU; false when no such geometry exists.
bool global_decode_geometry_capped(int B, int Hq, int Hkv, int d, int capacity,
                                   size_t max_bytes, int* nsplit, int* chunk,
                                   size_t* ws_bytes);
// Device address of the current device's no-allocation decode scratch (looked up once per
// device) and its size in bytes.
hipError_t decode_noalloc_scratch(void** ptr, size_t* bytes);

}  // namespace zg
