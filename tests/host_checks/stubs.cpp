// Test-only stand-ins for the kernel launchers and the three HIP runtime calls the C ABI
// makes, so that api.cpp (argument checks, workspace sizing, layer tables, per-device
// caches) runs on the CPU under sanitizers. No kernel runs and no memory is touched: the
// launchers record their arguments. Sizes follow the layouts the header documents.
#include "stubs.h"

namespace stub {
int valu_launches;
bool last_valu_f32;
int launches, prefill_launches, aux_launches, decode_launches, batched_layers,
    scratch_lookups;
int smem_attr_calls;
zg::PrefillArgs last_prefill;
zg::BackwardArgs last_backward;
zg::DecodeArgs last_decode;
alignas(256) static unsigned char scratch_buf[256];
void* const scratch = scratch_buf;
void reset() {
  launches = prefill_launches = aux_launches = decode_launches = batched_layers = 0;
  valu_launches = 0;
  scratch_lookups = 0;
}
}  // namespace stub

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) {
  __atomic_add_fetch(&stub::smem_attr_calls, 1, __ATOMIC_RELAXED);
  return hipSuccess;
}
}

namespace zg {
static hipError_t rec_prefill(const PrefillArgs& a) {
  ++stub::launches;
  ++stub::prefill_launches;
  stub::last_prefill = a;
  return hipSuccess;
}
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t) { return rec_prefill(a); }
hipError_t launch_prefill_valu(const PrefillArgs& a, bool f32, hipStream_t) {
  ++stub::valu_launches;
  stub::last_valu_f32 = f32;
  return rec_prefill(a);
}
bool prefill_bf16_supported(int d, int group, int rdim) {
  return (d == 64 || d == 128) && group >= 1 && 256 % group == 0 && (256 / group) % 32 == 0 &&
         rdim <= 64;
}
size_t prefill_vtiles_bytes(int B, int Hkv, int T, int d) {
  return (size_t)B * Hkv * ((T + 63) / 64) * 64 * d * 2;
}
size_t prefill_vtiles_bytes_varlen(int Hkv, int T, int n_docs, int d) {
  return (size_t)Hkv * (T / 64 + n_docs) * 64 * d * 2;
}
hipError_t launch_kv_prepass(const PrefillArgs&, hipStream_t) {
  ++stub::launches;
  ++stub::aux_launches;
  return hipSuccess;
}
hipError_t launch_qknorm_rope(const NormRopeArgs&, hipStream_t) {
  ++stub::launches;
  ++stub::aux_launches;
  return hipSuccess;
}
size_t backward_workspace_bytes(int B, int T, int Hq, int Hkv, int d) {
  return (size_t)B * T * (Hq + Hkv) * d * 16 + 4096;
}
hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t) {
  ++stub::launches;
  stub::last_backward = a;
  return hipSuccess;
}
static hipError_t rec_decode(const DecodeArgs& a) {
  ++stub::launches;
  ++stub::decode_launches;
  stub::last_decode = a;
  return hipSuccess;
}
hipError_t launch_swa_decode(const DecodeArgs& a, hipStream_t) { return rec_decode(a); }
hipError_t launch_global_decode(const DecodeArgs& a, hipStream_t) { return rec_decode(a); }
hipError_t launch_swa_decode_layers(const DecodeArgs& a, const LayerIO* io, int n, hipStream_t) {
  for (int i = 0; i < n; ++i)   // every entry must be readable
    if (!io[i].q || !io[i].k_cache) return hipErrorInvalidValue;
  stub::batched_layers += n;
  return rec_decode(a);
}
hipError_t launch_global_decode_layers(const DecodeArgs& a, const LayerIO* io, int n,
                                       hipStream_t) {
  for (int i = 0; i < n; ++i)
    if (!io[i].q || !io[i].ws) return hipErrorInvalidValue;
  stub::batched_layers += n;
  return rec_decode(a);
}
void global_decode_geometry(int B, int Hq, int d, int capacity, int* nsplit, int* chunk,
                            size_t* ws_bytes) {
  const int c = capacity <= 65536 ? 64 : 2048;
  *chunk = c;
  *nsplit = (capacity + c - 1) / c;
  *ws_bytes = ((size_t)B * Hq * d * (1 + (size_t)*nsplit) + (size_t)B * Hq * *nsplit * 2) * 4;
}
bool global_decode_geometry_capped(int B, int Hq, int, int d, int capacity, size_t max_bytes,
                                   int* nsplit, int* chunk, size_t* ws_bytes) {
  global_decode_geometry(B, Hq, d, capacity, nsplit, chunk, ws_bytes);
  return *ws_bytes <= max_bytes;
}
hipError_t decode_noalloc_scratch(void** ptr, size_t* bytes) {
  ++stub::scratch_lookups;
  *ptr = stub::scratch;
  *bytes = (size_t)64 << 20;
  return hipSuccess;
}
}  // namespace zg
