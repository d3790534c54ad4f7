// Test-only driver of the host-check build: every C-ABI entry point with valid and invalid
// arguments against the stub launchers (no GPU). Exits non-zero on the first failed check;
// the sanitizers (ASan + UBSan, or TSan) report memory errors, undefined behaviour and data
// races in the library's host code.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <thread>
#include <vector>

#include "stubs.h"
#include "zgattn.h"

#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      exit(1);                                                            \
    }                                                                     \
  } while (0)

static void* P(uintptr_t k) { return (void*)(uintptr_t)(0x100000 + 256 * k); }  // aligned, never read
static const float* W() { return (const float*)P(99); }

static zgattn_desc desc(int B, int T, int Hq, int Hkv, int d, int dtype = ZGATTN_BF16) {
  zgattn_desc x;
  x.batch = B;
  x.seq_len = T;
  x.n_q_heads = Hq;
  x.n_kv_heads = Hkv;
  x.head_dim = d;
  x.window = 128;
  x.rotary_dim = 2 * (int)floor(0.33 * d / 2);
  x.pos_offset = 0;
  x.rope_base = 10000.0f;
  x.rms_eps = 1e-6f;
  x.softmax_scale = 0.0f;
  x.dtype = dtype;
  return x;
}

static void prefill_checks() {
  zgattn_desc d = desc(2, 300, 8, 2, 128);
  stub::reset();
  CHECK(zgattn_swa_prefill(&d, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_OK);
  CHECK(stub::prefill_launches == 1);
  const zg::PrefillArgs& a = stub::last_prefill;
  CHECK(a.B == 2 && a.T == 300 && a.Hq == 8 && a.Hkv == 2 && a.d == 128 && a.window == 128);
  CHECK(a.rdim == 42 && a.swa == 1 && a.g == P(4) && a.out == P(5) && a.kt == nullptr);
  CHECK(fabsf(a.scale - 1.0f / sqrtf(128.0f)) < 1e-7f);
  CHECK(fabsf(a.fr.hi[0] - 0.15915494f) < 1e-7f && a.fr.hi[21] == 0.0f && a.fr.lo[63] == 0.0f);
  // every rejection happens before a launch
  struct Bad {
    int field, value, code;
  } bad[] = {{0, 0, ZGATTN_EINVAL},   {1, -1, ZGATTN_EINVAL},      {2, 7, ZGATTN_EINVAL},
             {4, 96, ZGATTN_EUNSUPPORTED}, {5, 0, ZGATTN_EINVAL}, {6, 43, ZGATTN_EINVAL},
             {6, 130, ZGATTN_EINVAL}, {7, -1, ZGATTN_ERANGE},    {11, 5, ZGATTN_EDTYPE}};
  for (const Bad& b : bad) {
    zgattn_desc x = d;
    int* f = (int*)&x;
    f[b.field] = b.value;
    stub::reset();
    CHECK(zgattn_swa_prefill(&x, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == b.code);
    CHECK(stub::launches == 0);
  }
  zgattn_desc x = d;
  x.pos_offset = (1 << 24) - 100;
  CHECK(zgattn_swa_prefill(&x, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_ERANGE);
  x = d;
  x.rms_eps = NAN;
  CHECK(zgattn_global_prefill(&x, P(1), P(2), P(3), W(), W(), nullptr, 0, P(5), nullptr, nullptr) == ZGATTN_EINVAL);
  CHECK(zgattn_swa_prefill(&d, P(1), P(2), P(3), nullptr, W(), W(), P(5), nullptr) == ZGATTN_ENULL);
  CHECK(zgattn_swa_prefill(&d, (char*)P(1) + 8, P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_EINVAL);
  CHECK(zgattn_swa_prefill(nullptr, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_ENULL);
  x = d;
  x.seq_len = 0;   // nothing to do: no launch, null pointers allowed
  stub::reset();
  CHECK(zgattn_swa_prefill(&x, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == ZGATTN_OK);
  CHECK(stub::launches == 0);
  // global: workspace sizing, pre-passes, fused fallback
  const size_t need = zgattn_global_prefill_workspace_bytes(&d);
  CHECK(need >= (size_t)2 * 2 * 300 * 128 * 2);
  stub::reset();
  CHECK(zgattn_global_prefill(&d, P(1), P(2), P(3), W(), W(), P(6), need - 1, P(5), nullptr, nullptr) == ZGATTN_EWORKSPACE);
  CHECK(stub::launches == 0);
  CHECK(zgattn_global_prefill(&d, P(1), P(2), P(3), W(), W(), P(6), need, P(5), nullptr, nullptr) == ZGATTN_OK);
  CHECK(stub::aux_launches == 1 && stub::prefill_launches == 1);
  CHECK(stub::last_prefill.kt == P(6) && stub::last_prefill.vt != nullptr && stub::last_prefill.swa == 0);
  CHECK(stub::last_prefill.lse == nullptr);
  stub::reset();
  CHECK(zgattn_global_prefill(&d, P(1), P(2), P(3), W(), W(), nullptr, 0, P(5), (float*)P(14), nullptr) == ZGATTN_OK);
  CHECK(stub::launches == 1 && stub::last_prefill.kt == nullptr && stub::last_prefill.lse == (float*)P(14));
  // the row log-sum-exp output: 4-byte aligned, bf16 only
  stub::reset();
  CHECK(zgattn_global_prefill(&d, P(1), P(2), P(3), W(), W(), nullptr, 0, P(5), (float*)((char*)P(14) + 2), nullptr) == ZGATTN_EINVAL);
  zgattn_desc f32d = desc(1, 64, 4, 1, 64, ZGATTN_F32);
  CHECK(zgattn_global_prefill(&f32d, P(1), P(2), P(3), W(), W(), nullptr, 0, P(5), (float*)P(14), nullptr) == ZGATTN_EUNSUPPORTED);
  CHECK(stub::launches == 0);
  // fp32, and bf16 shapes the MFMA kernels do not take (head group 16), go to the
  // vector-ALU kernel; the latter cannot give the log-sum-exp
  zgattn_desc f = desc(1, 64, 4, 1, 64, ZGATTN_F32);
  stub::reset();
  CHECK(zgattn_swa_prefill(&f, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_OK);
  CHECK(stub::valu_launches == 1 && stub::last_valu_f32);
  zgattn_desc g16 = desc(1, 64, 32, 2, 128);
  stub::reset();
  CHECK(zgattn_swa_prefill(&g16, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_OK);
  CHECK(stub::valu_launches == 1 && !stub::last_valu_f32);
  CHECK(zgattn_global_prefill(&g16, P(1), P(2), P(3), W(), W(), P(6), 1 << 30, P(5), nullptr, nullptr) == ZGATTN_OK);
  CHECK(stub::valu_launches == 2 && stub::aux_launches == 0);   // no pre-pass
  CHECK(zgattn_global_prefill(&g16, P(1), P(2), P(3), W(), W(), nullptr, 0, P(5), (float*)P(14), nullptr) == ZGATTN_EUNSUPPORTED);
  zgattn_desc model = desc(1, 64, 4, 1, 128);
  stub::reset();
  CHECK(zgattn_swa_prefill(&model, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_OK);
  CHECK(stub::valu_launches == 0 && stub::prefill_launches == 1);
  // varlen
  zgattn_desc v = desc(1, 1000, 8, 2, 128);
  stub::reset();
  CHECK(zgattn_swa_prefill_varlen(&v, (const int32_t*)P(7), 3, 600, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_OK);
  CHECK(stub::last_prefill.cu == P(7) && stub::last_prefill.n_docs == 3 && stub::last_prefill.max_len == 600);
  CHECK(zgattn_swa_prefill_varlen(&v, (const int32_t*)P(7), 0, 600, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_EINVAL);
  CHECK(zgattn_swa_prefill_varlen(&v, (const int32_t*)P(7), 3, 1001, P(1), P(2), P(3), P(4), W(), W(), P(5), nullptr) == ZGATTN_EINVAL);
  const size_t vneed = zgattn_global_prefill_varlen_workspace_bytes(&v, 3);
  CHECK(zgattn_global_prefill_varlen(&v, (const int32_t*)P(7), 3, 600, P(1), P(2), P(3), W(), W(), P(6), vneed - 16, P(5), nullptr) == ZGATTN_EWORKSPACE);
  CHECK(zgattn_global_prefill_varlen(&v, (const int32_t*)P(7), 3, 600, P(1), P(2), P(3), W(), W(), P(6), vneed, P(5), nullptr) == ZGATTN_OK);
  // backward
  const size_t bneed = zgattn_prefill_backward_workspace_bytes(&d);
  float* dw = (float*)P(20);
  CHECK(zgattn_swa_prefill_backward(&d, P(1), P(2), P(3), P(4), W(), W(), P(5), P(8), P(9), P(10), P(11), P(12), dw, dw, P(13), bneed - 1, nullptr) == ZGATTN_EWORKSPACE);
  CHECK(zgattn_global_prefill_backward(&d, P(1), P(2), P(3), W(), W(), P(5), nullptr, P(8), P(9), P(10), P(11), dw, dw, P(13), bneed, nullptr) == ZGATTN_OK);
  CHECK(stub::last_backward.lse == nullptr && stub::last_backward.swa == 0);
  CHECK(zgattn_global_prefill_backward(&d, P(1), P(2), P(3), W(), W(), P(5), (const float*)P(14), P(8), P(9), P(10), P(11), dw, dw, P(13), bneed, nullptr) == ZGATTN_OK);
  CHECK(stub::last_backward.lse == (const float*)P(14));
  CHECK(zgattn_global_prefill_backward(&d, P(1), P(2), P(3), W(), W(), P(5), (const float*)((char*)P(14) + 1), P(8), P(9), P(10), P(11), dw, dw, P(13), bneed, nullptr) == ZGATTN_EINVAL);
  CHECK(zgattn_swa_prefill_backward(&d, P(1), P(2), P(3), nullptr, W(), W(), P(5), P(8), P(9), P(10), P(11), P(12), dw, dw, P(13), bneed, nullptr) == ZGATTN_ENULL);
  CHECK(stub::last_backward.f32 == 0);
  // fp32 tensors and other head groups are accepted (the library picks the kernels)
  CHECK(zgattn_prefill_backward_workspace_bytes(&f) > 0);
  CHECK(zgattn_swa_prefill_backward(&f, P(1), P(2), P(3), P(4), W(), W(), P(5), P(8), P(9), P(10), P(11), P(12), dw, dw, P(13), zgattn_prefill_backward_workspace_bytes(&f), nullptr) == ZGATTN_OK);
  CHECK(stub::last_backward.f32 == 1 && stub::last_backward.swa == 1);
  CHECK(zgattn_global_prefill_backward(&g16, P(1), P(2), P(3), W(), W(), P(5), nullptr, P(8), P(9), P(10), P(11), dw, dw, P(13), zgattn_prefill_backward_workspace_bytes(&g16), nullptr) == ZGATTN_OK);
  CHECK(stub::last_backward.f32 == 0 && stub::last_backward.Hq == 32 && stub::last_backward.Hkv == 2);
}

static void decode_checks() {
  zgattn_desc d = desc(4, 1, 32, 8, 128);
  const int32_t* pos = (const int32_t*)P(30);
  stub::reset();
  CHECK(zgattn_swa_decode(&d, P(1), P(2), P(3), P(4), W(), W(), P(5), P(6), pos, P(7), nullptr) == ZGATTN_OK);
  CHECK(stub::decode_launches == 1 && stub::last_decode.window == 128 && stub::last_decode.g == P(4));
  zgattn_desc w = d;
  w.window = 5000;
  CHECK(zgattn_swa_decode(&w, P(1), P(2), P(3), P(4), W(), W(), P(5), P(6), pos, P(7), nullptr) == ZGATTN_EINVAL);
  const int cap = 262144;
  const size_t need = zgattn_global_decode_workspace_bytes(&d, cap);
  stub::reset();
  CHECK(zgattn_global_decode(&d, P(1), P(2), P(3), W(), W(), P(5), P(6), cap, pos, P(8), need - 1, P(7), nullptr) == ZGATTN_EWORKSPACE);
  CHECK(zgattn_global_decode(&d, P(1), P(2), P(3), W(), W(), P(5), P(6), 0, pos, P(8), need, P(7), nullptr) == ZGATTN_ERANGE);
  CHECK(stub::launches == 0);
  CHECK(zgattn_global_decode(&d, P(1), P(2), P(3), W(), W(), P(5), P(6), cap, pos, P(8), need, P(7), nullptr) == ZGATTN_OK);
  CHECK(stub::last_decode.S == cap && stub::last_decode.ws == (float*)P(8) && stub::last_decode.nsplit > 0);
  CHECK(stub::last_decode.f32 == 0);
  // fp32 tensors and caches: the same calls, flagged for the fp32 kernels
  zgattn_desc f = desc(4, 1, 32, 8, 128, ZGATTN_F32);
  CHECK(zgattn_global_decode(&f, P(1), P(2), P(3), W(), W(), P(5), P(6), cap, pos, P(8), need, P(7), nullptr) == ZGATTN_OK);
  CHECK(stub::last_decode.f32 == 1);
  CHECK(zgattn_swa_decode(&f, P(1), P(2), P(3), P(4), W(), W(), P(5), P(6), pos, P(7), nullptr) == ZGATTN_OK);
  CHECK(stub::last_decode.f32 == 1 && stub::last_decode.window == 128);
  // the no-allocation variant: scratch looked up only for calls that launch
  stub::reset();
  CHECK(zgattn_global_decode_noalloc(&d, P(1), P(2), P(3), W(), W(), P(5), P(6), cap, pos, P(7), nullptr) == ZGATTN_OK);
  CHECK(stub::scratch_lookups == 1 && stub::last_decode.ws == (float*)stub::scratch);
  zgattn_desc big = desc(1024, 1, 64, 8, 128);
  stub::reset();
  CHECK(zgattn_global_decode_noalloc(&big, P(1), P(2), P(3), W(), W(), P(5), P(6), cap, pos, P(7), nullptr) == ZGATTN_EWORKSPACE);
  CHECK(stub::scratch_lookups == 0 && stub::launches == 0);
  // a whole stack: 40 layers (every 6th global) in launches of at most 32 layers per kind
  const int n = 40;
  std::vector<int32_t> kinds(n);
  std::vector<zgattn_decode_layer> L(n);
  int n_glob = 0;
  for (int i = 0; i < n; ++i) {
    kinds[i] = (i + 1) % 6 == 0;
    n_glob += kinds[i];
    L[i] = zgattn_decode_layer{P(100 + 9 * i), P(101 + 9 * i), P(102 + 9 * i), P(103 + 9 * i),
                               W(), W(), P(105 + 9 * i), P(106 + 9 * i), P(107 + 9 * i)};
  }
  const size_t mneed = zgattn_model_decode_workspace_bytes(&d, n, kinds.data(), 4096);
  CHECK(mneed > 0);
  stub::reset();
  CHECK(zgattn_model_decode(&d, n, kinds.data(), L.data(), 4096, pos, P(900), mneed, nullptr) == ZGATTN_OK);
  CHECK(stub::batched_layers == n && stub::decode_launches == 2 + 1);   // 34 SWA = 32 + 2; 6 global
  stub::reset();
  CHECK(zgattn_model_decode(&d, n, kinds.data(), L.data(), 4096, pos, P(900), mneed - 1, nullptr) == ZGATTN_EWORKSPACE);
  L[17].out = nullptr;   // one invalid layer: nothing launches
  CHECK(zgattn_model_decode(&d, n, kinds.data(), L.data(), 4096, pos, P(900), mneed, nullptr) == ZGATTN_ENULL);
  CHECK(stub::launches == 0);
  CHECK(zgattn_model_decode(&d, 2000, kinds.data(), L.data(), 4096, pos, P(900), mneed, nullptr) == ZGATTN_EINVAL);
  // fp32: one single-layer launch sequence per layer, in layer order
  L[17].out = P(107 + 9 * 17);
  zgattn_desc f32 = desc(4, 1, 32, 8, 128, ZGATTN_F32);
  stub::reset();
  CHECK(zgattn_model_decode(&f32, n, kinds.data(), L.data(), 4096, pos, P(900), mneed, nullptr) == ZGATTN_OK);
  CHECK(stub::decode_launches == n && stub::batched_layers == 0);
  CHECK(stub::last_decode.f32 == 1 && stub::last_decode.out == P(107 + 9 * (n - 1)));
  CHECK(stub::last_decode.ws == (kinds[n - 1] ? (float*)((char*)P(900) + (n_glob - 1) * (mneed / n_glob)) : nullptr));
}

static void norm_rope_checks() {
  zgattn_desc d = desc(2, 37, 3, 3, 128);
  stub::reset();
  CHECK(zgattn_qknorm_rope(&d, 3, P(1), W(), nullptr, P(2), 3 * 64 * 128, 128, 64 * 128, nullptr) == ZGATTN_OK);
  CHECK(stub::aux_launches == 1);
  CHECK(zgattn_qknorm_rope(&d, 3, P(1), W(), nullptr, P(2), 3 * 64 * 128, 127, 64 * 128, nullptr) == ZGATTN_EINVAL);
  CHECK(zgattn_qknorm_rope(&d, 3, P(1), W(), nullptr, P(2), -128, 128, 64 * 128, nullptr) == ZGATTN_EINVAL);
  CHECK(zgattn_qknorm_rope(&d, 0, P(1), W(), nullptr, P(2), 0, 128, 128, nullptr) == ZGATTN_EINVAL);
  CHECK(zgattn_qknorm_rope(&d, 3, nullptr, W(), nullptr, P(2), 0, 128, 128, nullptr) == ZGATTN_ENULL);
  for (int s = -8; s < 8; ++s) CHECK(zgattn_strerror(s) != nullptr);
  CHECK(zgattn_abi_version() == ZGATTN_ABI_VERSION);
}

// The per-device caches (CU count, raised LDS limits) under concurrent callers.
static void cache_checks() {
  __atomic_store_n(&stub::smem_attr_calls, 0, __ATOMIC_RELAXED);
  std::vector<std::thread> th;
  for (int t = 0; t < 8; ++t)
    th.emplace_back([t] {
      for (int it = 0; it < 200; ++it) {
        int cus = 0;
        CHECK(zg::device_cu_count(&cus) == hipSuccess && cus == 256);
        const void* kern = P(5000 + (it + t) % 50);
        CHECK(zg::ensure_dynamic_smem(kern, 65536 + 1024 * ((it / 50) % 2)) == hipSuccess);
      }
    });
  for (auto& x : th) x.join();
  // each of the 50 kernels is raised at most twice (64 KiB, then 65 KiB)
  const int calls = __atomic_load_n(&stub::smem_attr_calls, __ATOMIC_RELAXED);
  CHECK(calls >= 50 && calls <= 100);
}

int main() {
  prefill_checks();
  decode_checks();
  norm_rope_checks();
  cache_checks();
  printf("host checks passed\n");
  return 0;
}
