// Test-only: what the stub launchers of the host-check build record.
#pragma once
#include "launch.h"

namespace stub {
extern int launches;              // kernel launches requested (any launcher)
extern int prefill_launches;      // launch_prefill_bf16 / launch_prefill_valu
extern int valu_launches;         // launch_prefill_valu alone
extern bool last_valu_f32;
extern int aux_launches;          // qknorm_rope / the global pre-pass
extern int decode_launches;       // single-layer and batched decode launchers
extern int batched_layers;        // layers passed to the batched decode launchers
extern int scratch_lookups;       // decode_noalloc_scratch calls
extern int smem_attr_calls;       // hipFuncSetAttribute calls
extern zg::PrefillArgs last_prefill;
extern zg::DecodeArgs last_decode;
extern zg::BackwardArgs last_backward;
extern void* const scratch;       // what decode_noalloc_scratch reports
void reset();
}  // namespace stub
