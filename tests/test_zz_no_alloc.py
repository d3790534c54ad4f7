"""zgattn_global_decode_noalloc (no workspace argument, no allocation: the split-K partials
go to the library's per-GPU scratch) against zgattn_global_decode (caller workspace).

Two calls in a row on the same GPU, the second with a smaller input, so the second reads a
scratch that still holds the first call's partials. The decode step followed is the global
layer of the "ZGCM-1-7B 完全解説" explainer, section アーキテクチャ (full-sequence cache);
the tolerance is the bf16 bar of the parity tests (2e-2 max-abs).
"""

import numpy as np
import pytest

from tests.gpu_util import TOL_BF16, host64, maxabs, need_gpu, say
from workloads import C5, decode_inputs, host_tensor, norm_weight

pytestmark = pytest.mark.gpu


def test_noalloc_decode_matches_workspace_decode_twice():
    need_gpu()
    import torch

    import global_attention_qk_amd as zg

    # 1) B = 32 at context 262144: the workspace call's split geometry needs 65.5 MiB of
    #    partials, more than the 64 MiB scratch, so this call runs longer cache chunks
    say("noalloc call 1: B=32 S=262144")
    x = decode_inputs(C5, device="cuda")
    S = C5.T
    pos = torch.tensor([S - 1 - 7919 * b for b in range(C5.B)], dtype=torch.int32,
                       device="cuda")
    ref = zg.global_decode(x["q"], x["k_new"], x["v_new"], x["wq"], x["wk"], x["k_cache"],
                           x["v_cache"], pos)
    kc_after = x["k_cache"][:, :, S - 1].clone()
    out = torch.full_like(ref, float("nan"))
    zg.global_decode_noalloc(x["q"], x["k_new"], x["v_new"], x["wq"], x["wk"], x["k_cache"],
                             x["v_cache"], pos, out=out)
    torch.cuda.synchronize()
    e1 = maxabs(host64(out), host64(ref))
    say("noalloc call 1 err", e1)
    assert e1 <= TOL_BF16
    # the cache append is the same (idempotent: same entry at the same index)
    assert torch.equal(x["k_cache"][:, :, S - 1], kc_after)
    del x, ref, out
    torch.cuda.empty_cache()

    # 2) smaller: B = 4, capacity 5000, positions 0 .. 4999; the workspace call's geometry
    #    fits the scratch, so the same kernels run on the same splits: identical outputs
    say("noalloc call 2: B=4 S=5000")
    B, Hq, Hkv, d, cap = 4, 32, 8, 128, 5000
    q = host_tensor((B, Hq, d), 51, "bf16").cuda()
    kn = host_tensor((B, Hkv, d), 52, "bf16").cuda()
    vn = host_tensor((B, Hkv, d), 53, "bf16").cuda()
    kc = host_tensor((B, Hkv, cap, d), 54, "bf16").cuda()
    vc = host_tensor((B, Hkv, cap, d), 55, "bf16").cuda()
    wq = torch.from_numpy(norm_weight(d, 56)).cuda()
    wk = torch.from_numpy(norm_weight(d, 57)).cuda()
    pos = torch.tensor([0, 17, 2500, cap - 1], dtype=torch.int32, device="cuda")
    kc2, vc2 = kc.clone(), vc.clone()
    ref = zg.global_decode(q, kn, vn, wq, wk, kc, vc, pos)
    out = torch.full_like(ref, float("nan"))
    zg.global_decode_noalloc(q, kn, vn, wq, wk, kc2, vc2, pos, out=out)
    torch.cuda.synchronize()
    e2 = maxabs(host64(out), host64(ref))
    say("noalloc call 2 err", e2, "identical", bool(torch.equal(out, ref)))
    assert e2 <= TOL_BF16
    assert torch.equal(out, ref)
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc)
