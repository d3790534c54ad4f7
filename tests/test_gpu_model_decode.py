"""Stack decode (zgattn_model_decode) against the fp64 oracle, layer by layer (GPU).

Each layer of the step is one gated-SWA or global decode on its own tensors; the batched
call must give every layer the single-layer result (oracle decode_swa / decode_global)
and update exactly that layer's cache slot.
"""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, TOL_F32, host64, maxabs, need_gpu, say
from workloads import host_tensor, norm_weight, stack_kinds

pytestmark = pytest.mark.gpu


def _layers(kinds, B, Hq, Hkv, d, W, cap, seed, dtype="bf16"):
    import torch
    out = []
    for i, kind in enumerate(kinds):
        s = seed + 100 * i
        S = cap if kind == "global" else W
        L = dict(kind=kind,
                 q=host_tensor((B, Hq, d), s, dtype),
                 g=host_tensor((B, Hq, d), s + 1, dtype) if kind == "swa" else None,
                 k_new=host_tensor((B, Hkv, d), s + 2, dtype),
                 v_new=host_tensor((B, Hkv, d), s + 3, dtype),
                 k_cache=host_tensor((B, Hkv, S, d), s + 4, dtype),
                 v_cache=host_tensor((B, Hkv, S, d), s + 5, dtype),
                 wq=torch.from_numpy(norm_weight(d, s + 6)),
                 wk=torch.from_numpy(norm_weight(d, s + 7)))
        out.append(L)
    return out


@pytest.mark.parametrize("n_layers,period,B,Hq,Hkv,d,cap,pos,dtype,W", [
    (12, 6, 3, 8, 2, 128, 3000, [0, 700, 2999], "bf16", 128),   # the model's 5:1 pattern
    (8, 4, 2, 32, 8, 128, 1024, [127, 1000], "bf16", 128),      # 3:1, the model's head counts
    (5, 1, 2, 4, 1, 64, 300, [5, 299], "bf16", 128),            # global only, d = 64
    (4, 1000, 4, 16, 2, 64, 1, [0, 1, 128, 5000], "bf16", 128), # SWA only (no workspace)
    # fp32 tensors and caches: the layers run through the single-layer kernels, so rings
    # above 128 slots are allowed too
    (6, 3, 2, 8, 2, 64, 500, [3, 499], "f32", 128),
    (4, 2, 2, 4, 1, 128, 700, [0, 650], "f32", 200),
])
def test_model_decode_vs_oracle(n_layers, period, B, Hq, Hkv, d, cap, pos, dtype, W):
    need_gpu()
    import torch
    import global_attention_qk_amd as zg
    kinds = stack_kinds(period, n_layers)
    host = _layers(kinds, B, Hq, Hkv, d, W, cap, 9000 + n_layers, dtype)
    dev = [{k: (v.cuda() if hasattr(v, "cuda") else v) for k, v in L.items()} for L in host]
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    outs = zg.model_decode(dev, posd, window=W, capacity=cap)
    torch.cuda.synchronize()
    r = zg.rotary_dim_for(d)
    for i, (L, D) in enumerate(zip(host, dev)):
        args = [host64(L[f]) for f in ("q", "k_new", "v_new")]
        if L["kind"] == "swa":
            want, ktn = O.decode_swa(*args, host64(L["g"]), host64(L["wq"]), host64(L["wk"]),
                                     host64(L["k_cache"]), host64(L["v_cache"]), np.array(pos),
                                     window=W, rotary_dim=r)
            slots = [p % W for p in pos]
        else:
            want, ktn = O.decode_global(*args, host64(L["wq"]), host64(L["wk"]),
                                        host64(L["k_cache"]), host64(L["v_cache"]),
                                        np.array(pos), rotary_dim=r)
            slots = list(pos)
        err = maxabs(host64(outs[i]), want)
        say("model_decode layer", i, L["kind"], dtype, err)
        assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)
        kc, vc = host64(D["k_cache"]), host64(D["v_cache"])
        for b, sl in enumerate(slots):
            assert maxabs(kc[b, :, sl], ktn[b]) <= (1e-5 if dtype == "f32" else 2e-2)
            assert np.array_equal(vc[b, :, sl], host64(L["v_new"])[b])
            keep = np.ones(kc.shape[2], bool)
            keep[sl] = False
            assert np.array_equal(kc[b, :, keep], host64(L["k_cache"])[b, :, keep])
