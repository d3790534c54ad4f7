"""Decode caches as the only state: checkpoint and resume (GPU).

The SWA layers keep a fixed 128-entry ring and the global layers the whole sequence
("ZGCM-1-7B 完全解説" explainer, section アーキテクチャ); nothing else carries over from one
decode step to the next. A stack of layers is decoded step by step; midway every ring and
cache is copied to the host, written to a file (safetensors), read back into fresh device
buffers, and decoding continues from both copies. The resumed run must match the
uninterrupted one bit for bit, outputs and caches alike.
"""

import numpy as np
import pytest

from tests.gpu_util import need_gpu, say
from workloads import host_tensor, norm_weight

pytestmark = pytest.mark.gpu


def _stack(kinds, B, Hq, Hkv, d, W, cap, T0, seed):
    """Per layer: norm weights and caches holding the first T0 tokens (post-norm/RoPE K
    from zgattn_qknorm_rope, raw V)."""
    import torch
    import global_attention_qk_amd as zg
    layers = []
    for i, kind in enumerate(kinds):
        s = seed + 100 * i
        wq = torch.from_numpy(norm_weight(d, s)).cuda()
        wk = torch.from_numpy(norm_weight(d, s + 1)).cuda()
        k = host_tensor((B, T0, Hkv, d), s + 2, "bf16").cuda()
        v = host_tensor((B, T0, Hkv, d), s + 3, "bf16").cuda()
        kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        zg.qknorm_rope(k, wk, out=kc.permute(0, 2, 1, 3)[:, :T0])
        vc.permute(0, 2, 1, 3)[:, :T0].copy_(v)
        if kind == "swa":
            kr = torch.zeros((B, Hkv, W, d), dtype=torch.bfloat16, device="cuda")
            vr = torch.zeros_like(kr)
            for p in range(max(0, T0 - W), T0):
                kr[:, :, p % W] = kc[:, :, p]
                vr[:, :, p % W] = vc[:, :, p]
            kc, vc = kr, vr
        layers.append(dict(kind=kind, wq=wq, wk=wk, k_cache=kc, v_cache=vc))
    return layers


def _step_inputs(kinds, B, Hq, Hkv, d, t, seed):
    out = []
    for i, kind in enumerate(kinds):
        s = seed + 7919 * t + 101 * i
        x = dict(q=host_tensor((B, Hq, d), s, "bf16").cuda(),
                 k_new=host_tensor((B, Hkv, d), s + 1, "bf16").cuda(),
                 v_new=host_tensor((B, Hkv, d), s + 2, "bf16").cuda())
        if kind == "swa":
            x["g"] = host_tensor((B, Hq, d), s + 3, "bf16").cuda()
        out.append(x)
    return out


def _decode(zg, layers, inputs, t, B, W, cap):
    import torch
    pos = torch.full((B,), t, dtype=torch.int32, device="cuda")
    step = [dict(L, **x) for L, x in zip(layers, inputs)]
    return [o.clone() for o in zg.model_decode(step, pos, window=W, capacity=cap)]


def test_decode_checkpoint_resume_is_bitwise(tmp_path):
    need_gpu()
    import torch
    from safetensors.torch import load_file, save_file

    import global_attention_qk_amd as zg
    B, Hq, Hkv, d, W, cap = 3, 8, 2, 128, 128, 512
    kinds = ["swa", "swa", "global", "swa"]
    T0, T_ckpt, T_end = 150, 190, 230
    layers = _stack(kinds, B, Hq, Hkv, d, W, cap, T0, 500)
    say("decode resume", kinds, T0, T_ckpt, T_end)
    for t in range(T0, T_ckpt):
        _decode(zg, layers, _step_inputs(kinds, B, Hq, Hkv, d, t, 77), t, B, W, cap)
    torch.cuda.synchronize()
    # checkpoint: every cache to a file on the host, back into fresh device buffers
    path = str(tmp_path / "decode_state.safetensors")
    save_file({f"{i}.{n}": L[n].cpu() for i, L in enumerate(layers)
               for n in ("k_cache", "v_cache")}, path)
    state = load_file(path)
    resumed = [dict(L, k_cache=state[f"{i}.k_cache"].cuda(), v_cache=state[f"{i}.v_cache"].cuda())
               for i, L in enumerate(layers)]
    for i, L in enumerate(layers):
        assert resumed[i]["k_cache"].data_ptr() != L["k_cache"].data_ptr()
    for t in range(T_ckpt, T_end):
        x = _step_inputs(kinds, B, Hq, Hkv, d, t, 77)
        a = _decode(zg, layers, x, t, B, W, cap)
        b = _decode(zg, resumed, x, t, B, W, cap)
        torch.cuda.synchronize()
        for i in range(len(kinds)):
            assert torch.isfinite(a[i].float()).all()
            assert torch.equal(a[i], b[i]), (t, i)
    for L, R in zip(layers, resumed):
        assert torch.equal(L["k_cache"], R["k_cache"]) and torch.equal(L["v_cache"], R["v_cache"])
