"""Backward pass (zgattn_*_prefill_backward) against the fp64 oracle's gradients (GPU).

Gradients of sum(dout * out) with dout ~ N(0, 1). Tolerance: max-abs error within 2e-2 of
max(1, max |reference|) per tensor: the products run on bf16 operands (Q~, K~, V, dA, P and
dS rounded to bf16, fp32 accumulation) and the inputs' bf16 rounding bounds the rest.
"""

import numpy as np
import pytest

from oracle import grad as OG
from tests.gpu_util import host64, need_gpu, say
from workloads import host_tensor, norm_weight

pytestmark = pytest.mark.gpu

REL = 2e-2


def _check(B, T, Hq, Hkv, d, window, seed, pos_offset=0):
    need_gpu()
    import torch
    import global_attention_qk_amd as zg
    q = host_tensor((B, T, Hq, d), seed, "bf16")
    k = host_tensor((B, T, Hkv, d), seed + 1, "bf16")
    v = host_tensor((B, T, Hkv, d), seed + 2, "bf16")
    g = host_tensor((B, T, Hq, d), seed + 3, "bf16", 2 ** 0.5) if window else None
    do = host_tensor((B, T, Hq, d), seed + 4, "bf16")
    wq = torch.from_numpy(norm_weight(d, seed + 5))
    wk = torch.from_numpy(norm_weight(d, seed + 6))
    r = zg.rotary_dim_for(d)
    cq, ck, cv, cdo, cwq, cwk = (t.cuda() for t in (q, k, v, do, wq, wk))
    cg = g.cuda() if g is not None else None
    if window:
        out = zg.swa_prefill(cq, ck, cv, cg, cwq, cwk, window=window, rotary_dim=r,
                             pos_offset=pos_offset)
    else:
        out = zg.global_prefill(cq, ck, cv, cwq, cwk, rotary_dim=r, pos_offset=pos_offset)
    dq, dk, dv, dg, dwq, dwk = zg.prefill_backward(cq, ck, cv, cg, cwq, cwk, out, cdo,
                                                   window=window, rotary_dim=r,
                                                   pos_offset=pos_offset)
    torch.cuda.synchronize()
    ref = OG.prefill_grads(host64(q), host64(k), host64(v), None if g is None else host64(g),
                           host64(wq), host64(wk), host64(do), window=window, rotary_dim=r,
                           pos_offset=pos_offset)
    got = dict(dq=dq, dk=dk, dv=dv, dwq=dwq, dwk=dwk)
    if window:
        got["dg"] = dg
    for name, t in got.items():
        want = ref[name]
        err = float(np.max(np.abs(host64(t) - want)))
        lim = REL * max(1.0, float(np.max(np.abs(want))))
        say("backward", (B, T, Hq, Hkv, d, window), name, f"err={err:.3e} lim={lim:.3e}")
        assert err <= lim, (name, err, lim)


@pytest.mark.parametrize("window", [None, 128, 50])
def test_backward_gqa_ragged(window):
    # 300 positions: several query and key tiles and a ragged tail; 4 query heads per KV head
    _check(2, 300, 8, 2, 128, window, 1200)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (16, 2)])
def test_backward_head_groups(Hq, Hkv):
    _check(1, 200, Hq, Hkv, 128, None, 1300 + Hq)
    _check(1, 200, Hq, Hkv, 128, 64, 1310 + Hq)


def test_backward_head_dim_64_and_offset():
    _check(1, 150, 4, 1, 64, None, 1400, pos_offset=1000)
    _check(1, 150, 4, 1, 64, 33, 1410, pos_offset=1000)


def test_backward_tiny_and_single_token():
    _check(1, 1, 4, 1, 128, None, 1500)
    _check(1, 3, 4, 1, 128, 2, 1510)


@pytest.mark.parametrize("window", [None, 128])
def test_backward_1024_positions(window):
    # longer rows: 16 key tiles per query row at the end of the sequence
    _check(1, 1024, 8, 2, 128, window, 1600)
