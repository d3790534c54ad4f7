"""Prefill parity: the HIP library (through the C ABI) against the fp64 oracle.

Sizes span several query and key tiles and a ragged tail; C1 and C2 run at their full
sizes. Tolerances: max-abs 1e-4 for fp32, 2e-2 for bf16 (fp32 accumulation).
"""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, TOL_F32, host64, maxabs, need_gpu, say, threads
from workloads import C1, C2, host_tensor, norm_weight, prefill_inputs

pytestmark = pytest.mark.gpu


def _zg():
    need_gpu()
    import global_attention_qk_amd as zg
    return zg


def _inputs(B, T, Hq, Hkv, d, dtype, seed, g_std=1.0):
    q = host_tensor((B, T, Hq, d), seed, dtype)
    k = host_tensor((B, T, Hkv, d), seed + 1, dtype)
    v = host_tensor((B, T, Hkv, d), seed + 2, dtype)
    g = host_tensor((B, T, Hq, d), seed + 3, dtype, g_std)
    import torch
    wq = torch.from_numpy(norm_weight(d, seed + 4))
    wk = torch.from_numpy(norm_weight(d, seed + 5))
    return q, k, v, g, wq, wk


def _cuda(*ts):
    return [None if t is None else t.cuda() for t in ts]


def _check(kind, q, k, v, g, wq, wk, *, window=128, rdim=None, pos_offset=0, tol,
           workspace="auto", rows=None):
    zg = _zg()
    import torch
    d = q.shape[-1]
    r = zg.rotary_dim_for(d) if rdim is None else rdim
    qd, kd, vd, gd, wqd, wkd = _cuda(q, k, v, g, wq, wk)
    if kind == "swa":
        out = zg.swa_prefill(qd, kd, vd, gd, wqd, wkd, window=window, rotary_dim=r,
                             pos_offset=pos_offset)
    else:
        out = zg.global_prefill(qd, kd, vd, wqd, wkd, rotary_dim=r, pos_offset=pos_offset,
                                workspace=workspace)
    torch.cuda.synchronize()
    T = q.shape[1]
    rows = np.arange(T) if rows is None else rows
    want = O.prefill_rows(host64(q), host64(k), host64(v),
                          host64(g) if kind == "swa" else None, host64(wq), host64(wk), rows,
                          window=window if kind == "swa" else None, rotary_dim=r,
                          pos_offset=pos_offset, threads=threads())
    got = host64(out)[:, rows]
    err = maxabs(got, want)
    say(kind, tuple(q.shape), tuple(k.shape), str(q.dtype), f"W={window} r={r} err={err:.3e}")
    assert err <= tol, err
    return out


def test_c1_full_fp32_swa():
    q, k, v, g, wq, wk = prefill_inputs(C1)
    _check("swa", q, k, v, g, wq, wk, window=C1.window, rdim=C1.rotary_dim, tol=TOL_F32)


def test_c1_shape_fp32_global():
    q, k, v, g, wq, wk = prefill_inputs(C1)
    _check("global", q, k, v, None, wq, wk, rdim=C1.rotary_dim, tol=TOL_F32)


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_fp32_ragged_gqa(kind):
    q, k, v, g, wq, wk = _inputs(2, 203, 6, 2, 128, "f32", 700)
    _check(kind, q, k, v, g, wq, wk, window=50, rdim=42, pos_offset=17, tol=TOL_F32)


@pytest.mark.parametrize("kind,ws", [("swa", None), ("global", "auto"), ("global", None)])
def test_bf16_ragged_multi_tile(kind, ws):
    # 300 positions: several 64-position query tiles, a ragged tail, 5 key tiles
    q, k, v, g, wq, wk = _inputs(2, 300, 8, 2, 128, "bf16", 100, g_std=2 ** 0.5)
    _check(kind, q, k, v, g, wq, wk, tol=TOL_BF16, workspace=ws)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (16, 2), (8, 1)])
@pytest.mark.parametrize("kind", ["swa", "global"])
def test_bf16_head_groups(Hq, Hkv, kind):
    q, k, v, g, wq, wk = _inputs(1, 520, Hq, Hkv, 128, "bf16", 200 + Hq * 10 + Hkv)
    _check(kind, q, k, v, g, wq, wk, tol=TOL_BF16)


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_bf16_head_dim_64(kind):
    q, k, v, g, wq, wk = _inputs(1, 333, 4, 1, 64, "bf16", 300)
    _check(kind, q, k, v, g, wq, wk, rdim=20, tol=TOL_BF16)


@pytest.mark.parametrize("window", [1, 7, 64, 129, 1000])
def test_bf16_windows(window):
    q, k, v, g, wq, wk = _inputs(1, 400, 8, 2, 128, "bf16", 400 + window)
    _check("swa", q, k, v, g, wq, wk, window=window, tol=TOL_BF16)


@pytest.mark.parametrize("rdim", [0, 2, 64])
def test_bf16_rotary_dims(rdim):
    q, k, v, g, wq, wk = _inputs(1, 257, 8, 2, 128, "bf16", 500 + rdim)
    _check("swa", q, k, v, g, wq, wk, rdim=rdim, tol=TOL_BF16)
    _check("global", q, k, v, None, wq, wk, rdim=rdim, tol=TOL_BF16)


def test_bf16_position_offset_large():
    # rotation angles at positions near 2.6e5, where fp32 angles would be inaccurate
    q, k, v, g, wq, wk = _inputs(1, 300, 8, 2, 128, "bf16", 600)
    _check("swa", q, k, v, g, wq, wk, pos_offset=262144 - 300, tol=TOL_BF16)
    _check("global", q, k, v, None, wq, wk, pos_offset=262144 - 300, tol=TOL_BF16)


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_fp32_position_offset_large(kind):
    # the fp32 tolerance resolves RoPE phase errors of ~1e-5 rad at positions near 2.6e5
    q, k, v, g, wq, wk = _inputs(1, 130, 4, 1, 128, "f32", 650)
    _check(kind, q, k, v, g, wq, wk, window=128, rdim=42, pos_offset=262144 - 130,
           tol=TOL_F32)


def test_tiny_sequences():
    for T in (1, 2, 31, 33, 64, 65):
        q, k, v, g, wq, wk = _inputs(1, T, 8, 2, 128, "bf16", 800 + T)
        _check("swa", q, k, v, g, wq, wk, tol=TOL_BF16)
        _check("global", q, k, v, None, wq, wk, tol=TOL_BF16)


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_c2_full(kind):
    q, k, v, g, wq, wk = prefill_inputs(C2, gated=(kind == "swa"))
    _check(kind, q, k, v, g, wq, wk, window=C2.window, rdim=C2.rotary_dim, tol=TOL_BF16)


# ---- invariants of the definition, on the GPU ------------------------------------------

def test_swa_wide_window_equals_global():
    zg = _zg()
    import torch
    q, k, v, g, wq, wk = _cuda(*_inputs(1, 300, 8, 2, 128, "bf16", 900))
    ginf = torch.full_like(g, float("inf"))
    a = zg.swa_prefill(q, k, v, ginf, wq, wk, window=300)
    b = zg.global_prefill(q, k, v, wq, wk)
    torch.cuda.synchronize()
    assert maxabs(host64(a), host64(b)) <= 1e-2


def test_gate_limits_and_constant_v():
    zg = _zg()
    import torch
    q, k, v, g, wq, wk = _cuda(*_inputs(1, 200, 8, 2, 128, "bf16", 910))
    ref = zg.global_prefill(q, k, v, wq, wk)
    ungated_swa_wide = zg.swa_prefill(q, k, v, torch.full_like(g, float("inf")), wq, wk,
                                      window=1000)
    zero = zg.swa_prefill(q, k, v, torch.full_like(g, float("-inf")), wq, wk)
    half = zg.swa_prefill(q, k, v, torch.zeros_like(g), wq, wk, window=1000)
    vc = torch.full_like(v, -1.75)
    const = zg.swa_prefill(q, k, vc, g, wq, wk)
    torch.cuda.synchronize()
    assert maxabs(host64(ungated_swa_wide), host64(ref)) <= 1e-2
    assert np.all(host64(zero) == 0.0)
    assert maxabs(host64(half), 0.5 * host64(ungated_swa_wide)) <= 4e-3
    want = -1.75 * O.sigmoid(host64(g))
    assert maxabs(host64(const), want) <= 1e-2


def test_deterministic_and_overwrites_poisoned_output():
    zg = _zg()
    import torch
    q, k, v, g, wq, wk = _cuda(*_inputs(2, 300, 8, 2, 128, "bf16", 920))
    for kind in ("swa", "global"):
        outs = []
        for _ in range(2):
            o = torch.full_like(q, float("nan"))
            if kind == "swa":
                zg.swa_prefill(q, k, v, g, wq, wk, out=o)
            else:
                zg.global_prefill(q, k, v, wq, wk, out=o)
            outs.append(o)
        torch.cuda.synchronize()
        assert torch.isfinite(outs[0].float()).all()
        assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("kind,ws,d", [("swa", None, 128), ("global", "auto", 128),
                                       ("global", None, 128), ("swa", None, 64),
                                       ("global", "auto", 64)])
def test_bf16_running_max_variant(kind, ws, d):
    # One large norm weight per branch lifts the score bound (qscale * d * max|wq| * max|wk|,
    # 2% margin) above the static-shift limit of 48 log2 units, so the kernels take their
    # running-max (online softmax) variant; the scores themselves stay moderate, because
    # RMSNorm scales the whole row and only one dim is amplified.
    q, k, v, g, wq, wk = _inputs(2, 300, 8, 2, d, "bf16", 950 + d, g_std=2 ** 0.5)
    wq[5] = 3.2
    wk[7] = -3.2
    qscale = d ** -0.5 * 1.4426950408889634
    bound = qscale * d * float(wq.abs().max()) * float(wk.abs().max()) * 1.02
    assert bound > 48.0, bound
    _check(kind, q, k, v, g, wq, wk, tol=TOL_BF16, workspace=ws)


def test_bf16_running_max_variant_loops_over_tiles():
    # 512 query tiles: more than the CUs of the device, so each workgroup of the looping
    # running-max grid takes several tiles; rows sampled over the whole sequence.
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count >= 512:
        pytest.skip("needs more query tiles than CUs")
    q, k, v, g, wq, wk = _inputs(2, 8192, 8, 2, 128, "bf16", 970)
    wq[5] = 3.2
    wk[7] = -3.2
    rows = np.unique(np.concatenate([np.arange(0, 8192, 131), [63, 64, 8191]]))
    _check("global", q, k, v, None, wq, wk, tol=TOL_BF16, rows=rows)
    _check("global", q, k, v, None, wq, wk, tol=TOL_BF16, rows=rows, workspace=None)


@pytest.mark.parametrize("kind", ["swa", "global"])
@pytest.mark.parametrize("Hq,Hkv,rdim", [(6, 2, 42), (4, 1, 128), (8, 8, 80)])
def test_bf16_shapes_off_the_mfma_paths(kind, Hq, Hkv, rdim):
    # head group 3, full rotary and rotary 80: bf16 tensors on the vector-ALU kernel
    q, k, v, g, wq, wk = _inputs(2, 230, Hq, Hkv, 128, "bf16", 3100 + Hq + rdim)
    _check(kind, q, k, v, g, wq, wk, window=70, rdim=rdim, pos_offset=9, tol=TOL_BF16)
