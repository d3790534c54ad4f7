"""Parity at the edges of the value range and with non-default layer parameters (GPU).

* Scores at the static-shift bound: constant q and k rows with rotary_dim 0 give every
  visible score the largest (or smallest) value RMSNorm allows, qscale * d * w^2. Just
  below the bound where the kernels switch variants (48 log2 units) the static-shift
  variant runs; just above it (w = 2.4, about 96) the running-max variant. V is scaled far
  up (1e6 .. 1e30) or down (1e-4) so that an accumulator that is not kept in range
  overflows or underflows. Judged on max-abs error relative to max |oracle|: the bf16
  output alone rounds each value by up to 2^-9 of itself.
* softmax_scale, rms_eps and rope_base away from their defaults, through the dense
  prefill calls (both SWA kernels, the global layer with and without its workspace) and
  both decode calls.
* Decode over a ring whose unwritten slots hold NaN (a freshly allocated ring, early in a
  sequence): slots the query does not see must not reach the output.

The definition followed (oracle) is the layer of the hyper.ai summary of arXiv 2609.13356,
section 方法 (GatedSWA equation) and the "ZGCM-1-7B 完全解説" explainer, section
アーキテクチャ: softmax attention is defined for any finite scores and values.
"""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, host64, maxabs, need_gpu, say, threads
from workloads import host_tensor, norm_weight, stratified_rows

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2   # max-abs error / max |oracle|


def _zg():
    need_gpu()
    import global_attention_qk_amd as zg
    return zg


def _rel(got, want):
    err = maxabs(got, want)
    return err / max(float(np.max(np.abs(want))), 1e-300)


def _bound_inputs(T, Hq, Hkv, d, w, v_scale, seed, k_sign=1.0, mixed_keys=True):
    """Constant q rows; k rows constant (sign k_sign) -- every other one random when
    mixed_keys -- so that the constant keys score exactly at the RMSNorm bound; V ~ N(0,1)
    * v_scale (rounded to bf16); norm weights all w."""
    import torch
    q = torch.ones((1, T, Hq, d), dtype=torch.bfloat16)
    k = torch.full((1, T, Hkv, d), k_sign, dtype=torch.bfloat16)
    if mixed_keys:
        k[:, 1::2] = host_tensor((1, T, Hkv, d), seed, "bf16")[:, 1::2]
    v = (host_tensor((1, T, Hkv, d), seed + 1, "f32") * v_scale).to(torch.bfloat16)
    g = host_tensor((1, T, Hq, d), seed + 2, "bf16")
    wq = torch.full((d,), w, dtype=torch.float32)
    wk = torch.full((d,), w, dtype=torch.float32)
    return q, k, v, g, wq, wk


def _run_prefill(zg, kind, q, k, v, g, wq, wk, *, window=128, rdim, ws="auto", **par):
    import torch
    qd, kd, vd, wqd, wkd = (t.cuda() for t in (q, k, v, wq, wk))
    if kind == "swa":
        out = zg.swa_prefill(qd, kd, vd, g.cuda(), wqd, wkd, window=window, rotary_dim=rdim,
                             **par)
    else:
        out = zg.global_prefill(qd, kd, vd, wqd, wkd, rotary_dim=rdim, workspace=ws, **par)
    torch.cuda.synchronize()
    return out


def _oracle_prefill(kind, q, k, v, g, wq, wk, rows, *, window=128, rdim, pos_offset=0,
                    scale=None, eps=1e-6, rope_base=10000.0):
    return O.prefill_rows(host64(q), host64(k), host64(v), host64(g) if kind == "swa" else None,
                          host64(wq), host64(wk), rows,
                          window=window if kind == "swa" else None, rotary_dim=rdim,
                          pos_offset=pos_offset, scale=scale, eps=eps, rope_base=rope_base,
                          threads=threads())


def _bound(d, w, scale=None):
    qscale = (d ** -0.5 if scale is None else scale) * 1.4426950408889634
    return qscale * d * w * w * 1.02


# ---- scores at the bound, values far from 1 -----------------------------------------------

@pytest.mark.parametrize("w,v_scale,ws", [(1.69, 1e6, "auto"), (1.69, 1e30, "auto"),
                                          (1.69, 1e6, None), (2.4, 1e6, "auto"),
                                          (2.4, 1e6, None)])
def test_global_scores_at_bound_large_v(w, v_scale, ws):
    zg = _zg()
    T, Hq, Hkv, d = 8192, 8, 2, 128
    b = _bound(d, w)
    assert (b <= 48.0) == (w < 2), b      # 1.69: static-shift variant; 2.4: running max
    q, k, v, g, wq, wk = _bound_inputs(T, Hq, Hkv, d, w, v_scale, 31)
    out = _run_prefill(zg, "global", q, k, v, g, wq, wk, rdim=0, ws=ws)
    rows = stratified_rows(T, 512, 32)
    want = _oracle_prefill("global", q, k, v, g, wq, wk, rows, rdim=0)
    rel = _rel(host64(out)[:, rows], want)
    say("global at bound", w, v_scale, ws, f"bound={b:.1f} rel={rel:.2e}")
    assert rel <= REL_TOL


@pytest.mark.parametrize("w,v_scale,rdim", [(1.69, 3e7, 0), (1.69, 3e7, 42), (1.69, 1e30, 42),
                                            (2.4, 3e7, 0), (2.4, 3e7, 42)])
def test_swa_scores_at_bound_large_v(w, v_scale, rdim):
    # rotary_dim 42 with 4 query heads per KV head runs the streaming SWA kernel, 0 the
    # tiled one
    zg = _zg()
    T, Hq, Hkv, d = 300, 8, 2, 128
    q, k, v, g, wq, wk = _bound_inputs(T, Hq, Hkv, d, w, v_scale, 41)
    out = _run_prefill(zg, "swa", q, k, v, g, wq, wk, rdim=rdim)
    rows = np.arange(T)
    want = _oracle_prefill("swa", q, k, v, g, wq, wk, rows, rdim=rdim)
    rel = _rel(host64(out), want)
    say("swa at bound", w, v_scale, rdim, f"rel={rel:.2e}")
    assert rel <= REL_TOL


@pytest.mark.parametrize("kind,rdim", [("global", 0), ("swa", 0), ("swa", 42)])
def test_scores_at_lower_bound_small_v(kind, rdim):
    # every score at -qscale*d*w^2: the static shift puts p at about 2^-94, still normal;
    # V ~ 1e-4 keeps the products p*v normal too
    zg = _zg()
    T, Hq, Hkv, d = 1000, 8, 2, 128
    q, k, v, g, wq, wk = _bound_inputs(T, Hq, Hkv, d, 1.69, 1e-4, 51, k_sign=-1.0,
                                       mixed_keys=False)
    out = _run_prefill(zg, kind, q, k, v, g, wq, wk, rdim=rdim)
    rows = np.arange(T)
    want = _oracle_prefill(kind, q, k, v, g, wq, wk, rows, rdim=rdim)
    rel = _rel(host64(out), want)
    say("lower bound small v", kind, rdim, f"rel={rel:.2e}")
    assert rel <= REL_TOL


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_small_v_random_scores(kind):
    zg = _zg()
    T, Hq, Hkv, d = 700, 8, 2, 128
    import torch
    q = host_tensor((1, T, Hq, d), 61, "bf16")
    k = host_tensor((1, T, Hkv, d), 62, "bf16")
    v = (host_tensor((1, T, Hkv, d), 63, "f32") * 1e-4).to(torch.bfloat16)
    g = host_tensor((1, T, Hq, d), 64, "bf16")
    wq = torch.from_numpy(norm_weight(d, 65))
    wk = torch.from_numpy(norm_weight(d, 66))
    out = _run_prefill(zg, kind, q, k, v, g, wq, wk, rdim=42)
    want = _oracle_prefill(kind, q, k, v, g, wq, wk, np.arange(T), rdim=42)
    rel = _rel(host64(out), want)
    say("small v", kind, f"rel={rel:.2e}")
    assert rel <= REL_TOL


# ---- non-default softmax_scale, rms_eps, rope_base ---------------------------------------

PARAMS = [  # (softmax_scale, rms_eps, rope_base, pos_offset)
    (0.05, 1e-6, 10000.0, 0),
    (0.2, 1e-6, 10000.0, 0),
    (0.0, 1e-2, 10000.0, 0),
    (0.0, 1e-6, 1e7, 200000),
    (0.2, 1e-2, 1e7, 200000),
]


def _param_id(p):
    return f"scale{p[0]}-eps{p[1]}-base{p[2]:g}-pos{p[3]}"


def _tol(scale, d=128):
    """The bf16 tolerance, grown with the softmax scale above the default 1/sqrt(d): the
    dominant error is the bf16 rounding of q~ and k~ inside the scores (about
    scale * sqrt(d) * |q~_c| |k~_c| * 2^-9 per score), which is proportional to the scale."""
    return TOL_BF16 * max(1.0, scale * d ** 0.5)


@pytest.mark.parametrize("par", PARAMS, ids=_param_id)
@pytest.mark.parametrize("kind,ws,Hq", [("swa", None, 8), ("swa", None, 4), ("global", "auto", 8),
                                        ("global", None, 8)])
def test_prefill_nondefault_parameters(par, kind, ws, Hq):
    # Hq 8 over 2 KV heads with rotary 42: the streaming SWA kernel; Hq 4 over 2: the tiled one
    zg = _zg()
    import torch
    scale, eps, base, po = par
    T, Hkv, d = 700, 2, 128
    q = host_tensor((1, T, Hq, d), 71, "bf16")
    k = host_tensor((1, T, Hkv, d), 72, "bf16")
    v = host_tensor((1, T, Hkv, d), 73, "bf16")
    g = host_tensor((1, T, Hq, d), 74, "bf16")
    # small rows make eps matter: eps 1e-2 against mean squares of about 0.04
    q[:, ::3] *= 0.2
    k[:, ::5] *= 0.2
    wq = torch.from_numpy(norm_weight(d, 75))
    wk = torch.from_numpy(norm_weight(d, 76))
    out = _run_prefill(zg, kind, q, k, v, g, wq, wk, rdim=42, ws=ws, pos_offset=po,
                       rope_base=base, eps=eps, scale=scale)
    want = _oracle_prefill(kind, q, k, v, g, wq, wk, np.arange(T), rdim=42, pos_offset=po,
                           scale=scale if scale > 0 else None, eps=eps, rope_base=base)
    err = maxabs(host64(out), want)
    say("prefill params", kind, ws, Hq, par, f"err={err:.2e}")
    assert err <= _tol(scale)
    if scale == 0.0 and eps == 1e-6 and base == 10000.0:
        return
    # the parameters must matter: the default-parameter oracle is far off
    dflt = _oracle_prefill(kind, q, k, v, g, wq, wk, np.arange(T), rdim=42, pos_offset=po)
    assert maxabs(dflt, want) > 5 * TOL_BF16


def _decode_tensors(B, Hq, Hkv, d, S, seed):
    q = host_tensor((B, Hq, d), seed, "bf16")
    g = host_tensor((B, Hq, d), seed + 1, "bf16")
    kn = host_tensor((B, Hkv, d), seed + 2, "bf16")
    vn = host_tensor((B, Hkv, d), seed + 3, "bf16")
    kc = host_tensor((B, Hkv, S, d), seed + 4, "bf16")
    vc = host_tensor((B, Hkv, S, d), seed + 5, "bf16")
    import torch
    q[::2] *= 0.2
    kn[1::2] *= 0.2
    wq = torch.from_numpy(norm_weight(d, seed + 6))
    wk = torch.from_numpy(norm_weight(d, seed + 7))
    return q, g, kn, vn, kc, vc, wq, wk


@pytest.mark.parametrize("par", PARAMS, ids=_param_id)
def test_decode_nondefault_parameters(par):
    zg = _zg()
    import torch
    scale, eps, base, po = par
    B, Hq, Hkv, d, S, W = 4, 8, 2, 128, 3000, 128
    pos = [po % S, (po + 5) % S, S - 1, 64]
    q, g, kn, vn, kc, vc, wq, wk = _decode_tensors(B, Hq, Hkv, d, S, 81)
    kr, vr = kc[:, :, :W].contiguous(), vc[:, :, :W].contiguous()
    r = 42
    kw = dict(rotary_dim=r, rope_base=base, eps=eps, scale=scale)
    okw = dict(rotary_dim=r, rope_base=base, eps=eps, scale=scale if scale > 0 else None)
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    og = zg.global_decode(q.cuda(), kn.cuda(), vn.cuda(), wq.cuda(), wk.cuda(), kc.cuda(),
                          vc.cuda(), posd, **kw)
    # ring positions past the window, so that the ring holds a full window
    pos_s = [p + 1000 for p in pos]
    os_ = zg.swa_decode(q.cuda(), kn.cuda(), vn.cuda(), g.cuda(), wq.cuda(), wk.cuda(),
                        kr.cuda(), vr.cuda(), torch.tensor(pos_s, dtype=torch.int32,
                                                           device="cuda"), **kw)
    torch.cuda.synchronize()
    want_g, _ = O.decode_global(host64(q), host64(kn), host64(vn), host64(wq), host64(wk),
                                host64(kc), host64(vc), np.array(pos), **okw)
    want_s, _ = O.decode_swa(host64(q), host64(kn), host64(vn), host64(g), host64(wq),
                             host64(wk), host64(kr), host64(vr), np.array(pos_s), window=W,
                             **okw)
    e1, e2 = maxabs(host64(og), want_g), maxabs(host64(os_), want_s)
    say("decode params", par, f"global={e1:.2e} swa={e2:.2e}")
    assert e1 <= _tol(scale) and e2 <= _tol(scale)


# ---- decode over a ring with unwritten (NaN) slots ----------------------------------------

@pytest.mark.parametrize("W,Hq,Hkv,d", [(128, 8, 2, 128), (128, 16, 2, 128), (100, 4, 1, 64)])
def test_swa_decode_nan_in_unwritten_slots(W, Hq, Hkv, d):
    zg = _zg()
    import torch
    pos = [0, 5, W - 2]
    B = len(pos)
    q, g, kn, vn, kc, vc, wq, wk = _decode_tensors(B, Hq, Hkv, d, W, 91)
    kr, vr = kc.clone(), vc.clone()
    for b, p in enumerate(pos):        # slots p .. W-1 never written: NaN
        kr[b, :, p:] = float("nan")
        vr[b, :, p:] = float("nan")
    r = zg.rotary_dim_for(d)
    krd, vrd = kr.cuda(), vr.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = zg.swa_decode(q.cuda(), kn.cuda(), vn.cuda(), g.cuda(), wq.cuda(), wk.cuda(), krd,
                        vrd, posd, rotary_dim=r)
    # the same step through the stack call (one SWA layer and one global layer)
    layers = [dict(kind="swa", q=q.cuda(), g=g.cuda(), k_new=kn.cuda(), v_new=vn.cuda(),
                   wq=wq.cuda(), wk=wk.cuda(), k_cache=kr.cuda(), v_cache=vr.cuda())]
    outs = zg.model_decode(layers, posd, window=W)
    torch.cuda.synchronize()
    want, _ = O.decode_swa(host64(q), host64(kn), host64(vn), host64(g), host64(wq),
                           host64(wk), host64(kr), host64(vr), np.array(pos), window=W,
                           rotary_dim=r)
    e1, e2 = maxabs(host64(out), want), maxabs(host64(outs[0]), want)
    say("swa decode NaN ring", W, Hq, Hkv, d, f"{e1:.2e} {e2:.2e}")
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16
