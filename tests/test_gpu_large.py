"""Full-size parity for the long-context workloads, in the launch configuration the
benchmark times.

* 256K prefill pair (B=1, T=262144, Hq=32, Hkv=8, d=128): 4096 stratified query rows per
  layer against the oracle (rows 0-15, window and tile edges, T-1, uniform rest).
* 32-sublayer hybrid stack at T=65536 (globals at 0-based 5, 11, 17, 23, 29): every layer
  launched back-to-back on one stream; 4096 sampled rows of each global layer and 1024 of
  each SWA layer against the oracle.
* Decode at context 262144, B=32: all 32 sequences of both layer kinds.
"""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, host64, maxabs, need_gpu, say, threads
from workloads import C3, C4, C5, decode_inputs, prefill_inputs, stratified_rows

pytestmark = pytest.mark.gpu


def f32(t):
    return t.detach().float().cpu().numpy()


# ---------------------------------------------------------------------------------------
# 256K prefill pair
# ---------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c4():
    need_gpu()
    import torch
    import global_attention_qk_amd as zg
    say("c4 setup: generating T=262144 inputs and running both layers")
    q, k, v, g, wq, wk = prefill_inputs(C4, device="cuda")
    out_s = zg.swa_prefill(q, k, v, g, wq, wk, window=C4.window, rotary_dim=C4.rotary_dim)
    out_g = zg.global_prefill(q, k, v, wq, wk, rotary_dim=C4.rotary_dim)
    torch.cuda.synchronize()
    rows = stratified_rows(C4.T, 4096, seed=4242, window=C4.window)
    ri = torch.from_numpy(rows).cuda()
    res = dict(rows=rows, k=f32(k), v=f32(v), q=f32(q[:, ri]), g=f32(g[:, ri]), wq=f32(wq),
               wk=f32(wk), out_s=f32(out_s[:, ri]), out_g=f32(out_g[:, ri]))
    del q, k, v, g, out_s, out_g
    torch.cuda.empty_cache()
    return res


def test_c4_swa_4096_rows(c4):
    want = O.prefill_rows(c4["q"], c4["k"], c4["v"], c4["g"], c4["wq"], c4["wk"], c4["rows"],
                          window=C4.window, rotary_dim=C4.rotary_dim, threads=threads())
    err = maxabs(c4["out_s"], want)
    say("c4 swa", len(c4["rows"]), "rows err", err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("part", range(4))
def test_c4_global_4096_rows(c4, part):
    sel = np.arange(part, len(c4["rows"]), 4)
    rows = c4["rows"][sel]
    want = O.prefill_rows(c4["q"][:, sel], c4["k"], c4["v"], None, c4["wq"], c4["wk"], rows,
                          rotary_dim=C4.rotary_dim, threads=threads(), row_block=64)
    err = maxabs(c4["out_g"][:, sel], want)
    say("c4 global part", part, len(rows), "rows err", err)
    assert err <= TOL_BF16


# ---------------------------------------------------------------------------------------
# 32-sublayer hybrid stack at T=65536
# ---------------------------------------------------------------------------------------

KINDS = O.layer_kinds(C3.n_layers)


@pytest.fixture(scope="module")
def c3():
    need_gpu()
    import torch
    import global_attention_qk_amd as zg
    say("c3 setup: 32 layers at T=65536")
    ins, outs = [], []
    for layer, kind in enumerate(KINDS):
        ins.append(prefill_inputs(C3, layer, device="cuda", gated=(kind == "swa")))
    torch.cuda.synchronize()
    for layer, kind in enumerate(KINDS):      # back-to-back on one stream
        q, k, v, g, wq, wk = ins[layer]
        if kind == "swa":
            outs.append(zg.swa_prefill(q, k, v, g, wq, wk, window=C3.window,
                                       rotary_dim=C3.rotary_dim))
        else:
            outs.append(zg.global_prefill(q, k, v, wq, wk, rotary_dim=C3.rotary_dim))
    torch.cuda.synchronize()
    res = {}
    for layer, kind in enumerate(KINDS):
        n = 4096 if kind == "global" else 1024
        rows = stratified_rows(C3.T, n, seed=3000 + layer, window=C3.window)
        ri = torch.from_numpy(rows).cuda()
        q, k, v, g, wq, wk = ins[layer]
        res[layer] = dict(rows=rows, k=f32(k), v=f32(v), q=f32(q[:, ri]),
                          g=None if g is None else f32(g[:, ri]), wq=f32(wq), wk=f32(wk),
                          out=f32(outs[layer][:, ri]))
    del ins, outs
    torch.cuda.empty_cache()
    return res


@pytest.mark.parametrize("layer", range(C3.n_layers))
def test_c3_stack_layer(c3, layer):
    r = c3[layer]
    kind = KINDS[layer]
    want = O.prefill_rows(r["q"], r["k"], r["v"], r["g"], r["wq"], r["wk"], r["rows"],
                          window=C3.window if kind == "swa" else None,
                          rotary_dim=C3.rotary_dim, threads=threads(), row_block=128)
    err = maxabs(r["out"], want)
    say("c3 layer", layer, kind, len(r["rows"]), "rows err", err)
    assert err <= TOL_BF16


# ---------------------------------------------------------------------------------------
# decode at context 262144, B = 32
# ---------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c5():
    need_gpu()
    import torch
    import global_attention_qk_amd as zg
    say("c5 setup: B=32 caches at context 262144")
    dec = decode_inputs(C5, device="cuda")
    S = C5.T
    pos = torch.full((C5.B,), S - 1, dtype=torch.int32, device="cuda")
    host_ring = (f32(dec["k_ring"]), f32(dec["v_ring"]))
    out_g = zg.global_decode(dec["q"], dec["k_new"], dec["v_new"], dec["wq"], dec["wk"],
                             dec["k_cache"], dec["v_cache"], pos, rotary_dim=C5.rotary_dim)
    out_s = zg.swa_decode(dec["q"], dec["k_new"], dec["v_new"], dec["g"], dec["wq"],
                          dec["wk"], dec["k_ring"], dec["v_ring"], pos,
                          rotary_dim=C5.rotary_dim)
    torch.cuda.synchronize()
    yield dict(dec=dec, out_g=f32(out_g), out_s=f32(out_s), ring=host_ring, S=S)
    del dec
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_c5_global_decode_all_sequences(c5, part):
    dec = c5["dec"]
    S = c5["S"]
    worst = 0.0
    for b in range(part * 8, part * 8 + 8):
        want, _ = O.decode_global(f32(dec["q"][b:b + 1]), f32(dec["k_new"][b:b + 1]),
                                  f32(dec["v_new"][b:b + 1]), f32(dec["wq"]), f32(dec["wk"]),
                                  f32(dec["k_cache"][b:b + 1]), f32(dec["v_cache"][b:b + 1]),
                                  np.array([S - 1]), rotary_dim=C5.rotary_dim)
        worst = max(worst, maxabs(c5["out_g"][b:b + 1], want))
    say("c5 global decode sequences", part * 8, "..", part * 8 + 7, "err", worst)
    assert worst <= TOL_BF16


def test_c5_swa_decode_all_sequences(c5):
    dec = c5["dec"]
    kr, vr = c5["ring"]
    want, _ = O.decode_swa(f32(dec["q"]), f32(dec["k_new"]), f32(dec["v_new"]), f32(dec["g"]),
                           f32(dec["wq"]), f32(dec["wk"]), kr, vr,
                           np.full(C5.B, c5["S"] - 1), window=C5.window,
                           rotary_dim=C5.rotary_dim)
    err = maxabs(c5["out_s"], want)
    say("c5 swa decode err", err)
    assert err <= TOL_BF16
