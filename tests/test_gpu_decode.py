"""Decode and standalone QK-norm/RoPE parity against the fp64 oracle (GPU)."""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, TOL_F32, host64, maxabs, need_gpu, say
from workloads import host_tensor, norm_weight

pytestmark = pytest.mark.gpu


def _zg():
    need_gpu()
    import global_attention_qk_amd as zg
    return zg


def _w(d, seed):
    import torch
    return torch.from_numpy(norm_weight(d, seed))


@pytest.mark.parametrize("dtype,tol,pos0,d", [("bf16", TOL_BF16, 1000, 128), ("f32", 2e-5, 1000, 128),
                                              ("f32", 2e-5, 262100, 128), ("f32", 2e-5, 7, 64),
                                              ("bf16", TOL_BF16, 0, 64)])
def test_qknorm_rope_into_cache_layout(dtype, tol, pos0, d):
    zg = _zg()
    import torch
    B, T, H, S = 2, 37, 3, 64
    x = host_tensor((B, T, H, d), 11, dtype)
    w = _w(d, 12)
    cache = torch.full((B, H, S, d), float("nan"), dtype=x.dtype, device="cuda")
    view = cache.permute(0, 2, 1, 3)[:, 5:5 + T]          # rows 5..5+T of each head
    zg.qknorm_rope(x.cuda(), w.cuda(), out=view, pos_offset=pos0)
    torch.cuda.synchronize()
    want = O.qknorm_rope(host64(x), host64(w), pos0 + np.arange(T)[None, :, None],
                         42 if d == 128 else 20)
    got = host64(cache).transpose(0, 2, 1, 3)[:, 5:5 + T]
    err = maxabs(got, want)
    say("qknorm_rope", dtype, err)
    assert err <= tol
    c = host64(cache)
    assert np.all(np.isnan(c[:, :, :5])) and np.all(np.isnan(c[:, :, 5 + T:]))


def test_qknorm_rope_position_array():
    zg = _zg()
    import torch
    B, T, H, d = 2, 10, 2, 64
    x = host_tensor((B, T, H, d), 21, "bf16")
    w = _w(d, 22)
    pos = np.random.default_rng(23).integers(0, 262144, size=(B, T)).astype(np.int32)
    out = zg.qknorm_rope(x.cuda(), w.cuda(), pos=torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    want = O.qknorm_rope(host64(x), host64(w), pos[:, :, None], 20)
    assert maxabs(host64(out), want) <= TOL_BF16


def _decode_case(B, Hq, Hkv, d, S, seed, dtype="bf16"):
    q = host_tensor((B, Hq, d), seed, dtype)
    g = host_tensor((B, Hq, d), seed + 1, dtype)
    kn = host_tensor((B, Hkv, d), seed + 2, dtype)
    vn = host_tensor((B, Hkv, d), seed + 3, dtype)
    kc = host_tensor((B, Hkv, S, d), seed + 4, dtype)
    vc = host_tensor((B, Hkv, S, d), seed + 5, dtype)
    return q, g, kn, vn, kc, vc, _w(d, seed + 6), _w(d, seed + 7)


@pytest.mark.parametrize("B,Hq,Hkv,d,S,pos", [
    (3, 8, 2, 128, 5000, [0, 1234, 4999]),
    (2, 32, 8, 128, 70000, [69999, 40000]),
    (2, 4, 4, 64, 300, [17, 299]),
    (1, 16, 2, 128, 2048, [2047]),
])
def test_global_decode_vs_oracle(B, Hq, Hkv, d, S, pos):
    zg = _zg()
    import torch
    q, g, kn, vn, kc, vc, wq, wk = _decode_case(B, Hq, Hkv, d, S, 1000 + S)
    kcd, vcd = kc.cuda(), vc.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = zg.global_decode(q.cuda(), kn.cuda(), vn.cuda(), wq.cuda(), wk.cuda(), kcd, vcd, posd)
    torch.cuda.synchronize()
    r = zg.rotary_dim_for(d)
    want, ktn = O.decode_global(host64(q), host64(kn), host64(vn), host64(wq), host64(wk),
                                host64(kc), host64(vc), np.array(pos), rotary_dim=r)
    err = maxabs(host64(out), want)
    say("global_decode", (B, Hq, Hkv, d, S), pos, err)
    assert err <= TOL_BF16
    kc2, vc2 = host64(kcd), host64(vcd)
    for b, p in enumerate(pos):
        assert maxabs(kc2[b, :, p], ktn[b]) <= 2e-2
        assert np.array_equal(vc2[b, :, p], host64(vn)[b])
        mask = np.ones(S, bool)
        mask[p] = False
        assert np.array_equal(kc2[b, :, mask], host64(kc)[b, :, mask])


# Rings of at most 128 slots take the MFMA kernel (instances for at most 4 and for 8 query
# heads per KV head); larger rings take the per-slot kernel.
@pytest.mark.parametrize("W,d,Hq,Hkv", [(128, 128, 8, 2), (128, 64, 8, 1), (50, 128, 2, 2),
                                        (77, 64, 16, 2), (1, 128, 4, 1), (300, 128, 8, 2),
                                        (128, 128, 16, 2), (100, 128, 8, 1), (33, 64, 2, 1)])
def test_swa_decode_vs_oracle(W, d, Hq, Hkv):
    zg = _zg()
    import torch
    pos = sorted({0, 5, max(W - 2, 0), W - 1, W, 300, 100000})
    B = len(pos)
    r = zg.rotary_dim_for(d)
    q, g, kn, vn, kr, vr, wq, wk = _decode_case(B, Hq, Hkv, d, W, 2000 + W)
    krd, vrd = kr.cuda(), vr.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = zg.swa_decode(q.cuda(), kn.cuda(), vn.cuda(), g.cuda(), wq.cuda(), wk.cuda(), krd,
                        vrd, posd, rotary_dim=r)
    torch.cuda.synchronize()
    want, ktn = O.decode_swa(host64(q), host64(kn), host64(vn), host64(g), host64(wq),
                             host64(wk), host64(kr), host64(vr), np.array(pos), window=W,
                             rotary_dim=r)
    err = maxabs(host64(out), want)
    say("swa_decode", W, d, Hq, Hkv, pos, err)
    assert err <= TOL_BF16
    kr2, vr2 = host64(krd), host64(vrd)
    for b, p in enumerate(pos):
        assert maxabs(kr2[b, :, p % W], ktn[b]) <= 2e-2
        assert np.array_equal(vr2[b, :, p % W], host64(vn)[b])
        others = np.ones(W, bool)
        others[p % W] = False
        assert np.array_equal(kr2[b, :, others], host64(kr)[b, :, others])


# fp32 tensors and caches (the per-slot SWA kernel and the global split kernel's fp32 form):
# parity at the fp32 tolerance, the new token's k~ within 1e-5 and its v copied exactly
@pytest.mark.parametrize("B,Hq,Hkv,d,S,pos", [(3, 8, 2, 128, 5000, [0, 1234, 4999]),
                                              (2, 4, 4, 64, 300, [17, 299]),
                                              (1, 16, 2, 128, 70000, [69999]),
                                              (2, 2, 1, 64, 1, [0, 0])])
def test_global_decode_fp32(B, Hq, Hkv, d, S, pos):
    zg = _zg()
    import torch
    q, g, kn, vn, kc, vc, wq, wk = _decode_case(B, Hq, Hkv, d, S, 4000 + S, "f32")
    kcd, vcd = kc.cuda(), vc.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = zg.global_decode(q.cuda(), kn.cuda(), vn.cuda(), wq.cuda(), wk.cuda(), kcd, vcd, posd)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    want, ktn = O.decode_global(host64(q), host64(kn), host64(vn), host64(wq), host64(wk),
                                host64(kc), host64(vc), np.array(pos),
                                rotary_dim=zg.rotary_dim_for(d))
    err = maxabs(host64(out), want)
    say("global_decode fp32", (B, Hq, Hkv, d, S), pos, err)
    assert err <= TOL_F32
    kc2, vc2 = host64(kcd), host64(vcd)
    for b, p in enumerate(pos):
        assert maxabs(kc2[b, :, p], ktn[b]) <= 1e-5
        assert np.array_equal(vc2[b, :, p], host64(vn)[b])
        mask = np.ones(S, bool)
        mask[p] = False
        assert np.array_equal(kc2[b, :, mask], host64(kc)[b, :, mask])


@pytest.mark.parametrize("W,d,Hq,Hkv", [(128, 128, 8, 2), (50, 64, 4, 1), (300, 128, 2, 2),
                                        (1, 64, 8, 1)])
def test_swa_decode_fp32(W, d, Hq, Hkv):
    zg = _zg()
    import torch
    pos = sorted({0, 5, max(W - 2, 0), W - 1, W, 300, 100000})
    B = len(pos)
    r = zg.rotary_dim_for(d)
    q, g, kn, vn, kr, vr, wq, wk = _decode_case(B, Hq, Hkv, d, W, 5000 + W, "f32")
    krd, vrd = kr.cuda(), vr.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = zg.swa_decode(q.cuda(), kn.cuda(), vn.cuda(), g.cuda(), wq.cuda(), wk.cuda(), krd,
                        vrd, posd, rotary_dim=r)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    want, ktn = O.decode_swa(host64(q), host64(kn), host64(vn), host64(g), host64(wq),
                             host64(wk), host64(kr), host64(vr), np.array(pos), window=W,
                             rotary_dim=r)
    err = maxabs(host64(out), want)
    say("swa_decode fp32", W, d, Hq, Hkv, pos, err)
    assert err <= TOL_F32
    kr2, vr2 = host64(krd), host64(vrd)
    for b, p in enumerate(pos):
        assert maxabs(kr2[b, :, p % W], ktn[b]) <= 1e-5
        assert np.array_equal(vr2[b, :, p % W], host64(vn)[b])
        others = np.ones(W, bool)
        others[p % W] = False
        assert np.array_equal(kr2[b, :, others], host64(kr)[b, :, others])


def test_decode_equals_prefill_row():
    """Caches built by qknorm_rope from a prefill's K/V: decode at t == prefill row t."""
    zg = _zg()
    import torch
    B, T, Hq, Hkv, d, W = 2, 300, 8, 2, 128, 128
    q = host_tensor((B, T, Hq, d), 3000, "bf16").cuda()
    k = host_tensor((B, T, Hkv, d), 3001, "bf16").cuda()
    v = host_tensor((B, T, Hkv, d), 3002, "bf16").cuda()
    g = host_tensor((B, T, Hq, d), 3003, "bf16").cuda()
    wq, wk = _w(d, 3004).cuda(), _w(d, 3005).cuda()
    pre_g = zg.global_prefill(q, k, v, wq, wk)
    pre_s = zg.swa_prefill(q, k, v, g, wq, wk, window=W)
    for t in (0, 1, 127, 128, 299):
        S = 512
        kc = torch.zeros((B, Hkv, S, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        if t > 0:
            zg.qknorm_rope(k[:, :t].contiguous(), wk, out=kc.permute(0, 2, 1, 3)[:, :t])
            vc.permute(0, 2, 1, 3)[:, :t].copy_(v[:, :t])
        pos = torch.full((B,), t, dtype=torch.int32, device="cuda")
        og = zg.global_decode(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                              wq, wk, kc, vc, pos)
        kr = torch.zeros((B, Hkv, W, d), dtype=torch.bfloat16, device="cuda")
        vr = torch.zeros_like(kr)
        for p in range(max(0, t - W + 1), t):
            kr[:, :, p % W] = kc[:, :, p]
            vr[:, :, p % W] = vc[:, :, p]
        os_ = zg.swa_decode(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                            g[:, t].contiguous(), wq, wk, kr, vr, pos)
        torch.cuda.synchronize()
        e1 = maxabs(host64(og), host64(pre_g[:, t]))
        e2 = maxabs(host64(os_), host64(pre_s[:, t]))
        say("decode==prefill row", t, e1, e2)
        assert e1 <= 2e-2 and e2 <= 2e-2


def test_decode_invalid_position_gives_nan_and_leaves_cache():
    zg = _zg()
    import torch
    B, Hq, Hkv, d, S = 2, 8, 2, 128, 1000
    q, g, kn, vn, kc, vc, wq, wk = _decode_case(B, Hq, Hkv, d, S, 4000)
    kcd, vcd = kc.cuda(), vc.cuda()
    pos = torch.tensor([-1, S], dtype=torch.int32, device="cuda")
    out = zg.global_decode(q.cuda(), kn.cuda(), vn.cuda(), wq.cuda(), wk.cuda(), kcd, vcd, pos)
    krd, vrd = kc[:, :, :128].contiguous().cuda(), vc[:, :, :128].contiguous().cuda()
    kr0 = krd.clone()
    pos2 = torch.tensor([-5, 1 << 24], dtype=torch.int32, device="cuda")
    out2 = zg.swa_decode(q.cuda(), kn.cuda(), vn.cuda(), g.cuda(), wq.cuda(), wk.cuda(), krd,
                         vrd, pos2)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(out2.float()).all()
    assert torch.equal(kcd.cpu(), kc) and torch.equal(krd, kr0)
