"""Randomised decode parity: seeded random batches, head groups, head dims, cache or ring
sizes and positions through both decode calls, against the fp64 oracle.

Global decode: caches of 1 .. 30,000 entries with every sequence at its own random
position (split-K chunks, their ragged last chunk and single-entry caches all occur). SWA
decode: rings of 1 .. 300 slots (both the MFMA kernel, rings up to 128, and the per-slot
kernel above) at positions up to 300,000, so that the ring has wrapped or is still
filling. Besides the output (max-abs 2e-2), each call must write k~ and v of the new token
into its slot and leave every other slot untouched.
"""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, host64, maxabs, need_gpu, say
from tests.test_gpu_decode import _decode_case

pytestmark = pytest.mark.gpu


def _zg():
    need_gpu()
    import global_attention_qk_amd as zg
    return zg


def _shape(rng):
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 5))
    return B, Hkv * group, Hkv, d


def _global_cases(n=8, seed=777001):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, Hq, Hkv, d = _shape(rng)
        S = int(rng.integers(1, 30001))
        pos = [int(x) for x in rng.integers(0, S, size=B)]
        if i % 3 == 0:
            pos[-1] = S - 1
        out.append((i, B, Hq, Hkv, d, S, pos))
    return out


def _swa_cases(n=8, seed=777002):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, Hq, Hkv, d = _shape(rng)
        W = int(rng.integers(1, 301))
        pos = [int(x) for x in rng.integers(0, 300001, size=B)]
        if i % 2 == 0:
            pos[0] = int(rng.integers(0, W))      # ring still filling
        out.append((i, B, Hq, Hkv, d, W, pos))
    return out


@pytest.mark.parametrize("case", _global_cases(), ids=lambda c: f"case{c[0]}")
def test_random_global_decode(case):
    zg = _zg()
    import torch
    i, B, Hq, Hkv, d, S, pos = case
    q, g, kn, vn, kc, vc, wq, wk = _decode_case(B, Hq, Hkv, d, S, 31000 + 10 * i)
    kcd, vcd = kc.cuda(), vc.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = zg.global_decode(q.cuda(), kn.cuda(), vn.cuda(), wq.cuda(), wk.cuda(), kcd, vcd, posd)
    torch.cuda.synchronize()
    r = zg.rotary_dim_for(d)
    want, ktn = O.decode_global(host64(q), host64(kn), host64(vn), host64(wq), host64(wk),
                                host64(kc), host64(vc), np.array(pos), rotary_dim=r)
    err = maxabs(host64(out), want)
    say("random global_decode", (B, Hq, Hkv, d, S), pos, f"{err:.3e}")
    assert err <= TOL_BF16
    kc2, vc2 = host64(kcd), host64(vcd)
    for b, p in enumerate(pos):
        assert maxabs(kc2[b, :, p], ktn[b]) <= 2e-2
        assert np.array_equal(vc2[b, :, p], host64(vn)[b])
        mask = np.ones(S, bool)
        mask[p] = False
        assert np.array_equal(kc2[b, :, mask], host64(kc)[b, :, mask])
        assert np.array_equal(vc2[b, :, mask], host64(vc)[b, :, mask])


@pytest.mark.parametrize("case", _swa_cases(), ids=lambda c: f"case{c[0]}")
def test_random_swa_decode(case):
    zg = _zg()
    import torch
    i, B, Hq, Hkv, d, W, pos = case
    r = zg.rotary_dim_for(d)
    q, g, kn, vn, kr, vr, wq, wk = _decode_case(B, Hq, Hkv, d, W, 32000 + 10 * i)
    krd, vrd = kr.cuda(), vr.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = zg.swa_decode(q.cuda(), kn.cuda(), vn.cuda(), g.cuda(), wq.cuda(), wk.cuda(), krd,
                        vrd, posd, rotary_dim=r)
    torch.cuda.synchronize()
    want, ktn = O.decode_swa(host64(q), host64(kn), host64(vn), host64(g), host64(wq),
                             host64(wk), host64(kr), host64(vr), np.array(pos), window=W,
                             rotary_dim=r)
    err = maxabs(host64(out), want)
    say("random swa_decode", (B, Hq, Hkv, d, W), pos, f"{err:.3e}")
    assert err <= TOL_BF16
    kr2, vr2 = host64(krd), host64(vrd)
    for b, p in enumerate(pos):
        assert maxabs(kr2[b, :, p % W], ktn[b]) <= 2e-2
        assert np.array_equal(vr2[b, :, p % W], host64(vn)[b])
        others = np.ones(W, bool)
        others[p % W] = False
        assert np.array_equal(kr2[b, :, others], host64(kr)[b, :, others])
        assert np.array_equal(vr2[b, :, others], host64(vr)[b, :, others])
