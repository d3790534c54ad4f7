"""Persistent global prefill launches.

With the K~ workspace, the global layer of a dense batch runs one workgroup per CU whenever
it has more query tiles than CUs; each workgroup walks its share of the tiles, dealt out in
snake order over the heavy-first list, grouped by XCD when the (batch, KV head) pairs
divide by 8 and over the plain list otherwise. A tile's arithmetic does not depend on which
workgroup runs it, so a persistent batch must match, bit for bit, the same sequences run one
batch element at a time (few enough tiles for one workgroup per tile), in the output and in
the row log-sum-exp; the output buffer starts as NaN, so a tile left out shows. Rows at
every query tile's first and last position are also checked against the fp64 oracle.
"""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, host64, maxabs, need_gpu, say, threads
from tests.test_gpu_prefill import _inputs

pytestmark = pytest.mark.gpu

# (B, T, Hq, Hkv, d): query tiles = B * Hkv * ceil(T / (256 / (Hq / Hkv)))
CASES = [
    (3, 5000, 8, 2, 128),    # 474 tiles, pairs not divisible by 8: plain snake order
    (2, 1100, 32, 8, 128),   # 288 tiles, the model's heads: per-XCD snake order
    (2, 2100, 16, 8, 64),    # 272 tiles, head dim 64, two query heads per KV head
]


def _tiles(B, T, Hq, Hkv):
    bmp = 256 // (Hq // Hkv)
    return B * Hkv * ((T + bmp - 1) // bmp), bmp


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_Hq{}_Hkv{}_d{}".format(*c))
def test_persistent_matches_single_sequences_and_oracle(case):
    need_gpu()
    import torch

    import global_attention_qk_amd as zg

    B, T, Hq, Hkv, d = case
    cus = torch.cuda.get_device_properties(0).multi_processor_count   # the persistent grid
    n_tiles, bmp = _tiles(B, T, Hq, Hkv)
    n_single, _ = _tiles(1, T, Hq, Hkv)
    assert n_tiles > cus >= n_single, (n_tiles, cus, n_single)   # persistent vs one tile each
    q, k, v, _, wq, wk = _inputs(B, T, Hq, Hkv, d, "bf16", 7100 + T)
    qd, kd, vd, wqd, wkd = (t.cuda() for t in (q, k, v, wq, wk))
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    zg.global_prefill(qd, kd, vd, wqd, wkd, out=out, lse=lse)
    singles, slse = [], []
    for b in range(B):
        o1 = torch.full_like(qd[b:b + 1], float("nan"))
        l1 = torch.full((1, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
        zg.global_prefill(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(),
                          vd[b:b + 1].contiguous(), wqd, wkd, out=o1, lse=l1)
        singles.append(o1)
        slse.append(l1)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert torch.equal(out, torch.cat(singles)), "persistent output differs from single runs"
    assert torch.equal(lse, torch.cat(slse)), "persistent lse differs from single runs"

    starts = np.arange(0, T, bmp)
    rows = np.unique(np.concatenate([starts, np.minimum(starts + bmp - 1, T - 1)]))
    want = O.prefill_rows(host64(q), host64(k), host64(v), None, host64(wq), host64(wk), rows,
                          rotary_dim=zg.rotary_dim_for(d), threads=threads())
    err = maxabs(host64(out)[:, rows], want)
    say("persistent", case, n_tiles, "tiles", len(rows), "rows err", f"{err:.3e}")
    assert err <= TOL_BF16, err
