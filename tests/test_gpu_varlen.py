"""Packed variable-length prefill and RoPE base 1e7 against the fp64 oracle (GPU).

Documents of a packed sequence are independent sequences (oracle ``prefill_varlen``);
lengths cover a single token, tile boundaries (63, 64, 65, 128, 129), and documents longer
than several tiles, so boundaries fall inside K/V tiles and query tiles.
"""

import numpy as np
import pytest

from oracle import attn as O
from tests.gpu_util import TOL_BF16, TOL_F32, host64, maxabs, need_gpu, say, threads
from workloads import host_tensor, norm_weight

pytestmark = pytest.mark.gpu


def _zg():
    need_gpu()
    import global_attention_qk_amd as zg
    return zg


def _packed(lens, Hq, Hkv, d, seed, dtype="bf16"):
    import torch
    T = int(sum(lens))
    q = host_tensor((T, Hq, d), seed, dtype)
    k = host_tensor((T, Hkv, d), seed + 1, dtype)
    v = host_tensor((T, Hkv, d), seed + 2, dtype)
    g = host_tensor((T, Hq, d), seed + 3, dtype, 2 ** 0.5)
    wq = torch.from_numpy(norm_weight(d, seed + 4))
    wk = torch.from_numpy(norm_weight(d, seed + 5))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, g, wq, wk, cu


def _run(kind, lens, Hq, Hkv, d, seed, *, window=128, workspace="auto", rope_base=10000.0,
         pos_offset=0, rows=None, dtype="bf16", rdim=None):
    zg = _zg()
    import torch
    q, k, v, g, wq, wk, cu = _packed(lens, Hq, Hkv, d, seed, dtype)
    r = zg.rotary_dim_for(d) if rdim is None else rdim
    dv = [t.cuda() for t in (q, k, v, g, wq, wk)]
    cud = torch.from_numpy(cu).cuda()
    mx = int(max(lens))
    if kind == "swa":
        out = zg.swa_prefill_varlen(dv[0], dv[1], dv[2], dv[3], dv[4], dv[5], cud, mx,
                                    window=window, rotary_dim=r, rope_base=rope_base,
                                    pos_offset=pos_offset)
    else:
        out = zg.global_prefill_varlen(dv[0], dv[1], dv[2], dv[4], dv[5], cud, mx,
                                       rotary_dim=r, rope_base=rope_base,
                                       pos_offset=pos_offset, workspace=workspace)
    torch.cuda.synchronize()
    want = O.prefill_varlen(host64(q), host64(k), host64(v),
                            host64(g) if kind == "swa" else None, host64(wq), host64(wk), cu,
                            rows=rows, window=window if kind == "swa" else None, rotary_dim=r,
                            rope_base=rope_base, pos_offset=pos_offset, threads=threads())
    got = host64(out) if rows is None else host64(out)[rows]
    err = maxabs(got, want)
    say("varlen", kind, dtype, d, Hq, Hkv, lens[:8], f"W={window} base={rope_base} err={err:.3e}")
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16), err


LENS = [1, 63, 64, 65, 300, 7, 129, 200, 128]


@pytest.mark.parametrize("ws", ["auto", None])
def test_global_varlen(ws):
    _run("global", LENS, 8, 2, 128, 500, workspace=ws)


def test_global_varlen_head_dim_64():
    _run("global", [70, 1, 190, 64], 4, 1, 64, 510)


@pytest.mark.parametrize("window", [128, 50])
def test_swa_varlen_model_shape(window):
    # d 128, four query heads per KV head, rotary 42: the streaming SWA kernel
    _run("swa", LENS, 8, 2, 128, 520, window=window)


def test_swa_varlen_other_shape():
    # d 64: the tiled SWA kernel
    _run("swa", [70, 1, 190, 64], 4, 1, 64, 530)


def test_varlen_single_document_and_empty_documents():
    # empty documents (repeated offsets) are skipped; one long document is the dense layer
    _run("global", [0, 300, 0, 0, 45, 0], 8, 2, 128, 540)
    _run("swa", [0, 300, 0, 0, 45, 0], 8, 2, 128, 550)


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_rope_base_ten_million(kind):
    # the 256K training stage's RoPE base (explainer, section 中訓練), large positions
    _run(kind, [200, 333], 8, 2, 128, 560, rope_base=1e7, pos_offset=200000)


def test_global_varlen_long_documents_sampled_rows():
    lens = [40000, 1, 20000, 5535]
    T = sum(lens)
    rng = np.random.default_rng(570)
    cu = np.concatenate([[0], np.cumsum(lens)])
    edges = np.concatenate([cu[:-1], cu[1:] - 1, cu[:-1] + 63, cu[:-1] + 64])
    rows = np.unique(np.concatenate([edges[(edges >= 0) & (edges < T)],
                                     rng.integers(0, T, 256)]))
    _run("global", lens, 8, 2, 128, 570, rows=rows)


def _random_packings(n=6, seed=990077):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        n_docs = int(rng.integers(1, 13))
        lens = [int(x) for x in rng.integers(0, 400, size=n_docs)]
        if sum(lens) == 0:
            lens[0] = 1
        model = i % 2 == 0   # the streaming SWA kernel's shape
        d = 128 if model else int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * (4 if model else int(rng.choice([1, 2, 4, 8])))
        window = int(rng.integers(1, 129 if model else 300))
        pos = int(rng.integers(0, 20_000))
        cases.append((i, lens, Hq, Hkv, d, window, pos))
    return cases


@pytest.mark.parametrize("case", _random_packings(), ids=lambda c: f"case{c[0]}")
def test_varlen_random_packings(case):
    # seeded random document counts and lengths (empty documents included), head shapes,
    # windows and position offsets through both packed layers
    i, lens, Hq, Hkv, d, window, pos = case
    _run("swa", lens, Hq, Hkv, d, 600 + 10 * i, window=window, pos_offset=pos)
    _run("global", lens, Hq, Hkv, d, 600 + 10 * i, pos_offset=pos)


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_varlen_fp32(kind):
    # fp32 packed documents on the vector-ALU kernel: empty and one-token documents, tile
    # boundaries, three query heads per KV head and a rotary dim the MFMA paths do not take
    lens = [0, 1, 63, 64, 65, 130, 0, 200]
    _run(kind, lens, 6, 2, 128, 580, window=50, dtype="f32", pos_offset=123, rdim=80)
    _run(kind, [70, 1, 190], 4, 1, 64, 590, window=128, dtype="f32")


@pytest.mark.parametrize("kind", ["swa", "global"])
def test_varlen_bf16_shape_off_the_mfma_paths(kind):
    # three query heads per KV head and rotary 80 (bf16): the vector-ALU kernel per document
    _run(kind, [0, 90, 1, 150], 6, 2, 128, 595, window=40, rdim=80)
