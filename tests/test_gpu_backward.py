"""Backward pass (zgattn_*_prefill_backward) against the fp64 oracle's gradients (GPU).

Gradients of sum(dout * out) with dout ~ N(0, 1). Tolerance: max-abs error within 2e-2 of
max(1, max |reference|) per tensor for bf16 tensors: the products run on bf16 operands (Q~,
K~, V, dA, P and dS rounded to bf16, fp32 accumulation) and the inputs' bf16 rounding bounds
the rest. fp32 tensors (the vector-ALU backward, fp32 throughout): 1e-4 of the same scale,
room for fp32 rounding summed over a thousand keys.
"""

import numpy as np
import pytest

from oracle import grad as OG
from tests.gpu_util import host64, need_gpu, say
from workloads import host_tensor, norm_weight

pytestmark = pytest.mark.gpu

REL = 2e-2
REL_F32 = 1e-4


def _check(B, T, Hq, Hkv, d, window, seed, pos_offset=0, fwd_lse=False, dtype="bf16",
           rdim=None):
    need_gpu()
    import torch
    import global_attention_qk_amd as zg
    q = host_tensor((B, T, Hq, d), seed, dtype)
    k = host_tensor((B, T, Hkv, d), seed + 1, dtype)
    v = host_tensor((B, T, Hkv, d), seed + 2, dtype)
    g = host_tensor((B, T, Hq, d), seed + 3, dtype, 2 ** 0.5) if window else None
    do = host_tensor((B, T, Hq, d), seed + 4, dtype)
    wq = torch.from_numpy(norm_weight(d, seed + 5))
    wk = torch.from_numpy(norm_weight(d, seed + 6))
    r = zg.rotary_dim_for(d) if rdim is None else rdim
    rel = REL_F32 if dtype == "f32" else REL
    cq, ck, cv, cdo, cwq, cwk = (t.cuda() for t in (q, k, v, do, wq, wk))
    cg = g.cuda() if g is not None else None
    if window:
        out = zg.swa_prefill(cq, ck, cv, cg, cwq, cwk, window=window, rotary_dim=r,
                             pos_offset=pos_offset)
        lse = None
    else:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda") if fwd_lse else None
        out = zg.global_prefill(cq, ck, cv, cwq, cwk, rotary_dim=r, pos_offset=pos_offset,
                                lse=lse)
    dq, dk, dv, dg, dwq, dwk = zg.prefill_backward(cq, ck, cv, cg, cwq, cwk, out, cdo,
                                                   window=window, rotary_dim=r,
                                                   pos_offset=pos_offset, lse=lse)
    torch.cuda.synchronize()
    ref = OG.prefill_grads(host64(q), host64(k), host64(v), None if g is None else host64(g),
                           host64(wq), host64(wk), host64(do), window=window, rotary_dim=r,
                           pos_offset=pos_offset)
    if lse is not None:
        # Scores come from bf16 operands (relative error <= 2^-8 each way) and the row sum
        # from bf16-rounded probabilities (2^-8 relative, 4e-3 in the log): the error is a
        # small multiple of 2^-8 of the largest |lse|.
        want = ref["lse"]
        err = float(np.max(np.abs(host64(lse) - want)))
        lim = 1e-2 * max(1.0, float(np.max(np.abs(want))))
        say("forward lse", (B, T, Hq, Hkv, d), f"err={err:.3e} lim={lim:.3e}")
        assert err <= lim, ("lse", err, lim)
    got = dict(dq=dq, dk=dk, dv=dv, dwq=dwq, dwk=dwk)
    if window:
        got["dg"] = dg
    for name, t in got.items():
        want = ref[name]
        err = float(np.max(np.abs(host64(t) - want)))
        lim = rel * max(1.0, float(np.max(np.abs(want))))
        say("backward", (B, T, Hq, Hkv, d, window, dtype, r), name,
            f"err={err:.3e} lim={lim:.3e}")
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


@pytest.mark.parametrize("T", [300, 1024])
def test_backward_global_with_forward_lse(T):
    # the forward's row log-sum-exp handed to the backward (no recomputation pass)
    _check(2 if T == 300 else 1, T, 8, 2, 128, None, 1700 + T, fwd_lse=True)


@pytest.mark.parametrize("window,lse", [(None, True), (None, False), (128, False)])
def test_backward_ragged_top_tile(window, lse):
    # T = 1000 (not a multiple of 64): each dK/dV workgroup of 256 keys meets a ragged last
    # query tile, a run of fully visible tiles and the diagonal tiles; B = 2, 4 query heads
    # per KV head
    _check(2, 1000, 8, 2, 128, window, 2000, fwd_lse=lse)


@pytest.mark.parametrize("window", [None, 128, 37])
def test_backward_f32(window):
    # fp32 tensors: the vector-ALU backward (forward on the vector-ALU prefill kernel),
    # several 64-row tiles, a ragged tail, 4 query heads per KV head
    _check(2, 300, 8, 2, 128, window, 2500, dtype="f32")


def test_backward_f32_head_dim_64_offset():
    _check(1, 200, 6, 2, 64, None, 2510, pos_offset=3000, dtype="f32")
    _check(1, 200, 6, 2, 64, 80, 2520, pos_offset=3000, dtype="f32")


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (3, 1), (32, 2)])
def test_backward_bf16_other_head_groups(Hq, Hkv):
    # head groups 3 and 16: bf16 tensors on the vector-ALU backward
    _check(1, 260, Hq, Hkv, 128, None, 2600 + Hq)
    _check(1, 260, Hq, Hkv, 64, 100, 2610 + Hq)


def test_backward_bf16_rotary_above_64():
    # a rotary dim the MFMA forward does not take (vector-ALU forward); the MFMA backward
    # handles any rotary dim
    _check(1, 200, 8, 2, 128, None, 2700, rdim=96)
    _check(1, 200, 8, 2, 128, 64, 2710, rdim=128)


def test_backward_forward_lse_head_dim_64_offset():
    _check(1, 150, 4, 1, 64, None, 1800, pos_offset=1000, fwd_lse=True)


def _spread_rows(T, n, seed):
    """Sorted positions: the first rows, tile and window edges, the middle, the last rows,
    and uniform draws up to n."""
    fixed = {0, 1, 2, 63, 64, 127, 128, 129, 255, 256, T // 2 - 1, T // 2, T - 65, T - 64,
             T - 2, T - 1}
    fixed = {x for x in fixed if 0 <= x < T}
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(T), np.array(sorted(fixed)))
    extra = rng.choice(pool, size=max(0, n - len(fixed)), replace=False)
    return np.sort(np.concatenate([np.array(sorted(fixed)), extra])).astype(np.int64)


@pytest.mark.parametrize("window", [None, 128])
def test_backward_sampled_rows_T8192(window):
    # 8192 positions with the model's head shape (d 128, rotary 42, 4 query heads per KV
    # head): the gradients at 48 spread query rows (dq, dg) and 48 spread keys (dk, dv, every
    # query row's contribution) against the oracle's closed-form backward, whose forward
    # runs over every row in fp64. The global layer takes the forward's log-sum-exp.
    need_gpu()
    import torch
    import global_attention_qk_amd as zg
    B, T, Hq, Hkv, d, seed = 1, 8192, 8, 2, 128, 1900
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
    lse = None
    if window:
        out = zg.swa_prefill(cq, ck, cv, cg, cwq, cwk, window=window, rotary_dim=r)
    else:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
        out = zg.global_prefill(cq, ck, cv, cwq, cwk, rotary_dim=r, lse=lse)
    dq, dk, dv, dg, _, _ = zg.prefill_backward(cq, ck, cv, cg, cwq, cwk, out, cdo,
                                               window=window, rotary_dim=r, lse=lse)
    torch.cuda.synchronize()
    rows, keys = _spread_rows(T, 48, seed + 7), _spread_rows(T, 48, seed + 8)
    say("backward sampled", (T, window), "oracle over every row (fp64)")
    ref = OG.prefill_grads_rows(host64(q), host64(k), host64(v),
                                None if g is None else host64(g), host64(wq), host64(wk),
                                host64(do), rows, keys, window=window, rotary_dim=r)
    got = dict(dq=(dq, rows), dk=(dk, keys), dv=(dv, keys))
    if window:
        got["dg"] = (dg, rows)
    for name, (t, at) in got.items():
        want = ref[name]
        err = float(np.max(np.abs(host64(t)[:, at] - want)))
        lim = REL * max(1.0, float(np.max(np.abs(want))))
        say("backward sampled", (T, window), name, f"err={err:.3e} lim={lim:.3e}")
        assert err <= lim, (name, err, lim)



def _random_cases(n=8, seed=880011):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        B = int(rng.choice([1, 2]))
        T = int(rng.integers(1, 701))
        window = None if i % 2 == 0 else int(rng.integers(1, 201))
        pos = int(rng.integers(0, 50_001))
        lse = bool(window is None and rng.integers(0, 2))
        cases.append((i, B, T, Hq, Hkv, d, window, pos, lse))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"case{c[0]}")
def test_backward_random_shapes(case):
    # seeded random batches, lengths (1 .. 700, ragged), head groups, head dims, windows,
    # position offsets and, for the global layer, with or without the forward's lse
    i, B, T, Hq, Hkv, d, window, pos, lse = case
    _check(B, T, Hq, Hkv, d, window, 2100 + 10 * i, pos_offset=pos, fwd_lse=lse)
