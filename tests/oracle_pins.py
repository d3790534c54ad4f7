"""Pin checks for the fp64 oracle, written against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with its anchor.
They look the oracle's functions up on the module at call time, so
``tests/test_oracle_mutations.py`` can plant a plausible mistake in the oracle and check
that at least one pin fails.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import attn as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------------------
# Independent pure-Python brute force (lists, math.exp/cos/sin, complex rotation).
# --------------------------------------------------------------------------------------

def _bf_norm(vec, w, eps):
    ms = sum(x * x for x in vec) / len(vec)
    inv = 1.0 / math.sqrt(ms + eps)
    return [x * inv * wi for x, wi in zip(vec, w)]


def _bf_rope(vec, p, r, base):
    out = list(vec)
    h = r // 2
    for k in range(h):
        theta = base ** (-2.0 * k / r)
        z = complex(vec[k], vec[k + h]) * complex(math.cos(p * theta), math.sin(p * theta))
        out[k], out[k + h] = z.real, z.imag
    return out


def brute_prefill(q, k, v, g, wq, wk, window, r, base=10000.0, eps=1e-6, pos_offset=0):
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    grp = Hq // Hkv
    sc = 1.0 / math.sqrt(d)
    out = np.zeros((B, T, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kv = h // grp
            for i in range(T):
                qi = _bf_rope(_bf_norm(list(q[b, i, h]), list(wq), eps), i + pos_offset, r, base)
                keys = [j for j in range(T) if j <= i and (window is None or j > i - window)]
                scores = []
                for j in keys:
                    kj = _bf_rope(_bf_norm(list(k[b, j, kv]), list(wk), eps), j + pos_offset, r, base)
                    scores.append(sc * sum(a * c for a, c in zip(qi, kj)))
                mx = max(scores)
                e = [math.exp(s - mx) for s in scores]
                tot = sum(e)
                for c in range(d):
                    acc = sum(e[n] / tot * v[b, j, kv, c] for n, j in enumerate(keys))
                    if g is not None:
                        acc *= 1.0 / (1.0 + math.exp(-g[b, i, h, c]))
                    out[b, i, h, c] = acc
    return out


# --------------------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------------------

def pin_worked_gate_example():
    """The review's window-4 example: the 4th token sees exactly 4 tokens including itself,
    and the gate multiplies the attention output elementwise."""
    gx = _golden("gate_worked_example.json")
    W, i = gx["window"], gx["query_index_0based"]
    A = np.array(gx["attention_output"])
    gate = np.array(gx["gate_sigmoid"])
    want = np.array(gx["gated_output_by_arithmetic"])
    T, d = len(gx["tokens"]), len(A)
    q = _rand((1, T, 1, d), 1)
    k = _rand((1, T, 1, d), 2)
    v = np.broadcast_to(A, (1, T, 1, d)).copy()      # every visible value row equals A
    g = np.broadcast_to(np.log(gate / (1.0 - gate)), (1, T, 1, d)).copy()
    w1 = np.ones(d)
    o = O.prefill(q, k, v, g, w1, w1, window=W, rotary_dim=0)
    assert np.allclose(o[0, i, 0], want, rtol=0, atol=1e-12), (o[0, i, 0], want)
    # count visible tokens with one-hot values over positions (d = T)
    d2 = 8
    T2 = 8
    q2 = _rand((1, T2, 1, d2), 3)
    k2 = _rand((1, T2, 1, d2), 4)
    v2 = np.eye(T2).reshape(1, T2, 1, d2)
    w2 = np.ones(d2)
    o2 = O.prefill(q2, k2, v2, None, w2, w2, window=W, rotary_dim=0)
    wts = o2[0, :, 0, :]                                   # row i = attention weights
    assert np.count_nonzero(wts[i] > 0) == gx["visible_tokens_including_self"]
    for row in range(T2):
        nz = np.nonzero(wts[row] > 0)[0].tolist()
        assert nz == list(range(max(0, row - W + 1), row + 1)), (row, nz)
        assert abs(wts[row].sum() - 1.0) < 1e-12


def pin_kv_footprint():
    gx = _golden("kv_footprint.json")
    H, d, by, T = gx["n_kv_heads"], gx["head_dim"], gx["bytes_per_elt"], gx["context_tokens"]
    full = O.kv_bytes_per_token(gx["full_attention"]["full_length_layers"], H, d, by)
    hyb = O.kv_bytes_per_token(gx["hybrid_swa_5to1"]["full_length_layers"], H, d, by)
    gdn = O.kv_bytes_per_token(gx["gdn_3to1_baseline"]["full_length_layers"], H, d, by)
    assert full == gx["full_attention"]["bytes_per_token"]
    assert hyb == gx["hybrid_swa_5to1"]["bytes_per_token"]
    assert full // 1024 == gx["full_attention"]["kib_per_token"]
    assert hyb // 1024 == gx["hybrid_swa_5to1"]["kib_per_token"]
    assert full * T / 2**30 == gx["full_attention"]["gib_at_context"]
    assert hyb * T / 2**30 == gx["hybrid_swa_5to1"]["gib_at_context"]
    assert gdn * T / 2**30 == gx["gdn_3to1_baseline"]["gib_at_context"]
    assert full / hyb == gx["reduction_full_over_hybrid"]


def pin_layer_schedule():
    gx = _golden("layer_schedule.json")
    kinds = O.layer_kinds(gx["n_layers"])
    glob = [i for i, kd in enumerate(kinds) if kd == "global"]
    assert [i + 1 for i in glob] == gx["global_layers_1based"]
    assert glob[-1] == gx["last_global_0based"]
    assert kinds.count("swa") == gx["n_swa"] and kinds.count("global") == gx["n_global"]
    assert all(kd == "swa" for kd in kinds[-gx["trailing_swa_layers"]:])
    for blk in range(5):
        assert kinds[6 * blk:6 * blk + 6] == ["swa"] * 5 + ["global"]


def pin_brute_force():
    """Oracle == independent pure-Python loops on tiny shapes (GQA, rope, window, gate)."""
    cases = [  # (B, T, Hq, Hkv, d, window, r, pos_offset)
        (1, 7, 2, 1, 8, 3, 2, 0),
        (2, 9, 4, 2, 8, None, 4, 0),
        (1, 10, 3, 3, 6, 4, 2, 5),
        (1, 6, 2, 2, 10, 128, 6, 0),
        (1, 12, 4, 1, 8, 1, 2, 3),
    ]
    for n, (B, T, Hq, Hkv, d, W, r, po) in enumerate(cases):
        q = _rand((B, T, Hq, d), 10 + n)
        k = _rand((B, T, Hkv, d), 20 + n)
        v = _rand((B, T, Hkv, d), 30 + n)
        g = _rand((B, T, Hq, d), 40 + n) if W is not None else None
        wq = 1 + 0.1 * _rand((d,), 50 + n)
        wk = 1 + 0.1 * _rand((d,), 60 + n)
        want = brute_prefill(q, k, v, g, wq, wk, W, r, pos_offset=po)
        got = O.prefill(q, k, v, g, wq, wk, window=W, rotary_dim=r, pos_offset=po)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (n, np.abs(got - want).max())


def pin_row_blocks_and_threads():
    """``prefill_rows`` as the long-context checks run it -- shuffled, sparse rows taken in
    blocks of 8 (so most blocks' key ranges start past position 0), four (batch, KV head)
    jobs on a 4-thread pool -- equals the pure-Python brute force, for a global layer and
    two windows."""
    B, T, Hq, Hkv, d, r, po = 2, 97, 4, 2, 8, 4, 3
    q = _rand((B, T, Hq, d), 70)
    k = _rand((B, T, Hkv, d), 71)
    v = _rand((B, T, Hkv, d), 72)
    g = _rand((B, T, Hq, d), 73)
    wq = 1 + 0.1 * _rand((d,), 74)
    wk = 1 + 0.1 * _rand((d,), 75)
    rng = np.random.default_rng(76)
    rows = rng.permutation(np.concatenate([[0, 1, T - 1],
                                           rng.choice(np.arange(2, T - 1), 50, replace=False)]))
    for W in (None, 5, 16):
        gg = None if W is None else g
        want = brute_prefill(q, k, v, gg, wq, wk, W, r, pos_offset=po)[:, rows]
        got = O.prefill_rows(q, k, v, gg, wq, wk, rows, window=W, rotary_dim=r, pos_offset=po,
                             row_block=8, threads=4)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (W, np.nanmax(np.abs(got - want)))


def pin_sdpa_rotary0():
    """rotary_dim 0: plain GQA attention on normed q/k == torch SDPA (fp64, explicit mask)."""
    import torch
    B, T, Hq, Hkv, d = 2, 37, 8, 2, 16
    q, k, v = _rand((B, T, Hq, d), 71), _rand((B, T, Hkv, d), 72), _rand((B, T, Hkv, d), 73)
    wq, wk = 1 + 0.1 * _rand((d,), 74), 1 + 0.1 * _rand((d,), 75)
    for W in (None, 5, 16):
        got = O.prefill(q, k, v, None, wq, wk, window=W, rotary_dim=0)
        qh = torch.from_numpy(O.rmsnorm(q, wq)).permute(0, 2, 1, 3)
        kh = torch.from_numpy(O.rmsnorm(k, wk)).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1)
        vh = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1)
        i = torch.arange(T)[:, None]
        j = torch.arange(T)[None, :]
        mask = j <= i
        if W is not None:
            mask &= j > i - W
        ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask)
        ref = ref.permute(0, 2, 1, 3).numpy()
        assert np.allclose(got, ref, rtol=0, atol=1e-12), (W, np.abs(got - ref).max())


def pin_rope_complex_and_invariants():
    d, r = 128, O.rotary_dim_for(128)
    assert r == 42 and O.rotary_dim_for(64) == 20
    x = _rand((5, 3, d), 81)
    pos = np.array([0, 1, 17, 4096, 262143])[:, None]
    y = O.partial_rope(x, pos, r)
    h = r // 2
    theta = 10000.0 ** (-2.0 * np.arange(h) / r)
    z = (x[..., :h] + 1j * x[..., h:r]) * np.exp(1j * pos[..., None] * theta)
    assert np.allclose(y[..., :h], z.real, atol=1e-9) and np.allclose(y[..., h:r], z.imag, atol=1e-9)
    assert np.array_equal(y[..., r:], x[..., r:])
    assert np.allclose(O.partial_rope(x, np.zeros((5, 3)), r), x, atol=0)   # position 0
    n0 = x[..., :h] ** 2 + x[..., h:r] ** 2
    n1 = y[..., :h] ** 2 + y[..., h:r] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)


def pin_relative_position():
    """Shifting every position by the same offset leaves attention unchanged."""
    B, T, Hq, Hkv, d = 1, 20, 2, 1, 16
    q, k, v = _rand((B, T, Hq, d), 91), _rand((B, T, Hkv, d), 92), _rand((B, T, Hkv, d), 93)
    w = np.ones(d)
    a = O.prefill(q, k, v, None, w, w, rotary_dim=6)
    b = O.prefill(q, k, v, None, w, w, rotary_dim=6, pos_offset=1234)
    assert np.allclose(a, b, atol=1e-9), np.abs(a - b).max()
    c = O.prefill(q, k, v, None, w, w, rotary_dim=0)
    assert not np.allclose(a, c, atol=1e-3)   # the rotation is not a no-op


def pin_rmsnorm():
    d = 16
    for c in (3.0, -0.25, 1e-2):
        x = np.full((d,), c)
        y = O.rmsnorm(x, np.ones(d), eps=1e-6)
        assert np.allclose(y, np.sign(c) * (1 + 1e-6 / c**2) ** -0.5, rtol=1e-14)
    x = _rand((4, d), 101)
    w = 1 + 0.1 * _rand((d,), 102)
    assert np.allclose(O.rmsnorm(7.5 * x, w, eps=0.0), O.rmsnorm(x, w, eps=0.0), rtol=1e-13)
    # per-head granularity: scaling one head of q leaves the attention output unchanged
    B, T, Hq, Hkv = 1, 9, 2, 1
    q, k, v = _rand((B, T, Hq, d), 103), _rand((B, T, Hkv, d), 104), _rand((B, T, Hkv, d), 105)
    q2 = q.copy()
    q2[:, :, 1] *= 9.0
    a = O.prefill(q, k, v, None, w, w, rotary_dim=4, eps=0.0)
    b = O.prefill(q2, k, v, None, w, w, rotary_dim=4, eps=0.0)
    assert np.allclose(a, b, atol=1e-12)


def pin_gate_limits_and_constants():
    B, T, Hq, Hkv, d, W = 1, 11, 4, 2, 8, 4
    q, k, v = _rand((B, T, Hq, d), 111), _rand((B, T, Hkv, d), 112), _rand((B, T, Hkv, d), 113)
    w = np.ones(d)
    ung = O.prefill(q, k, v, None, w, w, window=W, rotary_dim=2)
    for gval, fac in ((np.inf, 1.0), (0.0, 0.5), (-np.inf, 0.0)):
        g = np.full((B, T, Hq, d), gval)
        got = O.prefill(q, k, v, g, w, w, window=W, rotary_dim=2)
        assert np.array_equal(got, ung * fac), gval
    vc = np.full((B, T, Hkv, d), -1.75)
    got = O.prefill(q, k, vc, None, w, w, window=W, rotary_dim=2)
    assert np.allclose(got, -1.75, atol=1e-14)
    # row 0 sees only itself
    g = _rand((B, T, Hq, d), 114)
    got = O.prefill(q, k, v, g, w, w, window=W, rotary_dim=2)
    for h in range(Hq):
        assert np.allclose(got[0, 0, h], v[0, 0, h // 2] * O.sigmoid(g[0, 0, h]), atol=1e-14)


def pin_swa_wide_is_global():
    B, T, Hq, Hkv, d = 2, 25, 4, 2, 16
    q, k, v = _rand((B, T, Hq, d), 121), _rand((B, T, Hkv, d), 122), _rand((B, T, Hkv, d), 123)
    w = 1 + 0.1 * _rand((d,), 124)
    glob = O.prefill(q, k, v, None, w, w, rotary_dim=4)
    for W in (T, T + 1, 1000):
        sw = O.prefill(q, k, v, np.full((B, T, Hq, d), np.inf), w, w, window=W, rotary_dim=4)
        assert np.array_equal(sw, glob), W
    narrow = O.prefill(q, k, v, None, w, w, window=T - 1, rotary_dim=4)
    assert not np.allclose(narrow[:, -1], glob[:, -1])


def pin_decode_is_prefill_row():
    """Decode at step t over caches built from rows < t equals prefill row t."""
    B, T, Hq, Hkv, d, W = 2, 140, 4, 2, 16, 128
    r = 4
    q, k, v = _rand((B, T, Hq, d), 131), _rand((B, T, Hkv, d), 132), _rand((B, T, Hkv, d), 133)
    g = _rand((B, T, Hq, d), 134)
    wq, wk = 1 + 0.1 * _rand((d,), 135), 1 + 0.1 * _rand((d,), 136)
    pre_g = O.prefill(q, k, v, None, wq, wk, rotary_dim=r)
    pre_s = O.prefill(q, k, v, g, wq, wk, window=W, rotary_dim=r)
    kt = O.qknorm_rope(k, wk, np.arange(T)[None, :, None], r)          # [B,T,Hkv,d]
    for t in (0, 1, 5, 126, 127, 128, 129, 139):
        S = T
        kc = np.zeros((B, Hkv, S, d)); vc = np.zeros((B, Hkv, S, d))
        kc[:, :, :t] = kt[:, :t].transpose(0, 2, 1, 3)
        vc[:, :, :t] = v[:, :t].transpose(0, 2, 1, 3)
        kc[:, :, t:] = 1e3; vc[:, :, t:] = 1e3            # garbage beyond the prefix
        pos = np.full((B,), t)
        out, ktn = O.decode_global(q[:, t], k[:, t], v[:, t], wq, wk, kc, vc, pos, rotary_dim=r)
        assert np.allclose(out, pre_g[:, t], atol=1e-12), t
        assert np.allclose(ktn, kt[:, t], atol=1e-14)
        kr = np.full((B, Hkv, W, d), 1e3); vr = np.full((B, Hkv, W, d), 1e3)
        for p in range(max(0, t - W + 1), t):
            kr[:, :, p % W] = kt[:, p]
            vr[:, :, p % W] = v[:, p]
        out2, _ = O.decode_swa(q[:, t], k[:, t], v[:, t], g[:, t], wq, wk, kr, vr, pos,
                               window=W, rotary_dim=r)
        assert np.allclose(out2, pre_s[:, t], atol=1e-12), t


def pin_varlen_brute_force():
    """Packed documents == the independent pure-Python layer run on each document alone
    (positions restarting at pos_offset), for every packed row; documents of length 1,
    shorter and longer than the window."""
    lens = [1, 5, 9, 2, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d, r = int(cu[-1]), 4, 2, 8, 4
    q, k, v = _rand((T, Hq, d), 71), _rand((T, Hkv, d), 72), _rand((T, Hkv, d), 73)
    g = _rand((T, Hq, d), 74)
    wq, wk = 1 + 0.1 * _rand((d,), 75), 1 + 0.1 * _rand((d,), 76)
    for W, gg, po in ((None, None, 0), (3, g, 2)):
        got = O.prefill_varlen(q, k, v, gg, wq, wk, cu, window=W, rotary_dim=r, pos_offset=po)
        for i in range(len(lens)):
            s0, s1 = int(cu[i]), int(cu[i + 1])
            want = brute_prefill(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1],
                                 None if gg is None else gg[None, s0:s1], wq, wk, W, r,
                                 pos_offset=po)[0]
            assert np.allclose(got[s0:s1], want, rtol=0, atol=1e-12), (W, i)
    # a subset of rows in scrambled order gives the same rows
    rows = np.array([17, 0, 6, 23, 5, 15])
    sub = O.prefill_varlen(q, k, v, g, wq, wk, cu, rows=rows, window=3, rotary_dim=r)
    full = O.prefill_varlen(q, k, v, g, wq, wk, cu, window=3, rotary_dim=r)
    assert np.allclose(sub, full[rows], rtol=0, atol=1e-13)


def pin_varlen_equal_documents_are_a_batch():
    """n equal-length packed documents == the batched layer with B = n."""
    n, L, Hq, Hkv, d, r = 3, 11, 4, 1, 8, 4
    q, k, v = _rand((n, L, Hq, d), 81), _rand((n, L, Hkv, d), 82), _rand((n, L, Hkv, d), 83)
    wq, wk = 1 + 0.1 * _rand((d,), 84), 1 + 0.1 * _rand((d,), 85)
    cu = np.arange(n + 1) * L
    got = O.prefill_varlen(q.reshape(n * L, Hq, d), k.reshape(n * L, Hkv, d),
                           v.reshape(n * L, Hkv, d), None, wq, wk, cu, rotary_dim=r)
    want = O.prefill(q, k, v, None, wq, wk, rotary_dim=r).reshape(n * L, Hq, d)
    assert np.allclose(got, want, rtol=0, atol=1e-13)


def pin_varlen_isolation():
    """No key of another document contributes: one-hot V per packed token puts weight only
    on the row's own document (exactly min(i - start + 1, W) nonzero weights), and
    changing the other documents' tokens leaves a document's rows unchanged."""
    lens = [4, 6, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, d = int(cu[-1]), 16
    q, k = _rand((T, 1, d), 91), _rand((T, 1, d), 92)
    v = np.zeros((T, 1, d))
    v[np.arange(T), 0, np.arange(T)] = 1.0           # token t carries unit vector e_t
    w = np.ones(d)
    for W in (None, 2):
        out = O.prefill_varlen(q, k, v, None, w, w, cu, window=W, rotary_dim=4)[:, 0]
        for i in range(len(lens)):
            s0, s1 = int(cu[i]), int(cu[i + 1])
            for t in range(s0, s1):
                nz = np.nonzero(out[t, :T] > 0)[0]
                lo = s0 if W is None else max(s0, t - W + 1)
                assert list(nz) == list(range(lo, t + 1)), (W, t, nz)
    k2, v2 = k.copy(), v.copy()
    k2[:4] = _rand((4, 1, d), 93)
    v2[4:] *= 1.0
    v2[:4] = _rand((4, 1, d), 94)
    a = O.prefill_varlen(q, k, v, None, w, w, cu, rotary_dim=4)
    b = O.prefill_varlen(q, k2, v2, None, w, w, cu, rotary_dim=4)
    assert np.array_equal(a[4:], b[4:]) and not np.array_equal(a[:4], b[:4])


def pin_grad_forward_is_the_layer():
    """The differentiable restatement of the layer equals the oracle's forward, and its
    log-sum-exp equals the brute-force sum over each row's visible scores."""
    from oracle import grad as OG
    import torch
    B, T, Hq, Hkv, d, r = 2, 9, 4, 2, 8, 4
    q, k, v = _rand((B, T, Hq, d), 101), _rand((B, T, Hkv, d), 102), _rand((B, T, Hkv, d), 103)
    g = _rand((B, T, Hq, d), 104)
    wq, wk = 1 + 0.1 * _rand((d,), 105), 1 + 0.1 * _rand((d,), 106)
    for W, gg in ((None, None), (3, g)):
        want = O.prefill(q, k, v, gg, wq, wk, window=W, rotary_dim=r, pos_offset=7)
        out, lse = OG.layer_torch(*(torch.as_tensor(x) for x in (q, k, v)),
                                  None if gg is None else torch.as_tensor(gg),
                                  torch.as_tensor(wq), torch.as_tensor(wk), window=W,
                                  rotary_dim=r, pos_offset=7)
        assert np.allclose(out.numpy(), want, rtol=0, atol=1e-12), W
        qt = O.qknorm_rope(q, wq, 7 + np.arange(T)[None, :, None], r)
        kt = O.qknorm_rope(k, wk, 7 + np.arange(T)[None, :, None], r)
        for b in range(B):
            for h in range(Hq):
                for i in range(T):
                    js = [j for j in range(T) if j <= i and (W is None or j > i - W)]
                    s = [float(qt[b, i, h] @ kt[b, j, h // 2]) / math.sqrt(d) for j in js]
                    ref = math.log(sum(math.exp(x) for x in s))
                    assert abs(lse.numpy()[b, h, i] - ref) < 1e-12


def pin_grad_finite_differences():
    """Every gradient (q, k, v, g, w_q, w_k) equals central differences of the forward
    sum(dout * out) at sampled coordinates, for a gated window layer and a global layer."""
    from oracle import grad as OG
    B, T, Hq, Hkv, d, r = 1, 7, 4, 2, 8, 4
    q, k, v = _rand((B, T, Hq, d), 111), _rand((B, T, Hkv, d), 112), _rand((B, T, Hkv, d), 113)
    g, dout = _rand((B, T, Hq, d), 114), _rand((B, T, Hq, d), 115)
    wq, wk = 1 + 0.1 * _rand((d,), 116), 1 + 0.1 * _rand((d,), 117)
    rng = np.random.default_rng(118)
    h = 1e-5
    for W, gg in ((3, g), (None, None)):
        args = dict(q=q, k=k, v=v, g=gg, wq=wq, wk=wk)
        gr = OG.prefill_grads(q, k, v, gg, wq, wk, dout, window=W, rotary_dim=r, pos_offset=3)

        def loss(**kw):
            a = dict(args)
            a.update(kw)
            o = O.prefill(a["q"], a["k"], a["v"], a["g"], a["wq"], a["wk"], window=W,
                          rotary_dim=r, pos_offset=3)
            return float(np.sum(o * dout))

        for name in ("q", "k", "v", "g", "wq", "wk"):
            if args[name] is None:
                assert gr["dg"] is None
                continue
            x = args[name]
            for _ in range(6):
                idx = tuple(int(rng.integers(0, n)) for n in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                fd = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
                an = gr["d" + name][idx]
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (W, name, idx, fd, an)


def pin_grad_rows_match_autograd():
    """The closed-form gradients at sampled positions (prefill_grads_rows, used where the
    autograd graph does not fit) equal autograd's at those positions: a gated window layer
    and a global layer, GQA, row blocks smaller than the sequence, non-default scale and
    RoPE base."""
    from oracle import grad as OG
    B, T, Hq, Hkv, d, r = 2, 23, 4, 2, 8, 4
    q, k, v = _rand((B, T, Hq, d), 121), _rand((B, T, Hkv, d), 122), _rand((B, T, Hkv, d), 123)
    g, dout = _rand((B, T, Hq, d), 124), _rand((B, T, Hq, d), 125)
    wq, wk = 1 + 0.1 * _rand((d,), 126), 1 + 0.1 * _rand((d,), 127)
    rows, keys = [0, 1, 5, 13, 22], [0, 3, 7, 21, 22]
    for W, gg, sc, base in ((None, None, None, 10000.0), (5, g, 0.3, 1e7)):
        kw = dict(window=W, rotary_dim=r, pos_offset=3, scale=sc, rope_base=base)
        full = OG.prefill_grads(q, k, v, gg, wq, wk, dout, **kw)
        part = OG.prefill_grads_rows(q, k, v, gg, wq, wk, dout, rows, keys, block=7, **kw)
        for name, at in (("dq", rows), ("dg", rows), ("dk", keys), ("dv", keys)):
            if full[name] is None:
                assert part[name] is None
                continue
            err = np.max(np.abs(np.take(full[name], at, axis=1) - part[name]))
            assert err < 1e-10, (W, name, err)
        assert np.max(np.abs(full["lse"] - part["lse"])) < 1e-10

