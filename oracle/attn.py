"""fp64 NumPy oracle: the plain definition of the hybrid attention layer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never imports it.

Everything is computed in float64 from the exact input values (bf16 and fp32 inputs are
exactly representable in float64). There is no tiling, no online softmax and no rounding:
score rows are materialised, masked, max-subtracted, exponentiated and normalised. Long
inputs are only chunked over query rows (and over heads) so that memory stays bounded.

What each function follows, and how it is pinned (tests in ``tests/test_oracle_*.py``):

* ``rmsnorm`` -- QK normalisation by RMSNorm, applied to the q and k branches
  ("ZGCM-1-7B 完全解説" explainer, section アーキテクチャ; hyper.ai summary, section 方法).
  Pinned: closed form for a constant vector, scale invariance, brute-force loops.
  Granularity (per head over d, one [d] weight per branch) and eps are readings the pages
  leave open: *parity unpinned* by the pages for those two conventions.
* ``partial_rope`` -- partial RoPE with rotary ratio 0.33 (same two sections; also the
  jaehun.me review, section "1) 구조·시스템 공동 설계"). Pinned: independent complex-number
  form, identity at position 0, relative-position invariance of attention, pair norms.
  Which dims rotate, the pairing (k, k + r/2) and the frequency denominator are readings:
  *parity unpinned* by the pages for those conventions.
* ``visible_mask`` -- sliding window of the most recent W tokens, self included (explainer,
  section アーキテクチャ; jaehun.me review, section "게이트형 SWA의 동작", whose worked example
  with window 4 has the 4th token see 4 tokens including itself). Pinned: that example,
  one-hot brute force.
* ``prefill`` / ``prefill_rows`` -- causal GQA softmax attention, then the elementwise
  sigmoid gate for SWA layers (GatedSWA equation, hyper.ai summary section 方法; explainer
  section アーキテクチャ). Pinned: the worked gate example, pure-Python brute force,
  torch SDPA in fp64 for rotary_dim 0, gate limits, SWA(W >= T) == global, V == c.
  The softmax scale 1/sqrt(d) is the textbook reading (*parity unpinned* by the pages).
* ``prefill_varlen`` -- packed documents, each its own sequence (explainer, section 事後訓練:
  the 256K fine-tuning variant trains on packed tokens). Pinned: equal-length documents ==
  the batched layer, one-hot brute force of the document boundary, independence from the
  other documents' contents. No attention across documents is a reading (*parity
  unpinned* by the pages); restarting positions per document is one too, but with the
  masking in place it cannot change the outputs (RoPE attention depends on position
  differences only, pinned by the relative-position pin), only the rounding of angles.
* ``decode_global`` / ``decode_swa`` -- one new token against a full cache or a 128-entry
  ring (explainer, section アーキテクチャ: SWA layers keep a fixed 128 tokens, global layers
  the whole sequence). Pinned: decode at step t == prefill row t, ring-rotation invariance,
  row 0 == v_0.
* ``kv_bytes_per_token`` / ``layer_kinds`` -- the KV-byte arithmetic and the layer schedule
  (jaehun.me review, section "KV 캐시가 6.4배 줄어드는 이유"; explainer section アーキテクチャ).
  Pinned: the numbers the pages print (tests/golden/kv_footprint.json, layer_schedule.json).
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F64 = np.float64


def rotary_dim_for(head_dim: int, ratio: float = 0.33) -> int:
    """Number of rotated dims: the largest even count not above ratio * head_dim."""
    return 2 * int(math.floor(ratio * head_dim / 2.0))


def rmsnorm(x, w, eps: float = 1e-6):
    """x / sqrt(mean(x^2) + eps) * w over the last axis (one head's d dims)."""
    x = np.asarray(x, dtype=F64)
    w = np.asarray(w, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def partial_rope(x, pos, rotary_dim: int, base: float = 10000.0):
    """Rotate the leading ``rotary_dim`` dims of x in pairs (k, k + rotary_dim/2).

    ``pos`` broadcasts against ``x.shape[:-1]``. Pair k turns by pos * base**(-2k/rotary_dim);
    dims [rotary_dim, d) pass through unchanged.
    """
    x = np.asarray(x, dtype=F64)
    if rotary_dim == 0:
        return x.copy()
    half = rotary_dim // 2
    k = np.arange(half, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * k / rotary_dim)
    ang = np.asarray(pos, dtype=F64)[..., None] * inv_freq  # (..., half)
    c, s = np.cos(ang), np.sin(ang)
    out = x.copy()
    a = x[..., :half]
    b = x[..., half:rotary_dim]
    out[..., :half] = a * c - b * s
    out[..., half:rotary_dim] = b * c + a * s
    return out


def qknorm_rope(x, w, pos, rotary_dim: int, base: float = 10000.0, eps: float = 1e-6):
    """RMSNorm then partial RoPE: the transform applied to the q and k branches."""
    return partial_rope(rmsnorm(x, w, eps), pos, rotary_dim, base)


def sigmoid(x):
    """1 / (1 + exp(-x)); exactly 1 at +inf and 0 at -inf."""
    x = np.asarray(x, dtype=F64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def visible_mask(q_pos, k_pos, window=None):
    """Boolean [len(q_pos), len(k_pos)]: key j visible to query i iff i - W < j <= i."""
    qi = np.asarray(q_pos)[:, None]
    kj = np.asarray(k_pos)[None, :]
    m = kj <= qi
    if window is not None:
        m &= kj > qi - window
    return m


def _softmax_rows(s, mask):
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def prefill(q, k, v, g, wq, wk, *, window=None, rotary_dim=None, rope_base=10000.0,
            eps=1e-6, scale=None, pos_offset=0):
    """Whole-sequence layer output, float64 [B, T, Hq, d].

    q, g: [B, T, Hq, d]; k, v: [B, T, Hkv, d]; wq, wk: [d]. ``window`` None = global
    (ungated when g is None); an int = sliding window of that many tokens, self included.
    Query head h reads KV head h // (Hq // Hkv).
    """
    q = np.asarray(q, dtype=F64)
    B, T, Hq, d = q.shape
    rows = np.arange(T)
    return prefill_rows(q, k, v, g, wq, wk, rows, window=window, rotary_dim=rotary_dim,
                        rope_base=rope_base, eps=eps, scale=scale, pos_offset=pos_offset)


def _block_keys(ri, window):
    """Key positions a block of query rows ``ri`` can see: 0 .. max(ri) for a global layer
    (returned as that contiguous range), the union of the rows' windows
    ``max(0, i - W + 1) .. i`` for a sliding-window layer (so a windowed block touches, and
    normalises and rotates, only keys that some row of it sees)."""
    hi = int(np.max(ri)) + 1
    if window is None:
        return np.arange(hi)
    lo = np.maximum(np.asarray(ri) - window + 1, 0)
    return np.unique(np.concatenate([np.arange(a, r + 1) for a, r in zip(lo, ri)]))


def prefill_rows(q, k, v, g, wq, wk, rows, *, window=None, rotary_dim=None,
                 rope_base=10000.0, eps=1e-6, scale=None, pos_offset=0,
                 row_block=256, threads=1):
    """Layer output for the query rows ``rows`` only: float64 [B, len(rows), Hq, d].

    Same definition as ``prefill``. Rows are taken in blocks (in sorted order) of at most
    ``row_block``; a block scores only the keys ``_block_keys`` gives (every key visible
    to one of its rows; the mask removes the rest). A global layer's keys are normalised
    and rotated once per KV head, a windowed layer's per block, for that block's keys
    only. ``threads`` > 1 runs the (batch, KV head) pairs on a thread pool. ``q``/``g``
    may be given either full [B, T, Hq, d] or already restricted to ``rows``
    ([B, len(rows), Hq, d]); k and v are always full length.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    B, T, Hkv, d = k.shape
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(q)
    if q.shape[1] == len(rows) and q.shape[1] != T:
        q_rows = q
        g_rows = None if g is None else np.asarray(g)
    else:
        q_rows = q[:, rows]
        g_rows = None if g is None else np.asarray(g)[:, rows]
    Hq = q_rows.shape[2]
    grp = Hq // Hkv
    r = rotary_dim_for(d) if rotary_dim is None else rotary_dim
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((B, len(rows), Hq, d), dtype=F64)
    if len(rows) == 0:
        return out
    qpos = pos_offset + rows
    qt = qknorm_rope(q_rows, wq, qpos[None, :, None], r, rope_base, eps)  # [B,R,Hq,d]
    order = np.argsort(rows, kind="stable")

    def keys_of(b, kv, keys, kt_all, v_all):
        if kt_all is not None:      # global: a contiguous range of the transformed keys
            lo, hi = int(keys[0]), int(keys[-1]) + 1
            return kt_all[lo:hi], v_all[lo:hi]
        kt = qknorm_rope(np.asarray(k[b, keys, kv], dtype=F64), wk, pos_offset + keys, r,
                         rope_base, eps)
        return kt, np.asarray(v[b, keys, kv], dtype=F64)

    def one(b, kv):
        kt_all = v_all = None
        if window is None:
            kmax = int(rows.max()) + 1
            kt_all = qknorm_rope(np.asarray(k[b, :kmax, kv], dtype=F64), wk,
                                 pos_offset + np.arange(kmax), r, rope_base, eps)
            v_all = np.asarray(v[b, :kmax, kv], dtype=F64)
        for start in range(0, len(order), row_block):
            idx = order[start:start + row_block]
            ri = rows[idx]
            keys = _block_keys(ri, window)
            kt, vv = keys_of(b, kv, keys, kt_all, v_all)
            mask = visible_mask(ri, keys, window)
            for h in range(kv * grp, (kv + 1) * grp):
                s = sc * (qt[b, idx, h] @ kt.T)
                p = _softmax_rows(s, mask)
                out[b, idx, h] = p @ vv

    jobs = [(b, kv) for b in range(B) for kv in range(Hkv)]
    if threads > 1:
        # one BLAS thread per worker: the workers already cover the cores
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda a: one(*a), jobs))
    else:
        for a in jobs:
            one(*a)
    if g_rows is not None:
        out *= sigmoid(g_rows)
    return out


def _decode_one(q, k_new, v_new, wq, wk, k_cache, v_cache, pos, slots, *, rotary_dim,
                rope_base, eps, scale):
    """Shared single-sequence step: norm+RoPE q and k_new at ``pos``, write the new
    entry at cache index ``slots[-1]`` and attend over cache indices ``slots``."""
    Hq, d = q.shape
    Hkv = k_new.shape[0]
    grp = Hq // Hkv
    qt = qknorm_rope(q, wq, pos, rotary_dim, rope_base, eps)
    kt = qknorm_rope(k_new, wk, pos, rotary_dim, rope_base, eps)
    out = np.zeros((Hq, d), dtype=F64)
    for kv in range(Hkv):
        kc = np.array(k_cache[kv], dtype=F64, copy=True)
        vc = np.array(v_cache[kv], dtype=F64, copy=True)
        kc[slots[-1]] = kt[kv]
        vc[slots[-1]] = np.asarray(v_new[kv], dtype=F64)
        ks, vs = kc[slots], vc[slots]
        for h in range(kv * grp, (kv + 1) * grp):
            s = scale * (ks @ qt[h])
            p = np.exp(s - s.max())
            out[h] = (p / p.sum()) @ vs
    return out, kt


def prefill_varlen(q, k, v, g, wq, wk, cu_seqlens, *, rows=None, window=None,
                   rotary_dim=None, rope_base=10000.0, eps=1e-6, scale=None, pos_offset=0,
                   threads=1):
    """Packed documents: q, g [T, Hq, d]; k, v [T, Hkv, d]; cu_seqlens [n_docs + 1].

    Document i (tokens cu[i] .. cu[i+1]-1) is its own sequence: the layer of ``prefill``
    with positions pos_offset, pos_offset + 1, .. from its first token, and no key of
    another document visible (the pages say only that the 256K fine-tuning trains on
    packed tokens, explainer section 事後訓練; blocking attention across documents and
    restarting positions are the reading adopted). Returns float64 [len(rows), Hq, d] for
    the packed rows ``rows`` (all rows when None).
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    T = q.shape[0]
    cu = [int(x) for x in cu_seqlens]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), q.shape[1], q.shape[2]), dtype=F64)
    for i in range(len(cu) - 1):
        s0, s1 = cu[i], cu[i + 1]
        sel = np.nonzero((rows >= s0) & (rows < s1))[0]
        if len(sel) == 0:
            continue
        local = rows[sel] - s0
        gd = None if g is None else np.asarray(g)[None, s0:s1]
        out[sel] = prefill_rows(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], gd, wq, wk,
                                local, window=window, rotary_dim=rotary_dim,
                                rope_base=rope_base, eps=eps, scale=scale,
                                pos_offset=pos_offset, threads=threads)[0]
    return out


def decode_global(q, k_new, v_new, wq, wk, k_cache, v_cache, pos, *, rotary_dim=None,
                  rope_base=10000.0, eps=1e-6, scale=None):
    """One decode step of an ungated global layer for every sequence.

    q: [B, Hq, d]; k_new, v_new: [B, Hkv, d] (raw, before norm/RoPE); caches
    [B, Hkv, S, d] holding post-norm, post-RoPE K and raw V for positions < pos[b].
    The new token sits at absolute position pos[b] and cache index pos[b]; the query sees
    cache indices 0..pos[b]. Returns (out [B, Hq, d] float64, k_tilde_new [B, Hkv, d]).
    The caches are not modified.
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    r = rotary_dim_for(d) if rotary_dim is None else rotary_dim
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((B, Hq, d), dtype=F64)
    ktn = np.zeros((B, k_new.shape[1], d), dtype=F64)
    for b in range(B):
        p = int(pos[b])
        slots = np.arange(p + 1)
        out[b], ktn[b] = _decode_one(q[b], k_new[b], v_new[b], wq, wk, k_cache[b], v_cache[b],
                                     p, slots, rotary_dim=r, rope_base=rope_base, eps=eps,
                                     scale=sc)
    return out, ktn


def decode_swa(q, k_new, v_new, g, wq, wk, k_ring, v_ring, pos, *, window=128,
               rotary_dim=None, rope_base=10000.0, eps=1e-6, scale=None):
    """One decode step of a gated SWA layer over a ring of ``window`` entries.

    Position p lives in ring slot p % window. The new token (position pos[b]) is written
    to its slot; the query sees positions max(0, pos-window+1) .. pos, i.e. the slots of
    those positions. Output is gated by sigmoid(g). Returns (out, k_tilde_new).
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    r = rotary_dim_for(d) if rotary_dim is None else rotary_dim
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((B, Hq, d), dtype=F64)
    ktn = np.zeros((B, k_new.shape[1], d), dtype=F64)
    for b in range(B):
        p = int(pos[b])
        positions = np.arange(max(0, p - window + 1), p + 1)
        slots = positions % window
        out[b], ktn[b] = _decode_one(q[b], k_new[b], v_new[b], wq, wk, k_ring[b], v_ring[b],
                                     p, slots, rotary_dim=r, rope_base=rope_base, eps=eps,
                                     scale=sc)
    return out * sigmoid(g), ktn


def layer_kinds(n_layers: int = 32, period: int = 6):
    """Attention kind per 0-based layer: every ``period``-th layer (1-based) is global."""
    return ["global" if (i + 1) % period == 0 else "swa" for i in range(n_layers)]


def kv_bytes_per_token(n_full_layers: int, n_kv_heads: int = 8, head_dim: int = 128,
                       bytes_per_elt: int = 2) -> int:
    """K and V bytes one token adds to the layers that keep the whole sequence."""
    return 2 * n_full_layers * n_kv_heads * head_dim * bytes_per_elt
