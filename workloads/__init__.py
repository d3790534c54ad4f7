"""Seeded synthetic workloads: the five configurations and their input generators.

This module holds shapes, seeds and random-number draws only -- none of the layer's
arithmetic. It is the one piece shared by the tests, the benchmark and the oracle side:
the same seeded tensors feed both the HIP library and the fp64 oracle.

No public dataset is involved. The pages measure attention throughput on training runs
over their own corpus; seeded N(0, 1) tensors at the model's shapes (H_kv = 8,
d_head = 128 from the per-token KV-byte arithmetic in the jaehun.me review, section
"KV 캐시가 6.4배 줄어드는 이유"; Hq = 32 as in the workload table) stand in for it.

Seeds: ``seed = 1000 * config + 10 * layer + slot`` with slot Q=0, K=1, V=2, G=3, w_q=4,
w_k=5, k_new=6, v_new=7, pos=8, K cache=1, V cache=2 (decode configs use their own
config number, so streams never collide across configs).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SLOT = {"q": 0, "k": 1, "v": 2, "g": 3, "wq": 4, "wk": 5, "k_new": 6, "v_new": 7, "pos": 8}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config: int
    kind: str              # "swa", "global", "pair", "stack", "decode"
    dtype: str             # "f32" or "bf16"
    B: int
    T: int                 # sequence length (prefill) or cache context (decode)
    Hq: int
    Hkv: int
    d: int
    window: int = 128
    rotary_dim: int = 0
    g_std: float = 1.0
    n_layers: int = 1


def _rdim(d: int) -> int:
    return 2 * int(math.floor(0.33 * d / 2.0))


C1 = Workload("c1_swa_f32_T512", 1, "swa", "f32", 1, 512, 4, 1, 64, 128, _rdim(64))
C2 = Workload("c2_pair_bf16_B4_T4096", 2, "pair", "bf16", 4, 4096, 32, 8, 128, 128, _rdim(128),
              g_std=math.sqrt(2.0))
C3 = Workload("c3_stack32_bf16_T65536", 3, "stack", "bf16", 1, 65536, 32, 8, 128, 128,
              _rdim(128), n_layers=32)
C4 = Workload("c4_pair_bf16_T262144", 4, "pair", "bf16", 1, 262144, 32, 8, 128, 128,
              _rdim(128))
C5 = Workload("c5_decode_bf16_B32_ctx262144", 5, "decode", "bf16", 32, 262144, 32, 8, 128, 128,
              _rdim(128))
CONFIGS = {1: C1, 2: C2, 3: C3, 4: C4, 5: C5}

# Attention stacks of the 32-layer backbone compared in the stack sweep: the model's
# hybrid (every sixth layer global: 27 gated SWA + 5 global), the SWA 3:1 alternative
# (every fourth layer global: 24 + 8) and the full-attention baseline (32 global).
STACKS = {"hybrid_5to1": 6, "swa_3to1": 4, "full": 1}


def stack_kinds(period: int, n_layers: int = 32):
    """Per-layer kind ("swa" / "global") of a stack whose every ``period``-th layer
    (counting from 1) is global; period 1 makes every layer global."""
    return ["global" if (i + 1) % period == 0 else "swa" for i in range(n_layers)]


def seed_for(config: int, layer: int, slot: str) -> int:
    return 1000 * config + 10 * layer + SLOT[slot]


def host_normal(shape, seed: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 N(mean, std^2) from numpy's PCG64 stream ``seed``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def norm_weight(d: int, seed: int) -> np.ndarray:
    """RMSNorm weight ~ 1 + 0.1 * N(0, 1), float32 [d]."""
    return (1.0 + 0.1 * host_normal((d,), seed)).astype(np.float32)


def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def host_tensor(shape, seed: int, dtype: str, std: float = 1.0):
    """Seeded host draw rounded to ``dtype`` (bf16 by round-to-nearest-even) as a torch
    CPU tensor."""
    import torch
    return torch.from_numpy(host_normal(shape, seed, std)).to(torch_dtype(dtype))


def device_tensor(shape, seed: int, dtype: str, device="cuda", std: float = 1.0,
                  chunk_dim0: bool = False):
    """Seeded draw made on the device with torch's Philox generator, then rounded to
    ``dtype``. With ``chunk_dim0`` each index of the leading dim gets its own stream
    (seed * 4099 + i), which bounds the float32 staging memory for very large tensors."""
    import torch
    td = torch_dtype(dtype)
    out = torch.empty(tuple(shape), dtype=td, device=device)
    if chunk_dim0:
        for i in range(shape[0]):
            gen = torch.Generator(device=device)
            gen.manual_seed(seed * 4099 + i)
            tmp = torch.randn(tuple(shape[1:]), generator=gen, device=device,
                              dtype=torch.float32)
            if std != 1.0:
                tmp.mul_(std)
            out[i].copy_(tmp)
            del tmp
    else:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        tmp = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        out.copy_(tmp)
    return out


def prefill_inputs(w: Workload, layer: int = 0, *, device: Optional[str] = None,
                   T: Optional[int] = None, B: Optional[int] = None, gated: bool = True):
    """Seeded Q, K, V, G (G None when not gated) and fp32 norm weights for one layer.

    ``device`` None draws on the host (numpy PCG64); otherwise on that device (Philox).
    ``T``/``B`` override the workload's sizes (for reduced parity cases).
    """
    import torch
    T = w.T if T is None else T
    B = w.B if B is None else B
    qs, ks = (B, T, w.Hq, w.d), (B, T, w.Hkv, w.d)
    c = w.config
    if device is None:
        q = host_tensor(qs, seed_for(c, layer, "q"), w.dtype)
        k = host_tensor(ks, seed_for(c, layer, "k"), w.dtype)
        v = host_tensor(ks, seed_for(c, layer, "v"), w.dtype)
        g = host_tensor(qs, seed_for(c, layer, "g"), w.dtype, w.g_std) if gated else None
    else:
        q = device_tensor(qs, seed_for(c, layer, "q"), w.dtype, device)
        k = device_tensor(ks, seed_for(c, layer, "k"), w.dtype, device)
        v = device_tensor(ks, seed_for(c, layer, "v"), w.dtype, device)
        g = (device_tensor(qs, seed_for(c, layer, "g"), w.dtype, device, w.g_std)
             if gated else None)
    wq = torch.from_numpy(norm_weight(w.d, seed_for(c, layer, "wq")))
    wk = torch.from_numpy(norm_weight(w.d, seed_for(c, layer, "wk")))
    if device is not None:
        wq, wk = wq.to(device), wk.to(device)
    return q, k, v, g, wq, wk


def decode_inputs(w: Workload, *, device: Optional[str] = None, B: Optional[int] = None,
                  S: Optional[int] = None, layer: int = 0, kind: str = "both"):
    """Seeded decode-step inputs: q, g [B,Hq,d]; k_new, v_new [B,Hkv,d]; norm weights;
    global caches [B,Hkv,S,d]; SWA rings [B,Hkv,window,d]. Caches hold N(0,1) values that
    stand for already-normalised/rotated K and raw V. ``kind`` "swa" skips the global
    caches and "global" the rings (None in their place)."""
    import torch
    B = w.B if B is None else B
    S = w.T if S is None else S
    c = w.config
    qs, ns = (B, w.Hq, w.d), (B, w.Hkv, w.d)
    cs, rs = (B, w.Hkv, S, w.d), (B, w.Hkv, w.window, w.d)
    if device is None:
        mk = lambda shape, slot, lay=layer, std=1.0: host_tensor(shape, seed_for(c, lay, slot),
                                                                  w.dtype, std)
        q, g = mk(qs, "q"), mk(qs, "g")
        kn, vn = mk(ns, "k_new"), mk(ns, "v_new")
        kc, vc = (mk(cs, "k", 1), mk(cs, "v", 1)) if kind != "swa" else (None, None)
        kr, vr = (mk(rs, "k", 2), mk(rs, "v", 2)) if kind != "global" else (None, None)
    else:
        mk = lambda shape, slot, lay=layer, big=False: device_tensor(
            shape, seed_for(c, lay, slot), w.dtype, device, chunk_dim0=big)
        q, g = mk(qs, "q"), mk(qs, "g")
        kn, vn = mk(ns, "k_new"), mk(ns, "v_new")
        kc, vc = (mk(cs, "k", 1, True), mk(cs, "v", 1, True)) if kind != "swa" else (None, None)
        kr, vr = (mk(rs, "k", 2), mk(rs, "v", 2)) if kind != "global" else (None, None)
    wq = torch.from_numpy(norm_weight(w.d, seed_for(c, layer, "wq")))
    wk = torch.from_numpy(norm_weight(w.d, seed_for(c, layer, "wk")))
    if device is not None:
        wq, wk = wq.to(device), wk.to(device)
    return dict(q=q, g=g, k_new=kn, v_new=vn, wq=wq, wk=wk, k_cache=kc, v_cache=vc,
                k_ring=kr, v_ring=vr)


def stratified_rows(T: int, n: int, seed: int, window: int = 128) -> np.ndarray:
    """Sorted unique query rows for sampled checks: rows 0..15, the window edges
    (W-2 .. W+1), tile boundaries (multiples of 64 and 128, +-1) and T-1, topped up with
    uniform draws to ``n`` rows (all rows when T <= n)."""
    if T <= n:
        return np.arange(T)
    fixed = set(range(min(16, T)))
    fixed.update(x for x in (window - 2, window - 1, window, window + 1, T - 1, T - 2) if 0 <= x < T)
    rng = np.random.default_rng(seed)
    for m in rng.choice(np.arange(64, T, 64), size=min(64, (T - 1) // 64), replace=False):
        fixed.update(x for x in (m - 1, m, m + 1) if 0 <= x < T)
    rows = np.array(sorted(fixed), dtype=np.int64)
    if len(rows) >= n:
        return rows[:n]
    pool = np.setdiff1d(np.arange(T), rows)
    extra = rng.choice(pool, size=n - len(rows), replace=False)
    return np.sort(np.concatenate([rows, extra]))
