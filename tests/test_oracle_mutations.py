"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

A mutation that no pin detects would mean the oracle is only checked against itself.
"""

import numpy as np
import pytest

from oracle import attn as O
from tests import oracle_pins as P


def _rope_sign_flipped(x, pos, rotary_dim, base=10000.0):
    y = _ORIG["partial_rope"](x, pos, rotary_dim, base)
    h = rotary_dim // 2
    if h:
        # a - b*s  ->  a + b*s (a wrong sign in the rotation)
        x = np.asarray(x, dtype=np.float64)
        k = np.arange(h)
        ang = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * k / rotary_dim)
        y[..., :h] = x[..., :h] * np.cos(ang) + x[..., h:rotary_dim] * np.sin(ang)
    return y


def _rope_interleaved(x, pos, rotary_dim, base=10000.0):
    # pairs (2k, 2k+1) instead of (k, k + r/2)
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    h = rotary_dim // 2
    k = np.arange(h)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * k / rotary_dim)
    a, b = x[..., 0:rotary_dim:2], x[..., 1:rotary_dim:2]
    out[..., 0:rotary_dim:2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1:rotary_dim:2] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _rope_freq_over_d(x, pos, rotary_dim, base=10000.0):
    # frequency denominator d instead of rotary_dim: emulate with a larger effective r
    d = np.asarray(x).shape[-1]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    h = rotary_dim // 2
    k = np.arange(h)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * k / d)
    a, b = x[..., :h], x[..., h:rotary_dim]
    out[..., :h] = a * np.cos(ang) - b * np.sin(ang)
    out[..., h:rotary_dim] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _mask_off_by_one(q_pos, k_pos, window=None):
    qi = np.asarray(q_pos)[:, None]
    kj = np.asarray(k_pos)[None, :]
    m = kj <= qi
    if window is not None:
        m &= kj >= qi - window          # window of W + 1 tokens
    return m


def _mask_excludes_self(q_pos, k_pos, window=None):
    qi = np.asarray(q_pos)[:, None]
    kj = np.asarray(k_pos)[None, :]
    m = kj <= qi
    if window is not None:
        m &= kj > qi - window
    return m & ((kj < qi) | (qi == 0))


def _rmsnorm_no_weight(x, w, eps=1e-6):
    return _ORIG["rmsnorm"](x, np.ones_like(np.asarray(w, dtype=np.float64)), eps)


def _rmsnorm_no_sqrt(x, w, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, dtype=np.float64)


def _sigmoid_wrong(x):
    return np.asarray(x, dtype=np.float64)   # gate applied without the sigmoid


def _kv_bytes_no_factor2(n, h=8, d=128, by=2):
    return n * h * d * by                      # K only, V forgotten


def _layer_kinds_shifted(n=32, period=6):
    return ["global" if i % period == 0 else "swa" for i in range(n)]


def _varlen_boundary_shifted(q, k, v, g, wq, wk, cu_seqlens, **kw):
    # every interior document boundary one token late
    cu = [int(x) for x in cu_seqlens]
    moved = [cu[0]] + [min(c + 1, cu[-1]) for c in cu[1:-1]] + [cu[-1]]
    return _ORIG["prefill_varlen"](q, k, v, g, wq, wk, moved, **kw)


def _varlen_sees_previous_document(q, k, v, g, wq, wk, cu_seqlens, **kw):
    # each document also attends to the document before it
    cu = [int(x) for x in cu_seqlens]
    out = _ORIG["prefill_varlen"](q, k, v, g, wq, wk, cu_seqlens, **kw)
    if len(cu) > 2 and kw.get("rows") is None:
        merged = [cu[0]] + cu[2:]
        out2 = _ORIG["prefill_varlen"](q, k, v, g, wq, wk, merged, **kw)
        out[cu[1]:cu[2]] = out2[cu[1]:cu[2]]
    return out


def _block_keys_lo_off_by_one(ri, window):
    # a row block's key range starts one key late (its first visible key is dropped)
    return _ORIG["_block_keys"](ri, window)[1:]


from oracle import grad as OG

_ORIG_GRADS = OG.prefill_grads


def _grads_wk_forgotten(*a, **kw):
    r = _ORIG_GRADS(*a, **kw)
    r["dwk"] = np.zeros_like(r["dwk"])          # the norm weight of k left out
    return r


def _grads_dk_not_summed_over_group(*a, **kw):
    r = _ORIG_GRADS(*a, **kw)
    q = np.asarray(a[0])
    grp = q.shape[2] // r["dk"].shape[2]
    r["dk"] = r["dk"] / grp                     # one query head's share instead of the sum
    return r


def _softmax_vjp_without_d(p, dp, dsum):
    return p * dp                               # the row term D of the softmax Jacobian dropped


def _group_heads_first_only(kvh, grp):
    return range(kvh * grp, kvh * grp + 1)      # one query head of the group instead of all


_ORIG = {n: getattr(O, n) for n in ("partial_rope", "rmsnorm", "visible_mask", "sigmoid",
                                     "kv_bytes_per_token", "layer_kinds", "prefill_varlen",
                                     "_block_keys")}

MUTANTS = {
    "rope_sign": ("partial_rope", _rope_sign_flipped),
    "rope_interleaved": ("partial_rope", _rope_interleaved),
    "rope_freq_over_d": ("partial_rope", _rope_freq_over_d),
    "window_off_by_one": ("visible_mask", _mask_off_by_one),
    "window_excludes_self": ("visible_mask", _mask_excludes_self),
    "norm_drops_weight": ("rmsnorm", _rmsnorm_no_weight),
    "norm_no_sqrt": ("rmsnorm", _rmsnorm_no_sqrt),
    "gate_without_sigmoid": ("sigmoid", _sigmoid_wrong),
    "kv_bytes_k_only": ("kv_bytes_per_token", _kv_bytes_no_factor2),
    "schedule_shifted": ("layer_kinds", _layer_kinds_shifted),
    "varlen_boundary_shifted": ("prefill_varlen", _varlen_boundary_shifted),
    "grad_wk_forgotten": (OG, "prefill_grads", _grads_wk_forgotten),
    "grad_dk_one_head": (OG, "prefill_grads", _grads_dk_not_summed_over_group),
    "varlen_crosses_documents": ("prefill_varlen", _varlen_sees_previous_document),
    "row_block_lo_off_by_one": ("_block_keys", _block_keys_lo_off_by_one),
    "grad_rows_softmax_no_d": (OG, "_softmax_vjp", _softmax_vjp_without_d),
    "grad_rows_one_head": (OG, "_group_heads", _group_heads_first_only),
}

PINS = [getattr(P, n) for n in dir(P) if n.startswith("pin_")]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches(mutant, monkeypatch):
    spec = MUTANTS[mutant]
    mod, attr, fn = spec if len(spec) == 3 else (O, *spec)
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {mutant}"
