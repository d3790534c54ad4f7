"""Backward pass of the layer in fp64: gradients of the plain definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never imports it.

The layer (GatedSWA equation, hyper.ai summary of arXiv 2609.13356, section 方法; the
"ZGCM-1-7B 完全解説" explainer, section アーキテクチャ: QK-RMSNorm and partial RoPE on the q
and k branches, the elementwise sigmoid gate on SWA layers) is restated here with torch
float64 CPU tensors, exactly as ``attn.prefill`` defines it, and differentiated by torch's
reverse-mode autograd. Nothing is tiled or approximated. Pinned (tests/oracle_pins.py):
the restated forward equals ``attn.prefill``, and every gradient equals central finite
differences of that forward on small inputs.

The pages train the model (the explainer's training sections) but print no formula for
the backward pass; the gradient of the stated forward is the only reading.
"""

from __future__ import annotations

import math

import numpy as np

from .attn import rotary_dim_for


def _t(x):
    import torch
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def layer_torch(q, k, v, g, wq, wk, *, window=None, rotary_dim=4, rope_base=10000.0,
                eps=1e-6, scale=None, pos_offset=0):
    """The layer as torch float64 ops (differentiable): returns (out [B,T,Hq,d],
    lse [B,Hq,T]) with lse the natural-log sum of exp over each row's visible scores."""
    import torch
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    r = rotary_dim
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    pos = torch.arange(T, dtype=torch.float64) + pos_offset

    def norm_rope(x, w):
        xn = x / torch.sqrt(torch.mean(x * x, dim=-1, keepdim=True) + eps) * w
        if r == 0:
            return xn
        half = r // 2
        inv = torch.tensor([rope_base ** (-2.0 * j / r) for j in range(half)],
                           dtype=torch.float64)
        ang = pos[None, :, None, None] * inv                     # [1,T,1,half]
        c, s = torch.cos(ang), torch.sin(ang)
        a, b2 = xn[..., :half], xn[..., half:r]
        return torch.cat([a * c - b2 * s, b2 * c + a * s, xn[..., r:]], dim=-1)

    qt = norm_rope(q, wq)
    kt = norm_rope(k, wk)
    grp = Hq // Hkv
    kr = kt.repeat_interleave(grp, dim=2)                         # [B,T,Hq,d]
    vr = v.repeat_interleave(grp, dim=2)
    s = sc * torch.einsum("bihc,bjhc->bhij", qt, kr)              # [B,Hq,T,T]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    vis = j <= i
    if window is not None:
        vis = vis & (j > i - window)
    s = s.masked_fill(~vis, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)                              # [B,Hq,T]
    p = torch.exp(s - lse[..., None])
    a = torch.einsum("bhij,bjhc->bihc", p, vr)
    out = a * torch.sigmoid(g) if g is not None else a
    return out, lse


def prefill_grads(q, k, v, g, wq, wk, dout, *, window=None, rotary_dim=None,
                  rope_base=10000.0, eps=1e-6, scale=None, pos_offset=0):
    """Gradients of sum(dout * out) for the layer output out = prefill(...).

    q, g, dout: [B,T,Hq,d]; k, v: [B,T,Hkv,d]; wq, wk: [d]. Returns a dict of float64
    arrays: dq, dk, dv, dg (None for an ungated layer), dwq, dwk, and out, lse
    (natural-log row sums of exp over the visible scores, [B,Hq,T]).
    """
    import torch
    d = np.asarray(q).shape[-1]
    r = rotary_dim_for(d) if rotary_dim is None else rotary_dim
    ts = {n: _t(x).requires_grad_(True) for n, x in
          (("q", q), ("k", k), ("v", v), ("wq", wq), ("wk", wk))}
    tg = None if g is None else _t(g).requires_grad_(True)
    out, lse = layer_torch(ts["q"], ts["k"], ts["v"], tg, ts["wq"], ts["wk"], window=window,
                           rotary_dim=r, rope_base=rope_base, eps=eps, scale=scale,
                           pos_offset=pos_offset)
    loss = torch.sum(out * _t(dout))
    wrt = [ts["q"], ts["k"], ts["v"], ts["wq"], ts["wk"]] + ([tg] if tg is not None else [])
    grads = torch.autograd.grad(loss, wrt)
    res = {n: gr.detach().numpy() for n, gr in zip(("dq", "dk", "dv", "dwq", "dwk"), grads)}
    res["dg"] = grads[5].detach().numpy() if tg is not None else None
    res["out"] = out.detach().numpy()
    res["lse"] = lse.detach().numpy()
    return res
