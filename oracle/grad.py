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


# ---- gradients at sampled positions, from the closed-form backward ----------------------
# For long sequences the autograd graph above (every score of every head) does not fit. The
# gradient of the same forward is written out instead, step by step: with P the row-wise
# softmax of S = scale * q~ . k~ over the visible keys, A = P V, O = A * sigmoid(G) (O = A
# without a gate) and L = sum(dO * O):
#   dA = dO * sigmoid(G),  D_i = sum_c dO_ic O_ic = sum_c dA_ic A_ic,
#   dS = P * (dA V^T - D)   (the softmax Jacobian applied to dP = dA V^T),
#   dq~_i = scale * sum_j dS_ij k~_j,  dk~_j = scale * sum over the group's heads and rows
#   i of dS_ij q~_i,  dv_j = sum over the group's heads and rows i of P_ij dA_i,
#   dG = dO * A * sigmoid(G) * (1 - sigmoid(G)),
# and dq, dk are the vector-Jacobian products of the per-row norm/RoPE transform (autograd
# of that transform on the sampled rows only). The forward runs over every row (in row
# blocks) because dk and dv at a key need every query row's log-sum-exp and D.

def _norm_rope_rows(x, w, pos, r, rope_base, eps):
    """RMSNorm * w, then RoPE on the leading r dims, of rows x [..., d] at positions pos
    (broadcast against x's leading dims), torch float64."""
    import torch
    xn = x / torch.sqrt(torch.mean(x * x, dim=-1, keepdim=True) + eps) * w
    if r == 0:
        return xn
    half = r // 2
    inv = torch.tensor([rope_base ** (-2.0 * j / r) for j in range(half)], dtype=torch.float64)
    ang = pos[..., None] * inv
    c, s = torch.cos(ang), torch.sin(ang)
    a, b2 = xn[..., :half], xn[..., half:r]
    return torch.cat([a * c - b2 * s, b2 * c + a * s, xn[..., r:]], dim=-1)


def _softmax_vjp(p, dp, dsum):
    """dS = P * (dP - D): the softmax Jacobian applied to dP (D per row)."""
    return p * (dp - dsum)


def _group_heads(kvh, grp):
    """The query heads that read KV head kvh."""
    return range(kvh * grp, (kvh + 1) * grp)


def prefill_grads_rows(q, k, v, g, wq, wk, dout, q_rows, k_rows, *, window=None,
                       rotary_dim=None, rope_base=10000.0, eps=1e-6, scale=None, pos_offset=0,
                       block=512):
    """Gradients of sum(dout * out) at sampled positions (see the block comment above).

    q, g, dout: [B,T,Hq,d]; k, v: [B,T,Hkv,d]; wq, wk: [d]; q_rows, k_rows: positions.
    Returns float64 arrays: dq, dg (None without a gate) at q_rows [B, nq, Hq, d]; dk, dv at
    k_rows [B, nk, Hkv, d]; lse [B, Hq, T] (natural log)."""
    import torch
    qn, kn, vn = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, T, Hq, d = qn.shape
    Hkv = kn.shape[2]
    grp = Hq // Hkv
    r = rotary_dim_for(d) if rotary_dim is None else rotary_dim
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    qr = np.asarray(q_rows, dtype=np.int64)
    kr = np.asarray(k_rows, dtype=np.int64)
    with torch.no_grad():
        Q, K, V = _t(qn), _t(kn), _t(vn)
        Wq, Wk = _t(wq), _t(wk)
        dO = _t(dout)
        G = None if g is None else _t(g)
        pos = torch.arange(T, dtype=torch.float64) + pos_offset
        qt = _norm_rope_rows(Q, Wq, pos[None, :, None], r, rope_base, eps)   # [B,T,Hq,d]
        kt = _norm_rope_rows(K, Wk, pos[None, :, None], r, rope_base, eps)   # [B,T,Hkv,d]
        idx = torch.arange(T)

        def visible(i, j):            # i: query positions [n,1], j: key positions [1,m]
            m = j <= i
            if window is not None:
                m = m & (j > i - window)
            return m

        # forward over every row: log-sum-exp and A
        lse = torch.empty((B, Hq, T), dtype=torch.float64)
        A = torch.empty((B, T, Hq, d), dtype=torch.float64)
        for b in range(B):
            for h in range(Hq):
                kh = h // grp
                for i0 in range(0, T, block):
                    i1 = min(T, i0 + block)
                    s = sc * qt[b, i0:i1, h] @ kt[b, :, kh].T
                    s = s.masked_fill(~visible(idx[i0:i1, None], idx[None, :]), float("-inf"))
                    l = torch.logsumexp(s, dim=-1)
                    lse[b, h, i0:i1] = l
                    A[b, i0:i1, h] = torch.exp(s - l[:, None]) @ V[b, :, kh]
        sig = None if G is None else torch.sigmoid(G)
        O = A * sig if sig is not None else A
        dA = dO * sig if sig is not None else dO
        Dsum = torch.sum(dO * O, dim=-1)                                     # [B,T,Hq]

        # dq~ at the sampled query rows
        qi = torch.as_tensor(qr)
        dqt = torch.zeros((B, len(qr), Hq, d), dtype=torch.float64)
        for b in range(B):
            for h in range(Hq):
                kh = h // grp
                s = sc * qt[b, qi, h] @ kt[b, :, kh].T                       # [nq, T]
                vis = visible(qi[:, None], idx[None, :])
                p = torch.where(vis, torch.exp(s - lse[b, h, qi][:, None]), 0.0)
                dp = dA[b, qi, h] @ V[b, :, kh].T
                ds = _softmax_vjp(p, dp, Dsum[b, qi, h][:, None])
                dqt[b, :, h] = sc * ds @ kt[b, :, kh]

        # dk~ and dv at the sampled keys: every query row of the group's heads
        kj = torch.as_tensor(kr)
        dkt = torch.zeros((B, len(kr), Hkv, d), dtype=torch.float64)
        dv = torch.zeros((B, len(kr), Hkv, d), dtype=torch.float64)
        for b in range(B):
            for kh in range(Hkv):
                for h in _group_heads(kh, grp):
                    s = sc * qt[b, :, h] @ kt[b, kj, kh].T                   # [T, nk]
                    vis = visible(idx[:, None], kj[None, :])
                    p = torch.where(vis, torch.exp(s - lse[b, h][:, None]), 0.0)
                    dv[b, :, kh] += p.T @ dA[b, :, h]
                    dp = dA[b, :, h] @ V[b, kj, kh].T
                    ds = _softmax_vjp(p, dp, Dsum[b, :, h][:, None])
                    dkt[b, :, kh] += sc * ds.T @ qt[b, :, h]
        dg = None
        if sig is not None:
            dg = (dO[:, qi] * A[:, qi] * sig[:, qi] * (1.0 - sig[:, qi])).numpy()

    # norm/RoPE backward on the sampled rows
    xq = Q[:, qi].clone().requires_grad_(True)
    yq = _norm_rope_rows(xq, Wq, pos[qi][None, :, None], r, rope_base, eps)
    (dq,) = torch.autograd.grad(yq, xq, dqt)
    xk = K[:, kj].clone().requires_grad_(True)
    yk = _norm_rope_rows(xk, Wk, pos[kj][None, :, None], r, rope_base, eps)
    (dk,) = torch.autograd.grad(yk, xk, dkt)
    return {"dq": dq.numpy(), "dk": dk.numpy(), "dv": dv.numpy(), "dg": dg,
            "lse": lse.numpy()}
