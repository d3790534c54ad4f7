"""Thin Python entry points with the C ABI's names.

Argument marshalling only: every step of the layer runs in libzgattn's HIP kernels.
PyTorch supplies device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream()``); outputs are allocated with ``torch.empty`` when the
caller passes none.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from ._lib import BF16, F32, DecodeLayer, Desc, check, lib


def rotary_dim_for(head_dim: int, ratio: float = 0.33) -> int:
    """The largest even number of dims not above ``ratio * head_dim`` (42 for 128, 20 for 64)."""
    return 2 * int(math.floor(ratio * head_dim / 2.0))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_desc(*, batch, seq_len, n_q_heads, n_kv_heads, head_dim, window=128,
              rotary_dim=None, pos_offset=0, rope_base=10000.0, rms_eps=1e-6,
              softmax_scale=0.0, dtype=BF16) -> Desc:
    return Desc(batch, seq_len, n_q_heads, n_kv_heads, head_dim, window,
                rotary_dim_for(head_dim) if rotary_dim is None else rotary_dim,
                pos_offset, rope_base, rms_eps, softmax_scale, dtype)


def _prefill_desc(q, k, window, rotary_dim, pos_offset, rope_base, eps, scale):
    B, T, Hq, d = q.shape
    return make_desc(batch=B, seq_len=T, n_q_heads=Hq, n_kv_heads=k.shape[2], head_dim=d,
                     window=window, rotary_dim=rotary_dim, pos_offset=pos_offset,
                     rope_base=rope_base, rms_eps=eps, softmax_scale=scale,
                     dtype=_dtype_code(q))


def swa_prefill(q, k, v, g, wq, wk, *, window=128, rotary_dim=None, pos_offset=0,
                rope_base=10000.0, eps=1e-6, scale=0.0, out=None):
    """Gated sliding-window layer: [B,T,Hq,d] output of softmax-window attention * sigmoid(g)."""
    _dev(q, k, v, g, wq, wk, out)
    if out is None:
        out = torch.empty_like(q)
    d = _prefill_desc(q, k, window, rotary_dim, pos_offset, rope_base, eps, scale)
    check(lib().zgattn_swa_prefill(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(wq), _ptr(wk), _ptr(out), _stream()),
          "zgattn_swa_prefill")
    return out


def global_prefill_workspace_bytes(q, k, rotary_dim=None) -> int:
    d = _prefill_desc(q, k, 1, rotary_dim, 0, 10000.0, 1e-6, 0.0)
    return int(lib().zgattn_global_prefill_workspace_bytes(ctypes.byref(d)))


def global_prefill(q, k, v, wq, wk, *, rotary_dim=None, pos_offset=0, rope_base=10000.0,
                   eps=1e-6, scale=0.0, workspace="auto", out=None, lse=None):
    """Ungated full-causal layer. ``workspace``: "auto" allocates the K~ buffer, None runs
    the fused-K variant, or a caller-owned uint8 CUDA tensor. ``lse``: an fp32 CUDA tensor
    [B, Hq, T] that receives each row's log-sum-exp (for ``prefill_backward``), or None."""
    _dev(q, k, v, wq, wk, out, lse)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (q.shape[0], q.shape[2], q.shape[1])):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, T]")
    if out is None:
        out = torch.empty_like(q)
    d = _prefill_desc(q, k, 1, rotary_dim, pos_offset, rope_base, eps, scale)
    ws_bytes = int(lib().zgattn_global_prefill_workspace_bytes(ctypes.byref(d)))
    if isinstance(workspace, str):
        workspace = (torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
                     if ws_bytes > 0 else None)
    ws_ptr = _ptr(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().zgattn_global_prefill(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                      _ptr(wk), ws_ptr, nbytes, _ptr(out), _ptr(lse),
                                      _stream()),
          "zgattn_global_prefill")
    return out


def _varlen_desc(q, k, window, rotary_dim, pos_offset, rope_base, eps, scale):
    T, Hq, d = q.shape
    return make_desc(batch=1, seq_len=T, n_q_heads=Hq, n_kv_heads=k.shape[1], head_dim=d,
                     window=window, rotary_dim=rotary_dim, pos_offset=pos_offset,
                     rope_base=rope_base, rms_eps=eps, softmax_scale=scale,
                     dtype=_dtype_code(q))


def _cu(cu_seqlens):
    _dev(cu_seqlens)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-D int32 CUDA tensor")
    return cu_seqlens.numel() - 1


def swa_prefill_varlen(q, k, v, g, wq, wk, cu_seqlens, max_seqlen, *, window=128,
                       rotary_dim=None, pos_offset=0, rope_base=10000.0, eps=1e-6, scale=0.0,
                       out=None):
    """Gated SWA over packed documents: q, g [T, Hq, d]; k, v [T, Hkv, d]; document i is
    tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 (int32 on the device)."""
    _dev(q, k, v, g, wq, wk, out)
    n_docs = _cu(cu_seqlens)
    if out is None:
        out = torch.empty_like(q)
    d = _varlen_desc(q, k, window, rotary_dim, pos_offset, rope_base, eps, scale)
    check(lib().zgattn_swa_prefill_varlen(ctypes.byref(d), _ptr(cu_seqlens), n_docs,
                                          int(max_seqlen), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                          _ptr(wq), _ptr(wk), _ptr(out), _stream()),
          "zgattn_swa_prefill_varlen")
    return out


def global_prefill_varlen_workspace_bytes(q, k, n_docs: int, rotary_dim=None) -> int:
    d = _varlen_desc(q, k, 1, rotary_dim, 0, 10000.0, 1e-6, 0.0)
    return int(lib().zgattn_global_prefill_varlen_workspace_bytes(ctypes.byref(d), n_docs))


def global_prefill_varlen(q, k, v, wq, wk, cu_seqlens, max_seqlen, *, rotary_dim=None,
                          pos_offset=0, rope_base=10000.0, eps=1e-6, scale=0.0,
                          workspace="auto", out=None):
    """Global causal layer over packed documents (see swa_prefill_varlen for the layout)."""
    _dev(q, k, v, wq, wk, out)
    n_docs = _cu(cu_seqlens)
    if out is None:
        out = torch.empty_like(q)
    d = _varlen_desc(q, k, 1, rotary_dim, pos_offset, rope_base, eps, scale)
    ws_bytes = int(lib().zgattn_global_prefill_varlen_workspace_bytes(ctypes.byref(d), n_docs))
    if isinstance(workspace, str):
        workspace = (torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
                     if ws_bytes > 0 else None)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().zgattn_global_prefill_varlen(ctypes.byref(d), _ptr(cu_seqlens), n_docs,
                                             int(max_seqlen), _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(wq), _ptr(wk), _ptr(workspace), nbytes,
                                             _ptr(out), _stream()),
          "zgattn_global_prefill_varlen")
    return out


def _decode_desc(q, k_new, window, rotary_dim, rope_base, eps, scale):
    B, Hq, dd = q.shape
    return make_desc(batch=B, seq_len=1, n_q_heads=Hq, n_kv_heads=k_new.shape[1],
                     head_dim=dd, window=window, rotary_dim=rotary_dim, rope_base=rope_base,
                     rms_eps=eps, softmax_scale=scale, dtype=_dtype_code(q))


def swa_decode(q, k_new, v_new, g, wq, wk, k_ring, v_ring, pos, *, rotary_dim=None,
               rope_base=10000.0, eps=1e-6, scale=0.0, out=None):
    """One gated-SWA decode step; the ring size is the window. Updates the ring in place."""
    _dev(q, k_new, v_new, g, wq, wk, k_ring, v_ring, pos, out)
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if out is None:
        out = torch.empty_like(q)
    d = _decode_desc(q, k_new, k_ring.shape[2], rotary_dim, rope_base, eps, scale)
    check(lib().zgattn_swa_decode(ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(g),
                                  _ptr(wq), _ptr(wk), _ptr(k_ring), _ptr(v_ring), _ptr(pos),
                                  _ptr(out), _stream()),
          "zgattn_swa_decode")
    return out


def global_decode_workspace_bytes(q, k_new, capacity: int) -> int:
    d = _decode_desc(q, k_new, 1, None, 10000.0, 1e-6, 0.0)
    return int(lib().zgattn_global_decode_workspace_bytes(ctypes.byref(d), capacity))


def global_decode(q, k_new, v_new, wq, wk, k_cache, v_cache, pos, *, rotary_dim=None,
                  rope_base=10000.0, eps=1e-6, scale=0.0, workspace=None, out=None):
    """One global-layer decode step over a full cache; appends the new token in place."""
    _dev(q, k_new, v_new, wq, wk, k_cache, v_cache, pos, out)
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if out is None:
        out = torch.empty_like(q)
    cap = k_cache.shape[2]
    d = _decode_desc(q, k_new, 1, rotary_dim, rope_base, eps, scale)
    need = int(lib().zgattn_global_decode_workspace_bytes(ctypes.byref(d), cap))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    check(lib().zgattn_global_decode(ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(wq), _ptr(wk), _ptr(k_cache), _ptr(v_cache), cap,
                                     _ptr(pos), _ptr(workspace), nbytes, _ptr(out), _stream()),
          "zgattn_global_decode")
    return out


def global_decode_noalloc(q, k_new, v_new, wq, wk, k_cache, v_cache, pos, *, rotary_dim=None,
                          rope_base=10000.0, eps=1e-6, scale=0.0, out=None):
    """global_decode with the library's own per-GPU scratch instead of a workspace: the C
    call allocates nothing (pass ``out`` to keep this wrapper from allocating either).
    Calls that overlap on one GPU race on the shared scratch."""
    _dev(q, k_new, v_new, wq, wk, k_cache, v_cache, pos, out)
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if out is None:
        out = torch.empty_like(q)
    cap = k_cache.shape[2]
    d = _decode_desc(q, k_new, 1, rotary_dim, rope_base, eps, scale)
    check(lib().zgattn_global_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(k_new),
                                             _ptr(v_new), _ptr(wq), _ptr(wk), _ptr(k_cache),
                                             _ptr(v_cache), cap, _ptr(pos), _ptr(out),
                                             _stream()),
          "zgattn_global_decode_noalloc")
    return out


def qknorm_rope(x, w, *, pos=None, rotary_dim=None, pos_offset=0, rope_base=10000.0,
                eps=1e-6, out=None):
    """RMSNorm + partial RoPE of x [B,T,H,d]. ``out`` may be any strided view with the
    same logical shape (e.g. ``cache.permute(0, 2, 1, 3)[:, :T]``) whose last dim is dense."""
    _dev(x, w, pos)
    B, T, H, dd = x.shape
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.stride(3) != 1 or out.dtype != x.dtype or not out.is_cuda:
        raise ValueError("out must match x's shape/dtype with a dense last dim")
    if pos is not None and pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    d = make_desc(batch=B, seq_len=T, n_q_heads=H, n_kv_heads=H, head_dim=dd, window=1,
                  rotary_dim=rotary_dim, pos_offset=pos_offset, rope_base=rope_base,
                  rms_eps=eps, dtype=_dtype_code(x))
    sb, st, sh, _ = out.stride()
    check(lib().zgattn_qknorm_rope(ctypes.byref(d), H, _ptr(x), _ptr(w), _ptr(pos),
                                   _ptr(out), sb, st, sh, _stream()),
          "zgattn_qknorm_rope")
    return out


def _stack_tables(layers):
    n = len(layers)
    kinds = (ctypes.c_int32 * max(n, 1))(*[1 if L["kind"] == "global" else 0 for L in layers])
    return n, kinds


def model_decode_workspace_bytes(layers, capacity: int, *, rotary_dim=None) -> int:
    """Workspace bytes of a model_decode call over ``layers`` (global layers' partials)."""
    L0 = layers[0]
    n, kinds = _stack_tables(layers)
    d = _decode_desc(L0["q"], L0["k_new"], 1, rotary_dim, 10000.0, 1e-6, 0.0)
    return int(lib().zgattn_model_decode_workspace_bytes(ctypes.byref(d), n, kinds, capacity))


def model_decode(layers, pos, *, window=128, capacity=None, rotary_dim=None,
                 rope_base=10000.0, eps=1e-6, scale=0.0, workspace=None):
    """One decode step of a layer stack in a few launches.

    ``layers``: list of dicts with kind ("swa" / "global"), q, k_new, v_new, g (SWA only),
    wq, wk, k_cache, v_cache (SWA rings [B,Hkv,window,d] / global caches
    [B,Hkv,capacity,d]) and optional out. Returns the list of outputs; caches are updated
    in place.
    """
    if not layers:
        return []
    for L in layers:
        _dev(L["q"], L["k_new"], L["v_new"], L.get("g"), L["wq"], L["wk"], L["k_cache"],
             L["v_cache"], L.get("out"))
        if L.get("out") is None:
            L["out"] = torch.empty_like(L["q"])
    _dev(pos)
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if capacity is None:
        caps = [L["k_cache"].shape[2] for L in layers if L["kind"] == "global"]
        capacity = caps[0] if caps else 1
    n, kinds = _stack_tables(layers)
    L0 = layers[0]
    d = _decode_desc(L0["q"], L0["k_new"], window, rotary_dim, rope_base, eps, scale)
    if workspace is None:
        nbytes = int(lib().zgattn_model_decode_workspace_bytes(ctypes.byref(d), n, kinds,
                                                              capacity))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=L0["q"].device)
    tab = (DecodeLayer * n)(*[DecodeLayer(*[None if L.get(f) is None else L[f].data_ptr()
                                            for f in ("q", "k_new", "v_new", "g", "wq", "wk",
                                                      "k_cache", "v_cache", "out")])
                              for L in layers])
    check(lib().zgattn_model_decode(ctypes.byref(d), n, kinds, tab, capacity, _ptr(pos),
                                    _ptr(workspace), workspace.numel(), _stream()),
          "zgattn_model_decode")
    return [L["out"] for L in layers]


def prefill_backward_workspace_bytes(q, k) -> int:
    d = _prefill_desc(q, k, 1, None, 0, 10000.0, 1e-6, 0.0)
    return int(lib().zgattn_prefill_backward_workspace_bytes(ctypes.byref(d)))


def prefill_backward(q, k, v, g, wq, wk, out, dout, *, window=None, rotary_dim=None,
                     pos_offset=0, rope_base=10000.0, eps=1e-6, scale=0.0, workspace=None,
                     lse=None):
    """Gradients of sum(dout * out) for the layer that produced ``out``: a gated SWA layer
    when ``g`` is given (``window`` its width), else the global layer. ``lse``: the global
    forward's row log-sum-exp (``global_prefill(..., lse=...)``), or None to recompute it.
    Returns dq, dk, dv, dg (None for the global layer), dwq, dwk."""
    _dev(q, k, v, g, wq, wk, out, dout, lse)
    swa = g is not None
    if lse is not None and swa:
        raise ValueError("lse is taken by the global layer's backward only")
    d = _prefill_desc(q, k, window if swa else 1, rotary_dim, pos_offset, rope_base, eps, scale)
    if workspace is None:
        n = int(lib().zgattn_prefill_backward_workspace_bytes(ctypes.byref(d)))
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g) if swa else None
    dwq = torch.empty(q.shape[-1], dtype=torch.float32, device=q.device)
    dwk = torch.empty_like(dwq)
    nb = workspace.numel() * workspace.element_size()
    if swa:
        check(lib().zgattn_swa_prefill_backward(
            ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(wq), _ptr(wk), _ptr(out),
            _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dwq), _ptr(dwk),
            _ptr(workspace), nb, _stream()), "zgattn_swa_prefill_backward")
    else:
        check(lib().zgattn_global_prefill_backward(
            ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), _ptr(out),
            _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwq), _ptr(dwk),
            _ptr(workspace), nb, _stream()), "zgattn_global_prefill_backward")
    return dq, dk, dv, dg, dwq, dwk
