"""ctypes view of libzgattn.so (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzgattn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "zgattn.h")

F32, BF16 = 0, 1
STATUS = {0: "ZGATTN_OK", -1: "ZGATTN_EINVAL", -2: "ZGATTN_ENULL", -3: "ZGATTN_EDTYPE",
          -4: "ZGATTN_EUNSUPPORTED", -5: "ZGATTN_EWORKSPACE", -6: "ZGATTN_ERANGE",
          -7: "ZGATTN_EHIP"}


class Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("pos_offset", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class DecodeLayer(ctypes.Structure):
    """zgattn_decode_layer: one layer's device tensors in a stack decode step."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "k_new", "v_new", "g", "wq", "wk", "k_cache", "v_cache", "out")]


class ZgattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {STATUS.get(status, status)} "
                         f"({_lib.zgattn_strerror(status).decode() if _lib else ''})")


_lib = None
P = ctypes.c_void_p
DP = ctypes.POINTER(Desc)
I32, I64, SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

SIGNATURES = {
    "zgattn_abi_version": (ctypes.c_int, []),
    "zgattn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "zgattn_swa_prefill": (ctypes.c_int, [DP, P, P, P, P, P, P, P, P]),
    "zgattn_global_prefill": (ctypes.c_int, [DP, P, P, P, P, P, P, SZ, P, P, P]),
    "zgattn_global_prefill_workspace_bytes": (SZ, [DP]),
    "zgattn_swa_decode": (ctypes.c_int, [DP, P, P, P, P, P, P, P, P, P, P, P]),
    "zgattn_global_decode": (ctypes.c_int, [DP, P, P, P, P, P, P, P, I32, P, P, SZ, P, P]),
    "zgattn_global_decode_workspace_bytes": (SZ, [DP, I32]),
    "zgattn_global_decode_noalloc": (ctypes.c_int, [DP, P, P, P, P, P, P, P, I32, P, P, P]),
    "zgattn_qknorm_rope": (ctypes.c_int, [DP, I32, P, P, P, P, I64, I64, I64, P]),
    "zgattn_swa_prefill_varlen": (ctypes.c_int, [DP, P, I32, I32, P, P, P, P, P, P, P, P]),
    "zgattn_prefill_backward_workspace_bytes": (SZ, [DP]),
    "zgattn_swa_prefill_backward": (ctypes.c_int, [DP] + [P] * 15 + [SZ, P]),
    "zgattn_global_prefill_backward": (ctypes.c_int, [DP] + [P] * 14 + [SZ, P]),
    "zgattn_global_prefill_varlen": (ctypes.c_int, [DP, P, I32, I32, P, P, P, P, P, P, SZ, P,
                                                    P]),
    "zgattn_global_prefill_varlen_workspace_bytes": (SZ, [DP, I32]),
    "zgattn_model_decode": (ctypes.c_int, [DP, I32, ctypes.POINTER(I32),
                                           ctypes.POINTER(DecodeLayer), I32, P, P, SZ, P]),
    "zgattn_model_decode_workspace_bytes": (SZ, [DP, I32, ctypes.POINTER(I32), I32]),
}


def lib():
    """Load libzgattn.so once. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m global_attention_qk_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols():
    """Names of the functions include/zgattn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(zgattn_[a-z_0-9]+)\s*\(", text)))


def check(status: int, what: str):
    if status != 0:
        raise ZgattnError(status, what)
