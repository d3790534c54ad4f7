"""The C-ABI library loads and exports what include/zgattn.h declares; host-side argument
checks return their status codes before anything touches a GPU."""

import ctypes
import os

import pytest

from global_attention_qk_amd import _lib as L
from global_attention_qk_amd.api import make_desc

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH),
                                reason="libzgattn.so not built (run __graft_entry__.build())")

FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation first


def test_exports_every_declared_symbol():
    lib = L.lib()
    declared = L.header_symbols()
    assert len(declared) == 18
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(L.SIGNATURES)


def test_version_and_strerror():
    lib = L.lib()
    assert lib.zgattn_abi_version() == 2
    for code in L.STATUS:
        assert lib.zgattn_strerror(code)
    assert lib.zgattn_strerror(12345) == b"unknown status"


def _d(**kw):
    base = dict(batch=1, seq_len=16, n_q_heads=4, n_kv_heads=1, head_dim=128, window=128,
                rotary_dim=42, dtype=L.BF16)
    base.update(kw)
    return make_desc(**base)


def _swa(d, q=FAKE, g=FAKE, out=FAKE):
    return L.lib().zgattn_swa_prefill(ctypes.byref(d), q, FAKE, FAKE, g, FAKE, FAKE, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=6, n_kv_heads=4), -1),
    (dict(head_dim=96), -4),
    (dict(rotary_dim=43), -1),
    (dict(rotary_dim=130), -1),
    (dict(dtype=7), -3),
    (dict(window=0), -1),
    (dict(batch=0), -1),
    (dict(seq_len=-1), -1),
    (dict(pos_offset=-3), -6),
    (dict(pos_offset=(1 << 24) - 8, seq_len=16), -6),
    (dict(rope_base=-1.0), -1),
    (dict(rms_eps=float("nan")), -1),
])
def test_prefill_rejects(kw, code):
    assert _swa(_d(**kw)) == code


def test_nulls_and_alignment():
    assert _swa(_d(), q=None) == -2
    assert _swa(_d(), g=None) == -2
    assert _swa(_d(), out=ctypes.c_void_p(4100)) == -1
    assert L.lib().zgattn_swa_prefill(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2
    # empty sequence is a no-op that touches nothing
    assert _swa(_d(seq_len=0), q=None, g=None, out=None) == 0


def test_bf16_other_shapes_refuse_only_the_lse():
    # rotary_dim above 64 and head groups the 256-row tile cannot split run on the
    # vector-ALU kernel, which gives no log-sum-exp: asking for it is refused before launch
    lib = L.lib()
    for kw in (dict(rotary_dim=80), dict(n_q_heads=3, n_kv_heads=1)):
        d = _d(**kw)
        st = lib.zgattn_global_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                       FAKE, FAKE, None)
        assert st == -4


def test_global_prefill_workspace():
    lib = L.lib()
    d = _d(batch=2, seq_len=1000, n_q_heads=32, n_kv_heads=8)
    need = lib.zgattn_global_prefill_workspace_bytes(ctypes.byref(d))
    kbytes = (2 * 8 * 1000 + 64) * 128 * 2           # normalised K + a tile of slack
    vtiles = 2 * 8 * ((1000 + 63) // 64) * 64 * 128 * 2  # V as transposed 64-key tiles
    assert need == ((kbytes + 255) // 256) * 256 + vtiles
    st = lib.zgattn_global_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   need - 1, FAKE, None, None)
    assert st == -5


def test_decode_checks():
    lib = L.lib()
    d = _d(batch=4, seq_len=1, n_q_heads=32, n_kv_heads=8)
    cap = 262144
    need = lib.zgattn_global_decode_workspace_bytes(ctypes.byref(d), cap)
    assert need >= 4 * 32 * 128 * 4
    call = lambda **kw: lib.zgattn_global_decode(
        ctypes.byref(kw.get("d", d)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        kw.get("cap", cap), kw.get("pos", FAKE), kw.get("ws", FAKE), kw.get("nb", need),
        FAKE, None)
    assert call(ws=None) == -5
    assert call(nb=need - 1) == -5
    assert call(cap=0) == -6
    assert call(pos=None) == -2
    # fp32 passes the dtype check (its workspace check comes after it); nothing launches
    assert call(d=_d(batch=4, seq_len=1, n_q_heads=32, n_kv_heads=8, dtype=L.F32),
                nb=need - 1) == -5
    assert call(d=_d(n_q_heads=48, n_kv_heads=3)) == -4   # head group 16
    st = lib.zgattn_swa_decode(ctypes.byref(_d(window=0, n_q_heads=32, n_kv_heads=8)), FAKE,
                               FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == -1


def test_decode_noalloc_checks():
    # rejections happen on the host, before the scratch is looked up or anything launches
    lib = L.lib()
    call = lambda d, cap=4096, pos=FAKE: lib.zgattn_global_decode_noalloc(
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cap, pos, FAKE, None)
    ok = _d(batch=4, seq_len=1, n_q_heads=32, n_kv_heads=8)
    assert call(ok, cap=0) == -6
    assert call(ok, pos=None) == -2
    assert call(_d(dtype=L.F32, n_q_heads=32, n_kv_heads=8), cap=0) == -6   # fp32 accepted
    # partials of B * Hq * d = 2^23 values need 2 * 4 * 2^23 bytes even with one split:
    # more than the 64 MiB scratch
    big = _d(batch=1024, seq_len=1, n_q_heads=64, n_kv_heads=8)
    assert call(big, cap=262144) == -5


def test_qknorm_rope_checks():
    lib = L.lib()
    d = _d()
    ok_strides = (16 * 128, 128, 128 * 16)
    assert lib.zgattn_qknorm_rope(ctypes.byref(d), 0, FAKE, FAKE, None, FAKE, *ok_strides, None) == -1
    assert lib.zgattn_qknorm_rope(ctypes.byref(d), 4, FAKE, FAKE, None, FAKE, 16 * 128, 127, 128 * 16, None) == -1
    assert lib.zgattn_qknorm_rope(ctypes.byref(d), 4, None, FAKE, None, FAKE, *ok_strides, None) == -2


def test_model_decode_checks():
    lib = L.lib()
    d = _d(batch=4, seq_len=1, n_q_heads=32, n_kv_heads=8)
    cap = 4096
    kinds = (ctypes.c_int32 * 3)(0, 1, 0)
    lay = lambda **kw: L.DecodeLayer(*[kw.get(f, 4096) for f in (
        "q", "k_new", "v_new", "g", "wq", "wk", "k_cache", "v_cache", "out")])
    tab = (L.DecodeLayer * 3)(lay(), lay(), lay())
    need = lib.zgattn_model_decode_workspace_bytes(ctypes.byref(d), 3, kinds, cap)
    one = lib.zgattn_global_decode_workspace_bytes(ctypes.byref(d), cap)
    assert need == ((one + 255) // 256) * 256        # one global layer
    none = (ctypes.c_int32 * 2)(0, 0)
    assert lib.zgattn_model_decode_workspace_bytes(ctypes.byref(d), 2, none, cap) == 0
    call = lambda **kw: lib.zgattn_model_decode(
        ctypes.byref(kw.get("d", d)), kw.get("n", 3), kw.get("kinds", kinds),
        kw.get("tab", tab), kw.get("cap", cap), kw.get("pos", FAKE), kw.get("ws", FAKE),
        kw.get("nb", need), None)
    assert call(n=0, tab=None, kinds=None, pos=None) == 0    # nothing to do, nothing touched
    assert lib.zgattn_model_decode(None, 3, kinds, tab, cap, FAKE, FAKE, need, None) == -2
    assert call(tab=None) == -2
    assert call(kinds=None) == -2
    assert call(pos=None) == -2
    assert call(n=-1) == -1
    assert call(ws=None) == -5
    assert call(nb=need - 1) == -5
    assert call(cap=0) == -6
    bad = (L.DecodeLayer * 3)(lay(), lay(), lay(g=None))       # an SWA layer without gate
    assert call(tab=bad) == -2
    bad = (L.DecodeLayer * 3)(lay(), lay(out=4100), lay())     # misaligned output
    assert call(tab=bad) == -1
    assert call(d=_d(batch=4, seq_len=1, n_q_heads=32, n_kv_heads=8, window=129)) == -4
    # fp32 passes the dtype check (single-layer kernels per layer); its workspace check
    # still comes first, so nothing launches here
    f32 = _d(batch=4, seq_len=1, n_q_heads=32, n_kv_heads=8, dtype=L.F32)
    assert call(d=f32, nb=need - 1) == -5
    assert call(d=_d(batch=4, seq_len=1, n_q_heads=32, n_kv_heads=8, window=0)) == -1


def test_varlen_prefill_checks():
    lib = L.lib()
    d = _d(batch=1, seq_len=1000, n_q_heads=8, n_kv_heads=2)
    call = lambda **kw: lib.zgattn_swa_prefill_varlen(
        ctypes.byref(kw.get("d", d)), kw.get("cu", FAKE), kw.get("n", 3), kw.get("mx", 600),
        FAKE, FAKE, FAKE, kw.get("g", FAKE), FAKE, FAKE, FAKE, None)
    assert call(d=_d(batch=2, seq_len=1000, n_q_heads=8, n_kv_heads=2)) == -1   # B must be 1
    assert call(n=0) == -1
    assert call(mx=1001) == -1
    assert call(cu=None) == -2
    assert call(g=None) == -2
    # fp32 passes the dtype check (the vector-ALU kernel); the gate check still comes first
    assert call(d=_d(batch=1, seq_len=1000, n_q_heads=8, n_kv_heads=2, dtype=L.F32),
                g=None) == -2
    assert call(mx=0, cu=None, g=None) == 0                     # every document empty
    ws = lib.zgattn_global_prefill_varlen_workspace_bytes(ctypes.byref(d), 3)
    kbytes = (2 * 1000 + 64) * 128 * 2
    assert ws == ((kbytes + 255) // 256) * 256 + 2 * (1000 // 64 + 3) * 64 * 128 * 2
    st = lib.zgattn_global_prefill_varlen(ctypes.byref(d), FAKE, 3, 600, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, ws - 1, FAKE, None)
    assert st == -5


def test_backward_checks():
    lib = L.lib()
    d = _d(batch=2, seq_len=300, n_q_heads=8, n_kv_heads=2)
    need = lib.zgattn_prefill_backward_workspace_bytes(ctypes.byref(d))
    nq, nk = 2 * 300 * 8, 2 * 300 * 2
    a256 = lambda x: (x + 255) // 256 * 256
    n64 = (300 + 63) // 64
    assert need == (a256(nq * 128 * 2) + a256(nk * 128 * 2) + a256(nq * 128 * 2) + 2 * a256(nq * 4)
                    + a256(nq * 128 * 4) + a256(nk * 128 * 4) + a256(2 * 1024 * 128 * 4)
                    + 2 * a256(2 * 8 * n64 * 64 * 128 * 2) + a256(2 * 2 * n64 * 64 * 128 * 2))
    call = lambda **kw: lib.zgattn_swa_prefill_backward(
        ctypes.byref(kw.get("d", d)), FAKE, FAKE, FAKE, kw.get("g", FAKE), FAKE, FAKE, FAKE,
        kw.get("dout", FAKE), FAKE, FAKE, FAKE, kw.get("dg", FAKE), FAKE, FAKE,
        kw.get("ws", FAKE), kw.get("nb", need), None)
    assert call(ws=None) == -5
    assert call(nb=need - 1) == -5
    assert call(g=None) == -2
    assert call(dg=None) == -2
    assert call(dout=None) == -2
    assert call(dout=ctypes.c_void_p(4100)) == -1
    # fp32 tensors and head groups off the MFMA kernels take the vector-ALU backward: the
    # same checks, the same workspace size (the larger of the two paths' layouts)
    df = _d(batch=2, seq_len=300, n_q_heads=8, n_kv_heads=2, dtype=L.F32)
    assert lib.zgattn_prefill_backward_workspace_bytes(ctypes.byref(df)) == need
    assert call(d=df, nb=need - 1) == -5
    assert call(d=df, g=None) == -2
    dg16 = _d(batch=2, seq_len=300, n_q_heads=48, n_kv_heads=3)
    need16 = lib.zgattn_prefill_backward_workspace_bytes(ctypes.byref(dg16))
    assert need16 > need
    assert call(d=dg16, nb=need16 - 1) == -5
    assert call(d=dg16, ws=None, nb=need16) == -5
    assert call(d=_d(batch=2, seq_len=0, n_q_heads=8, n_kv_heads=2)) == 0
    st = lib.zgattn_global_prefill_backward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, need,
                                            None)
    assert st == -5
