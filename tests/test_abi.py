"""The C-ABI library loads, exports every declared entry point, and its
host-only calls and host-side argument checks behave (no GPU needed: every
call here returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import paged_fp8_kv_amd as P
from oracle import control as C
from oracle import layout as Lo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = P.lib()
    syms = declared_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(P._SIGS)


def test_abi_version():
    assert P.pkv_abi_version() == P.ABI_VERSION == 3


@pytest.mark.parametrize("nb,H,Bk,D", [(36175, 1, 128, 64), (20880, 8, 32, 64), (7, 3, 16, 64)])
def test_buffer_bytes_match_oracle(nb, H, Bk, D):
    half, total = P.pkv_kv_buffer_bytes(nb, H, Bk, D)
    assert half == Lo.half_bytes(nb, H, Bk, D) and total == Lo.buffer_bytes(nb, H, Bk, D)


@pytest.mark.parametrize("Bk", [16, 32, 64, 128])
def test_trimmed_width_matches_oracle(Bk):
    assert P.pkv_trimmed_width(128, Bk) == C.trimmed_width(128, Bk)
    for w in (1, 17, 100, 128, 129):
        for lag in (0, 1):
            assert P.pkv_trimmed_width(w, Bk, lag) == C.trimmed_width(w, Bk, lag), (w, lag)


def _attn(**over):
    a = dict(batch=2, q_heads=16, kv_heads=2, head_dim=64, block=32, num_blocks=10, window=0,
             q=None, k=None, k_packed=1, v=None, table=None, bt_stride=4, width=4, pos=None,
             rc=None, rs=None, ks=0.125, vs=0.0625, sm=0.125, out=None, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return P.lib().pkv_paged_decode_attn(*a.values())


def test_attention_argument_errors():
    assert _attn(head_dim=128) == P.PKV_ERR_UNSUPPORTED
    assert b"head_dim" in P.lib().pkv_last_error()
    assert _attn(block=24) == P.PKV_ERR_UNSUPPORTED
    assert _attn(q_heads=15) == P.PKV_ERR_ARG
    assert _attn(q_heads=32) == P.PKV_ERR_UNSUPPORTED      # group of 16
    assert _attn(kv_heads=0) == P.PKV_ERR_ARG
    assert _attn(batch=-1) == P.PKV_ERR_ARG
    assert _attn(width=5) == P.PKV_ERR_ARG                 # stride < width
    assert _attn() == P.PKV_ERR_ARG                        # null pointers
    assert _attn(batch=0) == P.PKV_OK                      # empty batch is a no-op
    fake = dict(q=0x1000, k=0x1000, v=0x1000, table=0x1000, pos=0x1000, out=0x1000)
    assert _attn(ks=1e30, sm=1e30, **fake) == P.PKV_ERR_ARG   # product overflows fp32
    assert _attn(ks=1e-30, sm=1e-30, **fake) == P.PKV_ERR_ARG  # product underflows to 0
    assert b"sm_scale * k_scale" in P.lib().pkv_last_error()


def test_rope_argument_errors():
    """Rejected before any launch (the fake addresses are never dereferenced)."""
    fake = dict(q=0x1000, k=0x1000, v=0x1000, table=0x1000, pos=0x1000, out=0x1000)
    assert _attn(rc=0x2000, **fake) == P.PKV_ERR_ARG
    assert b"rope" in P.lib().pkv_last_error()
    assert _attn(rs=0x2000, **fake) == P.PKV_ERR_ARG
    assert _attn(rc=0x2004, rs=0x2000, **fake) == P.PKV_ERR_ARG
    assert b"aligned" in P.lib().pkv_last_error()
    L = P.lib()
    assert L.pkv_kv_cache_update(1, 1, 64, 16, 4, 0x1000, 0x1000, 0x1000, 1, 0x1000, 0x1000,
                                 0x2000, None, 0.1, 0.1, None) == P.PKV_ERR_ARG
    assert b"rope" in L.pkv_last_error()


def test_update_and_setup_argument_errors():
    L = P.lib()
    assert L.pkv_kv_cache_update(1, 1, 32, 16, 4, None, None, None, 1, None, None,
                                 None, None, 0.1, 0.1, None) == P.PKV_ERR_UNSUPPORTED
    assert L.pkv_kv_cache_update(1, 1, 64, 16, 4, None, None, None, 1, None, None,
                                 None, None, 0.1, 0.1, None) == P.PKV_ERR_ARG
    assert L.pkv_kv_cache_update(0, 1, 64, 16, 4, None, None, None, 1, None, None,
                                 None, None, 0.1, 0.1, None) == P.PKV_OK
    assert L.pkv_setup_attn_control(1, 16, 128, 0, None, None, None, None, 4, None, 4, 4, None,
                                    None, None, 9, None, None, None, None) == P.PKV_ERR_ARG
    # anchor_lag other than 0 or 1 is refused before anything else
    assert L.pkv_setup_attn_control(1, 16, 128, 2, 0x100, 0x100, None, 0x100, 4, 0x100, 4, 4,
                                    0x100, 0x100, 0x100, 9, 0x100, 0x100, None,
                                    None) == P.PKV_ERR_ARG
    assert b"anchor_lag" in L.pkv_last_error()


def test_workspace_sizing():
    n = P.pkv_decode_workspace_bytes(64, 64, 8, 64, 32, 256, 0)
    assert n > 0 and n % 4 == 0
    assert P.lib().pkv_decode_workspace_bytes(1, 8, 1, 32, 16, 16, 0) == P.PKV_ERR_UNSUPPORTED
    assert P.pkv_decode_workspace_bytes(0, 8, 1, 64, 16, 16, 0) == 0


def test_decode_layer_rejects_both_or_neither_kv_form():
    s = P.PkvStep()
    s.batch, s.q_heads, s.kv_heads, s.head_dim, s.block = 1, 8, 1, 64, 16
    s.window, s.num_blocks, s.n_buffers, s.k_packed = 128, 4, 1, 1
    st = P.lib().pkv_decode_layer(ctypes.byref(s), 0, None, None, None, 0.1, 0.1, 0.1, None,
                                  None, 0, None)
    assert st == P.PKV_ERR_ARG and b"exactly one" in P.lib().pkv_last_error()
    arr = (ctypes.c_void_p * 1)(16)
    s.k_bufs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    s.v_bufs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    s.stacked = 256
    st = P.lib().pkv_decode_layer(ctypes.byref(s), 0, None, None, None, 0.1, 0.1, 0.1, None,
                                  None, 0, None)
    assert st == P.PKV_ERR_ARG and b"exactly one" in P.lib().pkv_last_error()


def test_noalloc_refuses_shapes_beyond_its_workspace():
    """The no-allocation layer call holds a 24 MiB workspace per GPU: shapes
    needing more are refused on the host, before anything is enqueued."""
    L = P.lib()
    s = P.PkvStep()
    s.batch, s.q_heads, s.kv_heads, s.head_dim, s.block = 8192, 256, 256, 64, 32
    s.window, s.num_blocks, s.n_buffers, s.k_packed = 128, 4, 1, 1
    ka = (ctypes.c_void_p * 1)(0x10000)
    va = (ctypes.c_void_p * 1)(0x20000)
    s.k_bufs = ctypes.cast(ka, ctypes.POINTER(ctypes.c_void_p))
    s.v_bufs = ctypes.cast(va, ctypes.POINTER(ctypes.c_void_p))
    s.bt_full = s.bt_swa_trim = s.pos_full = s.pos_swa = s.upd_full = s.upd_swa = 0x1000
    s.bt_full_stride = s.bt_full_width = 256
    s.trim_width = 5
    need = P.pkv_decode_workspace_bytes(8192, 256, 256, 64, 32, 256, 0)
    assert need > 24 << 20
    st = L.pkv_decode_layer_noalloc(ctypes.byref(s), 1, 0x1000, 0x1000, 0x1000, 0.125, 0.0625,
                                    0.125, 0x1000, None)
    assert st == P.PKV_ERR_WORKSPACE and b"library's own" in L.pkv_last_error()


def test_error_text_is_per_thread():
    """A call rejected on one thread sets that thread's error text only."""
    import threading
    lib = P.lib()
    seen = {}

    def bad():
        seen["bad"] = (lib.pkv_trimmed_width(0, 16, 0), lib.pkv_last_error())  # window < 1

    def good():
        seen["good"] = (lib.pkv_trimmed_width(128, 16, 0), lib.pkv_last_error())

    for f in (bad, good):
        t = threading.Thread(target=f)
        t.start()
        t.join()
    assert seen["bad"][0] < 0 and b"window" in seen["bad"][1]
    assert seen["good"][0] == 9 and b"window" not in (seen["good"][1] or b"")
