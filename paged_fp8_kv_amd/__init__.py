"""Thin Python binding of libpkv (include/pkv.h).

Argument marshalling only: every function has the name of the C entry point
it calls, takes torch tensors for device memory, passes their data pointers
and torch's current HIP stream, and raises on a negative status with the
library's own error text.  No computation happens here, and there is no
fallback: if the built library is missing the import of this module still
succeeds, but the first call raises.

Build the library with ``python -m paged_fp8_kv_amd.build``.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_ERR_DATA = -5

_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class PkvError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"pkv status {status}: {msg}")
        self.status = status


class PkvStep(ctypes.Structure):
    _fields_ = [
        ("batch", _i32), ("q_heads", _i32), ("kv_heads", _i32), ("head_dim", _i32),
        ("block", _i32), ("window", _i32), ("num_blocks", _i64), ("n_buffers", _i32),
        ("k_packed", _i32), ("k_bufs", ctypes.POINTER(_vp)), ("v_bufs", ctypes.POINTER(_vp)),
        ("stacked", _vp), ("bt_full", _vp), ("bt_full_stride", _i32), ("bt_full_width", _i32),
        ("bt_swa_trim", _vp), ("trim_width", _i32), ("pos_full", _vp), ("pos_swa", _vp),
        ("upd_full", _vp), ("upd_swa", _vp), ("rope_cos", _vp), ("rope_sin", _vp),
    ]


_SIGS = {
    "pkv_abi_version": ([], _i32),
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_kv_buffer_bytes": ([_i64, _i32, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)], _i32),
    "pkv_trimmed_width": ([_i32, _i32, _i32], _i32),
    "pkv_kv_budget": ([_i64, _i64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                       ctypes.POINTER(_i64)], _i32),
    "pkv_kv_num_blocks": ([_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(_i64)], _i32),
    "pkv_setup_attn_control": ([_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp], _i32),
    "pkv_setup_attn_control_csr": ([_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp],
                                   _i32),
    "pkv_kv_cache_update": ([_i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _i32, _vp, _vp,
                             _vp, _vp, _f32, _f32, _vp], _i32),
    "pkv_decode_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32], _i64),
    "pkv_paged_decode_attn": ([_i32, _i32, _i32, _i32, _i32, _i64, _i32, _vp, _vp, _i32, _vp,
                               _vp, _i32, _i32, _vp, _vp, _vp, _f32, _f32, _f32, _vp, _vp, _i64,
                               _vp], _i32),
    "pkv_decode_layer": ([ctypes.POINTER(PkvStep), _i32, _vp, _vp, _vp, _f32, _f32, _f32, _vp,
                          _vp, _i64, _vp], _i32),
    "pkv_decode_layer_noalloc": ([ctypes.POINTER(PkvStep), _i32, _vp, _vp, _vp, _f32, _f32, _f32,
                                  _vp, _vp], _i32),
    "pkv_validate_attn_control": ([_i32, _i32, _i32, _i64, _vp, _vp, _vp, _i32, _vp, _i32,
                                   _i32, _vp], _i32),
}

_lib = None
ABI_VERSION = 3  # PKV_ABI_VERSION these signatures follow


def lib():
    """The loaded libpkv (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m paged_fp8_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        if L.pkv_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI {L.pkv_abi_version()}, the binding expects "
                               f"{ABI_VERSION}: rebuild with `python -m paged_fp8_kv_amd.build`")
        _lib = L
    return _lib


def _check(status):
    if status < 0:
        raise PkvError(status, lib().pkv_last_error().decode())
    return status


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dev_ptr(t, dtype, name):
    if t is not None and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return _ptr(t, dtype, name)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def pkv_abi_version():
    return lib().pkv_abi_version()


def pkv_kv_buffer_bytes(num_blocks, kv_heads, block, head_dim):
    h, t = _i64(), _i64()
    _check(lib().pkv_kv_buffer_bytes(num_blocks, kv_heads, block, head_dim, ctypes.byref(h),
                                     ctypes.byref(t)))
    return h.value, t.value


def pkv_kv_budget(total_hbm_bytes, bytes_used, gmu, cap_fraction=0.30, min_kv_gib=1.0):
    """Bytes the KV cache may take; raises PkvError (PKV_ERR_DATA) below the minimum."""
    out = _i64()
    _check(lib().pkv_kv_budget(total_hbm_bytes, bytes_used, gmu, cap_fraction, min_kv_gib,
                               ctypes.byref(out)))
    return out.value


def pkv_kv_num_blocks(available_bytes, n_buffers, kv_heads, block, head_dim):
    out = _i64()
    _check(lib().pkv_kv_num_blocks(available_bytes, n_buffers, kv_heads, block, head_dim,
                                   ctypes.byref(out)))
    return out.value


def pkv_trimmed_width(window, block, anchor_lag=0):
    return _check(lib().pkv_trimmed_width(window, block, anchor_lag))


def pkv_setup_attn_control(seq_lens, active, bt_full, bt_swa, block, window, positions=None,
                           bt_width=None, out=None, stream=None, anchor_lag=0):
    """Returns a dict with pos_full, pos_swa, bt_swa_trim, upd_full, upd_swa, pos_abs."""
    B = seq_lens.shape[0]
    width = bt_full.shape[1] if bt_width is None else bt_width
    tw = pkv_trimmed_width(window, block, anchor_lag) if window > 0 else 0
    dev = seq_lens.device
    if out is None:
        out = dict(
            pos_full=torch.empty(B, dtype=torch.int32, device=dev),
            pos_swa=torch.empty(B, dtype=torch.int32, device=dev),
            bt_swa_trim=torch.empty(B, max(tw, 1), dtype=torch.int32, device=dev),
            upd_full=torch.empty(B, dtype=torch.int64, device=dev),
            upd_swa=torch.empty(B, dtype=torch.int64, device=dev),
            pos_abs=torch.empty(B, dtype=torch.int64, device=dev),
        )
    _check(lib().pkv_setup_attn_control(
        B, block, window, anchor_lag, _dev_ptr(seq_lens, torch.int32, "seq_lens"),
        _dev_ptr(active, torch.uint8, "active"), _dev_ptr(positions, torch.int64, "positions"),
        _dev_ptr(bt_full, torch.int32, "bt_full"), bt_full.shape[1],
        _dev_ptr(bt_swa, torch.int32, "bt_swa") if window > 0 else None,
        bt_swa.shape[1] if (window > 0 and bt_swa is not None) else 0, width,
        _dev_ptr(out["pos_full"], torch.int32, "pos_full"),
        _dev_ptr(out["pos_swa"], torch.int32, "pos_swa"),
        _dev_ptr(out["bt_swa_trim"], torch.int32, "bt_swa_trim"), tw,
        _dev_ptr(out["upd_full"], torch.int64, "upd_full"),
        _dev_ptr(out["upd_swa"], torch.int64, "upd_swa"),
        _dev_ptr(out["pos_abs"], torch.int64, "pos_abs"), _stream(stream)))
    return out


def _halves(buf, num_blocks, kv_heads, block, head_dim):
    half, total = pkv_kv_buffer_bytes(num_blocks, kv_heads, block, head_dim)
    if buf.dtype != torch.uint8 or buf.numel() != total or not buf.is_contiguous():
        raise ValueError(f"KV buffer must be a contiguous uint8 tensor of {total} bytes")
    if buf.device.type != "cuda":
        raise ValueError("KV buffer must be a device tensor")
    return buf.data_ptr(), buf.data_ptr() + half


def pkv_setup_attn_control_csr(kv_indptr, full_indices, swa_indices, last_page_len, active,
                               block, window, bt_width, positions=None, out=None, stream=None,
                               anchor_lag=0):
    """Control from compressed page lists.  Returns the dict of
    pkv_setup_attn_control plus seq_lens and the padded full table bt_full
    (written into `out` when given, e.g. for graph capture)."""
    B = kv_indptr.shape[0] - 1
    tw = pkv_trimmed_width(window, block, anchor_lag) if window > 0 else 0
    dev = kv_indptr.device
    if out is None:
        out = dict(
            bt_full=torch.empty(max(B, 1), bt_width, dtype=torch.int32, device=dev)[:B],
            seq_lens=torch.empty(B, dtype=torch.int32, device=dev),
            pos_full=torch.empty(B, dtype=torch.int32, device=dev),
            pos_swa=torch.empty(B, dtype=torch.int32, device=dev),
            bt_swa_trim=torch.empty(B, max(tw, 1), dtype=torch.int32, device=dev),
            upd_full=torch.empty(B, dtype=torch.int64, device=dev),
            upd_swa=torch.empty(B, dtype=torch.int64, device=dev),
            pos_abs=torch.empty(B, dtype=torch.int64, device=dev),
        )
    _check(lib().pkv_setup_attn_control_csr(
        B, block, window, anchor_lag, _dev_ptr(kv_indptr, torch.int32, "kv_indptr"),
        _dev_ptr(full_indices, torch.int32, "full_indices"),
        _dev_ptr(swa_indices, torch.int32, "swa_indices") if window > 0 else None,
        _dev_ptr(last_page_len, torch.int32, "last_page_len"),
        _dev_ptr(active, torch.uint8, "active"), _dev_ptr(positions, torch.int64, "positions"),
        _dev_ptr(out["bt_full"], torch.int32, "bt_full"), bt_width, bt_width,
        _dev_ptr(out["seq_lens"], torch.int32, "seq_lens"),
        _dev_ptr(out["pos_full"], torch.int32, "pos_full"),
        _dev_ptr(out["pos_swa"], torch.int32, "pos_swa"),
        _dev_ptr(out["bt_swa_trim"], torch.int32, "bt_swa_trim"), tw,
        _dev_ptr(out["upd_full"], torch.int64, "upd_full"),
        _dev_ptr(out["upd_swa"], torch.int64, "upd_swa"),
        _dev_ptr(out["pos_abs"], torch.int64, "pos_abs"), _stream(stream)))
    return out


def _rope(rope_cos, rope_sin, batch, head_dim):
    """Device pointers of the per-sequence rotary cos/sin (float32 [B, D/2]) or (None, None)."""
    if rope_cos is None and rope_sin is None:
        return None, None
    for t, n in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        if t is None or tuple(t.shape) != (batch, head_dim // 2):
            raise ValueError(f"{n} must be float32 [{batch}, {head_dim // 2}]")
    return (_dev_ptr(rope_cos, torch.float32, "rope_cos"),
            _dev_ptr(rope_sin, torch.float32, "rope_sin"))


def pkv_kv_cache_update(buf, k_new, v_new, slot_idx, block, num_blocks, k_scale, v_scale,
                        k_packed=True, stream=None, rope_cos=None, rope_sin=None):
    """buf: one shared buffer (uint8, K half then V half); k_new/v_new bf16 [B, Hkv, D];
    rope_cos/rope_sin: optional float32 [B, D/2] rotation of K."""
    B, H, D = k_new.shape
    kp, vp = _halves(buf, num_blocks, H, block, D)
    rc, rs = _rope(rope_cos, rope_sin, B, D)
    _check(lib().pkv_kv_cache_update(
        B, H, D, block, num_blocks, _dev_ptr(k_new, torch.bfloat16, "k_new"),
        _dev_ptr(v_new, torch.bfloat16, "v_new"), kp, int(bool(k_packed)), vp,
        _dev_ptr(slot_idx, torch.int64, "slot_idx"), rc, rs, float(k_scale), float(v_scale),
        _stream(stream)))


def pkv_decode_workspace_bytes(batch, q_heads, kv_heads, head_dim, block, table_width, window):
    return _check(lib().pkv_decode_workspace_bytes(batch, q_heads, kv_heads, head_dim, block,
                                                   table_width, window))


def new_workspace(batch, q_heads, kv_heads, head_dim, block, table_width, window, device):
    """A zero-filled workspace for pkv_paged_decode_attn (256-byte aligned by torch)."""
    n = pkv_decode_workspace_bytes(batch, q_heads, kv_heads, head_dim, block, table_width, window)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def pkv_paged_decode_attn(q, buf, block_table, frame_pos, block, num_blocks, window, k_scale,
                          v_scale, sm_scale, kv_heads, table_width=None, out=None,
                          workspace=None, k_packed=True, stream=None, rope_cos=None,
                          rope_sin=None):
    """q bf16 [B, Hq, D]; returns out bf16 [B, Hq, D].  rope_cos/rope_sin: optional
    float32 [B, D/2] rotation of the queries."""
    B, Hq, D = q.shape
    rc, rs = _rope(rope_cos, rope_sin, B, D)
    kp, vp = _halves(buf, num_blocks, kv_heads, block, D)
    width = block_table.shape[1] if table_width is None else table_width
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = new_workspace(B, Hq, kv_heads, D, block, width, window, q.device)
    _check(lib().pkv_paged_decode_attn(
        B, Hq, kv_heads, D, block, num_blocks, window, _dev_ptr(q, torch.bfloat16, "q"), kp,
        int(bool(k_packed)), vp, _dev_ptr(block_table, torch.int32, "block_table"),
        block_table.shape[1], width, _dev_ptr(frame_pos, torch.int32, "frame_pos"), rc, rs,
        float(k_scale), float(v_scale), float(sm_scale), _dev_ptr(out, torch.bfloat16, "out"),
        _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out


def make_step(bufs, ctl, bt_full, batch, q_heads, kv_heads, head_dim, block, window,
              num_blocks, k_packed=True, stacked=None, rope_cos=None, rope_sin=None):
    """Host pkv_step for the layer schedule.  bufs: list of shared buffers (per-buffer
    form) or None with `stacked` (one uint8 tensor of consecutive buffers);
    rope_cos/rope_sin: optional float32 [batch, head_dim/2] rotation of the step."""
    s = PkvStep()
    s.batch, s.q_heads, s.kv_heads, s.head_dim = batch, q_heads, kv_heads, head_dim
    s.block, s.window, s.num_blocks = block, window, num_blocks
    s.k_packed = int(bool(k_packed))
    half, total = pkv_kv_buffer_bytes(num_blocks, kv_heads, block, head_dim)
    keep = []
    if bufs is not None:
        n = len(bufs)
        ka = (_vp * n)(*[b.data_ptr() for b in bufs])
        va = (_vp * n)(*[b.data_ptr() + half for b in bufs])
        keep += [ka, va]
        s.k_bufs = ctypes.cast(ka, ctypes.POINTER(_vp))
        s.v_bufs = ctypes.cast(va, ctypes.POINTER(_vp))
        s.n_buffers = n
    if stacked is not None:
        s.stacked = stacked.data_ptr()
        if bufs is None:
            s.n_buffers = stacked.numel() // total
    s.bt_full = bt_full.data_ptr()
    s.bt_full_stride = bt_full.shape[1]
    s.bt_full_width = bt_full.shape[1]
    s.bt_swa_trim = ctl["bt_swa_trim"].data_ptr()
    s.trim_width = ctl["bt_swa_trim"].shape[1]
    s.pos_full = ctl["pos_full"].data_ptr()
    s.pos_swa = ctl["pos_swa"].data_ptr()
    s.upd_full = ctl["upd_full"].data_ptr()
    s.upd_swa = ctl["upd_swa"].data_ptr()
    s.rope_cos, s.rope_sin = _rope(rope_cos, rope_sin, batch, head_dim)
    keep += [rope_cos, rope_sin]
    s._keep = keep
    return s


def pkv_decode_layer(step, layer, q, k_new, v_new, k_scale, v_scale, sm_scale, out, workspace,
                     stream=None):
    _check(lib().pkv_decode_layer(
        ctypes.byref(step), layer, _dev_ptr(q, torch.bfloat16, "q"),
        _dev_ptr(k_new, torch.bfloat16, "k_new"), _dev_ptr(v_new, torch.bfloat16, "v_new"),
        float(k_scale), float(v_scale), float(sm_scale), _dev_ptr(out, torch.bfloat16, "out"),
        _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out


def pkv_decode_layer_noalloc(step, layer, q, k_new, v_new, k_scale, v_scale, sm_scale, out,
                             stream=None):
    """pkv_decode_layer with the library's own workspace (no allocation)."""
    _check(lib().pkv_decode_layer_noalloc(
        ctypes.byref(step), layer, _dev_ptr(q, torch.bfloat16, "q"),
        _dev_ptr(k_new, torch.bfloat16, "k_new"), _dev_ptr(v_new, torch.bfloat16, "v_new"),
        float(k_scale), float(v_scale), float(sm_scale), _dev_ptr(out, torch.bfloat16, "out"),
        _stream(stream)))
    return out


def pkv_validate_attn_control(seq_lens, active, bt_full, bt_swa, block, window, num_blocks,
                              stream=None):
    """Raises PkvError(PKV_ERR_DATA) on bad tables; synchronous."""
    B = seq_lens.shape[0]
    _check(lib().pkv_validate_attn_control(
        B, block, window, num_blocks, _dev_ptr(seq_lens, torch.int32, "seq_lens"),
        _dev_ptr(active, torch.uint8, "active"), _dev_ptr(bt_full, torch.int32, "bt_full"),
        bt_full.shape[1], _dev_ptr(bt_swa, torch.int32, "bt_swa") if window > 0 else None,
        bt_swa.shape[1] if window > 0 else 0, bt_full.shape[1], _stream(stream)))
