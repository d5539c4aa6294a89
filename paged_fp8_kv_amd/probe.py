"""Thin Python binding of libpkv_probe (include/pkv_probe.h): HBM
read-bandwidth probes, the measured ceiling the decode kernels are compared
with.  Argument marshalling only; each call enqueues one probe launch on
torch's current HIP stream and returns the bytes it reads."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv_probe.so")

PKV_PROBE_ERR_ARG = -1
PKV_PROBE_ERR_HIP = -4

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p

_SIGS = {
    "pkv_probe_stream_read": ([_vp, _i64, _i32, _i32, _vp, _vp], _i64),
    "pkv_probe_tile_read_bytes": ([_i64, _i32, _i32], _i64),
    "pkv_probe_tile_read": ([_vp, _i64, _i32, _i32, _i32, _vp, _vp], _i64),
}

_lib = None


def lib():
    """The loaded libpkv_probe (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m paged_fp8_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _check(n, what):
    if n < 0:
        raise RuntimeError(f"{what}: status {n}")
    return n


def _args(buf, sink, grid):
    if buf.device.type != "cuda" or sink.device.type != "cuda":
        raise ValueError("buffer and sink must be device tensors")
    if buf.dtype != torch.uint8 or not buf.is_contiguous():
        raise ValueError("buffer must be a contiguous uint8 tensor")
    if sink.dtype != torch.int32 or not sink.is_contiguous() or sink.numel() < grid:
        raise ValueError("sink must be a contiguous int32 tensor of at least `grid` elements")
    return buf.data_ptr(), buf.numel(), sink.data_ptr(), torch.cuda.current_stream().cuda_stream


def pkv_probe_stream_read(buf, grid, nontemporal, sink):
    p, n, s, st = _args(buf, sink, grid)
    return _check(lib().pkv_probe_stream_read(p, n, grid, int(bool(nontemporal)), s, st),
                  "pkv_probe_stream_read")


def pkv_probe_tile_read_bytes(nbytes, tile_bytes, grid):
    return _check(lib().pkv_probe_tile_read_bytes(nbytes, tile_bytes, grid), "pkv_probe_tile_read_bytes")


def pkv_probe_tile_read(buf, tile_bytes, grid, nontemporal, sink):
    p, n, s, st = _args(buf, sink, grid)
    return _check(lib().pkv_probe_tile_read(p, n, tile_bytes, grid, int(bool(nontemporal)), s, st),
                  "pkv_probe_tile_read")
