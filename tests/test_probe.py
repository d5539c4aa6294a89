"""The HBM read-bandwidth probes (libpkv_probe): exports, size arithmetic and
argument checks on the CPU; on the GPU, that each probe reads every byte it
says it reads exactly once (the XOR of the per-workgroup words it stores
equals the host's XOR of the same bytes)."""
import os
import re

import numpy as np
import pytest

from paged_fp8_kv_amd import probe as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "pkv_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    syms = sorted(set(re.findall(r"\b(pkv_probe_[a-z_]+)\s*\(", text)))
    assert syms == sorted(Q._SIGS)
    L = Q.lib()
    for s in syms:
        assert hasattr(L, s), s


@pytest.mark.parametrize("nbytes,tile,grid", [(1 << 26, 2048, 64), (1 << 32, 2048, 1024),
                                              (1 << 32, 16384, 2048), (1 << 20, 1024, 7),
                                              (1 << 14, 16384, 1)])
def test_tile_bytes_are_whole_groups(nbytes, tile, grid):
    n = Q.pkv_probe_tile_read_bytes(nbytes, tile, grid)
    waves, group = grid * 4, 16384 // tile
    per_wave = n // tile // waves
    assert n % (tile * waves) == 0 and per_wave % group == 0
    assert n <= nbytes < n + waves * group * tile  # as many whole groups as fit


def test_argument_errors():
    L = Q.lib()
    assert L.pkv_probe_tile_read_bytes(3 << 20, 2048, 8) == Q.PKV_PROBE_ERR_ARG   # not a power of two
    assert L.pkv_probe_tile_read_bytes(1 << 20, 512, 8) == Q.PKV_PROBE_ERR_ARG
    assert L.pkv_probe_tile_read_bytes(1 << 20, 32768, 8) == Q.PKV_PROBE_ERR_ARG
    assert L.pkv_probe_tile_read_bytes(1 << 20, 3072, 8) == Q.PKV_PROBE_ERR_ARG
    assert L.pkv_probe_tile_read_bytes(1 << 20, 2048, 0) == Q.PKV_PROBE_ERR_ARG
    # rejected before any launch: null, misaligned, bad sizes
    assert L.pkv_probe_stream_read(None, 1 << 20, 8, 1, 0x1000, None) == Q.PKV_PROBE_ERR_ARG
    assert L.pkv_probe_stream_read(0x1008, 1 << 20, 8, 1, 0x1000, None) == Q.PKV_PROBE_ERR_ARG
    assert L.pkv_probe_stream_read(0x1000, 1000, 8, 1, 0x1000, None) == Q.PKV_PROBE_ERR_ARG
    assert L.pkv_probe_stream_read(0x1000, 1 << 20, 8, 1, None, None) == Q.PKV_PROBE_ERR_ARG
    assert L.pkv_probe_tile_read(0x1000, 1 << 20, 2048, 8, 1, None, None) == Q.PKV_PROBE_ERR_ARG


def _xor_words(a):
    return int(np.bitwise_xor.reduce(a.view(np.uint32)))


@pytest.mark.gpu
@pytest.mark.parametrize("nt", [0, 1])
def test_gpu_probes_read_every_byte_once(gpu, nt):
    import torch
    g = torch.Generator(device="cpu").manual_seed(11)
    host = torch.randint(0, 256, (1 << 26,), dtype=torch.uint8, generator=g)
    buf = host.to(gpu)
    sink = torch.zeros(1024, dtype=torch.int32, device=gpu)
    cases = [
        ("stream whole", lambda: Q.pkv_probe_stream_read(buf, 1024, nt, sink), host.numpy()),
        # ragged: a tail of loads outside the unrolled loop
        ("stream ragged", lambda: Q.pkv_probe_stream_read(buf[: (1 << 26) - 4096 * 16 - 48], 96, nt, sink),
         host.numpy()[: (1 << 26) - 4096 * 16 - 48]),
        # 2^15 tiles of 2 KiB, 256 waves x 128 tiles: every tile once
        ("tiles 2K", lambda: Q.pkv_probe_tile_read(buf, 2048, 64, nt, sink), host.numpy()),
        ("tiles 16K", lambda: Q.pkv_probe_tile_read(buf, 16384, 32, nt, sink), host.numpy()),
    ]
    for name, run, ref in cases:
        sink.zero_()
        n = run()
        torch.cuda.synchronize()
        assert n == ref.size, name
        got = _xor_words(sink.cpu().numpy())
        assert got == _xor_words(ref), name
