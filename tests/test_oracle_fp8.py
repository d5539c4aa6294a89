"""Pins of the oracle's OCP E4M3 codec (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8_e4m3 as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch_all_codes():
    ours, ref = F.decode_table(), torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_spec_values():
    g = json.load(open(os.path.join(GOLD, "e4m3_code_values.json")))
    for code, v in g["values"].items():
        assert F.decode_value(int(code, 16)) == v, code
    for code in g["nan_codes"]:
        assert math.isnan(F.decode_value(int(code, 16)))
    nz = F.decode_value(int(g["negative_zero_code"], 16))
    assert nz == 0.0 and math.copysign(1.0, nz) < 0


def test_encode_roundtrip_all_finite_codes():
    vals = F.decode_table()
    for c in range(256):
        if math.isnan(vals[c]):
            continue
        assert F.encode_scalar(vals[c]) == c
    fin = ~np.isnan(vals)
    assert np.array_equal(F.encode(vals[fin]), np.arange(256)[fin].astype(np.uint8))


def _midpoints():
    v = np.sort(np.unique(F.decode_table()[:0x7F]))
    mids = (v[:-1] + v[1:]) / 2
    return v, mids


def test_encode_matches_torch_near_every_midpoint():
    v, mids = _midpoints()
    pts = []
    for m in mids:
        m32 = np.float32(m)
        pts += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))]
    pts = np.array(pts + list(v.astype(np.float32)), dtype=np.float32)
    pts = pts[np.abs(pts) <= 464]
    allp = np.concatenate([pts, -pts])
    assert np.array_equal(F.encode(allp.astype(np.float64)), torch_encode(allp))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(123)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-3, 0.1, 1, 8, 60)])
    x = x[np.abs(x) <= 464]
    assert np.array_equal(F.encode(x.astype(np.float64)), torch_encode(x))


def test_scalar_and_vector_encoders_agree():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(3000) * 30).astype(np.float32)
    assert [F.encode_scalar(float(t)) for t in x] == list(F.encode(x.astype(np.float64)))


def test_saturation_nan_and_signed_zero():
    assert list(F.encode([448.0, 455.0, 465.0, 1e6, math.inf])) == [0x7E] * 5
    assert list(F.encode([-465.0, -math.inf])) == [0xFE] * 2
    assert F.encode_scalar(float("nan")) == 0x7F
    assert F.encode_scalar(-float("nan")) == 0xFF
    assert F.encode_scalar(-0.0) == 0x80
    assert F.encode_scalar(0.0) == 0x00
    # ties to even at the subnormal end: 2^-10 sits between 0 and 2^-9
    assert F.encode_scalar(2.0 ** -10) == 0x00
    assert F.encode_scalar(3 * 2.0 ** -10) == 0x02


def test_encode_monotone():
    x = np.linspace(-460, 460, 200001)
    vals = F.decode(F.encode(x))
    assert np.all(np.diff(vals) >= 0)


@pytest.mark.parametrize("scale", [1.0 / 8, 1.0 / 16, 0.0173])
def test_quantize_is_fp32_division_then_encode(scale):
    rng = np.random.default_rng(9)
    x = torch.randn(50000, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).float().numpy()
    ref = torch_encode(torch.from_numpy(x).div(torch.tensor(scale, dtype=torch.float32)).numpy())
    keep = np.abs(x / np.float32(scale)) <= 464
    got = F.quantize(x, scale)
    assert np.array_equal(got[keep], ref[keep])
    del rng
