"""Pins of the oracle's rotary embedding (CPU only).

Each pin comes from outside the oracle's own formula: complex multiplication,
the relative-position property rotary embeddings exist for, exact quarter
turns, an fp32 rounding bound, and a hand-built case where a fused
multiply-add would round differently.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8_e4m3 as E
from oracle import rope as R
from oracle import update as U
from paged_build import bf16_values, build_halves, random_codes, rope_fma_trap


def _angles(pos, D, base=10000.0):
    inv = base ** (-2.0 * np.arange(D // 2) / D)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv


def test_is_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 64))
    th = rng.uniform(-np.pi, np.pi, (5, 1, 32))
    z = (x[..., :32] + 1j * x[..., 32:]) * np.exp(1j * th)
    want = np.concatenate([z.real, z.imag], axis=-1)
    got = R.rotate(x, np.cos(th), np.sin(th))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_scores_depend_on_relative_position_only():
    """<R(m) q, R(n) k> == <R(m - n) q, k> for angles linear in the position."""
    rng = np.random.default_rng(1)
    D = 64
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n in [(7, 3), (1000, 999), (3, 7), (123456, 100)]:
        tm, tn, td = _angles(m, D), _angles(n, D), _angles(m - n, D)
        lhs = R.rotate(q, np.cos(tm), np.sin(tm)) @ R.rotate(k, np.cos(tn), np.sin(tn))
        rhs = R.rotate(q, np.cos(td), np.sin(td)) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_orthogonal_and_invertible():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 64))
    th = rng.uniform(-10, 10, (4, 32))
    y = R.rotate(x, np.cos(th), np.sin(th))
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    back = R.rotate(y, np.cos(th), -np.sin(th))
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-13)


@pytest.mark.parametrize("fn", [R.rotate, R.rotate_f32])
def test_exact_quarter_turns(fn):
    rng = np.random.default_rng(3)
    x = bf16_values(rng, (6, 64)).astype(np.float32)
    a, b = x[:, :32], x[:, 32:]
    one, zero = np.ones((6, 32), np.float32), np.zeros((6, 32), np.float32)
    assert np.array_equal(fn(x, one, zero), x)
    assert np.array_equal(fn(x, zero, one), np.concatenate([-b, a], axis=-1))
    assert np.array_equal(fn(x, -one, zero), -x)
    assert np.array_equal(fn(x, zero, -one), np.concatenate([b, -a], axis=-1))


def test_f32_within_three_roundings_of_exact():
    rng = np.random.default_rng(4)
    x = bf16_values(rng, (64, 8, 64)).astype(np.float32)
    th = rng.uniform(-1e5, 1e5, (64, 1, 32))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    got = R.rotate_f32(x, c, s).astype(np.float64)
    want = R.rotate(x, c, s)  # exact up to fp64 rounding: same fp32 inputs
    a, b = x[..., :32].astype(np.float64), x[..., 32:].astype(np.float64)
    mag = np.concatenate([np.abs(a * c) + np.abs(b * s), np.abs(b * c) + np.abs(a * s)], axis=-1)
    u = 2.0 ** -24
    bound = u * mag * (1 + u) + u * np.abs(want) * (1 + 2 * u) + 1e-300
    assert np.all(np.abs(got - want) <= bound)
    assert np.any(got != want)  # it is the fp32 evaluation, not the exact one


def test_f32_rounds_each_product_before_the_sum():
    """A fused multiply-add would give 1.0625 + 2^-23 (another FP8 code) at each trap."""
    x, c, s, traps = rope_fma_trap()
    got = R.rotate_f32(x, c, s)
    exact = R.rotate(x, c, s)
    for r, d in traps:
        assert exact[r, d] == 1.0625 + 2.0 ** -24 + 2.0 ** -40
        assert got[r, d] == np.float32(1.0625)
    assert int(E.quantize(np.float32(1.0625), 1.0)) == 0x38
    assert int(E.quantize(np.float32(1.0625 + 2.0 ** -23), 1.0)) == 0x39


def test_update_rotates_k_only():
    rng = np.random.default_rng(5)
    nb, H, Bk, D, B = 4, 2, 8, 64, 2
    k = bf16_values(rng, (B, H, D))
    v = bf16_values(rng, (B, H, D))
    slots = np.array([Bk + 3, 2 * Bk], np.int64)
    zero, one = np.zeros((B, 32), np.float32), np.ones((B, 32), np.float32)
    # a quarter turn on every pair == writing [-k_hi, k_lo] without rotation
    kh1 = np.zeros(nb * H * Bk * D, np.uint8)
    vh1 = kh1.copy()
    U.kv_cache_update(kh1, vh1, k, v, slots, Bk, 0.125, 0.0625, True, zero, one)
    kh2, vh2 = kh1.copy() * 0, vh1.copy() * 0
    turned = np.concatenate([-k[..., 32:], k[..., :32]], axis=-1)
    U.kv_cache_update(kh2, vh2, turned, v, slots, Bk, 0.125, 0.0625, True)
    assert np.array_equal(kh1, kh2) and np.array_equal(vh1, vh2)


def test_attention_rotates_every_query_head():
    rng = np.random.default_rng(6)
    B, Hq, H, Bk, D, L = 2, 4, 2, 4, 64, 11
    nb = 2 * (-(-L // Bk)) + 1
    table = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    k_log = [random_codes(rng, (L, H, D)) for _ in range(B)]
    v_log = [random_codes(rng, (L, H, D), 1.0 / 16) for _ in range(B)]
    kh, vh = build_halves(k_log, v_log, [table[0], table[1]], nb, H, Bk, D, True)
    q = bf16_values(rng, (B, Hq, D))
    th = rng.uniform(-np.pi, np.pi, (B, 32))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    pos = np.array([L - 1, L - 1])
    got = A.paged_decode_attention(q, kh, vh, table, pos, 0, Bk, H, 0.125, 0.0625, 0.125,
                                   rope_cos=c, rope_sin=s)
    z = (q[..., :32] + 1j * q[..., 32:]) * (c + 1j * s.astype(np.float64))[:, None, :]
    qr = np.concatenate([z.real, z.imag], axis=-1)
    want = A.paged_decode_attention(qr, kh, vh, table, pos, 0, Bk, H, 0.125, 0.0625, 0.125)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    plain = A.paged_decode_attention(q, kh, vh, table, pos, 0, Bk, H, 0.125, 0.0625, 0.125)
    assert np.abs(got - plain).max() > 1e-3
