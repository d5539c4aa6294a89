"""Rotary position embedding of the new token's query and key.

"GPT-OSS-120B giga-kernel decode", section "Kernel contract": among the
layer-invariant attention-control tensors the kernel takes every step are the
RoPE cosines and sines, next to the absolute positions they come from.  The
pages give neither the pairing of dimensions nor the frequency schedule.

Readings (design notes):
  * cos/sin arrive per sequence for this step: ``cos[b, i]`` and ``sin[b, i]``,
    ``i < D/2``, are the cosine and sine of frequency ``i``'s angle at sequence
    ``b``'s absolute position; the caller builds them with its own frequency
    schedule.  One rotation serves every head of ``q`` and of the new ``k``;
    ``v`` is not rotated.
  * half-split pairing: dimension ``i`` pairs with ``i + D/2``, and the pair is
    turned by that angle -- as a complex number ``z_i = x_i + j x_{i+D/2}``
    is multiplied by ``cos + j sin``:
    ``x_i' = x_i cos - x_{i+D/2} sin``, ``x_{i+D/2}' = x_{i+D/2} cos + x_i sin``.
  * the rotated key goes straight from fp32 to its FP8 code (no bf16 rounding
    between); the fp32 rotation rounds each product to fp32, then their sum
    (no fused multiply-add), so the code is decided in one stated precision.

Parity pins: ``tests/test_oracle_rope.py`` (complex-multiply form, relative
position property, orthogonality, quarter turns, fp32 error bound).
"""
import numpy as np


def _split(x):
    x = np.asarray(x)
    h = x.shape[-1] // 2
    if 2 * h != x.shape[-1]:
        raise ValueError("head size must be even")
    return x[..., :h], x[..., h:]


def rotate(x, cos, sin):
    """Rotated copy of ``x`` in float64.

    x: [..., D]; cos, sin: broadcastable to [..., D/2].
    """
    a, b = _split(np.asarray(x, dtype=np.float64))
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rotate_f32(x, cos, sin):
    """Rotated copy of ``x`` in float32, one rounding per product and per sum.

    numpy's float32 multiply, subtract and add are single IEEE operations
    rounded to nearest even, and numpy never fuses them.
    """
    a, b = _split(np.asarray(x, dtype=np.float32))
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    lo = (a * c) - (b * s)
    hi = (b * c) + (a * s)
    return np.concatenate([lo, hi], axis=-1).astype(np.float32)
