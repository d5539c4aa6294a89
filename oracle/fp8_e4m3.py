"""OCP 8-bit floating point, E4M3 flavour ("e4m3fn"): the KV-cache element type.

The giga-kernel page ("GPT-OSS-120B giga-kernel decode", intro and "Kernel
contract") stores the KV cache as packed FP8; the FP8 flavour it uses is read
here as OCP E4M3 with one per-tensor dequantisation scale per K and per V.

Format (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits.
  * exponent field 0:      value = (-1)^s * (m / 8) * 2^(1 - 7)      (subnormal)
  * exponent field 1..15:  value = (-1)^s * (1 + m / 8) * 2^(e - 7)
  * S.1111.111 (0x7F, 0xFF) is NaN; there is no infinity; max finite = 448.

Encoding used by the cache write (a reading, stated in the design notes):
round to nearest, ties to the even code; magnitudes above 448 (and infinities)
saturate to +-448; NaN encodes as 0x7F with the input's sign bit; -0 -> 0x80.
"""
import numpy as np

NAN_CODE = 0x7F
MAX_FINITE = 448.0


def decode_value(code: int) -> float:
    """Value of one E4M3 code from the field definition above (float64)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


def decode_table() -> np.ndarray:
    """All 256 code values as float64, index = code."""
    return np.array([decode_value(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
# Non-negative finite codes 0x00..0x7E have strictly increasing values.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _TABLE[:0x7F]


def decode(codes) -> np.ndarray:
    """Element-wise decode of a uint8 array to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_scalar(y: float) -> int:
    """Nearest E4M3 code of one float (round half to even code, saturating)."""
    y = float(y)
    if np.isnan(y):
        return NAN_CODE | (0x80 if np.signbit(y) else 0)
    sign = 0x80 if np.signbit(y) else 0
    a = min(abs(y), MAX_FINITE)
    # index of the first representable magnitude >= a
    hi = int(np.searchsorted(_POS_VALUES, a, side="left"))
    if _POS_VALUES[hi] == a:
        return sign | int(_POS_CODES[hi])
    lo = hi - 1
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    if d_lo < d_hi:
        pick = lo
    elif d_hi < d_lo:
        pick = hi
    else:  # exact tie: the code whose mantissa LSB is 0
        pick = lo if (int(_POS_CODES[lo]) & 1) == 0 else hi
    return sign | int(_POS_CODES[pick])


def encode(values) -> np.ndarray:
    """Element-wise encode of a float array to uint8 codes (vectorised
    ``encode_scalar``: same nearest-value search and tie rule).

    The inputs are taken as exact float64 values; callers that quantise fp32
    quotients must do the fp32 division themselves (see ``quantize``).
    """
    v = np.asarray(values, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(np.nan_to_num(v, nan=0.0)), MAX_FINITE)
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    lo_even = (_POS_CODES[lo] & 1) == 0
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo_even, lo, hi)))
    pick = np.where(_POS_VALUES[hi] == a, hi, pick)
    code = sign | _POS_CODES[pick]
    code = np.where(np.isnan(v), NAN_CODE | sign, code)
    return code.astype(np.uint8)


def quantize(x_f32, scale: float) -> np.ndarray:
    """Cache code of x under dequant multiplier ``scale``: E(fp32(x) / fp32(scale)).

    The quotient is the IEEE fp32 round-to-nearest-even division (numpy's
    float32 / float32), so the rounding decision is taken in fp32 on both the
    device and here.
    """
    x32 = np.asarray(x_f32, dtype=np.float32)
    q32 = x32 / np.float32(scale)
    return encode(q32.astype(np.float64))
