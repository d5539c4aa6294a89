// Device-side helpers shared by the libpkv kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kHeadDim = 64;  // the only head size the kernels are built for

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Half-split rotary turn of one element: x at dimension d, xp its partner at
// d ^ (D/2), `upper` when d >= D/2, (c, s) the cosine and sine of the pair's
// angle.  The lower element becomes x*c - xp*s, the upper one x*c + xp*s
// (the pair, as x_lo + j*x_hi, times c + j*s).  Each product is rounded to
// fp32 before the sum (contraction off), so the value -- and an FP8 code
// taken from it -- is one defined fp32 result.
__device__ __forceinline__ float rope_turn(float x, float xp, float c, float s, bool upper) {
#pragma clang fp contract(off)
  const float xc = x * c;
  const float ps = xp * s;
  return upper ? xc + ps : xc - ps;
}

// OCP E4M3 code of an fp32 value: round to nearest, ties to the even code,
// |y| >= 448 (and +-inf) saturate to 0x7E|sign, NaN -> 0x7F|sign.
// Positive codes 0x00..0x7E are monotone in value with a carry-continuous
// (exponent,mantissa) field, so rounding up never needs a separate carry.
__device__ __forceinline__ uint8_t f32_to_e4m3_rne_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return static_cast<uint8_t>(sign | 0x7fu);
  if (mag >= 0x43e00000u) return static_cast<uint8_t>(sign | 0x7eu);  // >= 448
  const uint32_t ef = mag >> 23;                                     // biased fp32 exponent
  uint32_t code;
  if (ef < 121u) {
    // below 2^-6: multiples of 2^-9; scaling by 2^9 is exact, rintf rounds half-even
    code = static_cast<uint32_t>(rintf(__uint_as_float(mag) * 512.0f));
  } else {
    const uint32_t m = mag & 0x7fffffu;
    code = ((ef - 120u) << 3) | (m >> 20);
    const uint32_t rem = m & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;
  }
  return static_cast<uint8_t>(sign | code);
}

// Two FP8 codes (16-bit word HI_WORD of `w`) -> two fp16 / bf16, exactly
// (every E4M3 value is representable in both).
template <bool HI_WORD>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  f16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI_WORD);
  return __builtin_bit_cast(uint32_t, r);
}
template <bool HI_WORD>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI_WORD);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace pkv
