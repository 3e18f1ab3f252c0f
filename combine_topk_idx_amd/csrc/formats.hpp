// Device-side element codecs for gfx950: bf16, e4m3fn, e2m1, e8m0.
//
// Written from the public OCP definitions of the formats the "Low-Latency
// Mode API" page names for its receive buffers (float8_e4m3fn data,
// float4_e2m1fn_x2 data, float8_e8m0fnu scales) and from IEEE bf16.  All
// roundings are round-to-nearest, ties to even.  Encoders take float32 input
// already clamped to the format's largest finite value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

// bf16 <-> f32 ---------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even on the 16 dropped bits; NaN becomes a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// e4m3fn: bias 7, 3 mantissa bits, largest finite 448 ---------------------------

// |v| <= 448.  Below 2^-6 the format is subnormal with step 2^-9: scale by
// 2^9 (exact) and round to an integer.  Otherwise round the float32 mantissa
// to 3 bits with the usual add-half-minus-one-plus-lsb trick on the bit
// pattern (a carry propagates into the exponent) and rebias 127 -> 7.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t mag;
  if (a < 0x3c800000u) {
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    mag = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | mag;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t sign = (c & 0x80u) << 24;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;                               // m * 2^-9, exact
  } else if (e == 15 && m == 7) {
    mag = __uint_as_float(0x7fc00000u);
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// e2m1: bias 1, 1 mantissa bit, values 0 .5 1 1.5 2 3 4 6 ------------------------

// |v| <= 6.  Below 1 the step is 0.5 (subnormal); otherwise round the mantissa
// to one bit and rebias 127 -> 1.  Returns the 4-bit code, sign in bit 3.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 28) & 0x8u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t mag;
  if (a < 0x3f800000u) {
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
  } else {
    mag = ((a + 0x1fffffu + ((a >> 22) & 1u)) >> 22) - (126u << 1);
  }
  return sign | mag;
}

__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  // magnitudes x2: 0 1 2 3 4 6 8 12, halved exactly
  const uint32_t twice = (0xC8643210u >> ((c & 7u) * 4u)) & 0xFu;
  const float mag = (float)twice * 0.5f;
  return (c & 8u) ? -mag : mag;
}

// e8m0 -----------------------------------------------------------------------

// 2^(b-127) as float32; b = 0 gives the subnormal 2^-127; 0xFF is NaN.
__device__ __forceinline__ float e8m0_decode(uint32_t b) {
  if (b == 0xffu) return __uint_as_float(0x7fc00000u);
  if (b == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(b << 23);
}

// floor(log2(a)) of a positive finite float32 given by its bits (subnormals
// included).
__device__ __forceinline__ int floor_log2_bits(uint32_t a) {
  const int ef = (int)(a >> 23);
  return ef ? ef - 127 : (31 - __builtin_clz(a)) - 149;
}

}  // namespace ep
