// Device-side element codecs for gfx950: bf16, e4m3fn, e2m1, e8m0.
//
// The formats are the OCP ones the "Low-Latency Mode API" page names for its
// receive buffers (float8_e4m3fn data, float4_e2m1fn_x2 data, float8_e8m0fnu
// scales) and IEEE bf16.  All roundings are round-to-nearest, ties to even.
// The conversions use gfx950's hardware convert instructions.  Each wrapper
// states the inputs it is exact for; tests/test_gpu_codecs.py runs every
// wrapper over that whole domain (every code with every scale byte, every
// finite bf16 with every scale exponent, every rounding tie) and compares it
// bit for bit with the oracle's software codecs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ep {

// bf16 <-> f32 ---------------------------------------------------------------

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two float32 -> two bf16 (round to nearest even), element `lo` in bits 0-15.
// gfx950 converts in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// e8m0 -----------------------------------------------------------------------

// 2^(b-127) as float32; b = 0 gives the subnormal 2^-127; 0xFF is NaN.
__device__ __forceinline__ float e8m0_decode(uint32_t b) {
  uint32_t bits = b ? b << 23 : 0x00400000u;
  bits = b == 0xffu ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// floor(log2(a)) of a positive finite float32 given by its bits (subnormals
// included).
__device__ __forceinline__ int floor_log2_bits(uint32_t a) {
  const int ef = (int)(a >> 23);
  return ef ? ef - 127 : (31 - __builtin_clz(a)) - 149;
}

// ceil(log2 v) of a positive finite float32 from its bits `a`: floor, plus
// one unless v is a power of two (a normal with zero mantissa, or a
// subnormal with a single bit set)
__device__ __forceinline__ int ceil_log2_bits(uint32_t a) {
  const uint32_t mant = a & 0x7fffffu;
  const bool pow2 = (a >> 23) ? mant == 0 : (mant & (mant - 1)) == 0;
  return floor_log2_bits(a) + (pow2 ? 0 : 1);
}

// e4m3fn (bias 7, 3 mantissa bits, largest finite 448, no infinity) -----------
//
// gfx950's fp8 conversions use this OCP format.  The encoder below is exact
// round-to-nearest-even for every float32 input already clamped to +-448
// (the instruction itself would turn larger values into NaN instead of
// saturating, hence the clamp in the callers); the decoders are exact.
// Byte i of a word holds element i.

// 8 float32 (clamped to +-448) -> 8 codes, elements 0-3 in word 0.
__device__ __forceinline__ u32x2 e4m3x8_encode(const float (&v)[8]) {
  uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
  uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
  return u32x2{w0, w1};
}

// 8 codes -> exact float32 values.
__device__ __forceinline__ void e4m3x8_decode(const u32x2 &w, float (&y)[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
    y[4 * i] = a.x; y[4 * i + 1] = a.y; y[4 * i + 2] = b.x; y[4 * i + 3] = b.y;
  }
}

// 8 codes times the power of two `scale` (exact unless the product leaves
// float32's range).
__device__ __forceinline__ void e4m3x8_decode_scaled(const u32x2 &w, float scale, float (&y)[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], scale, false);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], scale, true);
    y[4 * i] = a.x; y[4 * i + 1] = a.y; y[4 * i + 2] = b.x; y[4 * i + 3] = b.y;
  }
}

// e2m1 (bias 1, 1 mantissa bit: 0 .5 1 1.5 2 3 4 6) --------------------------
//
// Nibble 2i of a word (low nibble of byte i) holds element 2i.

// 8 bf16 (4 words, element 2i in the low half of word i) divided by the power
// of two `scale` and rounded to e2m1, nearest even, saturating at +-6, sign
// kept.  One instruction per pair; exact for every finite bf16 input and
// every scale 2^-127 .. 2^126.
__device__ __forceinline__ uint32_t e2m1x8_encode_bf16(const u32x4 &r, float scale) {
  // copy the words to scalars first: bit-casting a vector element in place
  // makes this compiler pass element 0 to every call
  const uint32_t w0 = r.x, w1 = r.y, w2 = r.z, w3 = r.w;
  uint32_t q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, w0), scale, 0);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2, w1), scale, 1);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2, w2), scale, 2);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2, w3), scale, 3);
  return q;
}

// 8 nibbles times the power of two `scale`.
__device__ __forceinline__ void e2m1x8_decode_scaled(uint32_t w, float scale, float (&y)[8]) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
  y[0] = a.x; y[1] = a.y; y[2] = b.x; y[3] = b.y; y[4] = c.x; y[5] = c.y; y[6] = d.x; y[7] = d.y;
}

}  // namespace ep
