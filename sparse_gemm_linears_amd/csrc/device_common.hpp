// Device helpers shared by the fp8lin kernels (gfx950 only).
//
// Number formats: bf16 in/out (raw 16-bit patterns), OCP E4M3FN codes, fp32
// scales.  The e4m3 encoder works on the fp32 bit pattern with integer
// arithmetic: round to nearest, ties to even, saturating at +-448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

constexpr int kGroup = 128;  // activation group / weight block edge

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> E4M3FN code: RNE, saturating, NaN -> S|0x7F.
//  * normal range (|v| >= 2^-6): round the 23-bit mantissa to 3 bits on the
//    fp32 pattern; the carry moves into the exponent; rebias 127 -> 7.
//  * subnormal range: |v| * 2^9 is exact in fp32 and rint() rounds it to the
//    integer code 0..8 (8 is 2^-6, the smallest normal, code 0x08).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (a > 0x43E00000u) return sign | 0x7Eu;  // above 448 (and inf): saturate
  if (a >= 0x3C800000u) {                     // >= 2^-6
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - (120u << 3));
  }
  float f = __uint_as_float(a) * 512.0f;
  return sign | (uint32_t)__builtin_rintf(f);
}

// Code of x in a group with scale s = amax/448.  s == 0 only when every value
// of the group is +-0: the code is then the signed zero.  x / s is an IEEE
// (correctly rounded) fp32 division.
__device__ __forceinline__ uint32_t quantize(float x, float s) {
  return e4m3_encode(s == 0.0f ? x : x / s);
}

// |bf16| as an integer: ordering of non-NaN magnitudes is the integer ordering.
__device__ __forceinline__ uint32_t bf16_abs_bits(uint32_t b16) { return b16 & 0x7FFFu; }

// v_mfma_f32_16x16x128_f8f6f4 with both operands e4m3 and no block scale.
// A: 16 rows x 128 K, B: 128 K x 16 columns; lane l holds row / column l%16 and
// 32 K-bytes; D: lane l holds column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i &a, const v8i &b, const v4f &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace fp8lin
