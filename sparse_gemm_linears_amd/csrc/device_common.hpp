// Device helpers shared by the fp8lin kernels (gfx950 only).
//
// Number formats: bf16 in/out (raw 16-bit patterns), OCP E4M3FN codes, fp32
// scales.  Encoding to e4m3 rounds to nearest, ties to even, and saturates at
// +-448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

constexpr int kGroup = 128;  // activation group / weight block edge

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

typedef float v4f __attribute__((ext_vector_type(4)));

// A 16-byte load of data that is read once, with the non-temporal hint.  A
// streaming read over rotated copies of >= 1 GiB (timing probe on MI355X, 512
// workgroups, each load instruction covering whole 128-byte lines) took
// 18.1 us for 117 MB with it and 20.4 us without (6.5 against 5.7 TB/s);
// 59 MB: 10.4 against 11.4 us.  Used where a wave's load covers whole lines
// and A/B timing agreed: the decode weights read in whole rows, the weight
// quantizers' and the 2:4 pruner's inputs.  Loads that take a line in two
// halves (MFMA fragments of 64-byte runs) and the activation quantizer were
// slower with it.
__device__ __forceinline__ uint4 ldg16_stream(const void *p) {
  const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16, round to nearest even, by gfx950's v_cvt_pk_bf16_f32 (two
// values per instruction).  An in-bounds probe on MI355X compared it with the
// integer form (u + 0x7FFF + ((u >> 16) & 1)) >> 16 on all 2^32 fp32 bit
// patterns: equal on every non-NaN input; NaNs come out as quiet NaNs (the
// integer form turns some into infinities).
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t{lo, hi}), v2bf_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// Four E4M3FN codes packed little-endian into one word, from four fp32
// values, with the hardware conversion v_cvt_pk_fp8_f32: round to nearest
// even; the inputs are first clamped to +-448, which makes it saturating.  On
// gfx950 this equals an integer RNE-saturating encoder on every non-NaN input
// (checked over all exponents on a 2^-11-relative grid, +-40 ulp around every
// midpoint and 2M random values).
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
  q0 = __builtin_amdgcn_fmed3f(q0, -448.0f, 448.0f);
  q1 = __builtin_amdgcn_fmed3f(q1, -448.0f, 448.0f);
  q2 = __builtin_amdgcn_fmed3f(q2, -448.0f, 448.0f);
  q3 = __builtin_amdgcn_fmed3f(q3, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  return (uint32_t)w;
}

// Exact codes of four values of a group with scale s (IEEE divisions).
__device__ __forceinline__ uint32_t quantize4_exact(const float (&x)[4], float s) {
  float q[4];
#pragma unroll
  for (int j = 0; j < 4; j++) q[j] = s == 0.0f ? x[j] : x[j] / s;
  return e4m3_pack4(q[0], q[1], q[2], q[3]);
}

// Fast codes of four values: qa = x * rs with rs = rcp(s) (v_rcp_f32, within
// 1 ulp) is within 2 ulp of the correctly rounded quotient fl(x / s) (4 ulp
// across a binade edge), so the e4m3 rounding of qa and of fl(x / s) can only
// differ when qa lies that close to an e4m3 rounding midpoint.  Midpoints of
// the normal range have the 20 bits below the 3 kept mantissa bits equal to
// 0x80000; `need` gets a non-zero bit when some qa is within 8 ulp of one, or
// lies in the e4m3 subnormal range (0 < |qa| < 2^-6): the caller must then use
// quantize4_exact for these values.
__device__ __forceinline__ uint32_t quantize4_fast(const float (&x)[4], float rs, uint32_t &need) {
  float q[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    q[j] = x[j] * rs;
    const uint32_t b = __float_as_uint(q[j]);
    const uint32_t t = b & 0x7FFFFFFFu;
    need |= (((b & 0xFFFFFu) - 0x7FFF8u) < 17u) | ((t - 1u) < 0x3C7FFFFFu);
  }
  return e4m3_pack4(q[0], q[1], q[2], q[3]);
}

// Scales for which the fast path is valid: 2^-100 <= s < inf (rs finite, no
// overflow or underflow in x * rs for bf16 x with |x| <= 448 s).
__device__ __forceinline__ bool scale_fast_ok(float s) {
  const uint32_t b = __float_as_uint(s);
  return b >= 0x0D800000u && b < 0x7F800000u;
}

// UE8M0 (power-of-two) scales: byte e stands for 2^(e - 127).  The exponent of
// a group is the smallest e >= 0 with 448 * 2^(e - 127) >= amax.  With amax =
// (1 + f) 2^(E - 127) (fp32 fields E, f; 448 = 1.75 * 2^8) that is E - 8, plus
// one when f > 0.75, clamped at 0 (zero, subnormal and tiny groups).
__device__ __forceinline__ uint32_t ue8m0_exponent(uint32_t amax_f32_bits) {
  const int e = (int)(amax_f32_bits >> 23) - 8 + ((amax_f32_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < 0 ? 0u : (uint32_t)e;
}

// 2^(127 - e) as an fp32 normal (e <= 253, which every bf16 amax gives).
__device__ __forceinline__ float ue8m0_inverse(uint32_t e) { return __uint_as_float((254u - e) << 23); }

// Codes of four values with a power-of-two scale: x * 2^(127 - e) is exact
// (or so small that it rounds to a zero code either way), so one hardware RNE
// conversion gives the code of the exact quotient; |x| <= amax never saturates.
__device__ __forceinline__ uint32_t quantize4_pow2(const float (&x)[4], float inv) {
  return e4m3_pack4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
}

// |bf16| as an integer: ordering of non-NaN magnitudes is the integer ordering.
__device__ __forceinline__ uint32_t bf16_abs_bits(uint32_t b16) { return b16 & 0x7FFFu; }

// Codes of the 8 bf16 values packed in raw with one scale sc: the fast path,
// and the exact divisions when some value needs them or sc is out of the fast
// range.
__device__ __forceinline__ uint2 quantize8_scaled(const uint4 &raw, float sc) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  const float rs = __builtin_amdgcn_rcpf(sc);
  float v[2][4];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    v[i][0] = bf16_to_f32(w[2 * i] & 0xFFFFu);
    v[i][1] = __uint_as_float(w[2 * i] & 0xFFFF0000u);
    v[i][2] = bf16_to_f32(w[2 * i + 1] & 0xFFFFu);
    v[i][3] = __uint_as_float(w[2 * i + 1] & 0xFFFF0000u);
  }
  uint32_t need = scale_fast_ok(sc) ? 0u : 1u;
  uint32_t packed[2];
#pragma unroll
  for (int i = 0; i < 2; i++) packed[i] = quantize4_fast(v[i], rs, need);
  if (__builtin_expect(need != 0u, 0)) {
#pragma unroll
    for (int i = 0; i < 2; i++) packed[i] = quantize4_exact(v[i], sc);
  }
  return make_uint2(packed[0], packed[1]);
}

// Largest |x| of the 8 bf16 values packed in raw, as bf16 magnitude bits.
__device__ __forceinline__ uint32_t amax8_bits(const uint4 &raw) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) a = max(a, max(bf16_abs_bits(w[i] & 0xFFFFu), bf16_abs_bits(w[i] >> 16)));
  return a;
}

// Scale of a group whose largest magnitude amax is a bf16 value (given as
// fp32 bits): s = amax / 448 and rs = 1 / s, both IEEE divisions.  For
// 2^-90 <= amax < inf the e4m3 code of fl(x / s), for every bf16 x with
// |x| <= amax, equals the code of the quotient corrected once by FMA,
//   q0 = fl(x rs),  q = fl(q0 - fl(q0 s - x) rs)
// (fused operations; an exhaustive check over every such pair of bf16 amax
// and x, both signs; q itself can be one ulp off fl(x / s), but never next
// to an e4m3 rounding midpoint).  The remainder is taken as q0 s - x, not
// x - q0 s, so that x = -0 gives -0 (the other form gives +0 - 0 = +0).
// Below 2^-90 the remainder can underflow and the codes differ in a few
// cases, so zero, tiny and non-finite amax take the IEEE divisions.
struct GroupScale {
  float s, rs;
  bool fast;
};

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_f32_bits) {
  GroupScale g;
  g.s = __uint_as_float(amax_f32_bits) / 448.0f;
  g.rs = 1.0f / g.s;
  g.fast = amax_f32_bits >= 0x12800000u && amax_f32_bits < 0x7F800000u;
  return g;
}

// Codes of four values of a group with g.fast set (see group_scale).
__device__ __forceinline__ uint32_t quantize4_corrected(const float (&x)[4], const GroupScale &g) {
  float q[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const float q0 = x[j] * g.rs;
    const float r = __builtin_fmaf(q0, g.s, -x[j]);  // rounded, then negated as an operand
    q[j] = __builtin_fmaf(-r, g.rs, q0);
  }
  return e4m3_pack4(q[0], q[1], q[2], q[3]);
}

// Codes of four values of a group: corrected quotients, or the IEEE
// divisions when the scale is outside the checked range.
__device__ __forceinline__ uint32_t quantize4_group(const float (&x)[4], const GroupScale &g) {
  return g.fast ? quantize4_corrected(x, g) : quantize4_exact(x, g.s);
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), in every lane
// of the row: two quad permutations, then rotations of the row by 4 and 8.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
  return v;
}

// One 1x128 activation group held by 16 consecutive lanes (one DPP row; all
// 16 active), 8 bf16 values (16 bytes) per lane: returns this lane's 8 codes
// and the group scale.  The group amax is an integer max over |bf16| bit
// patterns; s = amax / 448 as an IEEE division; codes as in group_scale.
__device__ __forceinline__ uint2 quantize_group16(const uint4 &raw, float &s_out) {
  const GroupScale g = group_scale(row16_max(amax8_bits(raw)) << 16);
  s_out = g.s;
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[2][4];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    v[i][0] = bf16_to_f32(w[2 * i] & 0xFFFFu);
    v[i][1] = __uint_as_float(w[2 * i] & 0xFFFF0000u);
    v[i][2] = bf16_to_f32(w[2 * i + 1] & 0xFFFFu);
    v[i][3] = __uint_as_float(w[2 * i + 1] & 0xFFFF0000u);
  }
  if (__builtin_expect(g.fast, 1)) return make_uint2(quantize4_corrected(v[0], g), quantize4_corrected(v[1], g));
  return make_uint2(quantize4_exact(v[0], g.s), quantize4_exact(v[1], g.s));
}

// v_mfma_f32_16x16x128_f8f6f4 with both operands e4m3 and no block scale.
// A: 16 rows x 128 K, B: 128 K x 16 columns; lane l holds row / column l%16 and
// 32 K-bytes; D: lane l holds column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i &a, const v8i &b, const v4f &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace fp8lin
