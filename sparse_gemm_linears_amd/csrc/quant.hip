// Activation (per-token 1x128) and weight (128x128 block) e4m3 quantizers.
//
// Both are HBM-bound streaming kernels: 16-byte loads of bf16, the group /
// block maximum of |x| by cross-lane and LDS reductions, one IEEE fp32
// division per element, integer RNE encoding, packed stores.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8lin {

// ---------------------------------------------------------------------------
// Activations: 16 lanes own one 1x128 group (8 bf16 = 16 bytes per lane).  A
// 256-thread block covers 16 groups; groups are numbered row-major over
// [M, K/128], so consecutive lanes read consecutive bytes of a row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s,
                                                        int64_t n_groups) {
  const int lane16 = threadIdx.x & 15;
  const int64_t grp = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = grp < n_groups;
  // group grp covers elements [grp*128, grp*128+128) of the flattened [M,K] array
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(x + grp * kGroup + lane16 * 8);
  float sc;
  const uint2 packed = quantize_group16(raw, sc);
  if (live) {
    *reinterpret_cast<uint2*>(q + grp * kGroup + lane16 * 8) = packed;
    if (lane16 == 0) s[grp] = sc;
  }
}

// ---------------------------------------------------------------------------
// Weights: one 256-thread block per 128x128 block.  Thread t owns columns
// 8*(t%16) .. +7 of rows t/16 + 16*i, i = 0..7 (128 bytes of bf16).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_wblock_kernel(const uint16_t* __restrict__ w,
                                                           int64_t K, uint8_t* __restrict__ q,
                                                           float* __restrict__ s) {
  __shared__ uint32_t wave_max[4];
  const int t = threadIdx.x;
  const int KB = (int)(K / kGroup), nb = (int)blockIdx.x / KB, kb = (int)blockIdx.x % KB;
  const int col = 8 * (t & 15);
  const int64_t base = ((int64_t)nb * kGroup + (t >> 4)) * K + (int64_t)kb * kGroup + col;
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; i++) raw[i] = *reinterpret_cast<const uint4*>(w + base + (int64_t)i * 16 * K);
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint32_t v[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; j++)
      amax_bits = max(amax_bits, max(bf16_abs_bits(v[j] & 0xFFFFu), bf16_abs_bits(v[j] >> 16)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = amax_bits;
  __syncthreads();
  amax_bits = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  const float sc = bf16_to_f32(amax_bits) / 448.0f;
  const float rs = __builtin_amdgcn_rcpf(sc);
  const bool ok = scale_fast_ok(sc);
  if (t == 0) s[(int64_t)nb * KB + kb] = sc;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float v[2][4];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t lo = h ? raw[i].z : raw[i].x, hi = h ? raw[i].w : raw[i].y;
      v[h][0] = bf16_to_f32(lo & 0xFFFFu);
      v[h][1] = __uint_as_float(lo & 0xFFFF0000u);
      v[h][2] = bf16_to_f32(hi & 0xFFFFu);
      v[h][3] = __uint_as_float(hi & 0xFFFF0000u);
    }
    uint32_t need = ok ? 0u : 1u;
    uint32_t packed[2];
#pragma unroll
    for (int h = 0; h < 2; h++) packed[h] = quantize4_fast(v[h], rs, need);
    if (__builtin_expect(need != 0u, 0)) {
#pragma unroll
      for (int h = 0; h < 2; h++) packed[h] = quantize4_exact(v[h], sc);
    }
    *reinterpret_cast<uint2 *>(q + base + (int64_t)i * 16 * K) = make_uint2(packed[0], packed[1]);
  }
}

// ---------------------------------------------------------------------------
// UE8M0 variants: the same layouts with one exponent byte per group / block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_act_ue8m0_kernel(const uint16_t* __restrict__ x,
                                                              uint8_t* __restrict__ q,
                                                              uint8_t* __restrict__ e_out,
                                                              int64_t n_groups) {
  const int lane16 = threadIdx.x & 15;
  const int64_t grp = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = grp < n_groups;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(x + grp * kGroup + lane16 * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) amax = max(amax, max(bf16_abs_bits(w[i] & 0xFFFFu), bf16_abs_bits(w[i] >> 16)));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 16));
  const uint32_t e = ue8m0_exponent(amax << 16);
  const float inv = ue8m0_inverse(e);
  uint32_t packed[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const float v[4] = {bf16_to_f32(w[2 * i] & 0xFFFFu), __uint_as_float(w[2 * i] & 0xFFFF0000u),
                        bf16_to_f32(w[2 * i + 1] & 0xFFFFu), __uint_as_float(w[2 * i + 1] & 0xFFFF0000u)};
    packed[i] = quantize4_pow2(v, inv);
  }
  if (live) {
    *reinterpret_cast<uint2*>(q + grp * kGroup + lane16 * 8) = make_uint2(packed[0], packed[1]);
    if (lane16 == 0) e_out[grp] = (uint8_t)e;
  }
}

__global__ __launch_bounds__(256) void quant_wblock_ue8m0_kernel(const uint16_t* __restrict__ w,
                                                                 int64_t K, uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ e_out) {
  __shared__ uint32_t wave_max[4];
  const int t = threadIdx.x;
  const int KB = (int)(K / kGroup), nb = (int)blockIdx.x / KB, kb = (int)blockIdx.x % KB;
  const int col = 8 * (t & 15);
  const int64_t base = ((int64_t)nb * kGroup + (t >> 4)) * K + (int64_t)kb * kGroup + col;
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; i++) raw[i] = *reinterpret_cast<const uint4*>(w + base + (int64_t)i * 16 * K);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t v[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; j++) amax = max(amax, max(bf16_abs_bits(v[j] & 0xFFFFu), bf16_abs_bits(v[j] >> 16)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = amax;
  __syncthreads();
  amax = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  const uint32_t e = ue8m0_exponent(amax << 16);
  const float inv = ue8m0_inverse(e);
  if (t == 0) e_out[(int64_t)nb * KB + kb] = (uint8_t)e;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint32_t packed[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t lo = h ? raw[i].z : raw[i].x, hi = h ? raw[i].w : raw[i].y;
      const float v[4] = {bf16_to_f32(lo & 0xFFFFu), __uint_as_float(lo & 0xFFFF0000u), bf16_to_f32(hi & 0xFFFFu),
                          __uint_as_float(hi & 0xFFFF0000u)};
      packed[h] = quantize4_pow2(v, inv);
    }
    *reinterpret_cast<uint2*>(q + base + (int64_t)i * 16 * K) = make_uint2(packed[0], packed[1]);
  }
}

hipError_t launch_quant_act_ue8m0(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* e,
                                  hipStream_t stream) {
  const int64_t n_groups = M * (K / kGroup);
  hipLaunchKernelGGL(quant_act_ue8m0_kernel, dim3((unsigned)((n_groups + 15) / 16)), dim3(256), 0, stream, x, q, e,
                     n_groups);
  return hipGetLastError();
}

hipError_t launch_quant_wblock_ue8m0(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, uint8_t* e,
                                     hipStream_t stream) {
  hipLaunchKernelGGL(quant_wblock_ue8m0_kernel, dim3((unsigned)((N / kGroup) * (K / kGroup))), dim3(256), 0, stream,
                     w, K, q, e);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                            hipStream_t stream) {
  const int64_t n_groups = M * (K / kGroup);
  const int64_t blocks = (n_groups + 15) / 16;
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, s, n_groups);
  return hipGetLastError();
}

hipError_t launch_quant_wblock(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s,
                               hipStream_t stream) {
  hipLaunchKernelGGL(quant_wblock_kernel, dim3((unsigned)((N / kGroup) * (K / kGroup))), dim3(256), 0, stream, w,
                     K, q, s);
  return hipGetLastError();
}

}  // namespace fp8lin
