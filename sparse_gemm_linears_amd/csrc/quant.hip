// Activation (per-token 1x128) and weight (128x128 block) e4m3 quantizers.
//
// Both are HBM-bound streaming kernels: 16-byte loads of bf16, the group /
// block maximum of |x| by cross-lane and LDS reductions, the quotient x / s
// by a multiply and two FMAs (group_scale), hardware RNE encoding, packed
// stores.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8lin {

// ---------------------------------------------------------------------------
// Activations: 16 lanes own one 1x128 group at a time (8 bf16 = 16 bytes per
// lane), G groups 16 apart, with the G loads in flight together.  A 256-thread
// block covers 16 G consecutive groups; groups are numbered row-major over
// [M, K/128], so consecutive lanes read consecutive bytes of a row.  G = 2
// against one group per lane set (A/B on MI355X, inputs from HBM, identical
// outputs): 4096 x 14336 31.7 -> 28.3 us, 8192 x 7168 32.2 -> 28.8 us,
// 4096 x 4096 11.2 -> 10.8 us, level at 1-512 tokens; G = 4 was level with 2.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s,
                                                        int64_t n_groups) {
  const int lane16 = threadIdx.x & 15;
  int64_t grp[G];
  uint4 raw[G];
  // unconditional loads (a group past the end loads the last group): a branch
  // around them would make the first group's arithmetic wait for every load
#pragma unroll
  for (int j = 0; j < G; j++) {
    grp[j] = ((int64_t)blockIdx.x * G + j) * 16 + (threadIdx.x >> 4);
    const int64_t gl = grp[j] < n_groups ? grp[j] : n_groups - 1;
    raw[j] = *reinterpret_cast<const uint4*>(x + gl * kGroup + lane16 * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  // every group's codes before any store (a store behind a branch would make
  // the next group wait for it)
  float sc[G];
  uint2 packed[G];
#pragma unroll
  for (int j = 0; j < G; j++) packed[j] = quantize_group16(raw[j], sc[j]);
#pragma unroll
  for (int j = 0; j < G; j++) {
    if (grp[j] < n_groups) {
      *reinterpret_cast<uint2*>(q + grp[j] * kGroup + lane16 * 8) = packed[j];
      if (lane16 == 0) s[grp[j]] = sc[j];
    }
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
  for (int i = 0; i < 8; i++) raw[i] = ldg16_stream(w + base + (int64_t)i * 16 * K);
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
  const GroupScale g = group_scale(amax_bits << 16);
  if (t == 0) s[(int64_t)nb * KB + kb] = g.s;
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
    *reinterpret_cast<uint2 *>(q + base + (int64_t)i * 16 * K) =
        make_uint2(quantize4_group(v[0], g), quantize4_group(v[1], g));
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
  for (int i = 0; i < 8; i++) raw[i] = ldg16_stream(w + base + (int64_t)i * 16 * K);
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

// ---------------------------------------------------------------------------
// One scale for a whole tensor (dynamic per-tensor, or static): codes of the
// flattened tensor in 8-element chunks (16 bytes of bf16 per thread), and the
// scale written to every entry of the block-scale array, so the block-scaled
// GEMM takes the result unchanged.  The dynamic scale needs the amax of the
// whole tensor before any code: partial maxima per block are parked in the
// scale array itself (as bf16 magnitude bits), one block folds them into
// s[0] = amax / 448, and the quantizer reads its scale from s[0] and fills the
// rest of the array.  Three ordered launches on the stream; no atomics, no
// buffer beyond the outputs, and the result does not depend on the grid.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void amax_partial_kernel(const uint16_t* __restrict__ x, int64_t n_chunks,
                                                           uint32_t* __restrict__ part) {
  __shared__ uint32_t wave_max[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t a = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n_chunks; i += 4 * stride) {
    uint4 r[4];
#pragma unroll
    for (int u = 0; u < 4; u++) r[u] = *reinterpret_cast<const uint4*>(x + (i + u * stride) * 8);
#pragma unroll
    for (int u = 0; u < 4; u++) a = max(a, amax8_bits(r[u]));
  }
  for (; i < n_chunks; i += stride) a = max(a, amax8_bits(*reinterpret_cast<const uint4*>(x + i * 8)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
}

// One block: s[0] <- fp32(amax / 448) from the n_part partial maxima held as
// bits in s[0 .. n_part).  Every read is done before the barrier, the single
// write after it.
__global__ __launch_bounds__(256) void amax_finish_kernel(float* s, int n_part) {
  __shared__ uint32_t wave_max[4];
  const uint32_t* part = reinterpret_cast<const uint32_t*>(s);
  uint32_t a = 0;
  for (int i = threadIdx.x; i < n_part; i += 256) a = max(a, part[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0)
    s[0] = bf16_to_f32(max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]))) / 448.0f;
}

// Codes of chunk i with the scale *scale; thread i also writes s[i] for
// s_from <= i < n_s (the grid has at least n_s threads).  scale may point
// into s when s_from excludes that entry.
__global__ __launch_bounds__(256) void quant_scaled_kernel(const uint16_t* __restrict__ x, const float* scale,
                                                           int64_t n_chunks, uint8_t* __restrict__ q, float* s,
                                                           int64_t n_s, int64_t s_from) {
  const float sc = *scale;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n_chunks)
    *reinterpret_cast<uint2*>(q + i * 8) = quantize8_scaled(*reinterpret_cast<const uint4*>(x + i * 8), sc);
  if (i >= s_from && i < n_s) s[i] = sc;
}

hipError_t launch_amax_finish(float* s, int64_t n_part, hipStream_t stream) {
  hipLaunchKernelGGL(amax_finish_kernel, dim3(1), dim3(256), 0, stream, s, (int)n_part);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* s, int64_t n_s,
                               hipStream_t stream) {
  const int64_t n_chunks = n / 8;
  const int n_part = (int)(n_s < kTensorAmaxParts ? n_s : kTensorAmaxParts);
  hipLaunchKernelGGL(amax_partial_kernel, dim3((unsigned)n_part), dim3(256), 0, stream, x, n_chunks,
                     reinterpret_cast<uint32_t*>(s));
  hipLaunchKernelGGL(amax_finish_kernel, dim3(1), dim3(256), 0, stream, s, n_part);
  hipLaunchKernelGGL(quant_scaled_kernel, dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0, stream, x,
                     (const float*)s, n_chunks, q, s, n_s, (int64_t)1);
  return hipGetLastError();
}

hipError_t launch_quant_static(const uint16_t* x, const float* scale, int64_t n, uint8_t* q, float* s, int64_t n_s,
                               hipStream_t stream) {
  const int64_t n_chunks = n / 8;
  hipLaunchKernelGGL(quant_scaled_kernel, dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0, stream, x, scale,
                     n_chunks, q, s, n_s, (int64_t)0);
  return hipGetLastError();
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
  const int64_t blocks = (n_groups + 31) / 32;
  hipLaunchKernelGGL(quant_act_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, s, n_groups);
  return hipGetLastError();
}

hipError_t launch_quant_wblock(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s,
                               hipStream_t stream) {
  hipLaunchKernelGGL(quant_wblock_kernel, dim3((unsigned)((N / kGroup) * (K / kGroup))), dim3(256), 0, stream, w,
                     K, q, s);
  return hipGetLastError();
}

}  // namespace fp8lin
