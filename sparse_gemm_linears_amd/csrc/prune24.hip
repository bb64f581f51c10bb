// 2:4 pruning along K with post-prune 128x128 block scales and compression.
//
// One 256-thread block per 128x128 weight block.  Thread t owns the two
// groups of 4 at columns 8*(t%16) .. +7 of rows t/16 + 16*i (i = 0..7):
//   1. scores |w| * c formed in fp64 (a bf16 times an fp32 is exact there);
//   2. a position is kept when fewer than two positions of its group rank
//      before it (higher score, or equal score and lower index);
//   3. the block maximum of the kept magnitudes gives s = amax / 448;
//   4. the kept codes and the nibble i0 | i1 << 2 of each group are packed.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8lin {

struct Group4 {
  uint32_t i0, i1;  // kept positions, i0 < i1
};

__device__ __forceinline__ Group4 select_two(const float (&v)[4], const float (&c)[4]) {
  double sc[4];
#pragma unroll
  for (int j = 0; j < 4; j++) sc[j] = fabs((double)v[j]) * (double)c[j];
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    int ahead = 0;
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (i != j) ahead += (sc[i] > sc[j]) || (sc[i] == sc[j] && i < j);
    keep |= (ahead < 2 ? 1u : 0u) << j;
  }
  Group4 g;
  g.i0 = __builtin_ctz(keep);
  g.i1 = 31 - __builtin_clz(keep);
  return g;
}

__global__ __launch_bounds__(256) void prune24_kernel(const uint16_t* __restrict__ w,
                                                      const float* __restrict__ col_norm, int64_t K,
                                                      uint8_t* __restrict__ vals, uint8_t* __restrict__ meta,
                                                      float* __restrict__ s) {
  __shared__ uint32_t wave_max[4];
  const int t = threadIdx.x;
  const int64_t KB = K / kGroup, nb = blockIdx.x / KB, kb = blockIdx.x % KB;
  const int col = 8 * (t & 15);
  const int64_t row0 = nb * kGroup + (t >> 4);
  const int64_t kcol = kb * kGroup + col;

  float c[8];
  if (col_norm) {
    float4 c0 = *reinterpret_cast<const float4*>(col_norm + kcol);
    float4 c1 = *reinterpret_cast<const float4*>(col_norm + kcol + 4);
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = 1.0f;
  }

  float v[8][8];
  Group4 sel[8][2];
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint4 raw = *reinterpret_cast<const uint4*>(w + (row0 + 16 * i) * K + kcol);
    uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[i][2 * j] = bf16_to_f32(r[j] & 0xFFFFu);
      v[i][2 * j + 1] = bf16_to_f32(r[j] >> 16);
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      float gv[4] = {v[i][4 * h], v[i][4 * h + 1], v[i][4 * h + 2], v[i][4 * h + 3]};
      float gc[4] = {c[4 * h], c[4 * h + 1], c[4 * h + 2], c[4 * h + 3]};
      sel[i][h] = select_two(gv, gc);
      amax_bits = max(amax_bits, __float_as_uint(gv[sel[i][h].i0]) & 0x7FFFFFFFu);
      amax_bits = max(amax_bits, __float_as_uint(gv[sel[i][h].i1]) & 0x7FFFFFFFu);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = amax_bits;
  __syncthreads();
  amax_bits = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  const float sc = __uint_as_float(amax_bits) / 448.0f;
  if (t == 0) s[nb * KB + kb] = sc;

#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int64_t n = row0 + 16 * i;
    uint32_t word = 0, nibs = 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const Group4 g = sel[i][h];
      uint32_t a = quantize(v[i][4 * h + g.i0], sc);
      uint32_t b = quantize(v[i][4 * h + g.i1], sc);
      word |= (a | (b << 8)) << (16 * h);
      nibs |= (g.i0 | (g.i1 << 2)) << (4 * h);
    }
    *reinterpret_cast<uint32_t*>(vals + n * (K / 2) + kcol / 2) = word;
    meta[n * (K / 8) + kcol / 8] = (uint8_t)nibs;
  }
}

hipError_t launch_prune24(const uint16_t* w, const float* col_norm, int64_t N, int64_t K, uint8_t* vals,
                          uint8_t* meta, float* s, hipStream_t stream) {
  hipLaunchKernelGGL(prune24_kernel, dim3((unsigned)((N / kGroup) * (K / kGroup))), dim3(256), 0, stream, w,
                     col_norm, K, vals, meta, s);
  return hipGetLastError();
}

}  // namespace fp8lin
