// 2:4 pruning along K with post-prune 128x128 block scales and compression.
//
// One 256-thread block per 128x128 weight block.  Thread t owns the two
// groups of 4 at columns 8*(t%16) .. +7 of rows t/16 + 16*i (i = 0..7):
//   1. scores |w| * c formed in fp64 (a bf16 times an fp32 is exact there);
//   2. a position is kept when fewer than two positions of its group rank
//      before it (higher score, or equal score and lower index), from the six
//      pairwise comparisons of the group;
//   3. the block maximum of the kept magnitudes gives s = amax / 448;
//   4. the kept codes and the nibble i0 | i1 << 2 of each group are packed.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8lin {

// Kept pair of one group of 4: the two values in index order and the nibble
// i0 | i1 << 2.
struct Kept2 {
  float first, second;
  uint32_t nib;
};

// SC: score type (uint32 |w| bit patterns for magnitude, exact fp64 products
// for activation-aware).  gij (i < j) says position i ranks before position j
// (ties go to the lower index); a position is kept when fewer than two of the
// other three rank before it, i.e. when it ranks before at least two of them.
// Each comparison becomes a lane mask of the wave (one vector compare), the
// majorities are scalar bit operations on the masks, and the four keep flags
// go back to the lanes as select masks.  The values come in as four scalars
// and are picked with selects: from an array, the compiler turns the pick into
// an indexed load from scratch memory.  Against the same rule in plain bool
// logic, where the compiler repeated every comparison in negated form and
// spilled the masks (A/B on MI355X, weights from HBM, identical outputs):
// 6144 x 4096 19.0 -> 16.8 us, 4096 x 4096 14.4 -> 12.6 us, 28672 x 4096
// 63.6 -> 62.4 us, 4096 x 14336 34.4 -> 33.5 us (activation-aware).
typedef unsigned long long LaneMask;
__device__ __forceinline__ LaneMask lanes_where(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ bool lane_in(LaneMask m) { return __builtin_amdgcn_inverse_ballot_w64(m); }
__device__ __forceinline__ LaneMask majority3(LaneMask a, LaneMask b, LaneMask c) { return (a & b) | (c & (a | b)); }

template <bool kNib, typename SC>
__device__ __forceinline__ Kept2 select_two(float v0, float v1, float v2, float v3, SC s0, SC s1, SC s2, SC s3) {
  const LaneMask g01 = lanes_where(s0 >= s1), g02 = lanes_where(s0 >= s2), g03 = lanes_where(s0 >= s3);
  const LaneMask g12 = lanes_where(s1 >= s2), g13 = lanes_where(s1 >= s3), g23 = lanes_where(s2 >= s3);
  const bool k0 = lane_in(majority3(g01, g02, g03));
  const bool k1 = lane_in(majority3(~g01, g12, g13));
  const bool k2 = lane_in(majority3(~g02, ~g12, g23));
  const bool k3 = lane_in(majority3(~g03, ~g13, ~g23));
  Kept2 r;
  r.first = k0 ? v0 : (k1 ? v1 : v2);
  r.second = k3 ? v3 : (k2 ? v2 : v1);
  // made here, in registers: otherwise the compiler sinks the selects to their
  // uses after the block reduction and keeps (spills) every mask until then
  asm volatile("" : "+v"(r.first), "+v"(r.second));
  r.nib = 0;
  if constexpr (kNib) {
    const uint32_t i0 = k0 ? 0u : (k1 ? 1u : 2u);
    const uint32_t i1 = k3 ? 3u : (k2 ? 2u : 1u);
    r.nib = i0 | (i1 << 2);
  }
  return r;
}

// MODE 0: block scales (the kernel above).  The per-tensor form runs in three
// launches on the stream: MODE 1 writes each block's largest kept magnitude
// (bf16 bits) into its entry of s; amax_finish_kernel folds them into
// s[0] = amax / 448; MODE 2 quantizes the kept values with s[0] and writes it
// to every other entry.
template <bool AWARE, int MODE = 0>
__global__ __launch_bounds__(256) void prune24_kernel(const uint16_t* __restrict__ w,
                                                      const float* __restrict__ col_norm, int64_t K,
                                                      uint8_t* __restrict__ vals, uint8_t* __restrict__ meta,
                                                      float* s) {
  __shared__ uint32_t wave_max[4];
  const int t = threadIdx.x;
  // Block b runs on XCD b % 8.  Each XCD takes a contiguous range of blocks
  // (consecutive K blocks of a row band), so the lines of vals and meta, which
  // neighbouring K blocks write in 64- and 16-byte pieces, are completed in
  // one L2 instead of being merged from eight.
  const int KB = (int)(K / kGroup);
  const int b = (int)blockIdx.x, total = (int)gridDim.x;
  const int L = total % 8 == 0 ? (b % 8) * (total / 8) + b / 8 : b;
  const int nb = L / KB, kb = L % KB;
  const int col = 8 * (t & 15);
  const int64_t row0 = (int64_t)nb * kGroup + (t >> 4);
  const int64_t kcol = (int64_t)kb * kGroup + col;

  double c[8];
  if (AWARE) {
    const float4 c0 = *reinterpret_cast<const float4*>(col_norm + kcol);
    const float4 c1 = *reinterpret_cast<const float4*>(col_norm + kcol + 4);
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
  }

  // all eight row loads in flight before any arithmetic (interleaved with the
  // scoring, the compiler waits for each load before issuing the next)
  const uint16_t* wp = w + row0 * K + kcol;
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    // read once, except by the per-tensor form's first pass (its second pass
    // reads the weight again)
    const uint16_t* rp = wp + (int64_t)i * 16 * K;
    raw[i] = MODE == 1 ? *reinterpret_cast<const uint4*>(rp) : ldg16_stream(rp);
  }

  Kept2 kept[8][2];
  uint32_t mbs[8];
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t r[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t lo = r[2 * h], hi = r[2 * h + 1];
      const float v0 = bf16_to_f32(lo & 0xFFFFu), v1 = __uint_as_float(lo & 0xFFFF0000u);
      const float v2 = bf16_to_f32(hi & 0xFFFFu), v3 = __uint_as_float(hi & 0xFFFF0000u);
      if constexpr (AWARE) {
        // |w| * c is exact in fp64 (8 + 24 significant bits)
        kept[i][h] = select_two<MODE != 1>(v0, v1, v2, v3, fabs((double)v0) * c[4 * h],
                                           fabs((double)v1) * c[4 * h + 1], fabs((double)v2) * c[4 * h + 2],
                                           fabs((double)v3) * c[4 * h + 3]);
      } else {
        kept[i][h] = select_two<MODE != 1>(v0, v1, v2, v3, lo & 0x7FFFu, (lo >> 16) & 0x7FFFu, hi & 0x7FFFu,
                                           (hi >> 16) & 0x7FFFu);
      }
      amax_bits = max(amax_bits, max(__float_as_uint(kept[i][h].first) & 0x7FFFFFFFu,
                                     __float_as_uint(kept[i][h].second) & 0x7FFFFFFFu));
    }
    // the row's two meta nibbles, made now for the same reason
    mbs[i] = kept[i][0].nib | (kept[i][1].nib << 4);
    if constexpr (MODE != 1) asm volatile("" : "+v"(mbs[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = amax_bits;
  __syncthreads();
  amax_bits = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  if constexpr (MODE == 1) {
    if (t == 0) reinterpret_cast<uint32_t*>(s)[(int64_t)nb * KB + kb] = amax_bits >> 16;  // bf16 magnitude bits
    return;
  }
  GroupScale g;
  if constexpr (MODE == 2) {
    // the tensor scale (amax / 448 of every kept value): codes by the
    // reciprocal with a check near e4m3 rounding midpoints, else the IEEE
    // division (the static-scale quantizer's arithmetic)
    g.s = s[0];
    g.rs = __builtin_amdgcn_rcpf(g.s);
    g.fast = scale_fast_ok(g.s);
    if (t == 0 && (nb != 0 || kb != 0)) s[(int64_t)nb * KB + kb] = g.s;
  } else {
    g = group_scale(amax_bits);
    if (t == 0) s[(int64_t)nb * KB + kb] = g.s;
  }

#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int64_t n = row0 + 16 * i;
    const float kv[4] = {kept[i][0].first, kept[i][0].second, kept[i][1].first, kept[i][1].second};
    uint32_t word;
    if constexpr (MODE == 2) {
      uint32_t need = g.fast ? 0u : 1u;
      word = quantize4_fast(kv, g.rs, need);
      if (__builtin_expect(need != 0u, 0)) word = quantize4_exact(kv, g.s);
    } else {
      word = quantize4_group(kv, g);
    }
    *reinterpret_cast<uint32_t*>(vals + n * (K / 2) + kcol / 2) = word;
    // the 16 lanes of a row segment hold its 16 consecutive meta bytes: the
    // first lane of each quad gathers the bytes of lanes 1, 2, 3 of its quad
    // (DPP quad broadcasts) for one 4-byte store
    const uint32_t mb = mbs[i];
    const uint32_t m4 = mb | ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x55, 0xF, 0xF, false) << 8) |
                        ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xAA, 0xF, 0xF, false) << 16) |
                        ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xFF, 0xF, 0xF, false) << 24);
    if ((t & 3) == 0) *reinterpret_cast<uint32_t*>(meta + n * (K / 8) + kcol / 8) = m4;
  }
}

hipError_t launch_prune24_tensor(const uint16_t* w, const float* col_norm, int64_t N, int64_t K, uint8_t* vals,
                                 uint8_t* meta, float* s, hipStream_t stream) {
  const int64_t blocks = (N / kGroup) * (K / kGroup);
  const dim3 grid((unsigned)blocks);
  if (col_norm)
    hipLaunchKernelGGL((prune24_kernel<true, 1>), grid, dim3(256), 0, stream, w, col_norm, K, vals, meta, s);
  else
    hipLaunchKernelGGL((prune24_kernel<false, 1>), grid, dim3(256), 0, stream, w, col_norm, K, vals, meta, s);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_amax_finish(s, blocks, stream);
  if (e != hipSuccess) return e;
  if (col_norm)
    hipLaunchKernelGGL((prune24_kernel<true, 2>), grid, dim3(256), 0, stream, w, col_norm, K, vals, meta, s);
  else
    hipLaunchKernelGGL((prune24_kernel<false, 2>), grid, dim3(256), 0, stream, w, col_norm, K, vals, meta, s);
  return hipGetLastError();
}

hipError_t launch_prune24(const uint16_t* w, const float* col_norm, int64_t N, int64_t K, uint8_t* vals,
                          uint8_t* meta, float* s, hipStream_t stream) {
  const dim3 grid((unsigned)((N / kGroup) * (K / kGroup)));
  if (col_norm)
    hipLaunchKernelGGL(prune24_kernel<true>, grid, dim3(256), 0, stream, w, col_norm, K, vals, meta, s);
  else
    hipLaunchKernelGGL(prune24_kernel<false>, grid, dim3(256), 0, stream, w, col_norm, K, vals, meta, s);
  return hipGetLastError();
}

}  // namespace fp8lin
