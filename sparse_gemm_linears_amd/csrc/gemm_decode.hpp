// Decode-sized (M <= 64) block-scaled GEMM, shared by the dense and the 2:4
// kernels.  The weight is read once, straight from HBM into MFMA operand
// registers; the run is HBM-bound, so the kernel keeps D K blocks of loads in
// flight per wave and does nothing else of note.
//
// Workgroup: RT row tiles of 16 weight rows (one 128-row scale block holds all
// of them) and all of K.  Its NW waves take the K blocks round-robin (wave w:
// kb = w, w + NW, ...), so at any time the waves read neighbouring 128-byte
// pieces of the same rows; each wave accumulates its own partial sums, and the
// partials meet in LDS at the end (fixed order: deterministic).
// Tokens: CT column tiles of 16 (M <= 16*CT); rows past M re-read row M-1 and
// are never stored.
//
// The weight operand is a policy W:
//   typename W::Frag;                                  operand registers
//   Frag W::load(int64_t row, int kb, int g) const;    row's K block kb, lane group g
//   v4f  W::mma(const Frag &a, const v8i &b) const;    16x16 partial for one K block
#pragma once

#include "gemm_common.hpp"

namespace fp8lin {

template <class W, int RT, int CT, int NW, int D>
__global__ __launch_bounds__(NW * 64) void decode_kernel(W wop, const uint8_t *__restrict__ xq,
                                                         const float *__restrict__ xs, const float *__restrict__ ws,
                                                         int M, int N, int K, uint16_t *__restrict__ y) {
  static_assert(128 % (16 * RT) == 0, "a workgroup's rows must sit in one 128-row scale block");
  __shared__ v4f red[NW > 1 ? NW - 1 : 1][RT * CT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, lr = lane & 15;
  const int KB = K / kGroup;
  const int n0 = blockIdx.x * 16 * RT;
  const float *ws_row = ws + (int64_t)(n0 / kGroup) * KB;
  const int n_w = wave < KB ? (KB - wave + NW - 1) / NW : 0;  // K blocks of this wave

  const uint8_t *xrow[CT];
  const float *srow[CT];
#pragma unroll
  for (int c = 0; c < CT; c++) {
    const int m = min(16 * c + lr, M - 1);
    xrow[c] = xq + (int64_t)m * K;
    srow[c] = xs + (int64_t)m * KB;
  }

  typename W::Frag a[D][RT];
  v8i b[D][CT];
  float sx[D][CT], sw[D];
  auto load = [&](int slot, int i) {
    const int kb = wave + i * NW;
#pragma unroll
    for (int r = 0; r < RT; r++) a[slot][r] = wop.load(n0 + 16 * r + lr, kb, g);
#pragma unroll
    for (int c = 0; c < CT; c++) {
      b[slot][c] = load_frag_global(xrow[c] + (int64_t)kb * kGroup, g);
      sx[slot][c] = srow[c][kb];
    }
    sw[slot] = ws_row[kb];
  };

  v4f acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; r++)
#pragma unroll
    for (int c = 0; c < CT; c++) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int d = 0; d < D; d++)
    if (d < n_w) load(d, d);
  for (int i0 = 0; i0 < n_w; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      const int i = i0 + d;
      if (i < n_w) {
#pragma unroll
        for (int c = 0; c < CT; c++) {
          const float scl = sx[d][c] * sw[d];
#pragma unroll
          for (int r = 0; r < RT; r++) acc[r][c] += scl * wop.mma(a[d][r], b[d][c]);
        }
        if (i + D < n_w) load(d, i + D);
      }
    }
  }

  if (NW > 1) {
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < RT; r++)
#pragma unroll
        for (int c = 0; c < CT; c++) red[wave - 1][r * CT + c][lane] = acc[r][c];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < NW - 1; w++)
#pragma unroll
      for (int r = 0; r < RT; r++)
#pragma unroll
        for (int c = 0; c < CT; c++) acc[r][c] += red[w][r * CT + c][lane];
  }
#pragma unroll
  for (int c = 0; c < CT; c++) {
    const int m = 16 * c + lr;
    if (m >= M) continue;
#pragma unroll
    for (int r = 0; r < RT; r++) {
      const int n = n0 + 16 * r + 4 * g;
      *reinterpret_cast<uint2 *>(y + (int64_t)m * N + n) = pack_bf16x4(acc[r][c]);
    }
  }
}

}  // namespace fp8lin
