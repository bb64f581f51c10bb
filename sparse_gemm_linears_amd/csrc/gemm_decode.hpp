// Decode-sized (M <= 64) block-scaled GEMM, shared by the dense and the 2:4
// kernels.  The weight is read once, straight from HBM into MFMA operand
// registers; the run is HBM-bound, so the kernel keeps D K blocks of loads in
// flight per wave and does nothing else of note.
//
// Workgroup: RT row tiles of 16 weight rows (one 128-row scale block holds all
// of them) and all of K, or a quarter of it with S = 4 splits (below).  Its NW
// waves take the K blocks round-robin (wave w: kb = w, w + NW, ...), so at any
// time the waves read neighbouring 128-byte pieces of the same rows; each wave
// accumulates its own partial sums, and the partials meet in LDS at the end
// (fixed order: deterministic).
// Tokens: CT column tiles of 16 (M <= 16*CT); rows past M re-read row M-1 and
// are never stored.
//
// The weight operand is a policy W:
//   typename W::Frag;                                  operand registers
//   Frag W::load(int64_t row, int kb, int g) const;    row's K block kb, lane group g
//   v4f  W::mma(const Frag &a, const v8i &b) const;    16x16 partial for one K block
// and so is the token operand X:
//   typename X::Raw;                                   what a load leaves in registers
//   Raw  X::load(int m, int kb, int g) const;          token m's K block kb, lane group g
//   void X::make(const Raw &r, v8i &frag, float &s);   e4m3 fragment and the token's scale
//   kStaged                                            true: X::stage fills LDS first
// X::make runs with all 64 lanes active (it may reduce across lane groups).
#pragma once

#include <type_traits>

#include "gemm_common.hpp"

namespace fp8lin {

// Tokens already quantized by fp8_quant_act: codes and one scale per K block.
struct QuantTokens {
  const uint8_t *xq;
  const float *xs;
  int K;
  static constexpr bool kStaged = false, kE8 = false;
  typedef float Scale;
  struct Raw {
    v8i q;
    float s;
  };
  __device__ __forceinline__ void stage(uint8_t *, int, int, int) {}
  __device__ __forceinline__ Raw load(int m, int kb, int g) const {
    Raw r;
    r.q = load_frag_global(xq + (int64_t)m * K + (int64_t)kb * kGroup, g);
    r.s = xs[(int64_t)m * (K / kGroup) + kb];
    return r;
  }
  __device__ __forceinline__ void make(const Raw &r, v8i &frag, float &s) const {
    frag = r.q;
    s = r.s;
  }
};

// Tokens quantized by fp8_quant_act_ue8m0: codes and one exponent byte per K
// block; the MFMA applies 2^(e - 127) itself.
struct QuantTokensE8 {
  const uint8_t *xq;
  const uint8_t *xe;
  int K;
  static constexpr bool kStaged = false, kE8 = true;
  typedef uint8_t Scale;
  struct Raw {
    v8i q;
    uint32_t e;
  };
  __device__ __forceinline__ void stage(uint8_t *, int, int, int) {}
  __device__ __forceinline__ Raw load(int m, int kb, int g) const {
    Raw r;
    r.q = load_frag_global(xq + (int64_t)m * K + (int64_t)kb * kGroup, g);
    r.e = xe[(int64_t)m * (K / kGroup) + kb];
    return r;
  }
  __device__ __forceinline__ void make(const Raw &r, v8i &frag, uint32_t &e) const {
    frag = r.q;
    e = r.e;
  }
};

// bf16 tokens quantized once per workgroup into LDS before the GEMM loop (for
// small M, where M x K codes fit in LDS): 16 lanes per 1x128 group, the
// arithmetic of fp8_quant_act (quantize_group16), codes [M][K] and scales
// [M][K/128] in dynamically sized LDS.  Fragments then come from LDS.
struct StagedTokens {
  const uint16_t *x;
  int K;
  uint8_t *codes;
  float *scales;
  static constexpr bool kStaged = true, kE8 = false;
  typedef float Scale;
  struct Raw {
    v8i q;
    float s;
  };
  static size_t lds_bytes(int M, int K) { return (size_t)M * K + (size_t)4 * M * (K / kGroup); }
  static constexpr int kMaxPasses = 4;  // groups per 16-lane team
  // All threads of the workgroup take part (every 16-lane team stays active).
  // Every load is issued before any arithmetic, so the staging costs one
  // memory latency rather than one per pass.
  __device__ __forceinline__ void stage(uint8_t *lds, int M, int tid, int nthreads) {
    codes = lds;
    scales = reinterpret_cast<float *>(lds + (size_t)M * K);
    const int groups = M * (K / kGroup), teams = nthreads / 16, lane16 = tid & 15;
    const int passes = (groups + teams - 1) / teams;
    uint4 raw[kMaxPasses];
#pragma unroll
    for (int p = 0; p < kMaxPasses; p++) {
      // groups past the end repeat the last one and store nothing
      const int gc = min(p * teams + tid / 16, groups - 1);
      if (p < passes) raw[p] = *reinterpret_cast<const uint4 *>(x + (int64_t)gc * kGroup + lane16 * 8);
    }
#pragma unroll
    for (int p = 0; p < kMaxPasses; p++) {
      if (p < passes) {
        const int grp = p * teams + tid / 16, gc = min(grp, groups - 1);
        float s;
        const uint2 q = quantize_group16(raw[p], s);
        if (grp < groups) {
          *reinterpret_cast<uint2 *>(codes + (size_t)gc * kGroup + lane16 * 8) = q;
          if (lane16 == 0) scales[gc] = s;
        }
      }
    }
  }
  __device__ __forceinline__ Raw load(int m, int kb, int g) const {
    const uint8_t *row = codes + (size_t)m * K + (size_t)kb * kGroup;
    Raw r;
    r.q = make_v8i(*reinterpret_cast<const uint4 *>(row + 16 * g), *reinterpret_cast<const uint4 *>(row + 64 + 16 * g));
    r.s = scales[m * (K / kGroup) + kb];
    return r;
  }
  __device__ __forceinline__ void make(const Raw &r, v8i &frag, float &s) const {
    frag = r.q;
    s = r.s;
  }
};

// Staging pays while the per-workgroup quantization (M x K elements, redone by
// every workgroup) stays small next to the weight stream: measured on MI355X,
// the staged call beats fp8_quant_act + GEMM for one or two tokens and loses
// from three on.  The codes (plus the largest reduction buffer, 28 KB) must
// fit the default 64 KB of LDS per workgroup, and each 16-lane team stages at
// most kMaxPasses groups (64 teams in the 16-wave workgroup used for M <= 4).
inline bool staged_tokens_fit(int64_t M, int64_t K) {
  return M <= 2 && StagedTokens::lds_bytes((int)M, (int)K) <= 36 * 1024 &&
         M * (K / kGroup) <= StagedTokens::kMaxPasses * 64;
}

// S > 1 splits K over S workgroups per row band (blockIdx.y = split), for
// long-K weights with few row bands: each split stores its fp32 sums in
// part [S][M][N], and a separate kernel adds them in split order.
// A weight policy may load U consecutive K blocks at a time (W::kUnit, and
// mma(frag, b, u) for block u of the unit); without kUnit, U = 1.  The waves
// then take units round-robin, and K must hold a whole number of units.
template <class W, class = void>
struct weight_unit {
  static constexpr int value = 1;
};
template <class W>
struct weight_unit<W, std::void_t<decltype(W::kUnit)>> {
  static constexpr int value = W::kUnit;
};

template <class W, class X, int RT, int CT, int NW, int D, int S = 1>
__global__ __launch_bounds__(NW * 64) void decode_kernel(W wop, X xop, const typename X::Scale *__restrict__ ws,
                                                         int M, int N, int K, uint16_t *__restrict__ y,
                                                         float *__restrict__ part) {
  static_assert(128 % (16 * RT) == 0, "a workgroup's rows must sit in one 128-row scale block");
  __shared__ v4f red[NW > 1 ? NW - 1 : 1][RT * CT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, lr = lane & 15;
  constexpr int U = weight_unit<W>::value;
  const int KB = K / kGroup, KU = KB / U;  // K blocks, units of U blocks
  const int n0 = blockIdx.x * 16 * RT;
  const typename X::Scale *ws_row = ws + (int64_t)(n0 / kGroup) * KB;
  // this split's units: [kb0, kb0 + KBr)
  const int KBs = (KU + S - 1) / S, kb0 = S > 1 ? (int)blockIdx.y * KBs : 0;
  const int KBr = S > 1 ? max(0, min(KU, kb0 + KBs) - kb0) : KU;
  const int n_w = wave < KBr ? (KBr - wave + NW - 1) / NW : 0;  // units of this wave

  int mrow[CT];
#pragma unroll
  for (int c = 0; c < CT; c++) mrow[c] = min(16 * c + lr, M - 1);

  typename W::Frag a[D][RT];
  typename X::Raw b[D][CT][U];
  typename X::Scale sw[D][U];
  // The weight scale comes through a vector load like the other operands:
  // vector loads complete in order, so a wait can leave younger slots in
  // flight (scalar loads complete out of order and would need a full wait).
  const rsrc_t rws = make_rsrc(ws_row, (uint32_t)(KB * sizeof(typename X::Scale)));
  auto load_w = [&](int slot, int i) {
    const int kb = (kb0 + wave + i * NW) * U;  // first K block of the unit
#pragma unroll
    for (int r = 0; r < RT; r++) a[slot][r] = wop.load(n0 + 16 * r + lr, kb, g);
#pragma unroll
    for (int u = 0; u < U; u++) {
      if constexpr (X::kE8)
        sw[slot][u] = __builtin_amdgcn_raw_buffer_load_b8(rws, 0, kb + u, 0);
      else
        sw[slot][u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rws, 0, (kb + u) * 4, 0));
    }
  };
  auto load_x = [&](int slot, int i) {
    const int kb = (kb0 + wave + i * NW) * U;
#pragma unroll
    for (int c = 0; c < CT; c++)
#pragma unroll
      for (int u = 0; u < U; u++) b[slot][c][u] = xop.load(mrow[c], kb + u, g);
  };

  v4f acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; r++)
#pragma unroll
    for (int c = 0; c < CT; c++) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};

  // The first D slots.  A wave with fewer than D blocks fills the rest with
  // its last block again (in bounds; never consumed), so that every slot is
  // loaded on every path.
  if constexpr (X::kStaged) {
    // the first weight loads go out before the tokens are staged, so their
    // HBM latency overlaps the staging
    if (n_w > 0)
#pragma unroll
      for (int d = 0; d < D; d++) load_w(d, min(d, n_w - 1));
    extern __shared__ __align__(16) uint8_t staged_lds[];
    xop.stage(staged_lds, M, threadIdx.x, NW * 64);
    __syncthreads();
    if (n_w > 0)
#pragma unroll
      for (int d = 0; d < D; d++) load_x(d, min(d, n_w - 1));
  } else if (n_w > 0) {
    // slot by slot, in the loop's order (the waits count loads by age)
#pragma unroll
    for (int d = 0; d < D; d++) {
      load_w(d, min(d, n_w - 1));
      load_x(d, min(d, n_w - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  auto consume = [&](int d) {
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
      for (int c = 0; c < CT; c++) {
        v8i bf;
        if constexpr (X::kE8) {
          static_assert(U == 1, "scaled MFMAs take one K block at a time");
          uint32_t ex;
          xop.make(b[d][c][u], bf, ex);
#pragma unroll
          for (int r = 0; r < RT; r++) acc[r][c] = wop.mma_e8(a[d][r], bf, acc[r][c], sw[d][u], ex);
        } else {
          float sx;
          xop.make(b[d][c][u], bf, sx);
          const float scl = sx * sw[d][u];
#pragma unroll
          for (int r = 0; r < RT; r++) {
            if constexpr (U == 1)
              acc[r][c] += scl * wop.mma(a[d][r], bf);
            else
              acc[r][c] += scl * wop.mma(a[d][r], bf, u);
          }
        }
      }
  };
  // Rounds of D blocks.  While two more full rounds remain, every slot is
  // consumed and refilled on every path, so each wait counts loads exactly
  // and leaves the D - 1 younger slots in flight.  The last full round
  // refills only blocks that exist, and the remainder consumes what is left.
  int i0 = 0;
  for (; i0 + 2 * D <= n_w; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      consume(d);
      load_w(d, i0 + d + D);
      load_x(d, i0 + d + D);
      // keep slot d's refill ahead of slot d + 1's use (the scheduler would
      // sink it past, and the wait there would then drain every load)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (i0 + D <= n_w) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      consume(d);
      if (i0 + d + D < n_w) {
        load_w(d, i0 + d + D);
        load_x(d, i0 + d + D);
      }
    }
    i0 += D;
  }
#pragma unroll
  for (int d = 0; d < D - 1; d++)
    if (i0 + d < n_w) consume(d);

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
  if constexpr (S > 1) {
    const int sp = (int)blockIdx.y;
#pragma unroll
    for (int c = 0; c < CT; c++) {
      const int m = 16 * c + lr;
      if (m >= M) continue;
#pragma unroll
      for (int r = 0; r < RT; r++)
        *reinterpret_cast<v4f *>(part + ((int64_t)sp * M + m) * N + n0 + 16 * r + 4 * g) = acc[r][c];
    }
    return;
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
