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

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm_common.hpp"

namespace fp8lin {

// A 16-row x 128-byte operand tile in whole rows.  Read as an MFMA fragment
// (16 rows x 64 bytes per load instruction) the tile costs the memory
// pipeline a cache-line access per row for half a line; read as two runs of
// 8 whole rows it costs half as many.  Lane l loads row 8h + l / 8 at chunk
// position l % 8, holding logical chunk (l % 8) ^ swz(row), for h = 0 (lo)
// and 1 (hi); written to a 2 KB LDS tile in lane order, the tile then has
// logical chunk p ^ swz(r) at position p of row r, and the fragment reads back
// with the tile kernels' conflict-free offsets.  A tile is private to one
// wave, whose LDS operations complete in order: no barrier.
struct RowRuns {
  uint4 lo, hi;
};
// rows row0 .. row0 + 15 (each clamped to last_row) of a matrix with `stride`
// bytes per row, from byte `col` of each row; kStream: read-once data
template <bool kStream = false>
__device__ __forceinline__ RowRuns load_row_runs(const uint8_t *base, int64_t row0, int64_t last_row, int64_t stride,
                                                 int64_t col) {
  const int lane = threadIdx.x & 63, q = lane >> 3, p = lane & 7;
  const uint8_t *lo = base + min(row0 + q, last_row) * stride + col + 16 * (p ^ swz(q));
  const uint8_t *hi = base + min(row0 + 8 + q, last_row) * stride + col + 16 * (p ^ swz(q + 8));
  RowRuns x;
  x.lo = kStream ? ldg16_stream(lo) : ldg16(lo);
  x.hi = kStream ? ldg16_stream(hi) : ldg16(hi);
  return x;
}
__device__ __forceinline__ v8i row_runs_to_frag(const RowRuns &x, uint8_t *tile) {
  const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
  *reinterpret_cast<uint4 *>(tile + 16 * lane) = x.lo;
  *reinterpret_cast<uint4 *>(tile + 1024 + 16 * lane) = x.hi;
  return make_v8i(*reinterpret_cast<const uint4 *>(tile + lr * 128 + ((g ^ swz(lr)) << 4)),
                  *reinterpret_cast<const uint4 *>(tile + lr * 128 + (((g + 4) ^ swz(lr)) << 4)));
}

// Tokens already quantized by fp8_quant_act: codes and one scale per K block.
// Read as MFMA fragments, a 16-token tile of codes is 16 rows x 64 bytes per
// load instruction, and a fragment's scales are 16 words in 16 different
// 128-byte lines (one line per token row): both cost the memory pipeline a
// line access per row for half a line or less.  The modes:
//   0: both as fragments from global memory;
//   1: each code tile goes through one of the wave's LDS tiles in whole rows
//      (load_row_runs / row_runs_to_frag above); scales from global memory;
//   2: as 1, and the scales of the workgroup's K range are first copied into
//      LDS by linear loads (rows of `ss` floats, ss odd, so that the 16 tokens
//      of a fragment read 16 different banks), behind a barrier.
// launch_decode_kernel picks the mode per launch.
template <int kMode>
struct QuantTokensT {
  const uint8_t *xq;
  const float *xs;
  int K;
  const float *sl = nullptr;  // mode 2: LDS scales [M][ss] of K blocks kb_lo ..
  uint8_t *tl = nullptr;      // modes 1, 2: this wave's code tiles in LDS, 2 KB each
  int kb_lo = 0, ss = 1;
  static constexpr bool kStaged = false, kE8 = false, kCodeLds = kMode >= 1, kScaleLds = kMode == 2;
  typedef float Scale;
  struct RawFrag {
    v8i q;
    float s;
  };
  struct RawLin {
    uint4 lo, hi;                                // rows 0-7 and 8-15 of the tile, chunk position lane % 8
    std::conditional_t<kScaleLds, int, float> s;  // LDS index of the scale, or the scale
  };
  typedef std::conditional_t<kCodeLds, RawLin, RawFrag> Raw;
  static __host__ __device__ int scale_stride(int blocks) { return blocks | 1; }
  static __host__ __device__ size_t scale_lds_bytes(int M, int blocks) {
    return ((size_t)M * scale_stride(blocks) * sizeof(float) + 15) / 16 * 16;
  }
  // dynamic LDS of a workgroup: the scales (mode 2), then NW x CT code tiles
  static __host__ __device__ size_t lds_bytes(int M, int blocks, int NW, int CT) {
    return (kScaleLds ? scale_lds_bytes(M, blocks) : 0) + (size_t)NW * CT * 2048;
  }
  __device__ __forceinline__ void stage(uint8_t *, int, int, int) {}
  // Where the scales of K blocks kb0 .. kb0 + blocks - 1 and this wave's code
  // tiles go in LDS; before any load(), which records the LDS index of its
  // scale.
  __device__ __forceinline__ void bind(uint8_t *lds, int kb0, int blocks, int M, int wave, int CT) {
    sl = reinterpret_cast<const float *>(lds);
    kb_lo = kb0;
    ss = scale_stride(blocks);
    tl = lds + (kScaleLds ? scale_lds_bytes(M, blocks) : 0) + (size_t)wave * CT * 2048;
  }
  // Copies xs[m][kb_lo .. kb_lo + blocks) for every token into LDS, all
  // threads of the workgroup taking part, in passes of kScalePass words per
  // thread (past the end: the last word again, not stored).  The first pass
  // is split in two: load_scales issues its loads, store_scales waits for
  // them and writes LDS (and runs any further passes whole), so loads issued
  // in between stay in flight across the wait.  A barrier must follow before
  // make().
  static constexpr int kScalePass = 4;
  __device__ __forceinline__ void scale_pass_load(float (&v)[kScalePass], int q0, int M, int blocks, int tid,
                                                  int nthreads) const {
    const int KB = K / kGroup, total = M * blocks;
#pragma unroll
    for (int u = 0; u < kScalePass; u++) {
      const int q = min(q0 + u * nthreads + tid, total - 1);
      const int m = q / blocks;
      v[u] = xs[(int64_t)m * KB + kb_lo + (q - m * blocks)];
    }
  }
  __device__ __forceinline__ void scale_pass_store(const float (&v)[kScalePass], int q0, int M, int blocks, int tid,
                                                   int nthreads) const {
    float *lds = const_cast<float *>(sl);
    const int total = M * blocks;
#pragma unroll
    for (int u = 0; u < kScalePass; u++) {
      const int q = q0 + u * nthreads + tid;
      if (q < total) {
        const int m = q / blocks;
        lds[m * ss + (q - m * blocks)] = v[u];
      }
    }
  }
  __device__ __forceinline__ void load_scales(float (&v)[kScalePass], int M, int blocks, int tid, int nthreads) const {
    if (M * blocks > 0) scale_pass_load(v, 0, M, blocks, tid, nthreads);  // uniform
  }
  __device__ __forceinline__ void store_scales(const float (&v)[kScalePass], int M, int blocks, int tid,
                                               int nthreads) const {
    const int total = M * blocks;
    if (total == 0) return;
    scale_pass_store(v, 0, M, blocks, tid, nthreads);
    for (int q0 = kScalePass * nthreads; q0 < total; q0 += kScalePass * nthreads) {
      float w[kScalePass];
      scale_pass_load(w, q0, M, blocks, tid, nthreads);
      scale_pass_store(w, q0, M, blocks, tid, nthreads);
    }
  }
  // global-memory form: token m's fragment of K block kb, and its scale
  __device__ __forceinline__ RawFrag load(int m, int kb, int g) const {
    RawFrag r;
    r.q = load_frag_global(xq + (int64_t)m * K + (int64_t)kb * kGroup, g);
    r.s = xs[(int64_t)m * (K / kGroup) + kb];
    return r;
  }
  __device__ __forceinline__ void make(const RawFrag &r, v8i &frag, float &s) const {
    frag = r.q;
    s = r.s;
  }
  // LDS form: token tile c (rows 16c .., clamped to M - 1) of K block kb in
  // whole rows; m is this lane's token, for its scale
  __device__ __forceinline__ RawLin load_lin(int c, int m, int kb, int M) const {
    const RowRuns runs = load_row_runs(xq, 16 * c, M - 1, K, (int64_t)kb * kGroup);
    RawLin x;
    x.lo = runs.lo;
    x.hi = runs.hi;
    if constexpr (kScaleLds)
      x.s = m * ss + (kb - kb_lo);
    else
      x.s = xs[(int64_t)m * (K / kGroup) + kb];
    return x;
  }
  __device__ __forceinline__ void make_lin(int c, const RawLin &x, v8i &frag, float &s) const {
    frag = row_runs_to_frag(RowRuns{x.lo, x.hi}, tl + c * 2048);
    if constexpr (kScaleLds)
      s = sl[x.s];
    else
      s = x.s;
  }
  template <int kTo>
  QuantTokensT<kTo> as_mode() const {
    return QuantTokensT<kTo>{xq, xs, K};
  }
};
using QuantTokens = QuantTokensT<2>;

// Tokens quantized by fp8_quant_act_ue8m0: codes and one exponent byte per K
// block; the MFMA applies 2^(e - 127) itself.
struct QuantTokensE8 {
  const uint8_t *xq;
  const uint8_t *xe;
  int K;
  static constexpr bool kStaged = false, kE8 = true, kCodeLds = false, kScaleLds = false;
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
  static constexpr bool kStaged = true, kE8 = false, kCodeLds = false, kScaleLds = false;
  typedef float Scale;
  struct Raw {
    v8i q;
    float s;
  };
  static __host__ __device__ size_t lds_bytes(int M, int K) { return (size_t)M * K + (size_t)4 * M * (K / kGroup); }
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
// A weight policy with kRows loads its tiles in whole rows (its Frag) and
// turns them into MFMA operands (its MFrag) through a wave-private LDS tile of
// kTileBytes (to_frag) just before use.
template <class W, class = void>
struct weight_rows {
  static constexpr bool value = false;
};
template <class W>
struct weight_rows<W, std::void_t<decltype(W::kRows)>> {
  static constexpr bool value = W::kRows;
};

// Dynamic LDS of decode_kernel: the waves' weight tiles (kRows weights), then
// what the token policy stages (StagedTokens' codes and scales, or
// QuantTokensT's code tiles and scales), then the reduction buffer of
// the waves' partial sums.  Where the three pass the 160 KB of a workgroup,
// the reduction buffer starts at 0 instead, after a barrier at the end of the
// main loop (every wave is then past its last use of the rest).  The host and
// the kernel both lay it out with plan().
constexpr size_t kDecodeMaxLds = 160 * 1024;
template <class W, class = void>
struct weight_tile_bytes {
  static constexpr size_t value = 0;
};
template <class W>
struct weight_tile_bytes<W, std::void_t<decltype(W::kTileBytes)>> {
  static constexpr size_t value = W::kTileBytes;
};
template <class W, class X, int RT, int CT, int NW>
struct DecodeLds {
  static constexpr size_t kWeightTiles = weight_rows<W>::value ? (size_t)NW * RT * weight_tile_bytes<W>::value : 0;
  static constexpr size_t kRed = NW > 1 ? (size_t)(NW - 1) * RT * CT * 64 * sizeof(v4f) : 0;
  struct Plan {
    size_t tokens, red_off, bytes;
    bool alias;
  };
  static __host__ __device__ Plan plan(int M, int K, int S) {
    size_t tokens = 0;
    if constexpr (X::kStaged) {
      tokens = StagedTokens::lds_bytes(M, K);
    } else if constexpr (X::kCodeLds) {
      const int U = weight_unit<W>::value, KU = K / kGroup / U;
      tokens = X::lds_bytes(M, (KU + S - 1) / S * U, NW, CT);
    }
    const size_t front = (kWeightTiles + tokens + 15) / 16 * 16;
    if (front + kRed <= kDecodeMaxLds) return Plan{tokens, front, front + kRed, false};
    return Plan{tokens, 0, front > kRed ? front : kRed, true};
  }
};

template <class W, class X, int RT, int CT, int NW, int D, int S = 1>
__global__ __launch_bounds__(NW * 64) void decode_kernel(W wop, X xop, const typename X::Scale *__restrict__ ws,
                                                         int M, int N, int K, uint16_t *__restrict__ y,
                                                         float *__restrict__ part) {
  static_assert(128 % (16 * RT) == 0, "a workgroup's rows must sit in one 128-row scale block");
  using Lds = DecodeLds<W, X, RT, CT, NW>;
  extern __shared__ __align__(16) uint8_t decode_lds[];
  uint8_t *const token_lds = decode_lds + Lds::kWeightTiles;  // what the token policy stages
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // kRows weights: this wave's tiles
  uint8_t *const wtile = decode_lds + (size_t)wave * RT * weight_tile_bytes<W>::value;
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
  // unit i of this wave (with staged scales the first slots are loaded on
  // every path, also by a wave without units: its index is clamped into the
  // row, and those loads are never consumed)
  auto unit_of = [&](int i) { return X::kScaleLds ? min(kb0 + wave + i * NW, KU - 1) : kb0 + wave + i * NW; };
  auto load_w = [&](int slot, int i) {
    const int kb = unit_of(i) * U;  // first K block of the unit
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
    const int kb = unit_of(i) * U;
#pragma unroll
    for (int c = 0; c < CT; c++)
#pragma unroll
      for (int u = 0; u < U; u++) {
        if constexpr (X::kCodeLds)
          b[slot][c][u] = xop.load_lin(c, mrow[c], kb + u, M);
        else
          b[slot][c][u] = xop.load(mrow[c], kb + u, g);
      }
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
    xop.stage(token_lds, M, threadIdx.x, NW * 64);
    __syncthreads();
    if (n_w > 0)
#pragma unroll
      for (int d = 0; d < D; d++) load_x(d, min(d, n_w - 1));
  } else {
    // token scales of this split's K blocks: loads issued before the first
    // slots' loads, LDS writes after them (the wait covers only the former)
    float sv[4];
    if constexpr (X::kCodeLds) xop.bind(token_lds, kb0 * U, KBr * U, M, wave, CT);
    if constexpr (X::kScaleLds) {
      static_assert(X::kScalePass == 4, "sv holds one pass of scale words");
      xop.load_scales(sv, M, KBr * U, threadIdx.x, NW * 64);
    }
    // slot by slot, in the loop's order (the waits count loads by age); with
    // staged scales on every path, so that the wait for the scale loads can
    // leave these in flight (a branch around them would make it wait for all)
    if (X::kScaleLds || n_w > 0) {
#pragma unroll
      for (int d = 0; d < D; d++) {
        load_w(d, max(min(d, n_w - 1), 0));
        load_x(d, max(min(d, n_w - 1), 0));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (X::kScaleLds) {
      xop.store_scales(sv, M, KBr * U, threadIdx.x, NW * 64);
      __syncthreads();
    }
  }
  // consume slot d with its weight fragments `af` (a[d] itself, or for kRows
  // weights the fragments made from it through this wave's LDS tiles)
  auto consume_with = [&](int d, const auto &af) {
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
          for (int r = 0; r < RT; r++) acc[r][c] = wop.mma_e8(af[r], bf, acc[r][c], sw[d][u], ex);
        } else {
          float sx;
          if constexpr (X::kCodeLds)
            xop.make_lin(c, b[d][c][u], bf, sx);
          else
            xop.make(b[d][c][u], bf, sx);
          const float scl = sx * sw[d][u];
#pragma unroll
          for (int r = 0; r < RT; r++) {
            if constexpr (U == 1)
              acc[r][c] += scl * wop.mma(af[r], bf);
            else
              acc[r][c] += scl * wop.mma(af[r], bf, u);
          }
        }
      }
  };
  auto consume = [&](int d) {
    if constexpr (weight_rows<W>::value) {
      typename W::MFrag af[RT];
#pragma unroll
      for (int r = 0; r < RT; r++) af[r] = wop.to_frag(a[d][r], wtile + r * weight_tile_bytes<W>::value);
      consume_with(d, af);
    } else {
      consume_with(d, a[d]);
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
    // the partial sums of waves 1 .. NW - 1 meet in LDS (over the tiles and
    // staged tokens where those leave no room: every wave is then first past
    // its last use of them)
    const auto plan = Lds::plan(M, K, S);
    v4f *red = reinterpret_cast<v4f *>(decode_lds + plan.red_off);
    if (plan.alias) __syncthreads();
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < RT; r++)
#pragma unroll
        for (int c = 0; c < CT; c++) red[((wave - 1) * RT * CT + r * CT + c) * 64 + lane] = acc[r][c];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < NW - 1; w++)
#pragma unroll
      for (int r = 0; r < RT; r++)
#pragma unroll
        for (int c = 0; c < CT; c++) acc[r][c] += red[(w * RT * CT + r * CT + c) * 64 + lane];
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


// ===================================================== shared-token form ==
//
// The same GEMM for 3 to 16 quantized tokens on weights of many row bands:
// in decode_kernel every workgroup re-reads all M x K token codes from L2,
// which at 16 tokens doubles the bytes a CU takes in per weight byte (a 16-row
// band of a K = 4096 weight is 64 KB, and so are 16 tokens).  Here a grid of
// about one workgroup per compute unit stages the codes and scales of its K
// range in LDS once and then streams several row bands through it; the waves
// split each band's K units round-robin as in decode_kernel, keep D units of
// weight loads in flight across band boundaries, and meet once per band in
// LDS (or, with WB below, each wave takes whole bands).  Measured on MI355X
// (gate/up 28672 x 4096, weight from HBM), against decode_kernel: dense 3
// tokens 22.0 us against 25.5 us, 16 tokens 25.3 us against 27.4 us; 2:4 3
// tokens 16.6 us against 23.3 us, 16 tokens (WB) 17.7 us against 20.1 us.
//
// Work items: band b in [0, N / (16 RT)) and K split p in [0, S); workgroup
// w of the grid (G workgroups, G a multiple of S) takes split p = w % S and
// bands w / S, w / S + G / S, ...  Each split covers KB / S K blocks (a whole
// number of U-block units).  S = 1 stores y; S > 1 stores fp32 partials
// part[S][M][N] for launch_splitk_reduce.  Two ways to share a workgroup's
// bands among its waves:
//   * WB = false: every band's units round-robin over the waves (at least NW
//     units per split, so that every wave has work in every band), the waves'
//     partial sums meeting once per band;
//   * WB = true: whole bands round-robin over the waves (wave v takes the
//     workgroup's bands v, v + NW, ...), each wave streaming all units of its
//     bands and storing them itself: no partial sums, no barrier after the
//     staging.  Waves without a band only help stage the tokens.
//
// LDS: codes [M][XS] with XS an odd multiple of 128 bytes (the rows of a
// column of K blocks alternate 128-byte bank halves), chunk c of K block kb at
// kb * 128 + 16 * (c ^ swz(m)) as in the tile kernels, so 16-lane fragment
// reads of 16 tokens hit distinct banks; then scales [M][KBs + 1] (the extra
// word staggers the tokens' banks); then (split units only) the partial sums
// of the waves, double-buffered by band parity: the wave that adds band j's
// partials reads buffer j & 1 before the barrier of band j + 1, and the next
// writes to that buffer come after it; then (weights read in whole rows) each
// wave's weight tiles.
struct SharedTokenLayout {
  int KBs, XS, SS;
  size_t red_off, tiles_off, bytes;
  __host__ __device__ SharedTokenLayout(int M, int K, int S, int NW, int RT, size_t wtiles = 0) {
    KBs = K / kGroup / S;
    XS = (KBs + ((KBs & 1) ? 2 : 1)) * kGroup;
    SS = KBs + 1;
    red_off = ((size_t)M * XS + (size_t)4 * M * SS + 15) / 16 * 16;
    tiles_off = red_off + (size_t)2 * NW * RT * 64 * sizeof(v4f);
    bytes = tiles_off + wtiles;
  }
};
template <class W, bool R = weight_rows<W>::value>
struct weight_mfrag {
  typedef typename W::Frag type;
};
template <class W>
struct weight_mfrag<W, true> {
  typedef typename W::MFrag type;
};
template <class W, int RT, int NW>
constexpr size_t shared_weight_tiles() {
  return weight_rows<W>::value ? (size_t)NW * RT * weight_tile_bytes<W>::value : 0;
}

template <class W, int RT, int NW, int D, int S, bool WB = false>
__global__ __launch_bounds__(NW * 64) void decode_shared_kernel(W wop, const uint8_t *__restrict__ xq,
                                                                const float *__restrict__ xs,
                                                                const float *__restrict__ ws, int M, int N, int K,
                                                                uint16_t *__restrict__ y, float *__restrict__ part) {
  static_assert(128 % (16 * RT) == 0, "a band's rows must sit in one 128-row scale block");
  constexpr int U = weight_unit<W>::value;
  extern __shared__ __align__(16) uint8_t shared_tokens[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, lr = lane & 15;
  const SharedTokenLayout L(M, K, S, WB ? 0 : NW, RT, shared_weight_tiles<W, RT, NW>());
  const int KB = K / kGroup, US = L.KBs / U;  // K blocks per row, units per split
  // kRows weights: this wave's tiles
  uint8_t *const wtile = shared_tokens + L.tiles_off + (size_t)wave * RT * weight_tile_bytes<W>::value;
  uint8_t *codes = shared_tokens;
  float *scales = reinterpret_cast<float *>(shared_tokens + (size_t)M * L.XS);
  v4f *red = reinterpret_cast<v4f *>(shared_tokens + L.red_off);
  const int G = gridDim.x, b0 = blockIdx.x;
  const int sp = S > 1 ? b0 % S : 0, kb_lo = sp * L.KBs;
  const int bands = N / (16 * RT), first = b0 / S, stride = G / S;
  const int nbj = first < bands ? (bands - first + stride - 1) / stride : 0;  // bands of this workgroup
  // WB: each wave takes whole bands (the WG's bands wave, wave + NW, ...) and
  // all their units, so no partial sums meet; else the waves split each band's
  // units round-robin
  const int n_w = WB ? US : (US - wave + NW - 1) / NW;  // units per band of this wave (>= 1)
  const int nbw = WB ? (nbj > wave ? (nbj - wave + NW - 1) / NW : 0) : nbj;  // bands of this wave
  const int T = nbw * n_w;
  const int m = min(lr, M - 1);
  const rsrc_t rws = make_rsrc(ws, (uint32_t)((N / kGroup) * KB * (int)sizeof(float)));

  typename W::Frag a[D][RT];
  float sw[D][U];
  // Item (j, i) of this wave: band first + j * stride, unit wave + i * NW of
  // the split.  Items are walked by cursors, so the loop does no division.
  struct Item {
    int j, i;
  };
  auto next = [&](const Item &it) { return it.i + 1 == n_w ? Item{it.j + 1, 0} : Item{it.j, it.i + 1}; };
  auto item_at = [&](int t) {
    const int j = t / n_w;
    return Item{j, t - j * n_w};
  };
  auto band_of = [&](const Item &it) { return WB ? wave + it.j * NW : it.j; };   // index in the WG's band list
  auto unit_of = [&](const Item &it) { return WB ? it.i : wave + it.i * NW; };  // unit within the split
  auto load = [&](int slot, const Item &it) {
    const int n0 = (first + band_of(it) * stride) * 16 * RT, kb = kb_lo + unit_of(it) * U;
#pragma unroll
    for (int r = 0; r < RT; r++) a[slot][r] = wop.load(n0 + 16 * r + lr, kb, g);
#pragma unroll
    for (int u = 0; u < U; u++)
      sw[slot][u] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rws, 0, (uint32_t)((n0 / kGroup) * KB + kb + u) * 4u, 0));
  };
  // the first D items (a wave with fewer repeats its last one: in range, never
  // consumed) go out before the tokens are staged, so their HBM latency
  // overlaps the staging
  if (T > 0)
#pragma unroll
    for (int d = 0; d < D; d++) {
      load(d, item_at(min(d, T - 1)));
      __builtin_amdgcn_sched_barrier(0);
    }
  {
    // 16-byte chunks: every load of a pass is issued before its LDS writes.
    // Row and chunk of a chunk index come from a float reciprocal with one
    // correction step (indices stay below 2^13, so the estimate is off by at
    // most one) instead of an integer division.
    const int cpr = L.KBs * 8, chunks = M * cpr, NT = NW * 64;
    const float inv_cpr = 1.0f / (float)cpr, inv_kbs = 1.0f / (float)L.KBs;
    auto split = [](int q, int d, float inv, int &row, int &rem) {
      row = (int)((float)q * inv);
      rem = q - row * d;
      if (rem < 0) {
        row--;
        rem += d;
      } else if (rem >= d) {
        row++;
        rem -= d;
      }
    };
    for (int q0 = 0; q0 < chunks; q0 += 4 * NT) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        int mm, rem;
        split(min(q0 + u * NT + tid, chunks - 1), cpr, inv_cpr, mm, rem);  // past the end: the last chunk again
        v[u] = *reinterpret_cast<const uint4 *>(xq + (int64_t)mm * K + (int64_t)kb_lo * kGroup + rem * 16);
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int q = q0 + u * NT + tid;
        if (q < chunks) {
          int mm, rem;
          split(q, cpr, inv_cpr, mm, rem);
          const int kb = rem >> 3, c = rem & 7;
          *reinterpret_cast<uint4 *>(codes + mm * L.XS + kb * kGroup + ((c ^ swz(mm)) << 4)) = v[u];
        }
      }
    }
    for (int q = tid; q < M * L.KBs; q += NT) {
      int mm, kb;
      split(q, L.KBs, inv_kbs, mm, kb);
      scales[mm * L.SS + kb] = xs[(int64_t)mm * KB + kb_lo + kb];
    }
  }
  __syncthreads();

  v4f acc[RT];
#pragma unroll
  for (int r = 0; r < RT; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint8_t *xrow = codes + m * L.XS;
  const float *srow = scales + m * L.SS;
  const int f_lo = (g ^ swz(m)) << 4, f_hi = ((g + 4) ^ swz(m)) << 4;
  auto consume = [&](int d, const Item &it) {
    const int kr = unit_of(it) * U;  // first K block of the unit, relative to the split
    typename weight_mfrag<W>::type af[RT];
#pragma unroll
    for (int r = 0; r < RT; r++) {
      if constexpr (weight_rows<W>::value)
        af[r] = wop.to_frag(a[d][r], wtile + r * weight_tile_bytes<W>::value);
      else
        af[r] = a[d][r];
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint8_t *blk = xrow + (kr + u) * kGroup;
      const v8i bf = make_v8i(*reinterpret_cast<const uint4 *>(blk + f_lo), *reinterpret_cast<const uint4 *>(blk + f_hi));
      const float scl = srow[kr + u] * sw[d][u];
#pragma unroll
      for (int r = 0; r < RT; r++) {
        if constexpr (U == 1)
          acc[r] += scl * wop.mma(af[r], bf);
        else
          acc[r] += scl * wop.mma(af[r], bf, u);
      }
    }
  };
  // after item it: if it closed band j, the waves' partial sums meet in LDS
  // and wave j % NW adds them in wave order and stores the band
  auto flush = [&](const Item &it) {
    if (it.i != n_w - 1) return;
    if constexpr (WB) {
      const int n0 = (first + band_of(it) * stride) * 16 * RT;
      if (lr < M) {
#pragma unroll
        for (int r = 0; r < RT; r++) {
          const int n = n0 + 16 * r + 4 * g;
          if constexpr (S > 1)
            *reinterpret_cast<v4f *>(part + ((int64_t)sp * M + lr) * N + n) = acc[r];
          else
            *reinterpret_cast<uint2 *>(y + (int64_t)lr * N + n) = pack_bf16x4(acc[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < RT; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
      return;
    }
    const int j = it.j;
    v4f *buf = red + (size_t)(j & 1) * NW * RT * 64;
#pragma unroll
    for (int r = 0; r < RT; r++) buf[(wave * RT + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (wave == j % NW) {
      v4f sum[RT];
#pragma unroll
      for (int r = 0; r < RT; r++) sum[r] = buf[r * 64 + lane];
      for (int w = 1; w < NW; w++)
#pragma unroll
        for (int r = 0; r < RT; r++) sum[r] += buf[(w * RT + r) * 64 + lane];
      const int n0 = (first + j * stride) * 16 * RT;
      if (lr < M) {
#pragma unroll
        for (int r = 0; r < RT; r++) {
          const int n = n0 + 16 * r + 4 * g;
          if constexpr (S > 1)
            *reinterpret_cast<v4f *>(part + ((int64_t)sp * M + lr) * N + n) = sum[r];
          else
            *reinterpret_cast<uint2 *>(y + (int64_t)lr * N + n) = pack_bf16x4(sum[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RT; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  };
  // the slot schedule of decode_kernel over this wave's T items; t0 + d counts
  // items for the control flow, the cursors carry their (band, unit)
  Item cons{0, 0}, ld = item_at(D);
  int t0 = 0;
  for (; t0 + 2 * D <= T; t0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      consume(d, cons);
      load(d, ld);
      flush(cons);
      cons = next(cons);
      ld = next(ld);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (t0 + D <= T) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      consume(d, cons);
      if (t0 + d + D < T) load(d, ld);
      flush(cons);
      cons = next(cons);
      ld = next(ld);
    }
    t0 += D;
  }
#pragma unroll
  for (int d = 0; d < D - 1; d++)
    if (t0 + d < T) {
      consume(d, cons);
      flush(cons);
      cons = next(cons);
    }
}

// Host side of decode_kernel: its dynamic LDS (DecodeLds), and a launch that
// raises the kernel's LDS limit once per device where that passes 64 KB.
template <class W, class X, int RT, int CT, int NW>
inline size_t decode_lds_bytes(int M, int K, int S) {
  return DecodeLds<W, X, RT, CT, NW>::plan(M, K, S).bytes;
}

// decode_kernel<W, X, ...> itself, with the dynamic LDS its token policy needs
template <class W, class X, int RT, int CT, int NW, int D, int S>
hipError_t launch_decode_kernel_as(W wop, X xop, const typename X::Scale *ws, int M, int N, int K, uint16_t *y,
                                   float *part, hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> raised[kMaxDevices];
  const size_t lds = decode_lds_bytes<W, X, RT, CT, NW>(M, K, S);
  if (lds > 64 * 1024) {
    if (lds > kDecodeMaxLds) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!raised[dev].load(std::memory_order_acquire)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_kernel<W, X, RT, CT, NW, D, S>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecodeMaxLds);
      if (e != hipSuccess) return e;
      raised[dev].store(true, std::memory_order_release);
    }
  }
  const int bands = N / (16 * RT);
  hipLaunchKernelGGL((decode_kernel<W, X, RT, CT, NW, D, S>), dim3(bands, S), dim3(NW * 64), lds, stream, wop, xop, ws,
                     M, N, K, y, S > 1 ? part : nullptr);
  return hipGetLastError();
}

// The fewest U-block units a wave of any split gets (floor of the smallest
// split's units over the waves).
inline int min_units_per_wave(int K, int S, int U, int NW) {
  const int KU = K / kGroup / U, KBs = (KU + S - 1) / S;
  int fewest = KU;
  for (int sp = 0; sp < S; sp++) fewest = std::min(fewest, std::max(0, std::min(KU, (sp + 1) * KBs) - sp * KBs));
  return fewest / NW;
}

// Quantized tokens (QuantTokensT) take mode 2 (codes in whole rows through
// LDS, scales staged in LDS behind a barrier) from 17 tokens on (two or more
// token tiles) where every wave has at least two units, so that the staging
// and its barrier are spread over a pipeline of loads, and only for one-block
// units and at most 16 fragments of loads in flight per wave (RT * CT * D),
// where the kernel keeps its registers (the four-block 2:4 units and the
// three-deep 64-row bands spill); otherwise mode 1 (codes only, no barrier)
// from kCodeLdsMinTokens tokens on, and mode 0 below that.  Measured on MI355X
// against mode 0, Llama-3-8B weights from HBM (A/B in one process, results
// bit-identical), mode 2:
//   6144 x 4096   20 / 32 / 64 tokens 10.5 / 12.0 / 17.9 -> 9.1 / 10.1 / 12.9 us
//   4096 x 4096   32 / 64 tokens       9.9 / 13.0 -> 8.1 / 11.3 us
//   4096 x 14336  20 / 32 tokens       17.4 / 18.7 -> 16.9 / 17.8 us
//   2:4 at 64 tokens: 6144 x 4096 17.9 -> 12.6 us, 4096 x 4096 13.2 -> 10.9 us;
//   2:4 4096 x 14336 at 32 tokens 18.1 -> 16.4 us.
// The scale staging alone gave about half of that; up to 16 tokens it was
// level to 6 % slower, and so it was with a single unit per wave (the 2:4
// four-block units on K = 4096: 3 to 7 % slower).  Mode 1 against mode 0:
//   2:4 6144 x 4096 at 8 / 12 / 16 tokens 6.5 / 6.7 / 7.1 -> 6.0 / 6.3 / 6.5 us
//   2:4 4096 x 4096 at 16 / 24 / 32 tokens 5.7 / 6.7 / 7.5 -> 5.1 / 5.6 / 5.8 us
//   2:4 4096 x 14336 at 8 tokens 11.4 -> 10.3 us; dense level to 4 % faster;
// at 4 and 5 tokens level to 4 % slower.
constexpr int kScaleLdsMinTokens = 17, kScaleLdsMinUnitsPerWave = 2, kScaleLdsMaxFragsInFlight = 16;
constexpr int kCodeLdsMinTokens = 8;

template <class W, class X, int RT, int CT, int NW, int D, int S>
hipError_t launch_decode_kernel(W wop, X xop, const typename X::Scale *ws, int M, int N, int K, uint16_t *y,
                                float *part, hipStream_t stream) {
  constexpr int U = weight_unit<W>::value;
  if constexpr (X::kScaleLds) {
    constexpr bool kMode2Fits = U == 1 && CT >= 2 && RT * CT * D <= kScaleLdsMaxFragsInFlight;
    if constexpr (kMode2Fits) {
      if (M >= kScaleLdsMinTokens && min_units_per_wave(K, S, U, NW) >= kScaleLdsMinUnitsPerWave)
        return launch_decode_kernel_as<W, X, RT, CT, NW, D, S>(wop, xop, ws, M, N, K, y, part, stream);
    }
    // mode 1 where its registers fit (the four-block 2:4 units with more than
    // two fragments per slot spill)
    constexpr bool kMode1Fits = U == 1 ? RT * CT * D <= kScaleLdsMaxFragsInFlight : RT * CT <= 2;
    if constexpr (kMode1Fits) {
      if (M >= kCodeLdsMinTokens)
        return launch_decode_kernel_as<W, QuantTokensT<1>, RT, CT, NW, D, S>(wop, xop.template as_mode<1>(), ws, M, N,
                                                                             K, y, part, stream);
    }
    return launch_decode_kernel_as<W, QuantTokensT<0>, RT, CT, NW, D, S>(wop, xop.template as_mode<0>(), ws, M, N, K,
                                                                         y, part, stream);
  } else {
    return launch_decode_kernel_as<W, X, RT, CT, NW, D, S>(wop, xop, ws, M, N, K, y, part, stream);
  }
}

// Host side of the shared-token form.  The kernel's LDS (up to 160 KB) is
// dynamic, above the 64 KB a launch gets without asking, so each instance
// raises its limit once per device.
constexpr int kSharedTokenMaxLds = 160 * 1024;

// Grid of the shared-token form for this shape (0: the shape does not fit it):
// the split's K range must hold at least NW units of U blocks (unless each
// wave takes whole bands, WB), and the codes of the M tokens and the partial
// sums must fit the LDS.  One workgroup per compute unit per split, or two
// for at most 8 tokens with the split units (whose staging is cheaper;
// measured on MI355X), each streaming several row bands.
inline int shared_decode_grid(int M, int N, int K, int S, int U, int NW, int RT, int cus, bool wb = false,
                              size_t wtiles = 0) {
  const int KB = K / kGroup;
  if (M < 1 || M > 16 || N % (16 * RT) != 0 || KB % (S * U) != 0 || (!wb && KB / S / U < NW)) return 0;
  if (SharedTokenLayout(M, K, S, wb ? 0 : NW, RT, wtiles).bytes > (size_t)kSharedTokenMaxLds) return 0;
  const int bands = N / (16 * RT);
  return std::min(bands, (!wb && M <= 8 ? 2 : 1) * cus) * S;
}

template <class W, int RT, int NW, int D, int S, bool WB = false>
hipError_t launch_decode_shared(W wop, const uint8_t *xq, const float *xs, const float *ws, int M, int N, int K,
                                uint16_t *y, float *part, int grid, hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> raised[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!raised[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_shared_kernel<W, RT, NW, D, S, WB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kSharedTokenMaxLds);
    if (e != hipSuccess) return e;
    raised[dev].store(true, std::memory_order_release);
  }
  if (S > 1 && !part) return hipErrorInvalidValue;
  const SharedTokenLayout L(M, K, S, WB ? 0 : NW, RT, shared_weight_tiles<W, RT, NW>());
  hipLaunchKernelGGL((decode_shared_kernel<W, RT, NW, D, S, WB>), dim3(grid), dim3(NW * 64), L.bytes, stream, wop, xq,
                     xs, ws, M, N, K, y, part);
  return hipGetLastError();
}

}  // namespace fp8lin
