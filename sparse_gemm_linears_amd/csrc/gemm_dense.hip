// Dense block-scaled FP8 GEMM:  y[m,n] = bf16( sum_kb xs[m,kb] * ws[n/128,kb] * P(m,n,kb) ),
// P = the exact FP8 dot product over one 128-wide K block, accumulated in fp32 by
// v_mfma_f32_16x16x128_f8f6f4 (one instruction per 16x16 output tile and K block).
//
// The weight is MFMA operand A (rows = n) and the activations operand B
// (columns = m), so one lane's four results share a token m and a weight block
// row: the scale of a 16x16 partial is one fp32 product per lane, applied with
// four FMAs into the running fp32 accumulator.
//
// Two kernels:
//  * tile kernel (large M): BN x BM output tile per workgroup, 128-wide K steps
//    staged through double-buffered, swizzled LDS, one barrier per step,
//    coalesced bf16 stores through LDS at the end;
//  * decode kernel (M <= 64): the weight streams from HBM straight into MFMA
//    registers, the waves of a workgroup split K and meet in LDS at the end.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm_common.hpp"
#include "gemm_decode.hpp"
#include "launch.hpp"

namespace fp8lin {

// ============================================================== tile kernel ==

template <int BN, int BM, int WN, int WM>
struct DenseTile {
  static constexpr int kWaves = WN * WM, kThreads = kWaves * 64;
  static constexpr int kWaveN = BN / WN, kWaveM = BM / WM;
  static constexpr int RT = kWaveN / 16, CT = kWaveM / 16;
  static constexpr int kACopies = BN / 8 / kWaves, kBCopies = BM / 8 / kWaves;  // 1 KB = 8 rows per copy
  static constexpr int kATile = BN * 128, kBTile = BM * 128;
  static constexpr int kWavesPerSlice = WM;  // waves sharing a weight slice (one per token slice)
  static_assert(BN == 256 && (BM == 256 || BM == 128), "panels are addressed as 128-row halves");
  static_assert(128 % (8 * kWaves) == 0, "copy slabs tile the 128-row halves");
  static_assert(kWaves % 2 == 0, "copy slabs alternate 16-row parity per wave");
  static_assert(kWaveN == 128, "a wave covers one 128-row weight scale block (and 256-byte epilogue rows)");
  static_assert(BM <= kThreads, "one thread per token scale");
  static_assert(kWaves * 4096 <= kATile, "epilogue scratch fits in one weight stage");
};

// Arguments of the optional tile-kernel modes.
//  SwiGLU epilogue: h [M,I] bf16 is the kernel's y; when hq is not NULL, its
//  per-token 1x128 e4m3 codes hq [M,I] and scales hs [M,I/128] as well.
//  Grouped GEMM: G expert weights [G][N][K] (scales [G][N/128][K/128]); the
//  tokens of expert g are rows offsets[g] .. offsets[g+1] - 1 of X and Y.
//  Split K: workgroup (tile, s) covers K blocks [s * kb_split, +kb_split) and
//  writes its fp32 partial tile to part + s * M * N ([M][N]).
struct TileExtra {
  uint8_t *hq;
  float *hs;
  int I;
  const int32_t *offsets;
  int G;
  float *part;
  int kb_split;
};

// SwiGLU epilogue.  The two waves with the same token slice hold the gate
// (wn0 = 0) and up (wn0 = 128) sums of the same 128 outputs in the same
// register layout.  The work is split between them by token tile: in round p
// the gate wave finishes token tile 2p and the up wave token tile 2p + 1, each
// after receiving the other wave's sums of its tile through LDS (xch_g holds
// gate sums sent to the up wave, xch_u up sums sent to the gate wave).  A wave
// forms h = silu(g) * u = g * u / (1 + exp(-g)) in fp32, stores bf16(h) and, if
// asked, quantizes bf16(h) as fp8_quant_act would: the tile's 128 outputs are
// exactly one 1x128 group of a token, held by the four lane groups of the
// token's lanes (two xor-shuffles give the group amax).
template <class C>
__device__ __forceinline__ void swiglu_finish(const v4f (&gv)[C::RT], const v4f (&uv)[C::RT], uint8_t *scratch,
                                              uint16_t *h, const TileExtra &so, int M, int m0, int tn, int lane) {
  const int lr = lane & 15, g = lane >> 4;
  v4f hv[C::RT];
#pragma unroll
  for (int r = 0; r < C::RT; r++) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      // silu with the hardware exp2 and reciprocal (a few ulp in fp32, far
      // below the bf16 rounding that follows); the bf16 value is what h holds
      // in memory and what the codes are made from
      const float gg = gv[r][e];
      hv[r][e] = bf16_to_f32(f32_to_bf16_rne(gg * uv[r][e] * __builtin_amdgcn_rcpf(1.0f + __expf(-gg))));
    }
  }
  if (h) store_token_tile<C::RT>(scratch, hv, h, M, so.I, m0, 128 * tn, lane);
  if (!so.hq) return;
  uint32_t amax_bits = 0;
#pragma unroll
  for (int r = 0; r < C::RT; r++)
#pragma unroll
    for (int e = 0; e < 4; e++) amax_bits = max(amax_bits, __float_as_uint(hv[r][e]) & 0x7FFFFFFFu);
  amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 16, 64));
  amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 32, 64));
  const GroupScale gs = group_scale(amax_bits);
  uint32_t words[C::RT];
#pragma unroll
  for (int r = 0; r < C::RT; r++) {
    const float v[4] = {hv[r][0], hv[r][1], hv[r][2], hv[r][3]};
    words[r] = quantize4_group(v, gs);
  }
  // codes through the wave's LDS scratch (16 rows x 128 bytes, 16-byte chunks
  // XOR-swizzled by row) so that each row goes out as 128 contiguous bytes
#pragma unroll
  for (int r = 0; r < C::RT; r++)
    *reinterpret_cast<uint32_t *>(scratch + lr * 128 + ((r ^ (lr & 7)) << 4) + 4 * g) = words[r];
  if (g == 0 && m0 + lr < M) so.hs[(int64_t)(m0 + lr) * (so.I / kGroup) + tn] = gs.s;
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int row = 8 * p + (lane >> 3), chunk = lane & 7;
    const v4i v = *reinterpret_cast<const v4i *>(scratch + row * 128 + ((chunk ^ (row & 7)) << 4));
    if (m0 + row < M) *reinterpret_cast<v4i *>(so.hq + (int64_t)(m0 + row) * so.I + 128 * tn + 16 * chunk) = v;
  }
}

template <class C>
__device__ __forceinline__ void swiglu_epilogue(v4f (&acc)[C::RT][C::CT], v4f *xch_g, v4f *xch_u, uint8_t *scratch,
                                                uint16_t *h, const TileExtra &so, int M, int m_wave, int tn, int wave,
                                                int wn0, int lane) {
  static_assert(C::CT % 2 == 0, "token tiles are shared out in pairs");
  static_assert(C::kWavesPerSlice * C::RT * 64 * 16 <= C::kBTile, "one exchange direction fits in a token stage");
  const int slot = wave % C::kWavesPerSlice;
  const bool gate = wn0 == 0;
#pragma unroll
  for (int p = 0; p < C::CT / 2; p++) {
    constexpr int kRow = C::RT * 64;
    v4f *mine = (gate ? xch_g : xch_u) + slot * kRow + lane;  // what this wave sends
    const v4f *theirs = (gate ? xch_u : xch_g) + slot * kRow + lane;
    // the gate wave sends tile 2p + 1, the up wave tile 2p (compile-time
    // register indices in both branches)
    if (gate) {
#pragma unroll
      for (int r = 0; r < C::RT; r++) mine[r * 64] = acc[r][2 * p + 1];
    } else {
#pragma unroll
      for (int r = 0; r < C::RT; r++) mine[r * 64] = acc[r][2 * p];
    }
    __syncthreads();
    v4f other[C::RT];
#pragma unroll
    for (int r = 0; r < C::RT; r++) other[r] = theirs[r * 64];
    if (gate) {
      v4f gv[C::RT];
#pragma unroll
      for (int r = 0; r < C::RT; r++) gv[r] = acc[r][2 * p];
      swiglu_finish<C>(gv, other, scratch, h, so, M, m_wave + 32 * p, tn, lane);
    } else {
      v4f uv[C::RT];
#pragma unroll
      for (int r = 0; r < C::RT; r++) uv[r] = acc[r][2 * p + 1];
      swiglu_finish<C>(other, uv, scratch, h, so, M, m_wave + 32 * p + 16, tn, lane);
    }
    __syncthreads();
  }
}

// SB: K blocks per token-scale load (4 when K/128 is a multiple of 4, else 1).
// CR: the next K block's copies are issued across the first CR row tiles.
// SWIGLU: the weight is [gate; up] (2I rows); tile tn covers outputs
// [128 tn, 128 tn + 128) and reads gate rows there into the first panel half
// and up rows I + 128 tn .. into the second; y is h [M,I].
// E8: UE8M0 scales (xs, ws are exponent bytes) applied by the MFMA's block
// scaling, accumulating straight into the accumulators with no VALU work.
// GROUPED: tiles_m bounds the token tiles over all groups (the sum of
// ceil(rows_g / BM) <= ceil(M / BM) + G); the tiles that exist are counted
// from the offsets and ordered as in the plain kernel, and the workgroups
// beyond them return at once.
// PARTIAL: split K over blockIdx.y (so.kb_split K blocks each, a multiple of
// SB) and store unrounded fp32 partial tiles instead of y.
template <int BN, int BM, int WN, int WM, int SB, int CR, bool SWIGLU, bool E8 = false, bool GROUPED = false,
          bool PARTIAL = false>
__global__ __launch_bounds__(WN *WM * 64) void dense_tile_kernel(
    const uint8_t *__restrict__ xq, const std::conditional_t<E8, uint8_t, float> *__restrict__ xs,
    const uint8_t *__restrict__ wq_all, const std::conditional_t<E8, uint8_t, float> *__restrict__ ws_all,
    int M_all, int N, int K, uint16_t *__restrict__ y, int tiles_m, int tiles_n, int group_m, TileExtra so) {
  using C = DenseTile<BN, BM, WN, WM>;
  // One LDS object per stage and panel: copies into one stage and fragment
  // reads of the other are then known not to overlap, so reads never wait for
  // the copies in flight.
  __shared__ __align__(16) uint8_t lds_a0[C::kATile], lds_a1[C::kATile];
  __shared__ __align__(16) uint8_t lds_b0[C::kBTile], lds_b1[C::kBTile];
  __shared__ __align__(16) float lds_s[2 * SB * BM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, lr = lane & 15;
  const int cj = lane >> 3, cp = lane & 7;  // copy lane -> (row in an 8-row slab, chunk position)
  // KBs: K blocks per row (the stride of the scale rows); KB: K blocks this
  // workgroup accumulates, starting at block kb0
  const int KBs = K / kGroup, NB = N / kGroup;
  int kb0 = 0, KB = KBs;
  if constexpr (PARTIAL) {
    kb0 = blockIdx.y * so.kb_split;
    KB = min(so.kb_split, KBs - kb0);
  }

  int tm, tn, tiles_m_used = tiles_m;
  if constexpr (GROUPED) {
    // the launch covers the worst case; the tile order (and its split over the
    // XCDs) covers only the token tiles that exist, so that the surplus
    // workgroups, which return at once, are spread over every XCD instead of
    // taking whole XCDs at the end of the order
    int real = 0;
    for (int q = 0; q < so.G; q++) {
      const int o0 = min(max(so.offsets[q], 0), M_all), o1 = min(max(so.offsets[q + 1], o0), M_all);
      real += (o1 - o0 + BM - 1) / BM;
    }
    tiles_m_used = __builtin_amdgcn_readfirstlane(min(real, tiles_m));
    if (!tile_slot_used(blockIdx.x, tiles_m_used * tiles_n)) return;  // uniform: before any barrier
  }
  tile_coords(blockIdx.x, tiles_m_used, tiles_n, group_m, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  // token rows [m_base, M) of this tile and its weight
  int m_base = tm * BM, M = M_all;
  const uint8_t *wq = wq_all;
  const auto *ws = ws_all;
  if constexpr (GROUPED) {
    // token tiles are numbered group after group, ceil(rows_g / BM) per group
    int t = tm, sel = -1, m0 = 0, m1 = 0;
    // offsets are clamped into [0, M_all] and made nondecreasing, so that any
    // contents keep every access inside X and Y
    for (int q = 0; q < so.G; q++) {
      const int o0 = min(max(so.offsets[q], 0), M_all), o1 = min(max(so.offsets[q + 1], o0), M_all);
      const int nt = (o1 - o0 + BM - 1) / BM;
      if (t < nt) {
        sel = q;
        m0 = o0 + t * BM;
        m1 = o1;
        break;
      }
      t -= nt;
    }
    sel = __builtin_amdgcn_readfirstlane(sel);
    if (sel < 0) return;  // past the last group's tiles (uniform: before any barrier)
    m_base = __builtin_amdgcn_readfirstlane(m0);
    M = __builtin_amdgcn_readfirstlane(m1);
    wq = wq_all + (int64_t)sel * N * K;
    ws = ws_all + (int64_t)sel * (N / kGroup) * (K / kGroup);
  }
  const int n_base = tn * BN;
  const int wn0 = (wave / WM) * C::kWaveN, wm0 = (wave % WM) * C::kWaveM;

  // Copy slab i of this wave covers panel rows r0 = (i*kWaves + wave)*8 .. +7;
  // lane (cj, cp) writes LDS chunk position cp of row r0+cj, i.e. logical
  // chunk cp ^ swz(r0+cj); r0 % 16 = 8*(wave % 2) for every i.  Both panels
  // have K-byte rows, so one per-lane offset serves every copy; the slab and
  // the K block go into the scalar offset.
  const uint32_t copy_voff = (uint32_t)((wave * 8 + cj) * K + 16 * (cp ^ swz(cj + 8 * (wave & 1))));
  // first weight row of each 128-row panel half
  const int w_half0 = SWIGLU ? 128 * tn : n_base;
  const int w_half1 = SWIGLU ? so.I + 128 * tn : n_base + 128;
  // (a K range starting at block kb0 shifts every panel row by kb0 * 128
  // bytes; reads stay below row offset (kb0 + KB) * 128 <= K)
  const uint8_t *xpanel = xq + (int64_t)m_base * K + kb0 * kGroup;
  const rsrc_t rw0 = panel_rows128(wq + (int64_t)w_half0 * K + kb0 * kGroup, N - w_half0, 0, K);
  const rsrc_t rw1 = panel_rows128(wq + (int64_t)w_half1 * K + kb0 * kGroup, N - w_half1, 0, K);
  const rsrc_t rx0 = panel_rows128(xpanel, M - m_base, 0, K), rx1 = panel_rows128(xpanel, M - m_base, 128, K);
  std::conditional_t<E8, TokenExps<BM, SB>, TokenScales<BM, SB>> scales;
  scales.init(lds_s, xs + kb0, M, KBs, m_base, tid);

  // One 128-wide K block of the weight and token panels into LDS stage `st`.
  auto issue_copy = [&](int kb, int st, int j) {
    constexpr int kSlab = 8 * C::kWaves;  // panel rows covered by one copy of every wave
    const bool is_a = j < C::kACopies;
    const int first = (is_a ? j : j - C::kACopies) * kSlab;  // panel row of wave 0's slab
    const uint32_t soff = (uint32_t)kb * 128u + (uint32_t)(first % 128) * (uint32_t)K;
    const int lds_off = (first + wave * 8) * 128;
    if (is_a)
      buffer_copy16_to_lds(first < 128 ? rw0 : rw1, copy_voff, soff, (st ? lds_a1 : lds_a0) + lds_off);
    else
      buffer_copy16_to_lds(first < 128 ? rx0 : rx1, copy_voff, soff, (st ? lds_b1 : lds_b0) + lds_off);
  };
  constexpr int kCopies = C::kACopies + C::kBCopies;
  constexpr int kCopyRows = CR < C::RT ? CR : C::RT;  // copies are spread over the first kCopyRows row tiles
  constexpr int kCopiesPerRow = (kCopies + kCopyRows - 1) / kCopyRows;

  // per-lane fragment read offsets (row lr of a 16-row slab, chunks g and g+4)
  const int fr_lo = lr * 128 + ((g ^ swz(lr)) << 4);
  const int fr_hi = lr * 128 + (((g + 4) ^ swz(lr)) << 4);
  const int a_lo = wn0 * 128 + fr_lo, a_hi = wn0 * 128 + fr_hi;
  const int b_lo = wm0 * 128 + fr_lo, b_hi = wm0 * 128 + fr_hi;

  v4f acc[C::RT][C::CT];
#pragma unroll
  for (int r = 0; r < C::RT; r++)
#pragma unroll
    for (int c = 0; c < C::CT; c++) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nb_wave = min((wn0 == 0 ? w_half0 : w_half1) / kGroup, NB - 1);
  const auto *ws_row = ws + (int64_t)nb_wave * KBs + kb0;

  // Token fragments live in registers one K step ahead: bx[ST] holds this
  // step's, and the next step's are read from LDS during row tiles
  // kBReadRow.. of this step.  Token copies therefore run two steps ahead (the
  // stage they overwrite was drained into registers a step earlier) and the
  // weight copies one step ahead; every copy still has a whole step to land.
  v8i bx[2][C::CT];
  constexpr int kBReadRow = C::RT - C::CT;
  auto read_b = [&](const uint8_t *Bt, v8i (&dst)[C::CT], int c) {
    dst[c] = load_frag_at(Bt, b_lo, b_hi, c * 2048);
  };

  // One K step: A stage ST, B fragments in bx[ST].  The copies issued here
  // (weights of kb+1 into A stage ST^1, tokens of kb+2 into B stage ST) and,
  // once per scale group, the next token scales are in flight while the MFMAs
  // run.  The partial of each 16x16 tile is scaled into its accumulator while
  // the MFMA of the following tile executes.
  auto step = [&](int kb, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    const bool more_a = kb + 1 < KB, more_b = kb + 2 < KB;
    const bool scale_load = (kb % SB == 0) && (kb + SB < KB);
    if (scale_load) scales.load(kb / SB + 1);
    const uint8_t *At = ST ? lds_a1 : lds_a0;
    const uint8_t *Bn = ST ? lds_b0 : lds_b1;  // tokens of kb+1
    // fp32 scales: scl = xs * ws per token, applied by FMAs; UE8M0: the two
    // exponents go to the MFMA
    std::conditional_t<E8, uint32_t, float> scl[C::CT];
    const auto sw = ws_row[kb];
#pragma unroll
    for (int c = 0; c < C::CT; c++) {
      if constexpr (E8) scl[c] = scales.get(kb, wm0 + 16 * c + lr);
      else scl[c] = scales.get(kb, wm0 + 16 * c + lr) * sw;
    }
    v8i an = load_frag_at(At, a_lo, a_hi, 0);
    v4f p_prev, p_prev2;
#pragma unroll
    for (int r = 0; r < C::RT; r++) {
      if (r < kCopyRows) {
#pragma unroll
        for (int j = r * kCopiesPerRow; j < (r + 1) * kCopiesPerRow && j < kCopies; j++) {
          if (j < C::kACopies) {
            if (more_a) issue_copy(kb + 1, ST ^ 1, j);
          } else if (more_b) {
            issue_copy(kb + 2, ST, j);
          }
        }
      }
      const v8i af = an;
      // a compiler-only fence: the next row's fragment reads are not hoisted
      // above this row (with no VALU work between the MFMAs, the compiler
      // would read every fragment of the step up front and spill)
      if constexpr (E8) asm volatile("" ::: "memory");
      if (r + 1 < C::RT) an = load_frag_at(At, a_lo, a_hi, (r + 1) * 2048);
      if (r >= kBReadRow && more_a) read_b(Bn, bx[ST ^ 1], r - kBReadRow);
#pragma unroll
      for (int c = 0; c < C::CT; c++) {
        if constexpr (E8) {
          acc[r][c] = mfma_16x16x128_fp8_e8(af, bx[ST][c], acc[r][c], (uint32_t)sw, scl[c]);
          pin(acc[r][c]);  // keeps the MFMA in its row (nothing else reads acc until the epilogue)
        } else {
          const v4f p = mfma_16x16x128_fp8(af, bx[ST][c], v4f{0.f, 0.f, 0.f, 0.f});
          // scale the partial of two MFMAs back: its result is ready, so the
          // FMAs issue without hazard waits while this MFMA runs
          const int t = r * C::CT + c;
          if (t > 1) {
            const int pr = (t - 2) / C::CT, pc = (t - 2) % C::CT;
            acc[pr][pc] += scl[pc] * p_prev2;
            pin(acc[pr][pc]);
          }
          p_prev2 = p_prev;
          p_prev = p;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!E8) {
      acc[C::RT - 1][C::CT - 2] += scl[C::CT - 2] * p_prev2;
      pin(acc[C::RT - 1][C::CT - 2]);
      acc[C::RT - 1][C::CT - 1] += scl[C::CT - 1] * p_prev;
      pin(acc[C::RT - 1][C::CT - 1]);
    }
    if (more_a || scale_load) wait_global_loads();
    if (scale_load) scales.store(kb / SB + 1);
    __syncthreads();
  };

  // prologue: weights of K block 0, tokens of K blocks 0 and 1
#pragma unroll
  for (int j = 0; j < kCopies; j++) issue_copy(0, 0, j);
  if (KB > 1) {
#pragma unroll
    for (int j = C::kACopies; j < kCopies; j++) issue_copy(1, 1, j);
  }
  scales.load(0);
  wait_global_loads();
  scales.store(0);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < C::CT; c++) read_b(lds_b0, bx[0], c);
  __syncthreads();  // B stage 0 is refilled by step 0
  for (int kb = 0; kb < KB; kb += 2) {
    step(kb, std::integral_constant<int, 0>{});
    if (kb + 1 < KB) step(kb + 1, std::integral_constant<int, 1>{});
  }

  // epilogue through a wave-private 4 KB slice of the (now idle) weight stage 0
  uint8_t *scratch = lds_a0 + wave * 4096;
  if constexpr (PARTIAL) {
    float *part = so.part + (int64_t)blockIdx.y * M * N;
#pragma unroll
    for (int c = 0; c < C::CT; c++) {
      v4f col[C::RT];
#pragma unroll
      for (int r = 0; r < C::RT; r++) col[r] = acc[r][c];
      store_token_tile_f32<C::RT>(col, part, M, N, m_base + wm0 + 16 * c, n_base + wn0, lane);
    }
  } else if constexpr (!SWIGLU) {
#pragma unroll
    for (int c = 0; c < C::CT; c++) {
      v4f col[C::RT];
#pragma unroll
      for (int r = 0; r < C::RT; r++) col[r] = acc[r][c];
      store_token_tile<C::RT>(scratch, col, y, M, N, m_base + wm0 + 16 * c, n_base + wn0, lane);
    }
  } else {
    swiglu_epilogue<C>(acc, reinterpret_cast<v4f *>(lds_b0), reinterpret_cast<v4f *>(lds_b1), scratch, y, so, M,
                       m_base + wm0, tn, wave, wn0, lane);
  }
}


// ============================================================ decode kernel ==

// Weight operand of the decode kernel: 32 bytes of one row's K block per lane.
struct DenseWeight {
  typedef v8i Frag;
  const uint8_t *wq;
  int K;
  __device__ __forceinline__ Frag load(int64_t row, int kb, int g) const {
    return load_frag_global(wq + row * K + (int64_t)kb * kGroup, g);
  }
  __device__ __forceinline__ v4f mma(const v8i &a, const v8i &b) const {
    return mfma_16x16x128_fp8(a, b, v4f{0.f, 0.f, 0.f, 0.f});
  }
  __device__ __forceinline__ v4f mma_e8(const v8i &a, const v8i &b, const v4f &c, uint32_t ea, uint32_t eb) const {
    return mfma_16x16x128_fp8_e8(a, b, c, ea, eb);
  }
};

// The dense weight for decode_kernel: each 16-row tile is loaded as two runs
// of 8 whole rows and made into the MFMA fragment through the wave's LDS tile
// (load_row_runs / row_runs_to_frag).  Measured on MI355X against fragment
// loads (A/B in one process, weights from HBM, quantized tokens):
// 6144 x 4096 at 1 / 4 / 16 / 32 tokens 7.3 / 7.9 / 9.2 / 10.3 -> 6.8 / 6.8 /
// 8.0 / 9.5 us, 4096 x 4096 5.4 / 6.1 / 7.4 / 8.3 -> 5.3 / 5.4 / 6.7 / 8.0 us,
// 4096 x 14336 at 4 / 8 tokens 13.1 / 15.2 -> 12.5 / 13.2 us (level at 1 and
// 16).  Whole rows let the loads carry the non-temporal hint (each load
// instruction covers whole lines): against the same tiles with plain loads,
// 6144 x 4096 6.7 / 6.8 / 7.8 -> 6.4 / 6.3 / 7.2 us at 1 / 2 / 16 tokens,
// 4096 x 14336 12.4 / 13.3 -> 11.6 / 12.4 us at 2 / 8 tokens.  Fragment loads
// (half lines per instruction) were up to 13 % slower with the hint.
struct DenseWeightRows : DenseWeight {
  static constexpr bool kRows = true;
  static constexpr size_t kTileBytes = 2048;
  typedef RowRuns Frag;
  typedef v8i MFrag;
  // `row` is this lane's row of a 16-row tile starting at a multiple of 16
  __device__ __forceinline__ Frag load(int64_t row, int kb, int) const {
    const int64_t row0 = row & ~int64_t(15);
    return load_row_runs<true>(wq, row0, row0 + 15, K, (int64_t)kb * kGroup);
  }
  __device__ __forceinline__ v8i to_frag(const Frag &x, uint8_t *tile) const { return row_runs_to_frag(x, tile); }
};

// ===================================================== split-K reduction ==

// SwiGLU of summed partials, and optionally the group quantization of h:
// part [S][M][2I] fp32, gate sums in columns [0, I), up sums in [I, 2I).  16
// lanes own one 1x128 group of h (8 values each); h = bf16(silu(g) * u) as in
// the tile kernel's SwiGLU epilogue, codes and scale from quantize_group16 on
// the stored bf16 values (the arithmetic of fp8_quant_act).
__global__ __launch_bounds__(256) void swiglu_reduce_kernel(const float *__restrict__ part, int S, int M, int I,
                                                            uint16_t *__restrict__ h, uint8_t *__restrict__ hq,
                                                            float *__restrict__ hs) {
  const int lane16 = threadIdx.x & 15, gpr = I / kGroup;
  const int64_t grp = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = grp < (int64_t)M * gpr;  // uniform over the 16 lanes of a group
  const int64_t m = live ? grp / gpr : 0, col = (live ? grp % gpr : 0) * kGroup + lane16 * 8;
  const int64_t mn2 = (int64_t)M * 2 * I;
  v4f g[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}}, u[2] = {g[0], g[0]};
  if (live) {
    const float *pg = part + m * 2 * I + col, *pu = pg + I;
    for (int s = 0; s < S; s++) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        g[i] += *reinterpret_cast<const v4f *>(pg + (int64_t)s * mn2 + 4 * i);
        u[i] += *reinterpret_cast<const v4f *>(pu + (int64_t)s * mn2 + 4 * i);
      }
    }
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t b2[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const float gv = g[i / 2][2 * (i % 2) + j], uv = u[i / 2][2 * (i % 2) + j];
      b2[j] = f32_to_bf16_rne(gv * uv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)));
    }
    w[i] = b2[0] | (b2[1] << 16);
  }
  const uint4 raw = make_uint4(w[0], w[1], w[2], w[3]);
  if (live && h) *reinterpret_cast<uint4 *>(h + m * I + col) = raw;
  if (hq) {
    float sc;
    const uint2 codes = quantize_group16(raw, sc);
    if (live) {
      *reinterpret_cast<uint2 *>(hq + m * I + col) = codes;
      if (lane16 == 0) hs[m * gpr + col / kGroup] = sc;
    }
  }
}

// y = bf16(sum over s of part[s]), the S partials [S][M*N] added in order s =
// 0, 1, .. (deterministic); four elements per thread, grid-stride.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int S, int64_t mn,
                                                            uint16_t *__restrict__ y) {
  const int64_t n4 = mn / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    v4f acc = *reinterpret_cast<const v4f *>(part + 4 * i);
    for (int s = 1; s < S; s++) acc += *reinterpret_cast<const v4f *>(part + (int64_t)s * mn + 4 * i);
    *reinterpret_cast<uint2 *>(y + 4 * i) = pack_bf16x4(acc);
  }
}

hipError_t launch_splitk_reduce(const float *part, int splits, int64_t mn, uint16_t *y, hipStream_t stream) {
  const int64_t blocks = std::min<int64_t>((mn / 4 + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, mn, y);
  return hipGetLastError();
}

// ================================================================ dispatch ==

// Compute units of the current device (cached per device).
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Tile shape and K split of a tile-kernel GEMM.  A 256 x 128 tile costs
// about 0.62 of a 256 x 256 one (measured on the Llama-3-8B shapes), so it
// wins where the 256 x 256 grid leaves much of its last wave of workgroups
// (one per CU) idle.  When even that grid covers at most half of the CUs, K
// is split over up to 16 workgroups per tile, each with at least four K
// blocks (a multiple of four when the scales go four at a time); the fp32
// partials are summed in a second kernel.
TilePlan plan_tiles(int M, int N, int K, int cus) {
  const int tn = (N + 255) / 256;
  const int t256 = ((M + 255) / 256) * tn, t128 = ((M + 127) / 128) * tn;
  const double cost256 = (double)((t256 + cus - 1) / cus), cost128 = 0.62 * (double)((t128 + cus - 1) / cus);
  TilePlan p{cost128 < 0.97 * cost256 ? 128 : 256, 1, K / kGroup};
  const int tiles = p.bm == 128 ? t128 : t256, kb = K / kGroup;
  if (2 * tiles <= cus && kb >= 8) {
    const int step = kb % 4 == 0 ? 4 : 1;
    int s = std::min(std::min(cus / tiles, kb / 4), 16);
    if (s > 1) {
      int per = (kb + s - 1) / s;
      per = (per + step - 1) / step * step;
      p.splits = (kb + per - 1) / per;
      p.kb_split = per;
    }
  }
  return p;
}

// S: float (fp32 scales) or uint8_t (UE8M0 exponents, E8 = true).
// part != nullptr: fp32 partials (splits of kb_split K blocks) instead of y.
template <int BN, int BM, int WN, int WM, bool E8, class S>
static hipError_t launch_tile(const uint8_t *xq, const S *xs, const uint8_t *wq, const S *ws, int M, int N, int K,
                              uint16_t *y, int splits, int kb_split, float *part, hipStream_t stream) {
  using C = DenseTile<BN, BM, WN, WM>;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileExtra ex{nullptr, nullptr, 0, nullptr, 0, part, kb_split};
  const dim3 grid(tiles_m * tiles_n, splits);
  if (part) {
    if ((K / kGroup) % 4 == 0)
      hipLaunchKernelGGL((dense_tile_kernel<BN, BM, WN, WM, 4, 4, false, E8, false, true>), grid,
                         dim3(C::kThreads), 0, stream, xq, xs, wq, ws, M, N, K, y, tiles_m, tiles_n, 4, ex);
    else
      hipLaunchKernelGGL((dense_tile_kernel<BN, BM, WN, WM, 1, 4, false, E8, false, true>), grid,
                         dim3(C::kThreads), 0, stream, xq, xs, wq, ws, M, N, K, y, tiles_m, tiles_n, 4, ex);
  } else if ((K / kGroup) % 4 == 0) {
    hipLaunchKernelGGL((dense_tile_kernel<BN, BM, WN, WM, 4, 4, false, E8>), grid, dim3(C::kThreads), 0, stream, xq,
                       xs, wq, ws, M, N, K, y, tiles_m, tiles_n, 4, ex);
  } else {
    hipLaunchKernelGGL((dense_tile_kernel<BN, BM, WN, WM, 1, 4, false, E8>), grid, dim3(C::kThreads), 0, stream, xq,
                       xs, wq, ws, M, N, K, y, tiles_m, tiles_n, 4, ex);
  }
  return hipGetLastError();
}

// Tile-kernel GEMM with the planned tile height and K split (the reduction of
// the partials included; part holds them when K is split).
template <bool E8, class S>
static hipError_t tile_gemm(const uint8_t *xq, const S *xs, const uint8_t *wq, const S *ws, int m, int n, int k,
                            uint16_t *y, float *part, hipStream_t stream) {
  const TilePlan p = plan_tiles(m, n, k, device_cu_count());
  if (p.splits > 1 && !part) return hipErrorInvalidValue;
  float *pp = p.splits > 1 ? part : nullptr;
  hipError_t e = p.bm == 128
                     ? launch_tile<256, 128, 2, 4, E8>(xq, xs, wq, ws, m, n, k, y, p.splits, p.kb_split, pp, stream)
                     : launch_tile<256, 256, 2, 4, E8>(xq, xs, wq, ws, m, n, k, y, p.splits, p.kb_split, pp, stream);
  // (launch_tile writes y itself when it gets no partials)
  if (p.splits > 1 && e == hipSuccess) e = launch_splitk_reduce(part, p.splits, (int64_t)m * n, y, stream);
  return e;
}

template <class X, int RT, int CT, int NW, int D, int S = 1>
static hipError_t launch_decode(X xop, const uint8_t *wq, const typename X::Scale *ws, int M, int N, int K,
                                uint16_t *y, float *part, hipStream_t stream) {
  if (S > 1 && !part) return hipErrorInvalidValue;
  // whole-row weight tiles for up to 32 quantized tokens on weights of fewer
  // than 16384 rows (see DenseWeightRows).  Slower with them or level (A/B on
  // MI355X): the 28672-row gate/up weight at one or two tokens (5-16 %
  // slower, and still 12 % / 4 % with the non-temporal loads), the tokens
  // quantized in the kernel (one or two: 2-8 % on the smaller weights), and
  // 33-64 tokens (-3 to +4 %: there the tiles, the staged tokens and the
  // reduction buffer share LDS across a barrier).  The 4096 x 14336 weight at
  // one token had been 4 % slower with them; with the non-temporal loads it
  // is 5 % faster (11.7 -> 11.1 us).
  hipError_t e = hipSuccess;
  bool rows = false;
  if constexpr (std::is_same<X, QuantTokens>::value && CT <= 2) {
    rows = N < 16384 && M <= 32;
    if (rows)
      e = launch_decode_kernel<DenseWeightRows, X, RT, CT, NW, D, S>(DenseWeightRows{{wq, K}}, xop, ws, M, N, K, y,
                                                                     part, stream);
  }
  if (!rows)
    e = launch_decode_kernel<DenseWeight, X, RT, CT, NW, D, S>(DenseWeight{wq, K}, xop, ws, M, N, K, y, part, stream);
  if (S == 1 || e != hipSuccess) return e;
  return launch_splitk_reduce(part, S, (int64_t)M * N, y, stream);
}


// Decode configuration (measured on MI355X over the Llama-3-8B shapes): more
// rows per workgroup when N is large enough to keep every CU busy, since each
// workgroup re-reads the M x K activations from L2.
template <class X, int CT>
static hipError_t launch_decode_for(X xop, const uint8_t *wq, const typename X::Scale *ws, int M, int N, int K,
                                    uint16_t *y, float *part, hipStream_t stream) {
  // Long K on few row bands (N < 6144): 64-row bands read the tokens a
  // quarter as often per weight byte, and K split four ways (partials added
  // by a second kernel) fills the chip.  Measured on MI355X (4096 x 14336
  // weight, graph replay from HBM): 15 % faster at 16 tokens and 21-24 % at
  // 20, level at 8; with K = 4096 the second launch costs more than it saves.
  // Shorter K on few row bands at 33-64 tokens: 32-row bands, K split in two
  // (o_proj 4096 x 4096: 12-16 % faster; no gain at 32 tokens or fewer, and
  // 25 % slower on the 6144-row QKV weight).  decode_splits says which.
  const int splits = X::kStaged ? 1 : decode_splits(M, N, K);
  if constexpr (!X::kStaged && CT <= 2)
    if (splits == 4) {
      // 32-row bands, K in two splits (the partials hold four).  4096 x
      // 14336 from HBM (A/B, graph replay) against 64-row bands in four
      // splits: 12 / 16 tokens 14.8 / 15.0 -> 13.7 / 14.35 us (64-row bands
      // in two splits 17.9 / 18.5, 32-row bands in four 14.4 / 15.0); 20 / 24
      // / 32 tokens, one K block in flight per wave, 16.2 / 16.45 / 16.95 ->
      // 14.97 / 15.4 / 16.17 us (two in flight 15.2 / 15.5 / 16.2, four
      // splits 18.2 / 18.6 / 19.3).
      if constexpr (CT == 1) return launch_decode<X, 2, CT, 8, 2, 2>(xop, wq, ws, M, N, K, y, part, stream);
      return launch_decode<X, 2, CT, 8, 1, 2>(xop, wq, ws, M, N, K, y, part, stream);
    }
  if constexpr (!X::kStaged && CT == 4)
    if (splits == 2) return launch_decode<X, 2, CT, 8, 2, 2>(xop, wq, ws, M, N, K, y, part, stream);
  // Up to 4 tokens: 16 waves per workgroup taking one or two K blocks each, so
  // that every load of the row band is in flight at once; on long K (already
  // quantized tokens) four waves holding four blocks each, and 32-row bands
  // on 6144 to 16383 rows (measured on MI355X at one token, weights from HBM:
  // 4096 x 14336 11.6 us against 12.7 us, 6144 x 4096 7.2 us against 7.7 us).
  if constexpr (CT == 1)
    if (M <= 4) {
      if constexpr (!X::kStaged)
        if (K >= 8192) return launch_decode<X, 1, CT, 4, 4>(xop, wq, ws, M, N, K, y, part, stream);
      if (N >= 6144 && N < 16384) return launch_decode<X, 2, CT, 16, 2>(xop, wq, ws, M, N, K, y, part, stream);
      return launch_decode<X, 1, CT, 16, 2>(xop, wq, ws, M, N, K, y, part, stream);
    }
  if constexpr (CT <= 2)
    if (N >= 16384) return launch_decode<X, 4, CT, 8, 2>(xop, wq, ws, M, N, K, y, part, stream);
  if (N >= 6144) return launch_decode<X, 2, CT, 8, 2>(xop, wq, ws, M, N, K, y, part, stream);
  return launch_decode<X, 1, CT, 8, 1>(xop, wq, ws, M, N, K, y, part, stream);
}

template <class X>
static hipError_t launch_dense_decode(X xop, const uint8_t *wq, const typename X::Scale *ws, int M, int N, int K,
                                      uint16_t *y, float *part, hipStream_t stream) {
  if constexpr (X::kStaged) {
    return launch_decode_for<X, 1>(xop, wq, ws, M, N, K, y, part, stream);  // M <= 8
  } else {
    // 3 to 16 tokens on weights of at least 16384 rows and K < 8192: the
    // shared-token form (tokens staged in LDS once per workgroup, several row
    // bands per workgroup).  Measured on MI355X (gate/up 28672 x 4096, weight
    // from HBM): 22.0 / 22.5 / 25.3 us at 3 / 8 / 16 tokens against 25.5 /
    // 26.2 / 27.4 us.  Level or up to 5 % slower on the 4096- and 6144-row
    // weights, and not used on long K, which splits K instead.
    if constexpr (std::is_same<X, QuantTokens>::value) {
      if (M >= 3 && M <= 16 && K < 8192 && N >= 16384) {
        // whole-row weight tiles from 12 tokens, or from 5 on K >= 6144, where
        // they fit beside the staged tokens (A/B, weights from HBM, identical
        // outputs: 28672 x 4096 at 16 tokens 25.4 -> 23.6 us, 18432 x 7168 at
        // 8 tokens 30.1 -> 26.0 us; slower at 3 tokens, +2-5 %, and on
        // 28672 x 4096 at 8, +7 %)
        if (M >= 12 || (M >= 5 && K >= 6144)) {
          const int gr = shared_decode_grid(M, N, K, 1, 1, 16, 1, device_cu_count(), false,
                                            shared_weight_tiles<DenseWeightRows, 1, 16>());
          if (gr > 0)
            return launch_decode_shared<DenseWeightRows, 1, 16, 2, 1>(DenseWeightRows{{wq, K}}, xop.xq, xop.xs, ws, M,
                                                                      N, K, y, nullptr, gr, stream);
        }
        const int grid = shared_decode_grid(M, N, K, 1, 1, 16, 1, device_cu_count());
        if (grid > 0)
          return launch_decode_shared<DenseWeight, 1, 16, 2, 1>(DenseWeight{wq, K}, xop.xq, xop.xs, ws, M, N, K, y,
                                                                nullptr, grid, stream);
      }
    }
    if (M <= 16) return launch_decode_for<X, 1>(xop, wq, ws, M, N, K, y, part, stream);
    if (M <= 32) return launch_decode_for<X, 2>(xop, wq, ws, M, N, K, y, part, stream);
    return launch_decode_for<X, 4>(xop, wq, ws, M, N, K, y, part, stream);
  }
}

size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K, int cus) {
  int splits = 1;
  if (use_tile_kernel(M, N, K)) {
    splits = plan_tiles((int)M, (int)N, (int)K, cus).splits;
  } else {
    splits = decode_splits(M, N, K);
  }
  return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

size_t swiglu_partial_bytes(int64_t M, int64_t I, int64_t K, int cus) {
  const TilePlan p = plan_tiles((int)M, (int)(2 * I), (int)K, cus);
  if (p.bm == 256 && p.splits == 1) return 0;  // the fused kernel
  return (size_t)p.splits * (size_t)M * (size_t)(2 * I) * sizeof(float);
}

size_t linear_token_bytes(int64_t M, int64_t N, int64_t K, bool sparse) {
  if (linear_staged(M, N, K, sparse)) return 0;  // quantized inside the decode kernel
  return token_codes_bytes(M, K) + (size_t)M * (size_t)(K / kGroup) * sizeof(float);
}

hipError_t launch_dense_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M,
                             int64_t N, int64_t K, uint16_t *y, float *part, hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if (!use_tile_kernel(m, n, k))
    return launch_dense_decode(QuantTokens{xq, xs, k}, wq, ws, m, n, k, y, part, stream);
  return tile_gemm<false>(xq, xs, wq, ws, m, n, k, y, part, stream);
}

hipError_t launch_dense_gemm_swiglu(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                   int64_t M, int64_t I, int64_t K, uint16_t *h, uint8_t *hq, float *hs,
                                   float *part, hipStream_t stream) {
  using C = DenseTile<256, 256, 2, 4>;
  const int m = (int)M, k = (int)K, n2 = (int)(2 * I);
  const TilePlan p = plan_tiles(m, n2, k, device_cu_count());
  if (p.bm != 256 || p.splits > 1) {
    // few output tiles: the tile GEMM of the stacked weight into fp32 partials
    // (K split as planned), then SwiGLU and the quantization in one pass
    if (!part) return hipErrorInvalidValue;
    hipError_t e =
        p.bm == 128
            ? launch_tile<256, 128, 2, 4, false>(xq, xs, wq, ws, m, n2, k, nullptr, p.splits, p.kb_split, part, stream)
            : launch_tile<256, 256, 2, 4, false>(xq, xs, wq, ws, m, n2, k, nullptr, p.splits, p.kb_split, part, stream);
    if (e == hipSuccess) {
      const int64_t groups = (int64_t)m * (I / kGroup);
      hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, stream, part,
                         p.splits, m, (int)I, h, hq, hs);
      e = hipGetLastError();
    }
    return e;
  }
  const int tiles_m = (m + 255) / 256, tiles_n = (int)(I / 128);
  const TileExtra so{hq, hs, (int)I, nullptr, 0};
  if ((k / kGroup) % 4 == 0)
    hipLaunchKernelGGL((dense_tile_kernel<256, 256, 2, 4, 4, 4, true>), dim3(tiles_m * tiles_n), dim3(C::kThreads),
                       0, stream, xq, xs, wq, ws, m, (int)(2 * I), k, h, tiles_m, tiles_n, 4, so);
  else
    hipLaunchKernelGGL((dense_tile_kernel<256, 256, 2, 4, 1, 4, true>), dim3(tiles_m * tiles_n), dim3(C::kThreads),
                       0, stream, xq, xs, wq, ws, m, (int)(2 * I), k, h, tiles_m, tiles_n, 4, so);
  return hipGetLastError();
}

hipError_t launch_dense_gemm_ue8m0(const uint8_t *xq, const uint8_t *xe, const uint8_t *wq, const uint8_t *we,
                                   int64_t M, int64_t N, int64_t K, uint16_t *y, float *part, hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if (!use_tile_kernel(m, n, k))
    return launch_dense_decode(QuantTokensE8{xq, xe, k}, wq, we, m, n, k, y, part, stream);
  return tile_gemm<true>(xq, xe, wq, we, m, n, k, y, part, stream);
}

hipError_t launch_dense_grouped_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                    const int32_t *offsets, int64_t G, int64_t M, int64_t N, int64_t K, uint16_t *y,
                                    hipStream_t stream) {
  using C = DenseTile<256, 256, 2, 4>;
  const int m = (int)M, n = (int)N, k = (int)K;
  const int tiles_m = (m + 255) / 256 + (int)G, tiles_n = (n + 255) / 256;
  const TileExtra ex{nullptr, nullptr, 0, offsets, (int)G};
  if ((k / kGroup) % 4 == 0)
    hipLaunchKernelGGL((dense_tile_kernel<256, 256, 2, 4, 4, 4, false, false, true>), dim3(tiles_m * tiles_n),
                       dim3(C::kThreads), 0, stream, xq, xs, wq, ws, m, n, k, y, tiles_m, tiles_n, 4, ex);
  else
    hipLaunchKernelGGL((dense_tile_kernel<256, 256, 2, 4, 1, 4, false, false, true>), dim3(tiles_m * tiles_n),
                       dim3(C::kThreads), 0, stream, xq, xs, wq, ws, m, n, k, y, tiles_m, tiles_n, 4, ex);
  return hipGetLastError();
}

// One or two tokens on K < 8192: quantized inside the decode kernel
// (StagedTokens; linear_staged says where).  Otherwise fp8_quant_act into
// library scratch memory, then fp8_block_gemm (measured faster from three
// tokens on: every decode workgroup would re-quantize all M x K).
hipError_t launch_dense_linear(const uint16_t *x, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                               int64_t K, uint16_t *y, uint8_t *tokens, float *part, hipStream_t stream) {
  if (linear_staged(M, N, K, false))
    return launch_dense_decode(StagedTokens{x, (int)K, nullptr, nullptr}, wq, ws, (int)M, (int)N, (int)K, y, part,
                               stream);
  if (!tokens) return hipErrorInvalidValue;
  return quantize_then(x, M, K, tokens, stream, [&](const uint8_t *xq, const float *xs) {
    return launch_dense_gemm(xq, xs, wq, ws, M, N, K, y, part, stream);
  });
}

}  // namespace fp8lin
