// 2:4 sparse block-scaled FP8 GEMM on the gfx950 sparse MFMA
// (v_smfmac_f32_16x16x128_fp8_fp8): the compressed weight is operand A
// (16 rows x 64 kept values per 128-wide K block, plus one 32-bit index word
// per lane), the activations the dense operand B.
//
// Lane l of A (row l%16, lane group g = l/16) holds the 16 value bytes of
// groups 8g .. 8g+7 of the K block, i.e. vals[n, 64*kb + 16g .. +15], and the
// index word meta[n, 16*kb + 4g .. +3] read as a little-endian uint32: group
// 8g+j has its nibble i0 | i1 << 2 at bits 4j .. 4j+3, which is exactly the
// packed form prune24_compress writes.  B follows the shared dense layout
// (K bytes [16g, 16g+16) and [64+16g, 64+16g+16)).
//
// Scale handling, tiling and the two kernels (tile for large M, decode for
// M <= 64) mirror the dense GEMM.
#include <type_traits>

#include "gemm_common.hpp"
#include "gemm_decode.hpp"
#include "launch.hpp"

namespace fp8lin {

__device__ __forceinline__ v4f smfmac_16x16x128_fp8(const v4i &a, const v8i &b, int idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, v4f{0.f, 0.f, 0.f, 0.f}, idx, 0, 0);
}

// LDS row of 64 value bytes = four 16-byte chunks; chunk c of row r sits at
// position c ^ vswz(r).  A fragment read takes chunk column g = l / 16 of 16
// consecutive rows r = l % 16, served in the four 16-lane passes described at
// swz (gemm_common.hpp); four rows share a 256-byte bank line.  vswz (3 for
// bit 2 of r, xor 2 for bit 3) gives the 16 lanes of every pass distinct bank
// groups, also under the other two pass shapes named there; it depends on
// r % 16 only.  (Without it, or with (r >> 2) & 3, the reads conflict.)
__device__ __forceinline__ int vswz(int r) { return (((r >> 2) & 1) * 3) ^ (((r >> 3) & 1) << 1); }

// ============================================================== tile kernel ==

template <int BN, int BM, int WN, int WM>
struct SparseTile {
  static constexpr int kWaves = WN * WM, kThreads = kWaves * 64;
  static constexpr int kWaveN = BN / WN, kWaveM = BM / WM;
  static constexpr int RT = kWaveN / 16, CT = kWaveM / 16;
  // per K block: values 64 B/row (1 KB copy = 16 rows), index words 16 B/row
  // (1 KB copy = 64 rows), tokens 128 B/row (1 KB copy = 8 rows)
  static constexpr int kVCopies = BN / 16 / kWaves, kBCopies = BM / 8 / kWaves;
  static constexpr int kMCopyWaves = BN / 64;
  static constexpr int kVTile = BN * 64, kMTile = BN * 16, kBTile = BM * 128;
  static_assert(BN % (16 * kWaves) == 0 && BM % (8 * kWaves) == 0 && kMCopyWaves <= kWaves, "tile mismatch");
  static_assert(kWaves % 2 == 0, "copy slabs alternate 16-row parity per wave");
  static_assert(kWaves * 16 == 128 && BN == 256, "one value slab of every wave is one 128-row panel half");
  static_assert(kWaveN == 128, "a wave covers one 128-row weight scale block (and 256-byte epilogue rows)");
  static_assert(BM <= kThreads, "one thread per token scale");
  static_assert(kWaves * 4096 <= 2 * kBTile && kBTile % 4096 == 0, "epilogue scratch fits in the token stages");
  static constexpr int kScratchWavesPerStage = kBTile / 4096;
};

// SB: K blocks per token-scale load (4 when K/128 is a multiple of 4, else 1).
// CR: the next K block's copies are issued across the first CR row tiles.
// PARTIAL: split K over blockIdx.y (kb_split K blocks each, a multiple of
// SB) and store unrounded fp32 partial tiles to part + blockIdx.y * M * N.
// Unsplit 256x128 tiles are held to 128 registers (four waves per SIMD), so
// that two workgroups share a CU: the ratio form fits in that budget (the
// plain form spills a few registers there; it runs only for ill-conditioned
// scales).  Measured on QKV at M = 4096: 121 -> 99 us.  Split-K launches
// (mid-size M) have at most one workgroup per CU and keep the plain form.
template <int BN, int BM, int WN, int WM, int SB, int CR, bool PARTIAL = false>
__global__ __launch_bounds__(WN *WM * 64) __attribute__((amdgpu_waves_per_eu((BM == 128 && !PARTIAL) ? 4 : 1)))
void sparse_tile_kernel(const uint8_t *__restrict__ xq,
                                                                 const float *__restrict__ xs,
                                                                 const uint8_t *__restrict__ wv,
                                                                 const uint8_t *__restrict__ wm,
                                                                 const float *__restrict__ ws, int M, int N, int K,
                                                                 uint16_t *__restrict__ y, int tiles_m,
                                                                 int tiles_n, int group_m, float *part,
                                                                 int kb_split) {
  using C = SparseTile<BN, BM, WN, WM>;
  // one LDS object per stage and panel (see the dense tile kernel)
  __shared__ __align__(16) uint8_t lds_v0[C::kVTile], lds_v1[C::kVTile];
  __shared__ __align__(16) uint8_t lds_m0[C::kMTile], lds_m1[C::kMTile];
  __shared__ __align__(16) uint8_t lds_b0[C::kBTile], lds_b1[C::kBTile];
  __shared__ __align__(16) float lds_s[2 * SB * BM];
  __shared__ uint32_t xs_range[BM];  // per token: exponent range of its scales (see below)
  __shared__ uint32_t xs_const[BM];  // per token: all its scales over the K range equal
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, lr = lane & 15;
  const int cj = lane >> 3, cp = lane & 7;
  // KBs: K blocks per row (the stride of the scale rows); KB: K blocks this
  // workgroup accumulates, starting at block kb0 (every operand pointer below
  // is shifted to it; row strides are unchanged)
  const int KBs = K / kGroup, NB = N / kGroup;
  int kb0 = 0, KB = KBs;
  if constexpr (PARTIAL) {
    kb0 = blockIdx.y * kb_split;
    KB = min(kb_split, KBs - kb0);
  }
  const int64_t vrow_bytes = K / 2, mrow_bytes = K / 8;
  xq += kb0 * kGroup;
  xs += kb0;
  wv += kb0 * 64;
  wm += kb0 * 16;

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  const int m_base = tm * BM, n_base = tn * BN;
  const int wn0 = (wave / WM) * C::kWaveN, wm0 = (wave % WM) * C::kWaveM;

  // Copies through buffer resources over 128-row panel halves (rows past the
  // matrix edge read as zeros; their outputs are never stored), with one
  // per-lane offset per panel and the K block and half-panel row in the
  // scalar offset, so walking K costs no VALU.
  //  values: slab i covers rows r0 = (i*kWaves + wave)*16 .. +15 (half i*16*kWaves/128);
  //    lane l writes chunk position l%4 of row r0 + l/4 (logical chunk (l%4) ^ vswz(row));
  //  index words: one 64-row slab per wave for waves < kMCopyWaves;
  //  tokens: slab i covers rows (i*kWaves + wave)*8 .. +7, as in the dense kernel.
  const int vrow_in_slab = lane >> 2, vpos = lane & 3;
  const uint32_t v_voff =
      (uint32_t)((wave * 16 + vrow_in_slab) * vrow_bytes + 16 * (vpos ^ vswz(vrow_in_slab)));
  const uint32_t m_voff = (uint32_t)(((wave % 2) * 64 + lane) * mrow_bytes);
  const uint32_t b_voff = (uint32_t)((wave * 8 + cj) * K + 16 * (cp ^ swz(cj + 8 * (wave & 1))));
  const uint8_t *vpanel = wv + (int64_t)n_base * vrow_bytes, *mpanel = wm + (int64_t)n_base * mrow_bytes;
  const uint8_t *xpanel = xq + (int64_t)m_base * K;
  const rsrc_t rv0 = panel_rows128(vpanel, N - n_base, 0, (int)vrow_bytes);
  const rsrc_t rv1 = panel_rows128(vpanel, N - n_base, 128, (int)vrow_bytes);
  const rsrc_t rm0 = panel_rows128(mpanel, N - n_base, 0, (int)mrow_bytes);
  const rsrc_t rm1 = panel_rows128(mpanel, N - n_base, 128, (int)mrow_bytes);
  const rsrc_t rx0 = panel_rows128(xpanel, M - m_base, 0, K), rx1 = panel_rows128(xpanel, M - m_base, 128, K);
  TokenScales<BM, SB> scales;
  scales.init(lds_s, xs, M, KBs, m_base, tid);

  // copy j of a K block: 0 .. kVCopies-1 values, kVCopies the index words
  // (waves below kMCopyWaves), then the token panel
  auto issue_copy = [&](int kb, int st, int j) {
    if (j < C::kVCopies) {
      const int r0 = (j * C::kWaves + wave) * 16;  // rows j*128 + 16*wave .. +15: half j of the panel
      const uint32_t soff = (uint32_t)kb * 64u + (uint32_t)((j * C::kWaves * 16) % 128) * (uint32_t)vrow_bytes;
      buffer_copy16_to_lds((j * C::kWaves * 16) < 128 ? rv0 : rv1, v_voff, soff, (st ? lds_v1 : lds_v0) + r0 * 64);
    } else if (j == C::kVCopies) {
      if (wave < C::kMCopyWaves)
        buffer_copy16_to_lds(wave < 2 ? rm0 : rm1, m_voff, (uint32_t)kb * 16u, (st ? lds_m1 : lds_m0) + wave * 64 * 16);
    } else {
      const int i = j - C::kVCopies - 1;
      const int first = i * C::kWaves * 8;  // panel row of wave 0's slab
      const uint32_t soff = (uint32_t)kb * 128u + (uint32_t)(first % 128) * (uint32_t)K;
      buffer_copy16_to_lds(first < 128 ? rx0 : rx1, b_voff, soff, (st ? lds_b1 : lds_b0) + (first + wave * 8) * 128);
    }
  };
  constexpr int kCopies = C::kVCopies + 1 + C::kBCopies;
  constexpr int kCopyRows = CR < C::RT ? CR : C::RT;  // copies are spread over the first kCopyRows row tiles
  constexpr int kCopiesPerRow = (kCopies + kCopyRows - 1) / kCopyRows;
  auto issue_copies = [&](int kb, int st) {
#pragma unroll
    for (int j = 0; j < kCopies; j++) issue_copy(kb, st, j);
  };

  const int fr_lo = lr * 128 + ((g ^ swz(lr)) << 4);
  const int fr_hi = lr * 128 + (((g + 4) ^ swz(lr)) << 4);
  const int b_lo = wm0 * 128 + fr_lo, b_hi = wm0 * 128 + fr_hi;
  const int v_off = (wn0 + lr) * 64 + ((g ^ vswz(lr)) << 4);
  const int m_off = (wn0 + lr) * 16 + 4 * g;

  v4f acc[C::RT][C::CT];
#pragma unroll
  for (int r = 0; r < C::RT; r++)
#pragma unroll
    for (int c = 0; c < C::CT; c++) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nb_wave = min((n_base + wn0) / kGroup, NB - 1);
  const float *ws_row = ws + (int64_t)nb_wave * KBs + kb0;
  // the weight scale of the next step is loaded during this one, as a vector
  // (buffer) load counted with the copies: a scalar load can return out of
  // order, and while one is pending every LDS wait would have to drain all
  // LDS reads in flight
  const rsrc_t rws = make_rsrc(ws_row, (uint32_t)KB * 4u);
  float sw_cur = ws_row[0];
  // Ratio form of the scale accumulation (when every scale this wave uses is
  // well conditioned, see below): acc holds the running sum in units of the
  // current K block's scale, so each sparse MFMA accumulates straight into it
  // after one multiply by the ratio of the previous scale to the current one,
  // and the last scale is applied once at the end.  The plain form needs a
  // cleared partial per MFMA (the sparse MFMA accumulates into its
  // destination, so two register moves) and an FMA per output.
  // Unit form: where every scale product the wave uses is the same in every
  // K block (per-tensor scales, or per-token activation scales with one
  // weight scale per row block), the sparse MFMAs accumulate the unscaled
  // block sums straight into acc and the one scale is applied at the end: no
  // VALU work per MFMA at all.
  bool ratio_form = false, unit_form = false;
  float unit[C::CT];
#pragma unroll
  for (int c = 0; c < C::CT; c++) unit[c] = 1.f;

  // form_tag: 0 plain, 1 ratio, 2 unit
  auto step = [&](int kb, auto st_tag, auto form_tag) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr int kForm = decltype(form_tag)::value;
    constexpr bool kRatio = kForm == 1, kUnit = kForm == 2;
    const bool more = kb + 1 < KB;
    const bool scale_load = (kb % SB == 0) && (kb + SB < KB);
    if (scale_load) scales.load(kb / SB + 1);
    const float sw = sw_cur;
    const float sw_next = more ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                     rws, 0, (uint32_t)(kb + 1) * 4u, 0))
                               : 0.f;
    // the first row's weight fragment first: the first MFMAs wait only for it
    // and the token fragments they use
    const uint8_t *Vt = ST ? lds_v1 : lds_v0;
    const uint8_t *Mt = ST ? lds_m1 : lds_m0;
    v4i af_next = make_v4i(*reinterpret_cast<const uint4 *>(Vt + v_off));
    int ix_next = *reinterpret_cast<const int *>(Mt + m_off);
    v8i bf[C::CT];
    float scl[C::CT];
#pragma unroll
    for (int c = 0; c < C::CT; c++) {
      bf[c] = load_frag_at(ST ? lds_b1 : lds_b0, b_lo, b_hi, c * 2048);
      if constexpr (!kUnit) scl[c] = scales.get(kb, wm0 + 16 * c + lr) * sw;
    }
    if constexpr (kUnit) {
#pragma unroll
      for (int r = 0; r < C::RT; r++) {
        if (more && r < kCopyRows) {
#pragma unroll
          for (int j = r * kCopiesPerRow; j < (r + 1) * kCopiesPerRow && j < kCopies; j++)
            issue_copy(kb + 1, ST ^ 1, j);
        }
        const v4i af = af_next;
        const int ix = ix_next;
        if (r + 1 < C::RT) {
          af_next = make_v4i(*reinterpret_cast<const uint4 *>(Vt + v_off + (r + 1) * 1024));
          ix_next = *reinterpret_cast<const int *>(Mt + m_off + (r + 1) * 256);
        }
#pragma unroll
        for (int c = 0; c < C::CT; c++) {
          acc[r][c] = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(af, bf[c], acc[r][c], ix, 0, 0);
          pin(acc[r][c]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (kRatio) {
      float ratio[C::CT];
#pragma unroll
      for (int c = 0; c < C::CT; c++) {
        ratio[c] = unit[c] * __builtin_amdgcn_rcpf(scl[c]);
        unit[c] = scl[c];
      }
#pragma unroll
      for (int r = 0; r < C::RT; r++) {
        if (more && r < kCopyRows) {
#pragma unroll
          for (int j = r * kCopiesPerRow; j < (r + 1) * kCopiesPerRow && j < kCopies; j++)
            issue_copy(kb + 1, ST ^ 1, j);
        }
        const v4i af = af_next;
        const int ix = ix_next;
        if (r + 1 < C::RT) {
          af_next = make_v4i(*reinterpret_cast<const uint4 *>(Vt + v_off + (r + 1) * 1024));
          ix_next = *reinterpret_cast<const int *>(Mt + m_off + (r + 1) * 256);
        }
#pragma unroll
        for (int c = 0; c < C::CT; c++) {
          acc[r][c] = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(af, bf[c], acc[r][c] * ratio[c], ix, 0, 0);
          pin(acc[r][c]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      v4f p_prev[C::CT];
#pragma unroll
      for (int r = 0; r < C::RT; r++) {
        if (more && r < kCopyRows) {
#pragma unroll
          for (int j = r * kCopiesPerRow; j < (r + 1) * kCopiesPerRow && j < kCopies; j++)
            issue_copy(kb + 1, ST ^ 1, j);
        }
        const v4i af = af_next;
        const int ix = ix_next;
        if (r + 1 < C::RT) {
          af_next = make_v4i(*reinterpret_cast<const uint4 *>(Vt + v_off + (r + 1) * 1024));
          ix_next = *reinterpret_cast<const int *>(Mt + m_off + (r + 1) * 256);
        }
        v4f p_cur[C::CT];
#pragma unroll
        for (int c = 0; c < C::CT; c++) p_cur[c] = smfmac_16x16x128_fp8(af, bf[c], ix);
        if (r > 0) {
#pragma unroll
          for (int c = 0; c < C::CT; c++) {
            acc[r - 1][c] += scl[c] * p_prev[c];
            pin(acc[r - 1][c]);
          }
        }
#pragma unroll
        for (int c = 0; c < C::CT; c++) p_prev[c] = p_cur[c];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int c = 0; c < C::CT; c++) {
        acc[C::RT - 1][c] += scl[c] * p_prev[c];
        pin(acc[C::RT - 1][c]);
      }
    }
    // copies, token scales and the next weight scale have landed (vmcnt and
    // lgkmcnt drained: the LDS reads of this step are all consumed by now)
    if (more || scale_load) __builtin_amdgcn_s_waitcnt(0x0070);
    if (scale_load) scales.store(kb / SB + 1);
    sw_cur = sw_next;
    __syncthreads();
  };

  // The ratio form pays for its scan of the scales over long K ranges only
  // (short split-K ranges keep the plain form).
  constexpr int kRatioMinKB = 32;
  const bool try_ratio = KB >= kRatioMinKB;
  issue_copies(0, 0);
  scales.load(0);
  // While the first copies are in flight: the exponent range of every token
  // scale of the tile over this K range, per token (kTpt threads per token,
  // combined in consecutive lanes), into xs_range as (min << 8) | max of the
  // biased exponents, or ~0 when a scale is zero, subnormal or not finite;
  // and into xs_const whether all of the token's scales are the same bits.
  {
    constexpr int kTpt = C::kThreads / BM;
    static_assert(kTpt == 2 || kTpt == 4, "threads per token in the scale scan");
    const int tt = tid / kTpt, part = tid % kTpt;
    uint32_t lo = 255u, hi = 0u, odd = 0u, blo = ~0u, bhi = 0u;
    if (try_ratio && m_base + tt < M) {
      const float *row = xs + (int64_t)(m_base + tt) * KBs;
      const int chunk = (KB + kTpt - 1) / kTpt, k0 = part * chunk, k1 = min(KB, k0 + chunk);
#pragma unroll 8
      for (int kb = k0; kb < k1; kb++) {
        const uint32_t bits = __float_as_uint(row[kb]);
        const uint32_t e = (bits & 0x7FFFFFFFu) >> 23;
        odd |= (uint32_t)(e == 0u || e == 255u);
        lo = min(lo, e);
        hi = max(hi, e);
        blo = min(blo, bits);
        bhi = max(bhi, bits);
      }
    }
#pragma unroll
    for (int off = 1; off < kTpt; off <<= 1) {
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
      odd |= (uint32_t)__shfl_xor((int)odd, off, 64);
      blo = min(blo, (uint32_t)__shfl_xor((int)blo, off, 64));
      bhi = max(bhi, (uint32_t)__shfl_xor((int)bhi, off, 64));
    }
    if (part == 0) {
      xs_range[tt] = odd ? ~0u : (lo << 8) | hi;
      xs_const[tt] = blo == bhi ? 1u : 0u;
    }
  }
  // the same for this wave's weight scale row (every lane of the wave)
  uint32_t wlo = 255u, whi = 0u, wodd = 0u, wblo = ~0u, wbhi = 0u;
  for (int kb = try_ratio ? lane : KB; kb < KB; kb += 64) {
    const uint32_t bits = __float_as_uint(ws_row[kb]);
    const uint32_t e = (bits & 0x7FFFFFFFu) >> 23;
    wodd |= (uint32_t)(e == 0u || e == 255u);
    wlo = min(wlo, e);
    whi = max(whi, e);
    wblo = min(wblo, bits);
    wbhi = max(wbhi, bits);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    wlo = min(wlo, (uint32_t)__shfl_xor((int)wlo, off, 64));
    whi = max(whi, (uint32_t)__shfl_xor((int)whi, off, 64));
    wodd |= (uint32_t)__shfl_xor((int)wodd, off, 64);
    wblo = min(wblo, (uint32_t)__shfl_xor((int)wblo, off, 64));
    wbhi = max(wbhi, (uint32_t)__shfl_xor((int)wbhi, off, 64));
  }
  wait_global_loads();
  scales.store(0);
  __syncthreads();
  {
    // The ratio form is exact algebra; in fp32 it needs every scale product
    // xs * ws this wave uses to be a normal number in [2^-100, 2^100] and all
    // of them within 2^60 of each other: then no ratio, no rescaled sum (at
    // most K/128 * 2^25 * 2^60) and no rescaled partial (at least 2^-18 *
    // 2^-60) leaves the normal range, and the rescalings add a relative error
    // of about one ulp per K block.  A zero scale is excluded as well: the
    // form cannot skip a K block whose scale is zero while its codes are not.
    // Tokens past M are ignored (their outputs are never stored).  Each wave
    // decides for itself; otherwise it runs the plain form.
    bool ok = try_ratio && wodd == 0u;
#pragma unroll
    for (int c = 0; c < C::CT; c++) {
      const int tok = wm0 + 16 * c + lr;
      if (m_base + tok < M) {
        const uint32_t r = xs_range[tok];
        const int xlo = (int)(r >> 8), xhi = (int)(r & 0xFFu);
        ok = ok && r != ~0u && (xhi - xlo) + (int)(whi - wlo) + 2 <= 60 && xlo + (int)wlo >= 154 &&
             xhi + (int)whi <= 352;
      }
    }
    ratio_form = __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_ballot_w64(!ok) == 0)) != 0;
    // the unit form: every scale of the wave's tokens and of its weight block
    // row the same over the K range (any value, zero included: the sums are
    // exact block sums, scaled once)
    bool same = try_ratio && wblo == wbhi;
#pragma unroll
    for (int c = 0; c < C::CT; c++) {
      const int tok = wm0 + 16 * c + lr;
      if (m_base + tok < M) same = same && xs_const[tok] != 0u;
    }
    unit_form = __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_ballot_w64(!same) == 0)) != 0;
    if (unit_form) {
#pragma unroll
      for (int c = 0; c < C::CT; c++) unit[c] = scales.get(0, wm0 + 16 * c + lr) * sw_cur;
    }
  }
  // separate loops, one per form, so that each is register-allocated on its
  // own; every wave passes the same barriers in any of them
  if (unit_form) {
    for (int kb = 0; kb < KB; kb += 2) {
      step(kb, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
      if (kb + 1 < KB) step(kb + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
    }
  } else if (ratio_form) {
    for (int kb = 0; kb < KB; kb += 2) {
      step(kb, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      if (kb + 1 < KB) step(kb + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
    }
  } else {
    for (int kb = 0; kb < KB; kb += 2) {
      step(kb, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      if (kb + 1 < KB) step(kb + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
    }
  }

  // epilogue through a wave-private 4 KB slice of the (now idle) token stages
  constexpr int kPer = C::kScratchWavesPerStage;
  uint8_t *scratch = (wave < kPer ? lds_b0 : lds_b1) + (wave % kPer) * 4096;
#pragma unroll
  for (int c = 0; c < C::CT; c++) {
    v4f col[C::RT];
    const float u = (ratio_form || unit_form) ? unit[c] : 1.f;
#pragma unroll
    for (int r = 0; r < C::RT; r++) col[r] = acc[r][c] * u;
    if constexpr (PARTIAL)
      store_token_tile_f32<C::RT>(col, part + (int64_t)blockIdx.y * M * N, M, N, m_base + wm0 + 16 * c,
                                  n_base + wn0, lane);
    else
      store_token_tile<C::RT>(scratch, col, y, M, N, m_base + wm0 + 16 * c, n_base + wn0, lane);
  }
}

// ============================================================ decode kernel ==

// Weight operand of the decode kernel: 16 value bytes and one index word of
// one row's K block per lane.
struct SparseFrag {
  v4i v;
  int idx;
};
struct SparseWeight {
  typedef SparseFrag Frag;
  const uint8_t *wv, *wm;
  int K;
  __device__ __forceinline__ Frag load(int64_t row, int kb, int g) const {
    SparseFrag f;
    f.v = make_v4i(ldg16(wv + row * (K / 2) + (int64_t)kb * 64 + 16 * g));
    f.idx = *reinterpret_cast<const int *>(wm + row * (K / 8) + (int64_t)kb * 16 + 4 * g);
    return f;
  }
  __device__ __forceinline__ v4f mma(const Frag &a, const v8i &b) const { return smfmac_16x16x128_fp8(a.v, b, a.idx); }
};

// The same operand four K blocks at a time, for the weight-streaming kernel.
// One block's index words are 16 bytes per row, so loading them block by
// block costs as many memory requests as the values while carrying a quarter
// of the bytes (measured on MI355X: the 2:4 decode GEMMs ran 20-27 % faster
// with no index loads at all).  Here one 16-byte load per lane brings the
// words of four consecutive blocks: lane group g receives block kb + g's four
// words and needs word g of each block, so the four lane groups of a row
// exchange them (a 4x4 transpose by lane-permute swaps).
struct SparseFrag4 {
  v4i v[4];
  int idx[4];
};
struct SparseWeight4 {
  typedef SparseFrag4 Frag;
  static constexpr int kUnit = 4;
  const uint8_t *wv, *wm;
  int K;
  // kb: first of the four blocks.  All 64 lanes must call it together.
  __device__ __forceinline__ Frag load(int64_t row, int kb, int g) const {
    Frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) f.v[j] = make_v4i(ldg16(wv + row * (K / 2) + (int64_t)(kb + j) * 64 + 16 * g));
    load_idx(row, kb, g, f.idx);
    return f;
  }
  // the index words of the four blocks, word g of each in idx[0..3]
  __device__ __forceinline__ void load_idx(int64_t row, int kb, int g, int (&idx)[4]) const {
    const uint4 m = ldg16(wm + row * (K / 8) + (int64_t)kb * 16 + 16 * g);
    // Lane group g (the 16-lane row g of the wave) holds the four words of
    // block kb + g and needs word g of every block: a 4x4 transpose across the
    // rows.  Two 32-lane swaps (rows 2, 3 of one register with rows 0, 1 of
    // another), then two 16-lane swaps (odd rows with even rows), leave word g
    // of block kb + j in register j.  The swaps are VALU lane permutes: no LDS
    // round trip as with cross-lane shuffles (measured on MI355X: 4-10 % faster
    // 2:4 decode at 4-32 tokens, bit-identical results).
    const auto a = __builtin_amdgcn_permlane32_swap(m.x, m.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(m.y, m.w, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    idx[0] = (int)c[0];
    idx[1] = (int)c[1];
    idx[2] = (int)d[0];
    idx[3] = (int)d[1];
  }
  __device__ __forceinline__ v4f mma(const Frag &a, const v8i &b, int u) const {
    return smfmac_16x16x128_fp8(a.v[u], b, a.idx[u]);
  }
};

// The four-block operand with its values in whole rows, for decode_kernel: a
// 16-row tile's four blocks are 256 contiguous bytes per row, loaded as four
// runs of 4 rows (lane l: row 4i + l / 16, 16-byte chunk l % 16 of the row's
// 256 bytes) instead of four fragment loads of 16 rows x 64 bytes each (half
// as many cache-line accesses), then written to the wave's 4 KB LDS tile as
// four blocks of 16 rows x 64 bytes, chunk c of row r at position
// c ^ vswz(r) as in the tile kernel, and read back per block as the
// fragment.  The index words come as in SparseWeight4.  Used where the
// workgroup's outputs per lane group are one tile, or two row tiles (more
// spill registers).  Measured on MI355X against SparseWeight4 (A/B, weights
// from HBM): 4096 x 14336 at 1 / 4 / 8 tokens 9.8 / 10.5 / 10.2 -> 9.5 / 9.8 /
// 9.6 us, 4096 x 4096 at 1 / 5 / 8 tokens 6.5 / 6.3 / 6.2 -> 6.0 / 5.9 / 5.8
// us, 6144 x 4096 at 16 tokens 6.8 -> 6.4 us.  The value loads take the
// non-temporal hint (whole lines per load instruction): 6144 x 4096 at 8 / 16
// tokens 6.1 / 6.3 -> 5.75 / 5.8 us, 4096 x 14336 at 1 / 4 / 8 tokens 9.5 /
// 9.9 / 9.7 -> 9.3 / 9.4 / 9.2 us.
struct SparseFrag4Rows {
  uint4 v[4];
  int idx[4];
};
struct SparseWeight4Rows : SparseWeight4 {
  static constexpr bool kRows = true;
  static constexpr size_t kTileBytes = 4096;
  typedef SparseFrag4Rows Frag;
  typedef SparseFrag4 MFrag;
  // `row` is this lane's row of a 16-row tile starting at a multiple of 16
  __device__ __forceinline__ Frag load(int64_t row, int kb, int g) const {
    const int lane = threadIdx.x & 63;
    const uint8_t *base = wv + (row & ~int64_t(15)) * (K / 2) + (int64_t)kb * 64 + 16 * (lane & 15);
    Frag f;
#pragma unroll
    for (int i = 0; i < 4; i++) f.v[i] = ldg16_stream(base + (int64_t)(4 * i + (lane >> 4)) * (K / 2));
    load_idx(row, kb, g, f.idx);
    return f;
  }
  __device__ __forceinline__ MFrag to_frag(const Frag &f, uint8_t *tile) const {
    const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    const int u = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 4 * i + (lane >> 4);
      *reinterpret_cast<uint4 *>(tile + u * 1024 + r * 64 + 16 * (c ^ vswz(r))) = f.v[i];
    }
    MFrag m;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      m.v[b] = make_v4i(*reinterpret_cast<const uint4 *>(tile + b * 1024 + lr * 64 + 16 * (g ^ vswz(lr))));
      m.idx[b] = f.idx[b];
    }
    return m;
  }
};

// ================================================================ dispatch ==

template <int BN, int BM, int WN, int WM>
static hipError_t launch_tile(const uint8_t *xq, const float *xs, const uint8_t *wv, const uint8_t *wm,
                              const float *ws, int M, int N, int K, uint16_t *y, int splits, int kb_split,
                              float *part, hipStream_t stream) {
  using C = SparseTile<BN, BM, WN, WM>;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n, splits);
  if (splits > 1) {
    if ((K / kGroup) % 4 == 0)
      hipLaunchKernelGGL((sparse_tile_kernel<BN, BM, WN, WM, 4, 4, true>), grid, dim3(C::kThreads), 0, stream, xq, xs,
                         wv, wm, ws, M, N, K, y, tiles_m, tiles_n, 4, part, kb_split);
    else
      hipLaunchKernelGGL((sparse_tile_kernel<BN, BM, WN, WM, 1, 4, true>), grid, dim3(C::kThreads), 0, stream, xq, xs,
                         wv, wm, ws, M, N, K, y, tiles_m, tiles_n, 4, part, kb_split);
  } else if ((K / kGroup) % 4 == 0) {
    hipLaunchKernelGGL((sparse_tile_kernel<BN, BM, WN, WM, 4, 4>), grid, dim3(C::kThreads), 0, stream, xq, xs, wv, wm,
                       ws, M, N, K, y, tiles_m, tiles_n, 4, part, kb_split);
  } else {
    hipLaunchKernelGGL((sparse_tile_kernel<BN, BM, WN, WM, 1, 4>), grid, dim3(C::kThreads), 0, stream, xq, xs, wv, wm,
                       ws, M, N, K, y, tiles_m, tiles_n, 4, part, kb_split);
  }
  return hipGetLastError();
}

template <class Wt, class X, int RT, int CT, int NW, int D, int S>
static hipError_t launch_decode_with(Wt wop, X xop, const typename X::Scale *ws, int M,
                                int N, int K, uint16_t *y, float *part, hipStream_t stream) {
  if (S > 1 && !part) return hipErrorInvalidValue;
  const hipError_t e = launch_decode_kernel<Wt, X, RT, CT, NW, D, S>(wop, xop, ws, M, N, K, y, part, stream);
  if (S == 1 || e != hipSuccess) return e;
  return launch_splitk_reduce(part, S, (int64_t)M * N, y, stream);
}

// Four-block units (one unit in flight per wave: four blocks) where K holds a
// whole number of units, at least as many units as waves over the whole row,
// and the workgroup's outputs are at most four 16x16 tiles per lane group
// (RT * CT <= 4; beyond that the unit's registers spill).  A K split can still
// leave waves of a split without a unit: the 4096 x 14336 weight has 28 units,
// so its four splits get 7 each over 8 waves.  Measured on MI355X against one
// block at a time (graph replay from HBM, Llama-3-8B shapes): 15-20 % faster
// on down at 4-16 tokens (split four ways from 9 tokens, one wave per split
// idle), 15-19 % on QKV at 8-32, 13-14 % on gate/up at 8-16, 4-12 % on
// o_proj; with spills 17-22 % slower, and with half the waves idle over the
// whole row (gate/up at 1-4 tokens, 16 waves over 8 units) 3-8 % slower.
template <class X, int RT, int CT, int NW, int D, int S = 1>
static hipError_t launch_decode(X xop, const uint8_t *wv, const uint8_t *wm, const typename X::Scale *ws, int M,
                                int N, int K, uint16_t *y, float *part, hipStream_t stream) {
  constexpr int U = SparseWeight4::kUnit;
  if constexpr (RT * CT <= 4)
    if ((K / kGroup) % U == 0 && (K / kGroup) / U >= NW) {
      if constexpr (RT * CT == 1 || (RT == 2 && CT == 1))
        return launch_decode_with<SparseWeight4Rows, X, RT, CT, NW, 1, S>(SparseWeight4Rows{{wv, wm, K}}, xop, ws, M,
                                                                          N, K, y, part, stream);
      else
        return launch_decode_with<SparseWeight4, X, RT, CT, NW, 1, S>(SparseWeight4{wv, wm, K}, xop, ws, M, N, K, y,
                                                                      part, stream);
    }
  return launch_decode_with<SparseWeight, X, RT, CT, NW, D, S>(SparseWeight{wv, wm, K}, xop, ws, M, N, K, y, part,
                                                               stream);
}


// Up to 4 quantized tokens: K whose four-block units number 8 to 15 takes
// the whole-row four-block tiles over 4 or 8 waves (launch_decode_for).
static inline bool few_token_rows4(int64_t K) {
  const int64_t units = K / kGroup / SparseWeight4::kUnit;
  return (K / kGroup) % SparseWeight4::kUnit == 0 && units >= 8 && units < 16;
}

// Decode configuration (measured on MI355X over the Llama-3-8B shapes): more
// rows per workgroup when N is large enough to keep every CU busy, since each
// workgroup re-reads the M x K activations from L2.  K splits as in the dense
// GEMM (decode_splits).
template <class X, int CT>
static hipError_t launch_decode_for(X xop, const uint8_t *wv, const uint8_t *wm, const float *ws, int M, int N,
                                    int K, uint16_t *y, float *part, hipStream_t stream) {
  const int splits = X::kStaged ? 1 : decode_splits(M, N, K);
  if constexpr (!X::kStaged && CT <= 2)
    if (splits == 4) {
      // Whole-row four-block tiles over 32-row bands, K in two splits (the
      // partials hold four).  Measured on MI355X, 4096 x 14336 from HBM (A/B,
      // graph replay) against four splits of 64-row bands with fragment
      // loads: 12 / 16 tokens 13.1 / 13.45 -> 11.7 / 11.9 us (four splits of
      // 32-row bands over 4 waves 11.9 / 12.4, over 8 waves level, 16-row
      // bands 15.5 / 16.4; 64-row whole-row bands spill); 20 / 24 / 32 tokens
      // 16.5 / 16.9 / 17.3 -> 14.2 / 15.0 / 16.2 us (16-row bands 18.0 / 18.3
      // / 19.0, fragment loads 15.6 / 16.4 / 18.0).
      if ((K / kGroup) % SparseWeight4::kUnit == 0)
          return launch_decode_with<SparseWeight4Rows, X, 2, CT, 8, 1, 2>(SparseWeight4Rows{{wv, wm, K}}, xop, ws, M,
                                                                          N, K, y, part, stream);
      return launch_decode<X, 4, CT, 8, 2, 4>(xop, wv, wm, ws, M, N, K, y, part, stream);
    }
  if constexpr (!X::kStaged && CT == 4)
    if (splits == 2) return launch_decode<X, 2, CT, 8, 2, 2>(xop, wv, wm, ws, M, N, K, y, part, stream);
  if constexpr (CT == 1)
    if (M <= 4) {
      // Up to 4 quantized tokens on K with fewer four-block units than 16
      // waves (K < 8192): whole-row four-block tiles over fewer waves, each
      // wave with one or two units in flight.  Against one block at a time
      // over 16 waves (A/B, weights from HBM, outputs equal to 5e-5): 6144 x
      // 4096 at 1 / 2 / 4 tokens 7.4 / 8.0 / 8.6 -> 5.4 / 5.4 / 5.4 us (32-row
      // bands, 8 waves), 4096 x 4096 5.1 / 5.3 / 5.7 -> 4.7 / 4.7 / 4.7 us (8
      // waves), 28672 x 4096 at 1 / 2 tokens 20.4 / 22.0 -> 17.1 / 17.3 us (4
      // waves, two units in flight).
      if constexpr (!X::kStaged)
        if (few_token_rows4(K)) {
          const SparseWeight4Rows w4{{wv, wm, K}};
          if (N >= 16384)
            return launch_decode_with<SparseWeight4Rows, X, 1, CT, 4, 2, 1>(w4, xop, ws, M, N, K, y, part, stream);
          if (N >= 6144)
            return launch_decode_with<SparseWeight4Rows, X, 2, CT, 8, 1, 1>(w4, xop, ws, M, N, K, y, part, stream);
          return launch_decode_with<SparseWeight4Rows, X, 1, CT, 8, 1, 1>(w4, xop, ws, M, N, K, y, part, stream);
        }
      return launch_decode<X, 1, CT, 16, 2>(xop, wv, wm, ws, M, N, K, y, part, stream);
    }
  if constexpr (CT <= 2)
    if (N >= 16384) return launch_decode<X, 4, CT, 8, 3>(xop, wv, wm, ws, M, N, K, y, part, stream);
  if (N >= 6144) return launch_decode<X, 2, CT, 8, 2>(xop, wv, wm, ws, M, N, K, y, part, stream);
  return launch_decode<X, 1, CT, 8, 1>(xop, wv, wm, ws, M, N, K, y, part, stream);
}

template <class X>
static hipError_t launch_sparse_decode(X xop, const uint8_t *wv, const uint8_t *wm, const float *ws, int M, int N,
                                       int K, uint16_t *y, float *part, hipStream_t stream) {
  if constexpr (X::kStaged) {
    return launch_decode_for<X, 1>(xop, wv, wm, ws, M, N, K, y, part, stream);  // M <= 8
  } else {
    // 3 to 16 tokens on weights of at least 16384 rows and K < 8192: the
    // shared-token form.  From 5 tokens each wave takes whole bands (it
    // streams all units of its bands, so no partial sums meet and no barrier
    // follows the staging); at 3 or 4 the waves split each band's units.
    // Measured on MI355X, gate/up 28672 x 4096, weight from HBM (A/B):
    //   whole bands     16 tokens 17.7 us, 12: 17.3, 8: 17.0, 4: 16.4, 3: 16.4;
    //   split units                        12: 19.4 (*), 8: 17.4, 4: 15.9, 3: 15.8;
    //   (*) 12 and 16 tokens ran the weight-streaming kernel: 19.4 / 20.1 us.
    if constexpr (std::is_same<X, QuantTokens>::value) {
      if (M >= 3 && M <= 16 && K < 8192 && N >= 16384) {
        const int cus = device_cu_count();
        if (M >= 5) {
          // whole-row weight tiles where they fit beside the staged tokens
          // (A/B, weights from HBM, identical outputs: 28672 x 4096 at 5 / 8
          // / 12 / 16 tokens 16.9 / 16.8 / 17.4 / 18.0 -> 15.8 / 15.8 / 16.3
          // / 16.7 us, 18432 x 7168 at 5 / 8 / 12 tokens 20.0 / 20.5 / 21.6
          // -> 18.8 / 19.0 / 19.8 us)
          const int gr = shared_decode_grid(M, N, K, 1, SparseWeight4::kUnit, 16, 1, cus, true,
                                            shared_weight_tiles<SparseWeight4Rows, 1, 16>());
          if (gr > 0)
            return launch_decode_shared<SparseWeight4Rows, 1, 16, 2, 1, true>(
                SparseWeight4Rows{{wv, wm, K}}, xop.xq, xop.xs, ws, M, N, K, y, nullptr, gr, stream);
          const int grid = shared_decode_grid(M, N, K, 1, SparseWeight4::kUnit, 16, 1, cus, true);
          if (grid > 0)
            return launch_decode_shared<SparseWeight4, 1, 16, 2, 1, true>(SparseWeight4{wv, wm, K}, xop.xq, xop.xs,
                                                                          ws, M, N, K, y, nullptr, grid, stream);
        } else {
          const int grid = shared_decode_grid(M, N, K, 1, SparseWeight4::kUnit, 8, 1, cus);
          if (grid > 0)
            return launch_decode_shared<SparseWeight4, 1, 8, 1, 1>(SparseWeight4{wv, wm, K}, xop.xq, xop.xs, ws, M,
                                                                   N, K, y, nullptr, grid, stream);
        }
      }
    }
    if (M <= 16) return launch_decode_for<X, 1>(xop, wv, wm, ws, M, N, K, y, part, stream);
    if (M <= 32) return launch_decode_for<X, 2>(xop, wv, wm, ws, M, N, K, y, part, stream);
    return launch_decode_for<X, 4>(xop, wv, wm, ws, M, N, K, y, part, stream);
  }
}

hipError_t launch_sparse_gemm(const uint8_t *xq, const float *xs, const uint8_t *wv, const uint8_t *wm,
                              const float *ws, int64_t M, int64_t N, int64_t K, uint16_t *y, float *part,
                              hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if (!use_tile_kernel(m, n, k))
    return launch_sparse_decode(QuantTokens{xq, xs, k}, wv, wm, ws, m, n, k, y, part, stream);
  const TilePlan p = plan_tiles(m, n, k, device_cu_count());
  if (p.splits > 1 && !part) return hipErrorInvalidValue;
  float *pp = p.splits > 1 ? part : nullptr;
  hipError_t e = p.bm == 128
                     ? launch_tile<256, 128, 2, 4>(xq, xs, wv, wm, ws, m, n, k, y, p.splits, p.kb_split, pp, stream)
                     : launch_tile<256, 256, 2, 4>(xq, xs, wv, wm, ws, m, n, k, y, p.splits, p.kb_split, pp, stream);
  if (p.splits > 1 && e == hipSuccess) e = launch_splitk_reduce(part, p.splits, (int64_t)m * n, y, stream);
  return e;
}

// Where the GEMM itself takes a form that the in-kernel quantization does not
// have, the linear call runs the two calls: the 2:4 whole-row four-block tiles
// (few_token_rows4), and the dense four-wave form on K >= 8192 (measured on
// MI355X, 4096 x 14336 at one token: 13.4 us as two calls against 14.8 us
// quantized in the 16-wave kernel).
bool linear_staged(int64_t M, int64_t N, int64_t K, bool sparse) {
  if (use_tile_kernel(M, N, K) || !staged_tokens_fit(M, K)) return false;
  return sparse ? !few_token_rows4(K) : K < 8192;
}

// As the dense linear: in-kernel quantization for one or two tokens, else
// fp8_quant_act into the call's scratch tokens and fp8_sparse24_gemm.  The
// staged form sums in the order of the one-block kernel over 16 waves, so it
// is not used where fp8_sparse24_gemm takes the whole-row four-block tiles
// (few_token_rows4): there the two calls run, and the result stays
// bit-identical to them.
hipError_t launch_sparse_linear(const uint16_t *x, const uint8_t *wv, const uint8_t *wm, const float *ws, int64_t M,
                                int64_t N, int64_t K, uint16_t *y, uint8_t *tokens, float *part,
                                hipStream_t stream) {
  if (linear_staged(M, N, K, true))
    return launch_sparse_decode(StagedTokens{x, (int)K, nullptr, nullptr}, wv, wm, ws, (int)M, (int)N, (int)K, y,
                                part, stream);
  if (!tokens) return hipErrorInvalidValue;
  return quantize_then(x, M, K, tokens, stream, [&](const uint8_t *xq, const float *xs) {
    return launch_sparse_gemm(xq, xs, wv, wm, ws, M, N, K, y, part, stream);
  });
}

}  // namespace fp8lin
