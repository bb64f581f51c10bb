// Pieces shared by the dense and 2:4 sparse block-scaled GEMM kernels.
//
// Operand K layout inside one 128-wide K block (both GEMMs): lane group
// g = lane/16 holds K bytes [16g, 16g+16) in register bytes 0..15 and
// [64+16g, 64+16g+16) in bytes 16..31.  For the dense FP8 MFMA any layout
// shared by A and B is correct; this one is the layout the sparse MFMA
// expects of its dense operand when the compressed operand of lane group g
// covers the 8 groups of 4 at K = [32g, 32g+32) (16 contiguous value bytes
// and one 32-bit index word of the compressed weight).
//
// Output layout of a 16x16 MFMA with A = weight rows (n) and B = tokens (m):
// lane l holds token m = l%16 and rows n = 4*(l/16) .. +3.
#pragma once

#include "device_common.hpp"

namespace fp8lin {

__device__ __forceinline__ v8i make_v8i(const uint4 &lo, const uint4 &hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ v4i make_v4i(const uint4 &v) {
  v4i r;
  r[0] = (int)v.x; r[1] = (int)v.y; r[2] = (int)v.z; r[3] = (int)v.w;
  return r;
}

__device__ __forceinline__ uint4 ldg16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Dense operand fragment of one 128-wide K block straight from global memory:
// `row` points at the first byte of the K block of this lane's row.
__device__ __forceinline__ v8i load_frag_global(const uint8_t *row, int g) {
  return make_v8i(ldg16(row + 16 * g), ldg16(row + 64 + 16 * g));
}

// LDS tiles hold rows of 128 bytes as eight 16-byte chunks; chunk c of row r
// sits at chunk position c ^ swz(r).  A 16x16 fragment read (ds_read_b128)
// takes chunk column g = l / 16 of 16 consecutive rows r = l % 16.  The LDS
// (64 banks of 4 bytes) serves such a read in four passes of 16 lanes: lanes
// 0-31 and 32-63 apart, and within each half the lanes whose index bits 2, 3
// and 4 have even parity, then those with odd parity (measured on MI355X by
// pairing two lanes on one bank while all others read one word).  Row parity
// picks the bank half, and swz is chosen so that in every pass the 16 lanes
// touch 16 distinct 16-byte bank groups; it stays conflict-free if a pass were
// 16 consecutive lanes or lanes 8i..8i+7 with 32+8i..32+8i+7.  (A plain
// r ^ (r >> 3) spread costs a second cycle per pass.)  swz depends on r % 16
// only, so a fragment row r = 16*t + l%16 uses one per-lane address plus a
// compile-time offset 2048*t.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2); }

// Fragment read at precomputed per-lane byte offsets (lo, hi chunk) plus a
// compile-time displacement.
__device__ __forceinline__ v8i load_frag_at(const uint8_t *lds_base, int lo, int hi, int disp) {
  const uint4 a = *reinterpret_cast<const uint4 *>(lds_base + lo + disp);
  const uint4 b = *reinterpret_cast<const uint4 *>(lds_base + hi + disp);
  return make_v8i(a, b);
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4).
// The 64 lanes of a wave write 1 KB of LDS at `lds_wave_base` in lane order
// (lane l at +16*l); each lane supplies its own global source address.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

__device__ __forceinline__ void copy16_global_to_lds(const void *src, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void *)const_cast<void *>(src), (lds_void *)lds_wave_base, 16, 0, 0);
}

// Raw buffer resources (byte-addressed, no stride).  A load whose offset lies
// at or past `bytes` returns zeros.  Offsets are a per-lane 32-bit VGPR plus a
// wave-uniform 32-bit SGPR, so walking K costs scalar adds only.  The dword-3
// value 0x00020000 is the gfx9 raw-buffer format (32-bit data, no swizzle).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer resource over rows [row0, row0 + 128) of a panel of `row_bytes`-byte
// rows starting at `panel`, clipped to the `rows_left` rows that exist: rows
// past the matrix edge read as zeros (their results are never stored).  128
// rows of at most 2^24 bytes keep every offset below 2^31.  The clamp goes
// through readfirstlane so the resource stays in SGPRs (a VGPR resource
// would make every load a loop over lanes).
__device__ __forceinline__ rsrc_t panel_rows128(const uint8_t *panel, int rows_left, int row0, int row_bytes) {
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(128, rows_left - row0)));
  return make_rsrc(panel + (int64_t)row0 * row_bytes, (uint32_t)rows * (uint32_t)row_bytes);
}

// 16 bytes per lane from a buffer into registers.
__device__ __forceinline__ uint4 buffer_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// 16 bytes per lane from a buffer into LDS (buffer_load_dwordx4 ... lds): the
// 64 lanes write 1 KB at `lds_wave_base` in lane order.
__device__ __forceinline__ void buffer_copy16_to_lds(rsrc_t r, uint32_t voff, uint32_t soff, void *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_wave_base, 16, voff, soff, 0, 0);
}

// Wait until this wave's outstanding global loads (the LDS copies included)
// have landed: s_waitcnt vmcnt(0) (expcnt and lgkmcnt at their maxima, 7 and
// 15).  Issued through the builtin so that the compiler's own wait insertion
// knows the counter is drained and adds no later waits for these loads.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Pins a value in VGPRs at this point of the program: the computation that
// produces it cannot be sunk below the pin (keeps the partial-product scaling
// next to its MFMAs instead of piling up live partials).
__device__ __forceinline__ void pin(v4f &v) { asm volatile("" : "+v"(v)); }

// Pack four fp32 accumulators into four bf16 (RNE) for one 8-byte store.
__device__ __forceinline__ uint2 pack_bf16x4(const v4f &v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Token scales of a BM-row tile, staged in LDS in groups of SB K blocks
// (ring of two groups).  With SB = 4 (K/128 divisible by 4) each thread loads
// the four scales of its row with one 16-byte load, so the scattered per-row
// reads cost one request per four K blocks.
template <int BM, int SB>
struct TokenScales {
  float *lds;  // [2][SB][BM]
  const float *src;
  float4 reg;
  int tid;

  __device__ __forceinline__ void init(float *lds_, const float *xs, int M, int KB, int m_base, int tid_) {
    lds = lds_;
    tid = tid_;
    src = xs + (int64_t)min(m_base + min(tid, BM - 1), M - 1) * KB;
  }
  // registers <- scales of K blocks [SB*grp, SB*grp + SB)
  __device__ __forceinline__ void load(int grp) {
    if (tid < BM) {
      if (SB == 4) reg = *reinterpret_cast<const float4 *>(src + 4 * grp);
      else reg.x = src[grp];
    }
  }
  __device__ __forceinline__ void store(int grp) {
    if (tid < BM) {
      float *d = lds + (grp & 1) * SB * BM + tid;
      d[0] = reg.x;
      if (SB == 4) {
        d[BM] = reg.y;
        d[2 * BM] = reg.z;
        d[3 * BM] = reg.w;
      }
    }
  }
  __device__ __forceinline__ float get(int kb, int row) const {
    return lds[((kb / SB) & 1) * SB * BM + (kb % SB) * BM + row];
  }
};

// Token exponents (UE8M0 scales, one byte per token and K block) staged like
// TokenScales: registers <- SB exponent bytes of this thread's token (one
// 4-byte load when SB = 4), LDS [2][SB][BM] one word per exponent.
template <int BM, int SB>
struct TokenExps {
  uint32_t *lds;
  const uint8_t *src;
  uint32_t reg;
  int tid;

  __device__ __forceinline__ void init(float *lds_, const uint8_t *xe, int M, int KB, int m_base, int tid_) {
    lds = reinterpret_cast<uint32_t *>(lds_);
    tid = tid_;
    src = xe + (int64_t)min(m_base + min(tid, BM - 1), M - 1) * KB;
  }
  __device__ __forceinline__ void load(int grp) {
    if (tid < BM) {
      if (SB == 4) reg = *reinterpret_cast<const uint32_t *>(src + 4 * grp);
      else reg = src[grp];
    }
  }
  __device__ __forceinline__ void store(int grp) {
    if (tid < BM) {
      uint32_t *d = lds + (grp & 1) * SB * BM + tid;
      d[0] = reg & 0xFFu;
      if (SB == 4) {
        d[BM] = (reg >> 8) & 0xFFu;
        d[2 * BM] = (reg >> 16) & 0xFFu;
        d[3 * BM] = reg >> 24;
      }
    }
  }
  __device__ __forceinline__ uint32_t get(int kb, int row) const {
    return lds[((kb / SB) & 1) * SB * BM + (kb % SB) * BM + row];
  }
};

// v_mfma_scale_f32_16x16x128_f8f6f4, both operands e4m3, accumulating into c:
// products of A row i scaled by 2^(sa - 127) and of B column j by 2^(sb - 127),
// where sa / sb are byte 0 of the lane's scale operand (each lane covers its
// row / column and one 32-wide K quarter; all four quarters carry the same
// exponent here).
__device__ __forceinline__ v4f mfma_16x16x128_fp8_e8(const v8i &a, const v8i &b, const v4f &c, uint32_t sa,
                                                    uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

// Coalesced epilogue: a wave writes its 16 x (16*RT) bf16 sub-tile for token
// tile c into a private 16 x 256-byte LDS scratch (16-byte chunks XOR-swizzled
// by row), reads it back as whole rows and stores 256 contiguous bytes per
// row.  `acc_c` holds the RT 16x16 accumulators of token tile c (lane: token
// l%16, rows 4*(l/16)..+3 of each row tile).  Requires 16*RT*2 == 256.
// The stores are non-temporal: Y is written once and not read back by this
// kernel, and streaming it past the L2 keeps the end-of-tile write burst from
// stalling the next tile's operand loads.
template <int RT>
__device__ __forceinline__ void store_token_tile(uint8_t *scratch, const v4f (&acc_c)[RT], uint16_t *y, int M,
                                                 int N, int m0, int n0, int lane) {
  static_assert(RT == 8, "scratch rows are 256 bytes");
  const int lr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < RT; r++) {
    const int chunk = 2 * r + (g >> 1);
    *reinterpret_cast<uint2 *>(scratch + lr * 256 + ((chunk ^ lr) << 4) + 8 * (g & 1)) = pack_bf16x4(acc_c[r]);
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int row = 4 * j + g;  // lane l reads row 4j + l/16, chunk l%16
    const v4i v = *reinterpret_cast<const v4i *>(scratch + row * 256 + ((lr ^ row) << 4));
    const int m = m0 + row, n = n0 + 8 * lr;
    if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<v4i *>(y + (int64_t)m * N + n));
  }
}

// fp32 partial tile of token tile c straight from registers: lane (token
// l%16, rows 4*(l/16) + 16*r .. +3) stores 16 contiguous bytes per row tile,
// four lanes making 64 contiguous bytes of a token's row.  The partials are
// read back by the split-K reduction, so they go through the caches normally.
template <int RT>
__device__ __forceinline__ void store_token_tile_f32(const v4f (&acc_c)[RT], float *out, int M, int N, int m0, int n0,
                                                     int lane) {
  const int m = m0 + (lane & 15), g = lane >> 4;
  if (m >= M) return;
#pragma unroll
  for (int r = 0; r < RT; r++) {
    const int n = n0 + 16 * r + 4 * g;
    if (n < N) *reinterpret_cast<v4f *>(out + (int64_t)m * N + n) = acc_c[r];
  }
}

// Tile order.  Workgroups are dealt to the 8 XCDs round-robin (block b runs on
// XCD b % 8), each XCD with its own L2.  The remap gives every XCD one
// contiguous range of logical tile ids; the logical order then walks groups of
// `group_m` token tiles column by column, so an XCD's concurrent tiles share
// weight and activation panels in its L2.
// Whether workgroup b has a logical tile when only `total` tiles exist (a grid
// of at least `total` workgroups; the rest return): XCD x takes the first
// total / 8 (+1 for x < total % 8) of its workgroups b = x, x + 8, ...
__device__ __forceinline__ bool tile_slot_used(int b, int total) {
  const int q = total / 8, r = total % 8;
  return b / 8 < q + (b % 8 < r ? 1 : 0);
}

__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / 8, r = total % 8;
  const int xcd = b % 8, local = b / 8;
  const int logical = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int per_group = group_m * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in_group = logical % per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

}  // namespace fp8lin
