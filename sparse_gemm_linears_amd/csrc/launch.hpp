// Kernel launchers behind the C entry points.  Arguments are already
// validated; each returns the runtime's launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, hipStream_t stream);
hipError_t launch_quant_wblock(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, hipStream_t stream);
// Tile-kernel plan shared by the dense and 2:4 GEMMs: tile height (256 or 128
// tokens) and K split (splits workgroups per tile, kb_split K blocks each).
// Split GEMMs store fp32 partials [splits][M][N] that launch_splitk_reduce
// adds in order into y.
struct TilePlan {
  int bm, splits, kb_split;
};
int device_cu_count();
TilePlan plan_tiles(int M, int N, int K, int cus);
// Decode kernel or tile kernel: the decode kernel streams the weight once but
// re-reads the tokens per workgroup, so past about 20 tokens the tile kernel
// (split K) is faster on large weights (measured on MI355X, HIP-graph replay
// from HBM, on the 28672x4096 and 4096x14336 Llama-3-8B weights: at 16 tokens
// the decode kernel is faster, at 21 the two tie or the tile kernel leads by
// up to 11 %, at 32 the tile kernel leads by 6-21 %, dense and 2:4), while the
// 6144x4096 and 4096x4096 weights stay faster in the decode kernel up to 64.
// Long-K weights with N < 6144 take the decode kernel's split-K form up to 32
// tokens: on the 4096x14336 weight it beats the tile kernel by 19-23 % at 21
// to 32 tokens.
inline bool use_tile_kernel(int64_t M, int64_t N, int64_t K) {
  if (M > 64) return true;
  if (N < 6144 && K >= 8192) return M > 32;
  return M > 20 && N * K >= (int64_t(1) << 25);
}
hipError_t launch_splitk_reduce(const float *part, int splits, int64_t mn, uint16_t *y, hipStream_t stream);
// Library-owned scratch memory for the work a call puts on `stream`: kept
// between calls per (device, stream, slot), and per capture for calls under
// stream capture (a captured graph keeps its own).  Calls on one stream share
// it, so they must be issued in stream order (not from several host threads
// at once on one stream).  workspace_release returns it (a no-op unless the
// memory was a one-off allocation).
enum WorkspaceSlot { kSlotPartials = 0, kSlotTokens = 1 };
struct Workspace {
  void *p = nullptr;
  hipStream_t stream = nullptr;
  bool transient = false;
};
hipError_t workspace_acquire(Workspace *w, WorkspaceSlot slot, size_t bytes, hipStream_t stream);
hipError_t workspace_release(Workspace *w);

// Tokens quantized into library scratch memory, then the GEMM on them: exactly
// fp8_quant_act followed by gemm(xq, xs).
template <class Gemm>
inline hipError_t quantize_then(const uint16_t *x, int64_t M, int64_t K, hipStream_t stream, Gemm gemm) {
  const size_t q_bytes = ((size_t)M * (size_t)K + 255) / 256 * 256;
  const size_t s_bytes = (size_t)M * (size_t)(K / 128) * sizeof(float);
  Workspace ws;
  hipError_t e = workspace_acquire(&ws, kSlotTokens, q_bytes + s_bytes, stream);
  if (e != hipSuccess) return e;
  uint8_t *xq = static_cast<uint8_t *>(ws.p);
  float *xs = reinterpret_cast<float *>(xq + q_bytes);
  e = launch_quant_act(x, M, K, xq, xs, stream);
  if (e == hipSuccess) e = gemm(xq, xs);
  const hipError_t f = workspace_release(&ws);
  return e == hipSuccess ? f : e;
}

// One scale for a whole tensor of n bf16 values (n a multiple of 8), written
// to all n_s entries of s (n_s >= 1): the dynamic per-tensor amax / 448, or a
// static scale read from device memory.
constexpr int64_t kTensorAmaxParts = 1024;
hipError_t launch_quant_tensor(const uint16_t *x, int64_t n, uint8_t *q, float *s, int64_t n_s, hipStream_t stream);
hipError_t launch_quant_static(const uint16_t *x, const float *scale, int64_t n, uint8_t *q, float *s, int64_t n_s,
                               hipStream_t stream);
// UE8M0 (power-of-two) scale variants: one exponent byte per group / block.
hipError_t launch_quant_act_ue8m0(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *e, hipStream_t stream);
hipError_t launch_quant_wblock_ue8m0(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, uint8_t *e,
                                     hipStream_t stream);
hipError_t launch_dense_gemm_ue8m0(const uint8_t *xq, const uint8_t *xe, const uint8_t *wq, const uint8_t *we,
                                   int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream);
hipError_t launch_prune24(const uint16_t *w, const float *col_norm, int64_t N, int64_t K, uint8_t *vals,
                          uint8_t *meta, float *s, hipStream_t stream);
hipError_t launch_dense_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M,
                             int64_t N, int64_t K, uint16_t *y, hipStream_t stream);
hipError_t launch_sparse_gemm(const uint8_t *xq, const float *xs, const uint8_t *wv, const uint8_t *wm,
                              const float *ws, int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

// Grouped (MoE) dense GEMM: expert g multiplies rows offsets[g] .. offsets[g+1]-1
// (device int32 offsets, nondecreasing, offsets[0] = 0, offsets[G] = M).
hipError_t launch_dense_grouped_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                    const int32_t *offsets, int64_t G, int64_t M, int64_t N, int64_t K, uint16_t *y,
                                    hipStream_t stream);

// Dense GEMM on a [gate; up] weight (2I rows) with the SwiGLU epilogue:
// h = bf16(silu(g) * u), plus fp8_quant_act(h) when hq is not NULL.
hipError_t launch_dense_gemm_swiglu(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                   int64_t M, int64_t I, int64_t K, uint16_t *h, uint8_t *hq, float *hs,
                                   hipStream_t stream);

// Decode-sized (M <= 64) GEMMs on bf16 activations, quantized inside the kernel
// with the arithmetic of fp8_quant_act.
hipError_t launch_dense_linear(const uint16_t *x, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                               int64_t K, uint16_t *y, hipStream_t stream);
hipError_t launch_sparse_linear(const uint16_t *x, const uint8_t *wv, const uint8_t *wm, const float *ws, int64_t M,
                                int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

}  // namespace fp8lin
