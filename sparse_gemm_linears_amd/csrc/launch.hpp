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
// K split of the weight-streaming kernel (1 = none).  Long K on few row bands
// (N < 6144, K >= 8192) at 9 to 32 tokens splits four ways; shorter K on few
// row bands at 33 to 64 tokens two ways (both measured on MI355X; the
// launchers pick the matching kernel instance).  Never for one or two
// tokens, the range quantized inside the kernel.
inline int decode_splits(int64_t M, int64_t N, int64_t K) {
  if (M > 8 && M <= 32 && N < 6144 && K >= 8192) return 4;
  if (M > 32 && N < 6144 && K < 8192) return 2;
  return 1;
}
// Bytes of fp32 split-K partials that fp8_block_gemm, fp8_sparse24_gemm and
// fp8_block_gemm_ue8m0 need for this shape on a device with `cus` compute
// units (0 when K is not split): splits * M * N * 4.
size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K, int cus);
// The same for fp8_block_gemm_swiglu (the stacked [gate; up] GEMM of 2I rows
// when it runs on smaller tiles or split K).
size_t swiglu_partial_bytes(int64_t M, int64_t I, int64_t K, int cus);
// Whether the fused linear call quantizes the tokens inside the decode kernel
// (one or two tokens), for the dense or the 2:4 weight.
bool linear_staged(int64_t M, int64_t N, int64_t K, bool sparse);
// Scratch of the fused linear calls: the quantized tokens (codes, then fp32
// scales at a 256-byte aligned offset; 0 bytes when the tokens are quantized
// inside the decode kernel) and the partials of the GEMM that follows.
size_t linear_token_bytes(int64_t M, int64_t N, int64_t K, bool sparse);
inline size_t token_codes_bytes(int64_t M, int64_t K) { return ((size_t)M * (size_t)K + 255) / 256 * 256; }
hipError_t launch_splitk_reduce(const float *part, int splits, int64_t mn, uint16_t *y, hipStream_t stream);

// Scratch memory of one call, held from acquire() until release() (or the
// destructor): the split-K partials and the quantized tokens a call needs,
// found or made before the call's first launch, so that a failed acquisition
// enqueues no kernel.  While held it keeps the library's scratch lock, so that
// calls on one stream may come from several host threads: their launches and
// the stream-ordered frees of outgrown buffers are enqueued in call order.
//   * outside stream capture: one buffer per (device, stream, slot), from a
//     stream-ordered pool the library owns (hipStreamPerThread is keyed by the
//     calling thread too, since that one handle names a different stream in
//     each thread); a larger need allocates the new buffer first and then frees
//     the old one on the same stream, after the work queued on it;
//   * under stream capture: buffers of that capture (hipMalloc outside the
//     graph, kept until the process ends or fp8lin_release_graph_scratch),
//     at most 1 GiB in all; past it, allocation and free nodes in the graph.
class CallScratch {
 public:
  CallScratch() = default;
  CallScratch(const CallScratch &) = delete;
  CallScratch &operator=(const CallScratch &) = delete;
  ~CallScratch() { (void)release(); }
  hipError_t acquire(size_t partial_bytes, size_t token_bytes, hipStream_t stream);
  hipError_t release();
  float *partials() const { return static_cast<float *>(p_[0]); }
  uint8_t *tokens() const { return static_cast<uint8_t *>(p_[1]); }

 private:
  void *p_[2] = {nullptr, nullptr};
  bool transient_[2] = {false, false};
  hipStream_t stream_ = nullptr;
  bool locked_ = false;
};
// Frees the buffers kept for captured calls (all devices).  Only valid when no
// graph or executable graph that captured a library call exists any more.
hipError_t release_graph_scratch();
// The per-device address and size of the library's fixed scratch array (a
// file-scope device array, no allocation), looked up once per device.
hipError_t fixed_scratch(void **p, size_t *bytes);

// fp8_quant_act into `tokens` (linear_token_bytes of scratch: codes, then the
// scales at token_codes_bytes), then gemm(xq, xs) on them: exactly the two
// calls fp8_quant_act and the GEMM.
template <class Gemm>
inline hipError_t quantize_then(const uint16_t *x, int64_t M, int64_t K, uint8_t *tokens, hipStream_t stream,
                                Gemm gemm) {
  uint8_t *xq = tokens;
  float *xs = reinterpret_cast<float *>(tokens + token_codes_bytes(M, K));
  const hipError_t e = launch_quant_act(x, M, K, xq, xs, stream);
  return e == hipSuccess ? gemm(xq, xs) : e;
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
                                   int64_t M, int64_t N, int64_t K, uint16_t *y, float *part, hipStream_t stream);
hipError_t launch_prune24(const uint16_t *w, const float *col_norm, int64_t N, int64_t K, uint8_t *vals,
                          uint8_t *meta, float *s, hipStream_t stream);
// 2:4 prune with one per-tensor scale (three launches; s[0] holds partial
// maxima between them).
hipError_t launch_prune24_tensor(const uint16_t *w, const float *col_norm, int64_t N, int64_t K, uint8_t *vals,
                                 uint8_t *meta, float *s, hipStream_t stream);
// s[0] = (largest of the n_part bf16 magnitude bit patterns stored in s) / 448.
hipError_t launch_amax_finish(float *s, int64_t n_part, hipStream_t stream);
// part: fp32 partials of gemm_partial_bytes(M, N, K, device_cu_count()) bytes
// (may be NULL when that is 0).
hipError_t launch_dense_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M,
                             int64_t N, int64_t K, uint16_t *y, float *part, hipStream_t stream);
hipError_t launch_sparse_gemm(const uint8_t *xq, const float *xs, const uint8_t *wv, const uint8_t *wm,
                              const float *ws, int64_t M, int64_t N, int64_t K, uint16_t *y, float *part,
                              hipStream_t stream);

// Grouped (MoE) dense GEMM: expert g multiplies rows offsets[g] .. offsets[g+1]-1
// (device int32 offsets, nondecreasing, offsets[0] = 0, offsets[G] = M).
hipError_t launch_dense_grouped_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                    const int32_t *offsets, int64_t G, int64_t M, int64_t N, int64_t K, uint16_t *y,
                                    hipStream_t stream);

// Dense GEMM on a [gate; up] weight (2I rows) with the SwiGLU epilogue:
// h = bf16(silu(g) * u), plus fp8_quant_act(h) when hq is not NULL.
hipError_t launch_dense_gemm_swiglu(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                   int64_t M, int64_t I, int64_t K, uint16_t *h, uint8_t *hq, float *hs,
                                   float *part, hipStream_t stream);

// Decode-sized (M <= 64) GEMMs on bf16 activations, quantized inside the kernel
// with the arithmetic of fp8_quant_act.
// tokens: linear_token_bytes(M, N, K) bytes; part: gemm_partial_bytes(M, N, K, ..).
hipError_t launch_dense_linear(const uint16_t *x, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                               int64_t K, uint16_t *y, uint8_t *tokens, float *part, hipStream_t stream);
hipError_t launch_sparse_linear(const uint16_t *x, const uint8_t *wv, const uint8_t *wm, const float *ws, int64_t M,
                                int64_t N, int64_t K, uint16_t *y, uint8_t *tokens, float *part,
                                hipStream_t stream);

}  // namespace fp8lin
