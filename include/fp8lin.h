/*
 * fp8lin: FP8 block-scaled and 2:4-sparse FP8 linear layers for AMD MI355X (gfx950).
 *
 * C ABI.  All tensors are dense, row-major and contiguous in device memory.
 * bf16 values are passed as their raw 16-bit patterns (uint16_t).  FP8 codes
 * are OCP E4M3FN bytes (sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, 0x7F/0xFF = NaN, largest finite 448), view-compatible with
 * torch.float8_e4m3fn.  Scales are fp32.  G = 128 is the group / block edge.
 *
 * Ownership: the caller allocates every input and output; the library keeps
 * no pointer to them after a call returns.  Besides per-device architecture
 * and compute-unit counts, it keeps scratch memory of its own for the calls
 * that need one, until the process ends:
 *   fp8_block_gemm and fp8_sparse24_gemm on the tile kernel (M > 64, or
 *   M > 20 with N * K >= 2^25, except M <= 32 when N < 6144 and K >= 8192)
 *   with too few output tiles to cover half of the compute units split K,
 *   with S * M * N * 4 bytes of fp32 partials (S <= 16, at most 256 tiles'
 *   worth);
 *   the same two GEMMs on the weight-streaming kernel split K for weights
 *   with N < 6144: four ways at 9 to 32 tokens when K >= 8192, two ways at
 *   33 to 64 tokens when K < 8192 (S * M * N * 4 bytes of partials);
 *   fp8_block_linear and fp8_sparse24_linear from three tokens on quantize
 *   the tokens into M * K + 4 * M * K / 128 bytes (and may split K as above);
 *   fp8_block_gemm_swiglu with few tokens keeps the fp32 partials of the
 *   stacked GEMM (S * M * 2I * 4 bytes).
 * The scratch memory is held per device, stream and capture:
 *   - outside stream capture, one buffer per stream, from a stream-ordered
 *     pool the library creates once per device (hipMallocFromPoolAsync on
 *     `stream`; a larger need allocates the new buffer first, then frees the
 *     old one with hipFreeAsync on the same stream).  hipStreamPerThread names
 *     a different stream in each thread, so its buffers are kept per thread;
 *   - under stream capture, buffers of the capture's own (hipMalloc, made
 *     with the thread's capture mode relaxed for that call), kept because the
 *     graph holds their address: a replay shares no scratch memory with eager
 *     calls or with other graphs, and may run on any stream.  At most 1 GiB is
 *     kept for captures in all (buffers a capture outgrew included); past it a
 *     capture allocates inside the graph instead (stream-ordered pool
 *     allocation and free nodes).  fp8lin_release_graph_scratch frees the kept
 *     buffers once the caller has destroyed every such graph.
 * A call that needs scratch finds or makes all of it before its first launch
 * and holds the library's scratch lock until its last launch is enqueued, so
 * calls on one stream may come from any threads: they run in the order they
 * took the lock.  Calls on different streams never share scratch memory.
 * fp8_block_gemm_noalloc takes its partials from a fixed device array of the
 * library's instead and allocates nothing.
 *
 * Asynchrony: each call validates its arguments on the host, enqueues its
 * kernels on `stream` (NULL = the default stream) and returns without
 * synchronising.  A fault inside a kernel surfaces at the caller's next
 * synchronisation, as for any HIP launch.
 *
 * Errors: on any error no kernel is enqueued and every output is left untouched.
 *   FP8L_ERR_NULL    a required pointer is NULL;
 *   FP8L_ERR_SHAPE   M < 0, N <= 0, K <= 0, K % 128 != 0, N % 128 != 0, or a
 *                    dimension above 2^24, or a matrix above 2^36 elements
 *                    (and M > 64 for the two *_linear calls);
 *                    for fp8_block_gemm_swiglu I plays the part of N;
 *   FP8L_ERR_ALIGN   a pointer is not 16-byte aligned;
 *   FP8L_ERR_ALIAS   an output overlaps an input or another output;
 *   FP8L_ERR_DEVICE  the current HIP device is missing or is not gfx950;
 *   FP8L_ERR_LAUNCH  the kernel launch was rejected by the runtime;
 *   FP8L_ERR_MEMORY  scratch memory for the call could not be allocated (no
 *                    kernel runs);
 *   FP8L_ERR_SCRATCH fp8_block_gemm_noalloc: the call needs more scratch than
 *                    the fixed array holds (no kernel runs).
 * M == 0 (an empty batch) returns FP8L_OK without launching and without
 * looking at the M-sized buffers.  There is no fallback path: an unsupported
 * case is an error, never a silently slower kernel.
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int fp8l_status;
enum {
    FP8L_OK = 0,
    FP8L_ERR_NULL = 1,
    FP8L_ERR_SHAPE = 2,
    FP8L_ERR_ALIGN = 3,
    FP8L_ERR_ALIAS = 4,
    FP8L_ERR_DEVICE = 5,
    FP8L_ERR_LAUNCH = 6,
    FP8L_ERR_MEMORY = 7,
    FP8L_ERR_SCRATCH = 8
};

/*
 * Dynamic per-token activation quantization in 1x128 groups ("FP8 a
 * granularite fine", transformers docs: intro bullets, activations quantized
 * per token in groups of 128 input channels; section "Chemin rapide de
 * DeepGEMM": dynamic activation scheme).
 *
 *   x [M,K] bf16            activations, one token per row
 *   q [M,K] e4m3            q[m,k] = enc(fp32(x[m,k] / s[m,k/128]))
 *   s [M,K/128] fp32        s[m,kb] = fp32(amax / 448), amax = max |x[m,k]| over
 *                           the 128 channels of group kb; amax == 0 gives s = 0
 *                           and signed-zero codes
 * enc() rounds to nearest, ties to even, and saturates at +-448; both divisions
 * are IEEE fp32 divisions.
 */
fp8l_status fp8_quant_act(const uint16_t *x, int64_t M, int64_t K,
                          uint8_t *q, float *s, hipStream_t stream);

/*
 * Weight quantization in 128x128 blocks ("FP8 a granularite fine", intro
 * bullets: weight_block_size = (128, 128)).  W is nn.Linear.weight [N,K]
 * (K contiguous).
 *
 *   w [N,K] bf16
 *   q [N,K] e4m3            q[n,k] = enc(fp32(w[n,k] / s[n/128,k/128]))
 *   s [N/128,K/128] fp32    s = fp32(amax / 448), amax over the 128x128 block
 */
fp8l_status fp8_quant_weight_block(const uint16_t *w, int64_t N, int64_t K,
                                   uint8_t *q, float *s, hipStream_t stream);

/*
 * One scale for the whole tensor, in the block-scale layout: every entry of
 * the scale array holds the same fp32 s, so fp8_block_gemm and
 * fp8_sparse24_gemm take these codes and scales unchanged.
 *
 * fp8_quant_act_tensor: dynamic per-tensor scaling ("Deployer la parcimonie
 * 2:4 avec FP8 sur Hopper": pipeline step 3 and "Bonnes pratiques", FP8 with
 * a scale computed per tensor at run time).  s = fp32(amax / 448), amax the
 * largest |x| of the whole [M,K] tensor.  Three launches on the stream; s[0]
 * holds partial maxima between them, so s must not be read before the call's
 * work on the stream is done.
 *
 * fp8_quant_act_static: static activation scaling ("FP8 a granularite fine",
 * section "Chemin rapide de DeepGEMM": the static activation scheme, a scale
 * fixed ahead of time).  scale points to one fp32 in device memory (4-byte
 * aligned, not overlapping q or s), read by the kernel: 0 < *scale < inf is
 * the caller's contract; values beyond 448 * scale saturate to +-448.
 *
 * fp8_quant_weight_tensor: dynamic per-tensor weight scaling (the same
 * passage of "Deployer la parcimonie 2:4 avec FP8 sur Hopper"), s over all of
 * W [N,K] written to each of the [N/128,K/128] block scales.
 *
 *   x [M,K] bf16 / w [N,K] bf16
 *   q [M,K] / [N,K] e4m3      q = enc(fp32(x / s)), RNE, saturating at +-448
 *   s [M,K/128] / [N/128,K/128] fp32, every entry = s; amax == 0 gives s = 0
 *                             and signed-zero codes
 */
fp8l_status fp8_quant_act_tensor(const uint16_t *x, int64_t M, int64_t K,
                                 uint8_t *q, float *s, hipStream_t stream);
fp8l_status fp8_quant_act_static(const uint16_t *x, const float *scale, int64_t M, int64_t K,
                                 uint8_t *q, float *s, hipStream_t stream);
fp8l_status fp8_quant_weight_tensor(const uint16_t *w, int64_t N, int64_t K,
                                    uint8_t *q, float *s, hipStream_t stream);

/*
 * 2:4 pruning along K, post-prune block scales and compression ("Deployer la
 * parcimonie 2:4 avec FP8 sur Hopper": pipeline step 2, groups of 4
 * contiguous values along K; step 4, magnitude or activation-aware scores,
 * the two least important of every 4 dropped; step 6, FP8 scales re-derived
 * after pruning; step 7, pruned weights exported with their 2:4 masks.
 * "Combiner elagage et quantification", section "La cle": keep the two
 * largest of every four).
 *
 *   w [N,K] bf16
 *   col_norm [K] fp32 or NULL   score of w[n,k] = |w[n,k]| * col_norm[k]
 *                               (activation-aware), or |w[n,k]| when NULL
 *                               (magnitude); the product is compared exactly
 *   vals [N,K/2] e4m3           the two kept codes of each group, lower index first
 *   meta [N,K/8] u8             2-bit positions: group g of row n has nibble
 *                               i0 | (i1 << 2) (i0 < i1 the kept positions) at
 *                               bits 4*(g%2) .. 4*(g%2)+3 of meta[n, g/2]
 *   s [N/128,K/128] fp32        fp32(amax / 448), amax over the kept values of
 *                               the block; kept codes = enc(fp32(w / s))
 * Each group keeps exactly two positions, the two largest scores; equal scores
 * keep the lower index.
 */
fp8l_status prune24_compress(const uint16_t *w, const float *col_norm, int64_t N, int64_t K,
                             uint8_t *vals, uint8_t *meta, float *s, hipStream_t stream);

/*
 * The same 2:4 prune and compression with one scale for the whole tensor
 * ("Deployer la parcimonie 2:4 avec FP8 sur Hopper": pipeline step 3, FP8 with
 * a per-tensor scale; step 6, the scale re-derived after pruning).  The mask,
 * vals and meta follow prune24_compress; the scale is s = fp32(amax / 448)
 * with amax the largest kept magnitude of all of W, the kept codes are
 * enc(fp32(w / s)), and s is written to every entry of the [N/128,K/128] scale
 * array, so fp8_sparse24_gemm takes the result unchanged.  Three launches on
 * the stream; s[0] holds partial maxima between them, so s must not be read
 * before the call's work on the stream is done.
 */
fp8l_status prune24_compress_tensor(const uint16_t *w, const float *col_norm, int64_t N, int64_t K,
                                    uint8_t *vals, uint8_t *meta, float *s, hipStream_t stream);

/*
 * Block-scaled FP8 GEMM with fp32 accumulation ("FP8 a granularite fine",
 * section "Chemin rapide de DeepGEMM": every FP8 linear with (128,128) weight
 * blocks and dynamic activations runs as a block-scaled FP8 GEMM).
 *
 *   xq [M,K] e4m3, xs [M,K/128] fp32       from fp8_quant_act
 *   wq [N,K] e4m3, ws [N/128,K/128] fp32   from fp8_quant_weight_block
 *   y [M,N] bf16   y[m,n] = bf16_rne( sum_kb xs[m,kb] * ws[n/128,kb] *
 *                                     sum_{k in kb} dec(xq[m,k]) * dec(wq[n,k]) )
 * The inner block sums are exact FP8 products accumulated in fp32.  Small
 * batches (M <= 20, or M <= 32 when N < 6144 and K >= 8192, or M <= 64 when
 * N * K < 2^25) run a weight-streaming kernel; the rest run the tile kernel.
 * With few output tiles (tile kernel), or on weights with N < 6144 at 9 to 32
 * tokens with K >= 8192 or 33 to 64 tokens with K < 8192 (weight-streaming
 * kernel, four or two parts), the K blocks are summed in up to 16 fp32
 * partials (each in K order) that are then added in a fixed order, which
 * changes only the fp32 rounding order; results are deterministic either way.
 */
fp8l_status fp8_block_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                           int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

/*
 * fp8_block_gemm for callers that cannot allocate memory: code that must not
 * call hipMalloc (or add memory nodes to a graph being captured), tight
 * serving loops, harnesses that forbid allocation.  Same arguments, kernels
 * and results as fp8_block_gemm, bit for bit.  Where fp8_block_gemm splits K
 * (see above), the fp32 partials go to a fixed device array of the library
 * (32 MiB per device, a file-scope device variable that exists while the
 * library is loaded; enough for every split plan on a 256-CU MI355X) instead
 * of allocated scratch; every other case needs no scratch at all.  A call
 * whose partials would not fit returns FP8L_ERR_SCRATCH and launches nothing.
 * The array keeps the last call's partials and is overwritten before it is
 * read, so nothing needs clearing.  All calls on one device share it: calls
 * that can overlap on the GPU (different streams, or graphs replayed
 * concurrently) race on it and must be ordered by the caller.
 */
fp8l_status fp8_block_gemm_noalloc(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                   int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

/*
 * The same GEMM with a 2:4-compressed weight from prune24_compress ("Deployer
 * la parcimonie 2:4 avec FP8 sur Hopper", introduction and performance notes:
 * 2:4 GEMMs run on the sparse matrix units; here the sparse MFMA of gfx950).
 * The pruned positions contribute zero.
 *
 *   wvals [N,K/2] e4m3, wmeta [N,K/8], ws [N/128,K/128] fp32
 *
 * On the tile kernel, a workgroup that accumulates at least 32 K blocks may
 * keep its running sums in units of the current K block's scale (rescaled by
 * the ratio of consecutive scales, the last scale applied at the end) when
 * every scale product it uses is a normal fp32 number in [2^-100, 2^100], all
 * within 2^60 of each other, and no scale is zero; where every scale product
 * a wave uses is the same in all of those K blocks (per-tensor scales, as
 * from fp8_quant_act_tensor and prune24_compress_tensor), it sums the
 * unscaled block products and applies the one scale at the end; otherwise it
 * adds scaled partials.  The forms differ only in fp32 rounding (about one ulp
 * per K block for the rescaling); results are deterministic either way.
 */
fp8l_status fp8_sparse24_gemm(const uint8_t *xq, const float *xs, const uint8_t *wvals,
                              const uint8_t *wmeta, const float *ws, int64_t M, int64_t N,
                              int64_t K, uint16_t *y, hipStream_t stream);

/*
 * Grouped (mixture-of-experts) block-scaled FP8 GEMM, contiguous layout ("FP8
 * a granularite fine", section "Chemin rapide de DeepGEMM": the expert layers
 * of MoE models run as grouped FP8 GEMMs).  The tokens routed to expert g are
 * the rows offsets[g] .. offsets[g+1]-1 of X and Y; each group is
 * fp8_block_gemm with that expert's weight.
 *
 *   xq [M,K] e4m3, xs [M,K/128] fp32          tokens, sorted by expert
 *   wq [G,N,K] e4m3, ws [G,N/128,K/128] fp32  one 128x128-block-scaled weight per expert
 *   offsets [G+1] int32, device memory        offsets[0] = 0, nondecreasing,
 *                                             offsets[G] = M (empty groups allowed)
 *   y [M,N] bf16
 * The group sizes stay on the device: the launch covers the worst case
 * (ceil(M/256) + G token tiles) and surplus workgroups exit at once, so no
 * host synchronisation is needed.  Offsets that break the rules give
 * unspecified rows but never an access outside X, Y or the weights.
 * 1 <= G <= 4096, G*N*K <= 2^36.
 */
fp8l_status fp8_grouped_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                             const int32_t *offsets, int64_t G, int64_t M, int64_t N, int64_t K, uint16_t *y,
                             hipStream_t stream);

/*
 * Power-of-two (UE8M0) scales ("FP8 a granularite fine", section "Format
 * d'echelle UE8M0": scales stored as float8_e8m0fnu bytes, as some
 * checkpoints do and some kernels require).  A byte e stands for 2^(e - 127).
 * The group / block exponent is the smallest e >= 0 with 448 * 2^(e - 127) >=
 * amax, the smallest power of two not below amax / 448, so no value
 * saturates; amax == 0 gives e = 0.  Codes are enc(x * 2^(127 - e)), one
 * rounding of an exact quotient.  Layouts are those of the fp32-scale calls
 * with one byte per scale: e [M,K/128] for activations, [N/128,K/128] for
 * weights.
 */
fp8l_status fp8_quant_act_ue8m0(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *e,
                                hipStream_t stream);
fp8l_status fp8_quant_weight_block_ue8m0(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, uint8_t *e,
                                         hipStream_t stream);

/*
 * Block-scaled FP8 GEMM with UE8M0 scales, applied by the gfx950 MFMA's own
 * block scaling (no per-block multiply in the kernel):
 *   y[m,n] = bf16_rne( sum_kb 2^(xe[m,kb] - 127) * 2^(we[n/128,kb] - 127) *
 *                      sum_{k in kb} dec(xq[m,k]) * dec(wq[n,k]) ), fp32 accumulation.
 * Dense weights only: the 2:4 sparse MFMA of gfx950 has no block-scaled form.
 */
fp8l_status fp8_block_gemm_ue8m0(const uint8_t *xq, const uint8_t *xe, const uint8_t *wq, const uint8_t *we,
                                 int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

/*
 * Gated-MLP up projection with the SwiGLU activation in the GEMM epilogue
 * ("FP8 Quantization" (TensorRT-LLM), section "GEMM + SwiGLU Fusion in
 * Gated-MLP": the gate and up matmuls and the SwiGLU run as one kernel).  With
 * block scales every scale of both GEMMs is kept; the fused result differs
 * from two GEMMs and an elementwise pass only in skipping the bf16 rounding of
 * the gate and up sums.
 *
 *   xq [M,K], xs [M,K/128]          from fp8_quant_act
 *   wq [2I,K], ws [2I/128,K/128]    rows 0..I-1 the gate projection, I..2I-1 the
 *                                   up projection (nn.Linear weights stacked)
 *   h  [M,I] bf16                   h = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g)),
 *                                   g, u the fp32 block-scaled sums of fp8_block_gemm
 *                                   (NULL: not stored; then hq and hs are required)
 *   hq [M,I] e4m3, hs [M,I/128]     fp8_quant_act(h), the next layer's input
 *                                   (both NULL: not produced)
 * A caller that feeds only the next FP8 layer passes h = NULL and saves the
 * M * I * 2 bytes of bf16 output; hq and hs are the same as with h stored
 * (made from the same bf16-rounded values).  FP8L_ERR_NULL when h and hq are
 * both NULL, or exactly one of hq, hs is.
 * I must be a positive multiple of 128.  Prefill-sized M runs the fused
 * kernel (256-token tiles, SwiGLU and the quantization in the epilogue).
 * Where that grid would leave compute units idle (few tokens), the stacked
 * GEMM runs on smaller tiles and/or split K into fp32 partials held in library
 * scratch memory (S * M * 2I * 4 bytes), and one more kernel sums them and applies
 * SwiGLU and the quantization with the same arithmetic.
 */
fp8l_status fp8_block_gemm_swiglu(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                  int64_t M, int64_t I, int64_t K, uint16_t *h, uint8_t *hq, float *hs,
                                  hipStream_t stream);

/*
 * Decode-sized linear layer on bf16 activations: fp8_quant_act and
 * fp8_block_gemm in one kernel ("FP8 a granularite fine", intro bullets and
 * section "Chemin rapide de DeepGEMM": the activations are quantized per token
 * and group of 128 channels, dynamically, right before the block-scaled FP8
 * GEMM; "FP8 Quantization" (TensorRT-LLM), section "Low Latency GEMM Plugin":
 * small-batch FP8 GEMMs are latency-bound, and one launch less matters there).
 *
 *   x [M,K] bf16, M <= 64
 *   wq [N,K] e4m3, ws [N/128,K/128] fp32   from fp8_quant_weight_block
 *   y [M,N] bf16
 * y is bit-identical to fp8_quant_act(x) followed by fp8_block_gemm on the
 * resulting codes and scales.  One or two tokens (with the M x K codes fitting
 * in 36 KB of LDS, and K < 8192, where fp8_block_gemm streams the weight over
 * four waves) are quantized inside the weight-streaming kernel: every
 * workgroup quantizes the tokens into LDS and the codes are never written out.
 * Otherwise, where re-quantizing in every workgroup would cost more than it
 * saves, the call is those two calls, with the codes in library scratch memory.
 * M > 64 is FP8L_ERR_SHAPE: for a larger batch, quantize it once with
 * fp8_quant_act and call fp8_block_gemm.
 * Measured on MI355X (Llama-3-8B shapes, HIP graphs), one or two tokens save
 * 0.2-2.5 us per call against the two calls.
 */
fp8l_status fp8_block_linear(const uint16_t *x, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                             int64_t K, uint16_t *y, hipStream_t stream);

/*
 * The same fused decode-sized linear with a 2:4-compressed weight from
 * prune24_compress; bit-identical to fp8_quant_act then fp8_sparse24_gemm.
 * One or two tokens are quantized inside the kernel as above, except on K a
 * multiple of 512 from 4096 to 7680, where fp8_sparse24_gemm streams the
 * weight in whole-row four-block tiles faster than the in-kernel form: there
 * the call is the two calls.
 *
 *   x [M,K] bf16, M <= 64; wvals [N,K/2], wmeta [N,K/8], ws [N/128,K/128]; y [M,N] bf16
 */
fp8l_status fp8_sparse24_linear(const uint16_t *x, const uint8_t *wvals, const uint8_t *wmeta, const float *ws,
                                int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

/*
 * Frees the scratch memory the library keeps for calls made under stream
 * capture (on every device).  Call it only once no graph and no executable
 * graph that captured a library call exists, and no capture is in progress;
 * it synchronises the devices it frees memory on.  Returns FP8L_OK, or
 * FP8L_ERR_LAUNCH if the runtime refused a free.
 */
fp8l_status fp8lin_release_graph_scratch(void);

/* Static, never NULL, English text for a status code. */
const char *fp8lin_status_str(fp8l_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
