// C entry points: host-side validation, then the launches on the caller's
// stream.  Validation order: shapes (M == 0 returns here), NULL pointers,
// alignment, aliasing, device; then the call's scratch memory, all of it
// before the first launch.  No call enqueues a kernel before every check has
// passed.
#include <atomic>
#include <cstring>

#include "../../include/fp8lin.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 = unknown, 1 = gfx950, 2 = other

struct Range {
  const void *p;
  int64_t bytes;
};

bool overlaps(const Range &a, const Range &b) {
  if (a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Every output range against every input range and every other output range.
bool any_alias(const Range *outs, int n_out, const Range *ins, int n_in) {
  for (int i = 0; i < n_out; i++) {
    for (int j = 0; j < n_in; j++)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; j++)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}

fp8l_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FP8L_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int known = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (known) return known == 1 ? FP8L_OK : FP8L_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return FP8L_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FP8L_OK : FP8L_ERR_DEVICE;
}

constexpr int64_t kMaxElems = int64_t(1) << 36;  // keeps every grid and index in range

bool bad_mk(int64_t M, int64_t K) {
  return M < 0 || K <= 0 || K % 128 != 0 || M > kMaxDim || K > kMaxDim || M * K > kMaxElems;
}
bool bad_nk(int64_t N, int64_t K) {
  return N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0 || N > kMaxDim || K > kMaxDim || N * K > kMaxElems;
}
bool bad_mn(int64_t M, int64_t N) { return M * N > kMaxElems; }

constexpr int64_t kMaxLinearM = 64;  // the fused-quantization calls are the decode form
constexpr int64_t kMaxGroups = 4096;   // experts of one grouped GEMM

fp8l_status launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? FP8L_ERR_MEMORY : FP8L_ERR_LAUNCH;
  }
  return FP8L_OK;
}

// Status of a call that held scratch memory: the launches' status first, then
// that of handing the scratch back (a one-off allocation's stream-ordered free).
fp8l_status finished(hipError_t e, fp8lin::CallScratch &sc) {
  const hipError_t f = sc.release();
  return launched(e != hipSuccess ? e : f);
}

}  // namespace

extern "C" {

fp8l_status fp8_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, hipStream_t stream) {
  if (bad_mk(M, K)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!x || !q || !s) return FP8L_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{x, M * K * 2}};
  const Range outs[] = {{q, M * K}, {s, M * (K / 128) * 4}};
  if (any_alias(outs, 2, ins, 1)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_quant_act(x, M, K, q, s, stream));
}

fp8l_status fp8_quant_act_tensor(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s,
                                 hipStream_t stream) {
  if (bad_mk(M, K)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!x || !q || !s) return FP8L_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{x, M * K * 2}};
  const Range outs[] = {{q, M * K}, {s, M * (K / 128) * 4}};
  if (any_alias(outs, 2, ins, 1)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_quant_tensor(x, M * K, q, s, M * (K / 128), stream));
}

fp8l_status fp8_quant_act_static(const uint16_t *x, const float *scale, int64_t M, int64_t K, uint8_t *q, float *s,
                                 hipStream_t stream) {
  if (bad_mk(M, K)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!x || !scale || !q || !s) return FP8L_ERR_NULL;
  if (!aligned16(x) || ((uintptr_t)scale & 3u) || !aligned16(q) || !aligned16(s)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{x, M * K * 2}, {scale, 4}};
  const Range outs[] = {{q, M * K}, {s, M * (K / 128) * 4}};
  if (any_alias(outs, 2, ins, 2)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_quant_static(x, scale, M * K, q, s, M * (K / 128), stream));
}

fp8l_status fp8_quant_weight_tensor(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                    hipStream_t stream) {
  if (bad_nk(N, K)) return FP8L_ERR_SHAPE;
  if (!w || !q || !s) return FP8L_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{w, N * K * 2}};
  const Range outs[] = {{q, N * K}, {s, (N / 128) * (K / 128) * 4}};
  if (any_alias(outs, 2, ins, 1)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_quant_tensor(w, N * K, q, s, (N / 128) * (K / 128), stream));
}

fp8l_status fp8_quant_weight_block(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                   hipStream_t stream) {
  if (bad_nk(N, K)) return FP8L_ERR_SHAPE;
  if (!w || !q || !s) return FP8L_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{w, N * K * 2}};
  const Range outs[] = {{q, N * K}, {s, (N / 128) * (K / 128) * 4}};
  if (any_alias(outs, 2, ins, 1)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_quant_wblock(w, N, K, q, s, stream));
}

fp8l_status prune24_compress(const uint16_t *w, const float *col_norm, int64_t N, int64_t K, uint8_t *vals,
                             uint8_t *meta, float *s, hipStream_t stream) {
  if (bad_nk(N, K)) return FP8L_ERR_SHAPE;
  if (!w || !vals || !meta || !s) return FP8L_ERR_NULL;
  if (!aligned16(w) || !aligned16(vals) || !aligned16(meta) || !aligned16(s) ||
      (col_norm && !aligned16(col_norm)))
    return FP8L_ERR_ALIGN;
  const Range ins[] = {{w, N * K * 2}, {col_norm, col_norm ? K * 4 : 0}};
  const Range outs[] = {{vals, N * K / 2}, {meta, N * K / 8}, {s, (N / 128) * (K / 128) * 4}};
  if (any_alias(outs, 3, ins, 2)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_prune24(w, col_norm, N, K, vals, meta, s, stream));
}

fp8l_status prune24_compress_tensor(const uint16_t *w, const float *col_norm, int64_t N, int64_t K, uint8_t *vals,
                                    uint8_t *meta, float *s, hipStream_t stream) {
  if (bad_nk(N, K)) return FP8L_ERR_SHAPE;
  if (!w || !vals || !meta || !s) return FP8L_ERR_NULL;
  if (!aligned16(w) || !aligned16(vals) || !aligned16(meta) || !aligned16(s) ||
      (col_norm && !aligned16(col_norm)))
    return FP8L_ERR_ALIGN;
  const Range ins[] = {{w, N * K * 2}, {col_norm, col_norm ? K * 4 : 0}};
  const Range outs[] = {{vals, N * K / 2}, {meta, N * K / 8}, {s, (N / 128) * (K / 128) * 4}};
  if (any_alias(outs, 3, ins, 2)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_prune24_tensor(w, col_norm, N, K, vals, meta, s, stream));
}

fp8l_status fp8_block_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M,
                           int64_t N, int64_t K, uint16_t *y, hipStream_t stream) {
  if (bad_mk(M, K) || bad_nk(N, K) || bad_mn(M, N)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!xq || !xs || !wq || !ws || !y) return FP8L_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(y)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{xq, M * K}, {xs, M * (K / 128) * 4}, {wq, N * K}, {ws, (N / 128) * (K / 128) * 4}};
  const Range outs[] = {{y, M * N * 2}};
  if (any_alias(outs, 1, ins, 4)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  fp8lin::CallScratch sc;
  if (hipError_t e = sc.acquire(fp8lin::gemm_partial_bytes(M, N, K, fp8lin::device_cu_count()), 0, stream))
    return launched(e);
  const hipError_t e = fp8lin::launch_dense_gemm(xq, xs, wq, ws, M, N, K, y, sc.partials(), stream);
  return finished(e, sc);
}

fp8l_status fp8_block_gemm_noalloc(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                   int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream) {
  if (bad_mk(M, K) || bad_nk(N, K) || bad_mn(M, N)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!xq || !xs || !wq || !ws || !y) return FP8L_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(y)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{xq, M * K}, {xs, M * (K / 128) * 4}, {wq, N * K}, {ws, (N / 128) * (K / 128) * 4}};
  const Range outs[] = {{y, M * N * 2}};
  if (any_alias(outs, 1, ins, 4)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  const size_t need = fp8lin::gemm_partial_bytes(M, N, K, fp8lin::device_cu_count());
  float *part = nullptr;
  if (need > 0) {
    // the device's copy of the fixed array (address looked up once per device)
    void *p = nullptr;
    size_t cap = 0;
    if (fp8lin::fixed_scratch(&p, &cap) != hipSuccess) {
      (void)hipGetLastError();
      return FP8L_ERR_DEVICE;
    }
    if (need > cap) return FP8L_ERR_SCRATCH;
    part = static_cast<float *>(p);
  }
  return launched(fp8lin::launch_dense_gemm(xq, xs, wq, ws, M, N, K, y, part, stream));
}

fp8l_status fp8_sparse24_gemm(const uint8_t *xq, const float *xs, const uint8_t *wvals, const uint8_t *wmeta,
                              const float *ws, int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream) {
  if (bad_mk(M, K) || bad_nk(N, K) || bad_mn(M, N)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!xq || !xs || !wvals || !wmeta || !ws || !y) return FP8L_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wvals) || !aligned16(wmeta) || !aligned16(ws) ||
      !aligned16(y))
    return FP8L_ERR_ALIGN;
  const Range ins[] = {{xq, M * K},        {xs, M * (K / 128) * 4}, {wvals, N * K / 2},
                       {wmeta, N * K / 8}, {ws, (N / 128) * (K / 128) * 4}};
  const Range outs[] = {{y, M * N * 2}};
  if (any_alias(outs, 1, ins, 5)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  fp8lin::CallScratch sc;
  if (hipError_t e = sc.acquire(fp8lin::gemm_partial_bytes(M, N, K, fp8lin::device_cu_count()), 0, stream))
    return launched(e);
  const hipError_t e = fp8lin::launch_sparse_gemm(xq, xs, wvals, wmeta, ws, M, N, K, y, sc.partials(), stream);
  return finished(e, sc);
}

fp8l_status fp8_quant_act_ue8m0(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *e, hipStream_t stream) {
  if (bad_mk(M, K)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!x || !q || !e) return FP8L_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(e)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{x, M * K * 2}};
  const Range outs[] = {{q, M * K}, {e, M * (K / 128)}};
  if (any_alias(outs, 2, ins, 1)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_quant_act_ue8m0(x, M, K, q, e, stream));
}

fp8l_status fp8_quant_weight_block_ue8m0(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, uint8_t *e,
                                         hipStream_t stream) {
  if (bad_nk(N, K)) return FP8L_ERR_SHAPE;
  if (!w || !q || !e) return FP8L_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(e)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{w, N * K * 2}};
  const Range outs[] = {{q, N * K}, {e, (N / 128) * (K / 128)}};
  if (any_alias(outs, 2, ins, 1)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_quant_wblock_ue8m0(w, N, K, q, e, stream));
}

fp8l_status fp8_block_gemm_ue8m0(const uint8_t *xq, const uint8_t *xe, const uint8_t *wq, const uint8_t *we,
                                 int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream) {
  if (bad_mk(M, K) || bad_nk(N, K) || bad_mn(M, N)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!xq || !xe || !wq || !we || !y) return FP8L_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xe) || !aligned16(wq) || !aligned16(we) || !aligned16(y)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{xq, M * K}, {xe, M * (K / 128)}, {wq, N * K}, {we, (N / 128) * (K / 128)}};
  const Range outs[] = {{y, M * N * 2}};
  if (any_alias(outs, 1, ins, 4)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  fp8lin::CallScratch sc;
  if (hipError_t e = sc.acquire(fp8lin::gemm_partial_bytes(M, N, K, fp8lin::device_cu_count()), 0, stream))
    return launched(e);
  const hipError_t e = fp8lin::launch_dense_gemm_ue8m0(xq, xe, wq, we, M, N, K, y, sc.partials(), stream);
  return finished(e, sc);
}

fp8l_status fp8_grouped_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                             const int32_t *offsets, int64_t G, int64_t M, int64_t N, int64_t K, uint16_t *y,
                             hipStream_t stream) {
  if (G <= 0 || G > kMaxGroups || bad_mk(M, K) || bad_nk(N, K) || bad_mn(M, N) || G * N * K > kMaxElems)
    return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!xq || !xs || !wq || !ws || !offsets || !y) return FP8L_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(offsets) || !aligned16(y))
    return FP8L_ERR_ALIGN;
  const Range ins[] = {{xq, M * K},
                       {xs, M * (K / 128) * 4},
                       {wq, G * N * K},
                       {ws, G * (N / 128) * (K / 128) * 4},
                       {offsets, (G + 1) * 4}};
  const Range outs[] = {{y, M * N * 2}};
  if (any_alias(outs, 1, ins, 5)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  return launched(fp8lin::launch_dense_grouped_gemm(xq, xs, wq, ws, offsets, G, M, N, K, y, stream));
}

fp8l_status fp8_block_gemm_swiglu(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M,
                                  int64_t I, int64_t K, uint16_t *h, uint8_t *hq, float *hs, hipStream_t stream) {
  if (I <= 0 || I % 128 != 0 || bad_mk(M, K) || bad_nk(2 * I, K) || bad_mn(M, I)) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!xq || !xs || !wq || !ws || (!hq != !hs) || (!h && !hq)) return FP8L_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || (h && !aligned16(h)) ||
      (hq && (!aligned16(hq) || !aligned16(hs))))
    return FP8L_ERR_ALIGN;
  const Range ins[] = {{xq, M * K}, {xs, M * (K / 128) * 4}, {wq, 2 * I * K}, {ws, (2 * I / 128) * (K / 128) * 4}};
  const Range outs[] = {{h, h ? M * I * 2 : 0}, {hq, hq ? M * I : 0}, {hs, hs ? M * (I / 128) * 4 : 0}};
  if (any_alias(outs, 3, ins, 4)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  fp8lin::CallScratch sc;
  if (hipError_t e = sc.acquire(fp8lin::swiglu_partial_bytes(M, I, K, fp8lin::device_cu_count()), 0, stream))
    return launched(e);
  const hipError_t e = fp8lin::launch_dense_gemm_swiglu(xq, xs, wq, ws, M, I, K, h, hq, hs, sc.partials(), stream);
  return finished(e, sc);
}

fp8l_status fp8_block_linear(const uint16_t *x, const uint8_t *wq, const float *ws, int64_t M, int64_t N, int64_t K,
                             uint16_t *y, hipStream_t stream) {
  if (bad_mk(M, K) || bad_nk(N, K) || bad_mn(M, N) || M > kMaxLinearM) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!x || !wq || !ws || !y) return FP8L_ERR_NULL;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(ws) || !aligned16(y)) return FP8L_ERR_ALIGN;
  const Range ins[] = {{x, M * K * 2}, {wq, N * K}, {ws, (N / 128) * (K / 128) * 4}};
  const Range outs[] = {{y, M * N * 2}};
  if (any_alias(outs, 1, ins, 3)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  fp8lin::CallScratch sc;
  const size_t tokens = fp8lin::linear_token_bytes(M, N, K, false);
  if (hipError_t e = sc.acquire(fp8lin::gemm_partial_bytes(M, N, K, fp8lin::device_cu_count()), tokens, stream))
    return launched(e);
  const hipError_t e = fp8lin::launch_dense_linear(x, wq, ws, M, N, K, y, sc.tokens(), sc.partials(), stream);
  return finished(e, sc);
}

fp8l_status fp8_sparse24_linear(const uint16_t *x, const uint8_t *wvals, const uint8_t *wmeta, const float *ws,
                                int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream) {
  if (bad_mk(M, K) || bad_nk(N, K) || bad_mn(M, N) || M > kMaxLinearM) return FP8L_ERR_SHAPE;
  if (M == 0) return FP8L_OK;
  if (!x || !wvals || !wmeta || !ws || !y) return FP8L_ERR_NULL;
  if (!aligned16(x) || !aligned16(wvals) || !aligned16(wmeta) || !aligned16(ws) || !aligned16(y))
    return FP8L_ERR_ALIGN;
  const Range ins[] = {{x, M * K * 2}, {wvals, N * K / 2}, {wmeta, N * K / 8}, {ws, (N / 128) * (K / 128) * 4}};
  const Range outs[] = {{y, M * N * 2}};
  if (any_alias(outs, 1, ins, 4)) return FP8L_ERR_ALIAS;
  if (fp8l_status st = check_device()) return st;
  fp8lin::CallScratch sc;
  const size_t tokens = fp8lin::linear_token_bytes(M, N, K, true);
  if (hipError_t e = sc.acquire(fp8lin::gemm_partial_bytes(M, N, K, fp8lin::device_cu_count()), tokens, stream))
    return launched(e);
  const hipError_t e = fp8lin::launch_sparse_linear(x, wvals, wmeta, ws, M, N, K, y, sc.tokens(), sc.partials(),
                                                    stream);
  return finished(e, sc);
}

fp8l_status fp8lin_release_graph_scratch(void) {
  const hipError_t e = fp8lin::release_graph_scratch();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return FP8L_ERR_LAUNCH;
  }
  return FP8L_OK;
}

const char *fp8lin_status_str(fp8l_status status) {
  switch (status) {
    case FP8L_OK: return "ok";
    case FP8L_ERR_NULL: return "a required pointer is NULL";
    case FP8L_ERR_SHAPE:
      return "unsupported shape (K and N must be positive multiples of 128, M >= 0, each <= 2^24; M <= 64 for the "
             "*_linear calls)";
    case FP8L_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FP8L_ERR_ALIAS: return "an output overlaps an input or another output";
    case FP8L_ERR_DEVICE: return "no gfx950 (MI355X) device is current";
    case FP8L_ERR_LAUNCH: return "kernel launch failed";
    case FP8L_ERR_MEMORY: return "scratch memory for the call could not be allocated";
    case FP8L_ERR_SCRATCH: return "the call needs more scratch memory than the library's fixed array holds";
    default: return "unknown status";
  }
}

}  // extern "C"
