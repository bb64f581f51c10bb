// Scratch memory of the GEMM calls: split-K fp32 partials and tokens quantized
// inside a fused linear call.
//
// A stream-ordered allocation per call costs about 10 us on MI355X, host side
// when eager and as graph memory nodes when captured, which is as much as a
// whole decode-sized GEMM.  So the library keeps the memory between calls:
//
//   * eager calls: one buffer per (device, stream, slot), taken from a
//     library-owned pool on that stream.  Calls on one stream run in stream
//     order, so they can share it; when a call needs more, the old buffer is
//     freed on the same stream (after the work that uses it) and a larger one
//     allocated;
//   * calls under stream capture: one buffer per (device, stream, capture,
//     slot), allocated outside the graph and kept until the process ends,
//     because the graph (and every executable made from it) holds its address.
//     A replayed graph therefore never shares scratch with eager work or with
//     another graph.  Beyond 1 GiB of such buffers, or if the allocation fails,
//     the call falls back to an allocation inside the graph.
//
// Two slots per stream, so that one call can hold quantized tokens and split-K
// partials at once.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "launch.hpp"

namespace fp8lin {
namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kRound = size_t(1) << 20;            // buffer sizes in whole MiB
constexpr size_t kCaptureLimit = size_t(1) << 30;     // bytes kept for captured graphs
constexpr size_t kMaxEagerBuffers = 512;              // (device, stream, slot) entries

struct Buffer {
  void *p = nullptr;
  size_t bytes = 0;
};

std::mutex g_mu;
hipMemPool_t g_pools[kMaxDevices] = {};
std::map<std::tuple<int, hipStream_t, int>, Buffer> g_eager;
std::map<std::tuple<int, hipStream_t, unsigned long long, int>, Buffer> g_captured;
std::vector<void *> g_outgrown;  // captured buffers replaced by larger ones; graphs may still use them
size_t g_captured_bytes = 0;

// One pool per device that keeps up to 256 MB cached between calls (the
// default pool hands memory back to the driver at every synchronisation).
hipError_t pool_locked(int dev, hipMemPool_t *out) {
  if (!g_pools[dev]) {
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    hipError_t e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = uint64_t(256) << 20;
    if ((e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pools[dev] = pool;
  }
  *out = g_pools[dev];
  return hipSuccess;
}

size_t rounded(size_t bytes) { return (bytes + kRound - 1) / kRound * kRound; }

// Stream-ordered allocation released by workspace_release (inside a graph when
// the stream is capturing).
hipError_t transient_locked(int dev, Workspace *w, size_t bytes, hipStream_t stream) {
  hipMemPool_t pool;
  const hipError_t e = pool_locked(dev, &pool);
  if (e != hipSuccess) return e;
  w->transient = true;
  w->stream = stream;
  return hipMallocFromPoolAsync(&w->p, bytes, pool, stream);
}

hipError_t eager_locked(int dev, Workspace *w, int slot, size_t bytes, hipStream_t stream) {
  const auto key = std::make_tuple(dev, stream, slot);
  auto it = g_eager.find(key);
  if (it != g_eager.end() && it->second.bytes >= bytes) {
    w->p = it->second.p;
    return hipSuccess;
  }
  if (it == g_eager.end() && g_eager.size() >= kMaxEagerBuffers) return transient_locked(dev, w, bytes, stream);
  hipMemPool_t pool;
  hipError_t e = pool_locked(dev, &pool);
  if (e != hipSuccess) return e;
  if (it != g_eager.end()) {
    // earlier calls on this stream may still use it: free in stream order
    e = hipFreeAsync(it->second.p, stream);
    g_eager.erase(it);
    if (e != hipSuccess) return e;
  }
  Buffer b;
  b.bytes = rounded(bytes);
  if ((e = hipMallocFromPoolAsync(&b.p, b.bytes, pool, stream)) != hipSuccess) return e;
  g_eager[key] = b;
  w->p = b.p;
  return hipSuccess;
}

hipError_t captured_locked(int dev, Workspace *w, int slot, size_t bytes, hipStream_t stream,
                           unsigned long long capture) {
  const auto key = std::make_tuple(dev, stream, capture, slot);
  auto it = g_captured.find(key);
  if (it != g_captured.end() && it->second.bytes >= bytes) {
    w->p = it->second.p;
    return hipSuccess;
  }
  const size_t want = rounded(bytes);
  if (g_captured_bytes + want > kCaptureLimit) return transient_locked(dev, w, bytes, stream);
  // an ordinary allocation, outside the graph: the capture mode of this thread
  // is relaxed for the call so that the capture in progress stays valid
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  hipError_t e = hipThreadExchangeStreamCaptureMode(&mode);
  if (e != hipSuccess) return e;
  void *p = nullptr;
  const hipError_t m = hipMalloc(&p, want);
  e = hipThreadExchangeStreamCaptureMode(&mode);
  if (m != hipSuccess) {
    (void)hipGetLastError();  // not left for the next launch check to report
    return e != hipSuccess ? e : transient_locked(dev, w, bytes, stream);
  }
  if (e != hipSuccess) return e;
  if (it != g_captured.end()) g_outgrown.push_back(it->second.p);
  g_captured[key] = Buffer{p, want};
  g_captured_bytes += want;
  w->p = p;
  return hipSuccess;
}

}  // namespace

hipError_t workspace_acquire(Workspace *w, WorkspaceSlot slot, size_t bytes, hipStream_t stream) {
  *w = Workspace{};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
  unsigned long long capture = 0;
  if ((e = hipStreamGetCaptureInfo(stream, &status, &capture)) != hipSuccess) return e;
  if (status == hipStreamCaptureStatusInvalidated) return hipErrorStreamCaptureInvalidated;
  std::lock_guard<std::mutex> lock(g_mu);
  if (status == hipStreamCaptureStatusActive) return captured_locked(dev, w, (int)slot, bytes, stream, capture);
  return eager_locked(dev, w, (int)slot, bytes, stream);
}

hipError_t workspace_release(Workspace *w) {
  if (!w->transient || !w->p) return hipSuccess;
  const hipError_t e = hipFreeAsync(w->p, w->stream);
  *w = Workspace{};
  return e;
}

}  // namespace fp8lin
