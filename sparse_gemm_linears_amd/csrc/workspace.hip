// Scratch memory of the GEMM calls: split-K fp32 partials and tokens quantized
// inside a fused linear call.
//
// A stream-ordered allocation per call costs about 10 us on MI355X, host side
// when eager and as graph memory nodes when captured, which is as much as a
// whole decode-sized GEMM.  So the library keeps the memory between calls:
//
//   * eager calls: one buffer per (device, stream, slot), taken from a
//     library-owned pool on that stream.  Calls on one stream run in stream
//     order, so they can share it; when a call needs more, the larger buffer
//     is allocated first and the old one then freed on the same stream (after
//     the work that uses it).  hipStreamPerThread is one handle value that
//     names a different stream in every thread, so its buffers are also keyed
//     by the calling thread;
//   * calls under stream capture: one buffer per (device, stream, capture,
//     slot), allocated outside the graph and kept, because the graph (and every
//     executable made from it) holds its address.  A replayed graph therefore
//     never shares scratch with eager work or with another graph.  At most
//     1 GiB is kept that way in all (outgrown buffers included); past it, or if
//     the allocation fails, the call allocates inside the graph instead.
//     release_graph_scratch() frees what is kept once the caller has destroyed
//     every graph that holds it.
//
// A call holds the scratch lock from acquire() to release(): its launches go
// out under it, so calls on one stream from several host threads enqueue their
// kernels and the frees of outgrown buffers in the order they took the lock.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <thread>
#include <tuple>
#include <vector>

#include "launch.hpp"

namespace fp8lin {
namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kRound = size_t(1) << 20;            // buffer sizes in whole MiB
constexpr size_t kCaptureLimit = size_t(1) << 30;     // bytes kept for captured graphs
constexpr size_t kMaxEagerBuffers = 512;              // (device, stream, thread, slot) entries

struct Buffer {
  void *p = nullptr;
  size_t bytes = 0;
};

// The thread part of a stream's key: only hipStreamPerThread depends on the
// calling thread (every other handle names one stream for all threads).
std::thread::id stream_thread(hipStream_t stream) {
  return stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
}

std::mutex g_mu;
hipMemPool_t g_pools[kMaxDevices] = {};
std::map<std::tuple<int, hipStream_t, std::thread::id, int>, Buffer> g_eager;
std::map<std::tuple<int, hipStream_t, unsigned long long, int>, Buffer> g_captured;
std::vector<std::pair<int, void *>> g_outgrown;  // captured buffers replaced by larger ones (graphs hold them)
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

// What one slot of a call resolved to: an existing buffer (nothing to do), a
// new kept buffer (entry to record, an old one to free or keep), or a one-off
// allocation freed when the call releases it.
struct Pending {
  void *p = nullptr;
  bool fresh = false, transient = false, captured = false;
  size_t bytes = 0;
  void *old = nullptr;  // the buffer a fresh one replaces
};

hipError_t transient_locked(int dev, size_t bytes, hipStream_t stream, Pending *out) {
  hipMemPool_t pool;
  const hipError_t e = pool_locked(dev, &pool);
  if (e != hipSuccess) return e;
  out->transient = true;
  return hipMallocFromPoolAsync(&out->p, bytes, pool, stream);
}

hipError_t eager_locked(int dev, int slot, size_t bytes, hipStream_t stream, Pending *out) {
  const auto key = std::make_tuple(dev, stream, stream_thread(stream), slot);
  auto it = g_eager.find(key);
  if (it != g_eager.end() && it->second.bytes >= bytes) {
    out->p = it->second.p;
    return hipSuccess;
  }
  if (it == g_eager.end() && g_eager.size() >= kMaxEagerBuffers) return transient_locked(dev, bytes, stream, out);
  hipMemPool_t pool;
  const hipError_t e = pool_locked(dev, &pool);
  if (e != hipSuccess) return e;
  out->bytes = rounded(bytes);
  out->fresh = true;
  out->old = it != g_eager.end() ? it->second.p : nullptr;
  return hipMallocFromPoolAsync(&out->p, out->bytes, pool, stream);
}

hipError_t captured_locked(int dev, int slot, size_t bytes, hipStream_t stream, unsigned long long capture,
                           Pending *out) {
  const auto key = std::make_tuple(dev, stream, capture, slot);
  auto it = g_captured.find(key);
  if (it != g_captured.end() && it->second.bytes >= bytes) {
    out->p = it->second.p;
    return hipSuccess;
  }
  const size_t want = rounded(bytes);
  if (g_captured_bytes + want > kCaptureLimit) return transient_locked(dev, bytes, stream, out);
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
    return e != hipSuccess ? e : transient_locked(dev, bytes, stream, out);
  }
  if (e != hipSuccess) {
    (void)hipFree(p);
    return e;
  }
  out->p = p;
  out->bytes = want;
  out->fresh = true;
  out->captured = true;
  out->old = it != g_captured.end() ? it->second.p : nullptr;
  return hipSuccess;
}

// Undo the allocations of a failed acquisition (nothing of them was used).
void discard_locked(Pending *pend, int n, hipStream_t stream) {
  for (int i = 0; i < n; i++) {
    if (!pend[i].p || (!pend[i].fresh && !pend[i].transient)) continue;
    if (pend[i].captured) {
      hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
      if (hipThreadExchangeStreamCaptureMode(&mode) == hipSuccess) {
        (void)hipFree(pend[i].p);
        (void)hipThreadExchangeStreamCaptureMode(&mode);
      }
    } else {
      (void)hipFreeAsync(pend[i].p, stream);
    }
  }
  (void)hipGetLastError();
}

}  // namespace

hipError_t CallScratch::acquire(size_t partial_bytes, size_t token_bytes, hipStream_t stream) {
  const size_t need[2] = {partial_bytes, token_bytes};
  if (need[0] == 0 && need[1] == 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
  unsigned long long capture = 0;
  if ((e = hipStreamGetCaptureInfo(stream, &status, &capture)) != hipSuccess) return e;
  if (status == hipStreamCaptureStatusInvalidated) return hipErrorStreamCaptureInvalidated;
  g_mu.lock();
  locked_ = true;
  stream_ = stream;
  // every slot is resolved (and any new buffer allocated) before anything is
  // recorded or freed, so that a failure leaves the kept buffers as they were
  Pending pend[2];
  for (int slot = 0; slot < 2; slot++) {
    if (need[slot] == 0) continue;
    e = status == hipStreamCaptureStatusActive ? captured_locked(dev, slot, need[slot], stream, capture, &pend[slot])
                                                : eager_locked(dev, slot, need[slot], stream, &pend[slot]);
    if (e != hipSuccess) {
      discard_locked(pend, slot + 1, stream);
      locked_ = false;
      g_mu.unlock();
      return e;
    }
  }
  for (int slot = 0; slot < 2; slot++) {
    Pending &pd = pend[slot];
    p_[slot] = pd.p;
    transient_[slot] = pd.transient;
    if (!pd.fresh) continue;
    if (pd.captured) {
      if (pd.old) g_outgrown.emplace_back(dev, pd.old);
      g_captured[std::make_tuple(dev, stream, capture, slot)] = Buffer{pd.p, pd.bytes};
      g_captured_bytes += pd.bytes;
    } else {
      // earlier calls on this stream may still use the old buffer: freed in
      // stream order, after their work
      if (pd.old) (void)hipFreeAsync(pd.old, stream);
      g_eager[std::make_tuple(dev, stream, stream_thread(stream), slot)] = Buffer{pd.p, pd.bytes};
    }
  }
  return hipSuccess;
}

hipError_t CallScratch::release() {
  hipError_t e = hipSuccess;
  for (int slot = 0; slot < 2; slot++) {
    if (transient_[slot] && p_[slot]) {
      const hipError_t f = hipFreeAsync(p_[slot], stream_);
      if (e == hipSuccess) e = f;
    }
    p_[slot] = nullptr;
    transient_[slot] = false;
  }
  if (locked_) {
    locked_ = false;
    g_mu.unlock();
  }
  return e;
}

hipError_t release_graph_scratch() {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_captured.empty() && g_outgrown.empty()) return hipSuccess;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  std::vector<std::pair<int, void *>> all(g_outgrown);
  for (const auto &kv : g_captured) all.emplace_back(std::get<0>(kv.first), kv.second.p);
  for (const auto &b : all) {
    hipError_t f = hipSetDevice(b.first);
    if (f == hipSuccess) f = hipFree(b.second);
    if (e == hipSuccess) e = f;
  }
  const hipError_t f = hipSetDevice(cur);
  if (e == hipSuccess) e = f;
  g_outgrown.clear();
  g_captured.clear();
  g_captured_bytes = 0;
  return e;
}

}  // namespace fp8lin
