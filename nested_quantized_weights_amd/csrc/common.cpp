// Error state of the C ABI.
#include "common.h"

namespace nest {

std::string& last_error() {
  static thread_local std::string msg;
  return msg;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  last_error() = buf;
  return code;
}

int ok() {
  last_error().clear();
  return NEST_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(NEST_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace nest

extern "C" const char* nest_last_error(void) { return nest::last_error().c_str(); }

#include <map>
#include <mutex>
#include <utility>

namespace nest {

namespace {
std::mutex g_occ_mu;
}

int resident_blocks(const void* kernel, int threads, size_t dyn_lds) {
  static std::map<std::pair<const void*, size_t>, int> cache;
  static int cus = 0;
  std::lock_guard<std::mutex> lk(g_occ_mu);
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  const auto key = std::make_pair(kernel, dyn_lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn_lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int n = per_cu * cus;
  cache[key] = n;
  return n;
}

}  // namespace nest

#include <thread>

namespace nest {

namespace {
std::mutex g_counter_mu;

// A stream's identity for per-stream library state. The per-thread default
// stream is one handle for every host thread but a different stream in each,
// so it is told apart by the calling thread.
using StreamKey = std::pair<hipStream_t, std::thread::id>;
StreamKey stream_key(hipStream_t stream) {
  return {stream, stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
}
}

unsigned* stream_counter(hipStream_t stream) {
  // One zeroed word per (device, stream). Kernels on one stream run one
  // after another, and a kernel that counts its blocks with it leaves it at
  // zero when it ends, so two running kernels never share one.
  static std::map<std::pair<int, StreamKey>, unsigned*> slots;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_counter_mu);
  const auto key = std::make_pair(dev, stream_key(stream));
  auto it = slots.find(key);
  if (it != slots.end()) return it->second;
  void* p = nullptr;
  if (hipMalloc(&p, 256) != hipSuccess) return nullptr;
  if (hipMemset(p, 0, 256) != hipSuccess) {
    (void)hipFree(p);
    return nullptr;
  }
  slots[key] = static_cast<unsigned*>(p);
  return static_cast<unsigned*>(p);
}

}  // namespace nest

namespace nest {

namespace {
std::mutex g_scratch_mu;
}

void* stream_scratch(hipStream_t stream, size_t bytes) {
  // One buffer per (device, stream), grown on demand and kept until the
  // process ends. Calls on one stream run in order, so each call's use of
  // it ends before the next call's begins; before a smaller buffer is
  // replaced, the stream is drained (work queued on it may still read it).
  static std::map<std::pair<int, StreamKey>, std::pair<void*, size_t>> bufs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto& e = bufs[std::make_pair(dev, stream_key(stream))];
  if (e.first && e.second >= bytes) return e.first;
  if (e.first) {
    if (hipStreamSynchronize(stream) != hipSuccess) return nullptr;
    (void)hipFree(e.first);
    e = {nullptr, 0};
  }
  size_t n = bytes < (size_t{1} << 20) ? (size_t{1} << 20) : bytes;
  void* p = nullptr;
  if (hipMalloc(&p, n) != hipSuccess) return nullptr;
  e = {p, n};
  return p;
}

}  // namespace nest
