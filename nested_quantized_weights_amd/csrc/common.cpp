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
