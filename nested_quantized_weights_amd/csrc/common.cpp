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
