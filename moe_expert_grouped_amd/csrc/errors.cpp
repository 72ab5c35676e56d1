// Thread-local error message of the C ABI.
#include "common.hpp"

namespace mi {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

mi_status launch_status(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("%s: HIP error %d (%s)", what, static_cast<int>(err), hipGetErrorString(err));
    return MI_EHIP;
  }
  return MI_OK;
}

}  // namespace mi

extern "C" const char* mi_last_error(void) { return mi::g_last_error.c_str(); }

extern "C" int mi_abi_version(void) { return 9; }
