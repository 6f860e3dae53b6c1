// Status strings, per-thread error messages and launch checks of libdsa.
#include <stdarg.h>
#include <stdio.h>

#include "dsa_common.h"

namespace dsa {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

dsa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: HIP launch failed: %s", what, hipGetErrorString(e));
    return DSA_ERR_HIP;
  }
  return DSA_OK;
}

}  // namespace dsa

extern "C" const char* dsa_status_str(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape not supported";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP runtime error";
    default: return "unknown dsa_status";
  }
}

extern "C" const char* dsa_last_error(void) { return dsa::g_last_error; }

extern "C" int dsa_abi_version(void) { return DSA_ABI_VERSION; }
