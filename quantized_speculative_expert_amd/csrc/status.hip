// Status codes and thread-local error text of the libsmoe C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "smoe_internal.hpp"

namespace smoe {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

smoe_status check_launch(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(err));
    return SMOE_EHIP;
  }
  return SMOE_OK;
}

}  // namespace smoe

extern "C" {

int smoe_abi_version(void) { return 4; }

const char* smoe_status_string(smoe_status status) {
  switch (status) {
    case SMOE_OK: return "SMOE_OK";
    case SMOE_EINVAL: return "SMOE_EINVAL: invalid argument";
    case SMOE_EUNSUPPORTED: return "SMOE_EUNSUPPORTED: outside the kernels' limits";
    case SMOE_EHIP: return "SMOE_EHIP: HIP launch error";
    default: return "unknown smoe_status";
  }
}

const char* smoe_last_error(void) { return smoe::g_last_error; }

}  // extern "C"
