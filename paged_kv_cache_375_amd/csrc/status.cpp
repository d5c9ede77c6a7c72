// Status strings and the per-thread error detail of the C ABI.
#include <cstdio>

#include "internal.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace pa {

pa_status fail(pa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

pa_status ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_status_str(pa_status s) noexcept {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_UNKNOWN_SEQ: return "PA_ERR_UNKNOWN_SEQ";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_HOST_MEMORY: return "PA_ERR_HOST_MEMORY";
  }
  return "PA_ERR_UNKNOWN_STATUS";
}

extern "C" const char* pa_last_error(void) noexcept { return g_last_error; }
