// Status codes, per-thread error messages and the library version. Plain
// host C++ (no HIP), shared by every translation unit of the library.
#include <cstdarg>
#include <cstdio>

#include "pagedkv.h"
#include "status.h"

namespace pa {

namespace {
thread_local char g_msg[512] = "";
}  // namespace

pa_status fail(pa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace pa

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_OOM: return "out of free blocks";
    case PA_ERR_STATE: return "invalid allocator state (unknown or duplicate sequence)";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return pa::g_msg; }

int32_t pa_version(void) { return 1 * 10000 + 1 * 100 + 0; }

}  // extern "C"
