// Status strings and the per-thread last-error message.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ra_internal.h"

namespace ra {
namespace {
thread_local char g_last_error[512] = "";
}

ra_status fail(ra_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

ra_status hip_check(hipError_t err, const char *what) {
  if (err == hipSuccess) return RA_OK;
  return fail(RA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(err), static_cast<int>(err));
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace ra

extern "C" const char *ra_status_str(int32_t status) {
  switch (status) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARG: return "RA_ERR_INVALID_ARG: invalid argument";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED: unsupported dtype or head dim";
    case RA_ERR_HIP: return "RA_ERR_HIP: a HIP runtime call failed";
    default: return "unknown ra_status";
  }
}

extern "C" const char *ra_last_error(void) { return ra::g_last_error; }
