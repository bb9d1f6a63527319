// ABI version, status names and the per-thread error message.
#include <stdarg.h>
#include <stdio.h>

#include "pf_internal.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace pf {

pf_status fail(pf_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return st;
}

pf_status ok() {
  g_msg[0] = '\0';
  return PF_OK;
}

pf_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PF_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace pf

extern "C" {

int pf_abi_version(void) { return PF_ABI_VERSION; }

const char* pf_status_name(int status) {
  switch (status) {
    case PF_OK: return "PF_OK";
    case PF_ERR_NULL: return "PF_ERR_NULL";
    case PF_ERR_SHAPE: return "PF_ERR_SHAPE";
    case PF_ERR_UNSUPPORTED: return "PF_ERR_UNSUPPORTED";
    case PF_ERR_MISALIGNED: return "PF_ERR_MISALIGNED";
    case PF_ERR_RANGE: return "PF_ERR_RANGE";
    case PF_ERR_WORKSPACE: return "PF_ERR_WORKSPACE";
    case PF_ERR_HIP: return "PF_ERR_HIP";
    default: return "PF_UNKNOWN";
  }
}

const char* pf_last_error_message(void) { return g_msg; }

}  // extern "C"
