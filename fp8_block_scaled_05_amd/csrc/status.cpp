#include "status.hpp"

#include <cstdarg>
#include <cstdio>
#include <hip/hip_runtime_api.h>

namespace {
thread_local char g_last_error[512] = "";
}

namespace fp8bs {

fp8bs_status fail(fp8bs_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void begin_launch() { (void)hipGetLastError(); }

fp8bs_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FP8BS_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return FP8BS_OK;
}

}  // namespace fp8bs

extern "C" const char* fp8bs_last_error(void) { return g_last_error; }

extern "C" const char* fp8bs_version(void) { return "fp8bs 0.1.0 gfx950"; }
