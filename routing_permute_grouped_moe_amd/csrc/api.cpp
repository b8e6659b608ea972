// Host side of the C ABI: status text, last-error detail, launch checks and
// the per-device compute-unit count used to size persistent grids.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.hpp"

#define MOE_ABI_VERSION 11

static thread_local char g_last_error[512];

int moe_fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int moe_check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return moe_fail(MOE_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

int moe_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

int moe_abi_version(void) { return MOE_ABI_VERSION; }

}  // extern "C"
