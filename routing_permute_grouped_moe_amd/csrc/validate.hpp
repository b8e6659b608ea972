// Host-side argument checks shared by the C-ABI entry points.  They run
// before any HIP call, so they can be exercised without a GPU.
#pragma once

#include <stdint.h>

#include "common.hpp"

#define MOE_MAX_E 1024

#define MOE_TRY(expr)            \
  do {                           \
    int _st = (expr);            \
    if (_st != MOE_OK) return _st; \
  } while (0)

static inline int moe_need_ptr(const void* p, const char* fn, const char* name, int align = 16) {
  if (p == nullptr) return moe_fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (((uintptr_t)p) % (uintptr_t)align != 0)
    return moe_fail(MOE_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", fn, name, align);
  return MOE_OK;
}

static inline int moe_opt_ptr(const void* p, const char* fn, const char* name, int align = 16) {
  return p == nullptr ? MOE_OK : moe_need_ptr(p, fn, name, align);
}

static inline int moe_need_dt(int dt, const char* fn) {
  if (dt != MOE_F32 && dt != MOE_BF16)
    return moe_fail(MOE_ERR_INVALID_ARG, "%s: dtype %d is neither MOE_F32 nor MOE_BF16", fn, dt);
  return MOE_OK;
}

static inline int moe_dt_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

static inline int moe_need_nonneg(long long v, const char* fn, const char* name) {
  if (v < 0) return moe_fail(MOE_ERR_INVALID_ARG, "%s: %s = %lld is negative", fn, name, v);
  return MOE_OK;
}

static inline int moe_need_mult64(long long v, const char* fn, const char* name) {
  if (v <= 0 || v % 64 != 0)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: %s = %lld must be a positive multiple of 64", fn,
                    name, v);
  return MOE_OK;
}

static inline int moe_need_ek(int E, int k, const char* fn) {
  if (E < 1 || E > MOE_MAX_E)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: E = %d outside [1, %d]", fn, E, MOE_MAX_E);
  if (k < 1 || k > E)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: k = %d outside [1, E=%d]", fn, k, E);
  return MOE_OK;
}

// Every tensor must have fewer than 2^31 elements and fewer than 2^32 bytes
// per buffer window (row offsets are 32-bit inside the kernels).
static inline int moe_need_elems(long long rows, long long cols, int bytes, const char* fn,
                                 const char* name) {
  long long n = rows * cols;
  if (n >= (1LL << 31) || n * bytes >= (1LL << 32))
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: %s has %lld x %lld elements, above the limit", fn,
                    name, rows, cols);
  return MOE_OK;
}
