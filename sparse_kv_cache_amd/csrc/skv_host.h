// skv_host.h -- host-side argument checking and error reporting shared by the
// entry points of libsparsekv.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/sparsekv.h"

namespace skv {

void set_error(const char* fmt, ...);
void clear_error();

}  // namespace skv

// Reject a bad scalar before anything is enqueued.
#define SKV_REQUIRE(cond, ...)                 \
  do {                                         \
    if (!(cond)) {                             \
      skv::set_error(__VA_ARGS__);             \
      return SKV_EINVAL;                       \
    }                                          \
  } while (0)

// Reject a NULL pointer that the call needs.
#define SKV_REQUIRE_PTR(p)                                   \
  do {                                                       \
    if ((p) == nullptr) {                                    \
      skv::set_error("%s: %s must not be NULL", __func__, #p); \
      return SKV_EFAULT;                                     \
    }                                                        \
  } while (0)

// The same check for a helper shared by several entry points: `who` names
// the entry point the caller used.
#define SKV_REQUIRE_PTR_W(who, p)                             \
  do {                                                       \
    if ((p) == nullptr) {                                    \
      skv::set_error("%s: %s must not be NULL", (who), #p);  \
      return SKV_EFAULT;                                     \
    }                                                        \
  } while (0)

// Report a failed launch (or success) and return from the entry point.
#define SKV_CHECK_LAUNCH() SKV_CHECK_LAUNCH_W(__func__)

// The same for a helper shared by several entry points.
#define SKV_CHECK_LAUNCH_W(who)                                         \
  do {                                                                  \
    hipError_t e_ = hipGetLastError();                                  \
    if (e_ != hipSuccess) {                                             \
      skv::set_error("%s: launch failed: %s", (who),                    \
                     hipGetErrorString(e_));                            \
      return SKV_EIO;                                                   \
    }                                                                   \
    skv::clear_error();                                                 \
    return SKV_OK;                                                      \
  } while (0)

// Round a float to the nearest bf16 value (ties to even), on the host.
static inline float skv_host_round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  float r;
  memcpy(&r, &u, sizeof r);
  return r;
}

static inline bool skv_supported_page_size(int p) {
  return p == 1 || p == 2 || p == 4 || p == 8 || p == 16;
}
