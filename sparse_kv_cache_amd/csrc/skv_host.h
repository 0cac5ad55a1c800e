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

// The token-level accumulator's first pass, for a kernel that folds the
// update pass into itself (h2o.hip; used by sparse_decode.hip).  out
// describes where the pass left its results in the caller's scratch.
struct H2oPass {
  const float* logits;      // [B, rows, bt_ld], base-2 scaled logits
  const float* part;        // [B, rows, nchunk, 2] chunk (max, sum)
  const uint16_t* snap;     // [B, H_kv, bt_ld] the accumulator before the step
  int nchunk, chunk;        // chunks per row, tokens per chunk
  float decay;              // the decay as applied (its bf16 value)
};
int h2o_logits_pass(const char* fn, bool per_head, const float* q, int B, int H_q, int H_kv,
                    int D, const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                    const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                    int reserved_bos, int reserved_eos, float scale, float decay,
                    uint16_t* hh_score, float* scratch, int64_t scratch_floats,
                    hipStream_t stream, H2oPass* out, const uint16_t* k_new = nullptr,
                    const uint16_t* v_new = nullptr, uint16_t* kv_w = nullptr);
// floats of scratch h2o_logits_pass needs (-1 on bad arguments)
int64_t h2o_pass_scratch_floats(int B, int rows, int H_kv, int64_t max_tokens);

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
