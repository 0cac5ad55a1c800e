// page_topk.hip -- per-row top-k selection with the reserved pages forced in,
// ties to the lower index, output ascending.
//
// Selection: EntmaxKV README "How it works" (keep topk_pages per query head;
// the budget counts pages and includes the always-attended tail page);
// vortex_torch pull request "flow: add H2O sparse attention", hardware
// follow-up (the reserved leading bos and trailing eos entries are kept and
// only the window between them is ranked).
//
// Method: skv_topk.h (one block per row).
#include "skv_device.h"
#include "skv_host.h"
#include "skv_topk.h"

namespace {

// EAGER: the block reads its whole stored row (score_ld entries) before the
// request's length arrives, so the key loads overlap that round trip; for a
// launch of few rows that latency is the cost that matters.  Otherwise only
// the N valid entries are read (ragged rows of a large batch would read up
// to twice the bytes).
template <int BLOCK, int ITEMS, bool EAGER>
__global__ __launch_bounds__(BLOCK) void page_topk_kernel(
    const float* __restrict__ scores, int64_t score_ld, int H_sel,
    const int32_t* __restrict__ seq_lens, int P, int topk_pages,
    double topk_frac, int bos, int eos, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_cnt, int k_cap, const int32_t* __restrict__ bt,
    int64_t bt_ld, int32_t* __restrict__ sel_blk) {
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / H_sel);
  const float* srow = scores + row * score_ld;
  const bool aligned = ((score_ld & 3) == 0) &&
                       ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
  uint32_t key[ITEMS];
  if constexpr (EAGER) skv::load_row_keys<ITEMS>(srow, aligned, score_ld, key);
  int64_t N64 = (static_cast<int64_t>(seq_lens[b]) + P - 1) / P;
  if (N64 > score_ld) N64 = score_ld;
  if (N64 < 0) N64 = 0;
  const int N = static_cast<int>(N64);
  const int32_t* btr = sel_blk != nullptr ? bt + static_cast<int64_t>(b) * bt_ld : nullptr;
  int32_t* bout = sel_blk != nullptr ? sel_blk + row * k_cap : nullptr;
  // 8-bit digits; the outputs go to global memory only, so no closing barrier
  int total;
  if constexpr (EAGER) {
    total = skv::topk_row_keys<BLOCK, ITEMS, 8, false>(key, N, topk_pages, topk_frac, bos,
                                                       eos, btr, bt_ld, sel_idx + row * k_cap,
                                                       bout, k_cap);
  } else {
    total = skv::topk_row<BLOCK, ITEMS, 8, false>(srow, aligned, N, topk_pages, topk_frac,
                                                  bos, eos, btr, bt_ld, sel_idx + row * k_cap,
                                                  bout, k_cap);
  }
  if (threadIdx.x == 0) sel_cnt[row] = total;
}

// Launches of up to this many rows take the wide-block mapping and read their
// rows eagerly; larger launches take 256-thread blocks and read only the
// valid entries.
constexpr int64_t kEagerRows = 1024;

template <int BLOCK, int ITEMS, bool EAGER>
void launch_topk(int64_t rows, hipStream_t stream, const float* scores,
                 int64_t score_ld, int H_sel, const int32_t* seq_lens, int P,
                 int topk_pages, double topk_frac, int bos, int eos,
                 int32_t* sel_idx, int32_t* sel_cnt, int k_cap, const int32_t* bt,
                 int64_t bt_ld, int32_t* sel_blk) {
  hipLaunchKernelGGL((page_topk_kernel<BLOCK, ITEMS, EAGER>), dim3(static_cast<unsigned>(rows)),
                     dim3(BLOCK), 0, stream, scores, score_ld, H_sel, seq_lens, P,
                     topk_pages, topk_frac, bos, eos, sel_idx, sel_cnt, k_cap, bt,
                     bt_ld, sel_blk);
}

}  // namespace

namespace {

// Validation and dispatch shared by page_topk and page_topk_blk.
int topk_impl(const char* who, const float* scores, int64_t score_ld, int B, int H_sel,
              const int32_t* seq_lens, int page_size, int topk_pages, float topk_frac,
              int reserved_bos, int reserved_eos, int32_t* sel_idx, int32_t* sel_cnt,
              int k_cap, const int32_t* block_table, int64_t bt_ld, int32_t* sel_blk,
              hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_sel > 0, "%s: need B >= 0 and H_sel > 0", who);
  SKV_REQUIRE(score_ld > 0 && score_ld <= 32768,
              "%s: score_ld must be in [1, 32768] (got %lld)", who, (long long)score_ld);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "%s: page_size must be 1, 2, 4, 8 or 16 (got %d)", who, page_size);
  SKV_REQUIRE(topk_pages >= 1, "%s: topk_pages must be >= 1 (got %d)", who,
              topk_pages);
  SKV_REQUIRE(topk_frac >= 0.0f && topk_frac <= 1.0f,
              "%s: topk_frac must be in [0, 1]", who);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", who);
  const double frac = static_cast<double>(topk_frac);
  int64_t need = topk_pages;
  const int64_t fk = static_cast<int64_t>(floor(frac * static_cast<double>(score_ld)));
  if (fk > need) need = fk;
  if (static_cast<int64_t>(reserved_bos) + reserved_eos > need)
    need = static_cast<int64_t>(reserved_bos) + reserved_eos;
  if (need > score_ld) need = score_ld;
  SKV_REQUIRE(k_cap >= need, "%s: k_cap %d < largest possible selection %lld", who,
              k_cap, (long long)need);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(who, scores);
  SKV_REQUIRE_PTR_W(who, seq_lens);
  SKV_REQUIRE_PTR_W(who, sel_idx);
  SKV_REQUIRE_PTR_W(who, sel_cnt);
  if (sel_blk != nullptr) {
    SKV_REQUIRE_PTR_W(who, block_table);
    SKV_REQUIRE(bt_ld > 0, "%s: bt_ld must be > 0 when sel_blk is given", who);
  }
  const int64_t rows = static_cast<int64_t>(B) * H_sel;
  SKV_REQUIRE(rows <= 0x7fffffff, "%s: too many rows", who);
#define SKV_TOPK(BL, IT, EA)                                                          \
  launch_topk<BL, IT, EA>(rows, stream, scores, score_ld, H_sel, seq_lens, page_size, \
                          topk_pages, frac, reserved_bos, reserved_eos, sel_idx,      \
                          sel_cnt, k_cap, block_table, bt_ld, sel_blk)
  if (rows <= kEagerRows) {
    // few rows, each latency-bound: the widest block that still gives each
    // thread at least 4 entries, so every pass is short
    if (score_ld <= 1024) SKV_TOPK(256, 4, true);
    else if (score_ld <= 2048) SKV_TOPK(512, 4, true);
    else if (score_ld <= 4096) SKV_TOPK(1024, 4, true);
    else if (score_ld <= 8192) SKV_TOPK(1024, 8, true);
    else if (score_ld <= 16384) SKV_TOPK(1024, 16, true);
    else SKV_TOPK(1024, 32, true);
  } else {
    // rows enough to fill the chip: 256-thread blocks, several per CU
    if (score_ld <= 1024) SKV_TOPK(256, 4, false);
    else if (score_ld <= 2048) SKV_TOPK(256, 8, false);
    else if (score_ld <= 4096) SKV_TOPK(256, 16, false);
    else if (score_ld <= 8192) SKV_TOPK(512, 16, false);
    else if (score_ld <= 16384) SKV_TOPK(1024, 16, false);
    else SKV_TOPK(1024, 32, false);
  }
#undef SKV_TOPK
  SKV_CHECK_LAUNCH_W(who);
}

}  // namespace

extern "C" int page_topk(const float* scores, int64_t score_ld, int B, int H_sel,
                         const int32_t* seq_lens, int page_size, int topk_pages,
                         float topk_frac, int reserved_bos, int reserved_eos,
                         int32_t* sel_idx, int32_t* sel_cnt, int k_cap,
                         hipStream_t stream) {
  return topk_impl("page_topk", scores, score_ld, B, H_sel, seq_lens, page_size,
                   topk_pages, topk_frac, reserved_bos, reserved_eos, sel_idx, sel_cnt,
                   k_cap, nullptr, 0, nullptr, stream);
}

extern "C" int page_topk_blk(const float* scores, int64_t score_ld, int B, int H_sel,
                             const int32_t* seq_lens, int page_size, int topk_pages,
                             float topk_frac, int reserved_bos, int reserved_eos,
                             int32_t* sel_idx, int32_t* sel_cnt, int k_cap,
                             const int32_t* block_table, int64_t bt_ld, int32_t* sel_blk,
                             hipStream_t stream) {
  return topk_impl("page_topk_blk", scores, score_ld, B, H_sel, seq_lens, page_size,
                   topk_pages, topk_frac, reserved_bos, reserved_eos, sel_idx, sel_cnt,
                   k_cap, block_table, bt_ld, sel_blk, stream);
}
