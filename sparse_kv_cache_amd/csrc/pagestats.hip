// pagestats.hip -- per-page key statistics (k_min, k_max, k_mean), either
// rebuilt for every page or refreshed for the tail page fused with the KV
// append of a decode step (and the reset of the written hh slot).
//
// Statistics: vortex_torch pull request "flow: add H2O sparse attention",
// "Page-level variants" (element-wise max / min envelope and mean of the keys
// of a page); EntmaxKV README "How it works" (statistics per page of the
// [2, num_blocks, page_size, H_kv, D] cache).  Append: EntmaxKV "Quick start"
// (the decode call appends k_new / v_new).  Reset: vortex_torch pull request,
// "Token-level variants" point 2 (a written slot's score is zeroed so a
// recycled page does not inherit it).
//
// Layout: one token row of a block is H_kv * D contiguous bf16 values, and
// the statistics of a block are [H_kv, D] contiguous, so a thread owns one
// 16-byte vector (8 values) of the row across all rows of the page: loads and
// stores are 16-byte and coalesced across threads.  min / max are taken on
// the exact bf16 values and stored back as bf16 (exact); the mean is an fp32
// sum divided by the valid row count.
#include "skv_device.h"
#include "skv_host.h"

namespace {

using skv::unpack8;

struct Stats8 {
  float mn[8], mx[8], sm[8];
  __device__ void init(const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) { mn[i] = x[i]; mx[i] = x[i]; sm[i] = x[i]; }
  }
  __device__ void add(const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn[i] = fminf(mn[i], x[i]);
      mx[i] = fmaxf(mx[i], x[i]);
      sm[i] += x[i];
    }
  }
  // min / max are bf16 values held exactly in fp32: their top 16 bits are
  // the bf16 pattern.
  __device__ void store(uint16_t* kmin, uint16_t* kmax, float* kmean,
                        int64_t off, int n) const {
    uint32_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = (__float_as_uint(mn[2 * i]) >> 16) |
             (__float_as_uint(mn[2 * i + 1]) & 0xffff0000u);
      b[i] = (__float_as_uint(mx[2 * i]) >> 16) |
             (__float_as_uint(mx[2 * i + 1]) & 0xffff0000u);
    }
    *reinterpret_cast<uint4*>(kmin + off) = make_uint4(a[0], a[1], a[2], a[3]);
    *reinterpret_cast<uint4*>(kmax + off) = make_uint4(b[0], b[1], b[2], b[3]);
    const float inv = 1.0f / static_cast<float>(n);
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = sm[i] * inv;
    float4* dst = reinterpret_cast<float4*>(kmean + off);
    dst[0] = make_float4(m[0], m[1], m[2], m[3]);
    dst[1] = make_float4(m[4], m[5], m[6], m[7]);
  }
};

// Rebuild: one block per (logical page, request); blocks past N_b exit.
__global__ __launch_bounds__(256) void pagestats_rebuild_kernel(
    const uint16_t* __restrict__ kv, int64_t num_blocks, int P, int row_vecs,
    uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
    float* __restrict__ kmean, const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens) {
  const int b = blockIdx.y;
  const int p = blockIdx.x;
  const int S = seq_lens[b];
  int64_t N = (static_cast<int64_t>(S) + P - 1) / P;
  if (N > bt_ld) N = bt_ld;
  if (p >= N) return;
  const int n = min(P, S - p * P);
  const int64_t blk = bt[static_cast<int64_t>(b) * bt_ld + p];
  const int64_t row_elems = static_cast<int64_t>(row_vecs) * 8;
  const uint16_t* page = kv + blk * P * row_elems;   // K half, block blk
  for (int v = threadIdx.x; v < row_vecs; v += blockDim.x) {
    float x[8];
    Stats8 st;
    unpack8(*reinterpret_cast<const uint4*>(page + v * 8), x);
    st.init(x);
    for (int t = 1; t < n; ++t) {
      unpack8(*reinterpret_cast<const uint4*>(page + t * row_elems + v * 8), x);
      st.add(x);
    }
    st.store(kmin, kmax, kmean, blk * row_elems + v * 8, n);
  }
}

// Append: one block per request.  Writes token S_b - 1, zeroes its hh slot,
// and recomputes the statistics of its page from the cached rows before it
// plus the new row (taken from the input, not re-read).
__global__ __launch_bounds__(256) void pagestats_append_kernel(
    uint16_t* __restrict__ kv, int64_t num_blocks, int P, int H_kv,
    int row_vecs, uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
    float* __restrict__ kmean, const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint16_t* __restrict__ hh) {
  const int b = blockIdx.x;
  const int pos = seq_lens[b] - 1;
  if (pos < 0) return;
  const int page = pos / P;
  if (page >= bt_ld) return;
  const int row = pos % P;
  const int64_t blk = bt[static_cast<int64_t>(b) * bt_ld + page];
  const int64_t row_elems = static_cast<int64_t>(row_vecs) * 8;
  uint16_t* kpage = kv + blk * P * row_elems;
  uint16_t* vpage = kv + (num_blocks + blk) * P * row_elems;
  const uint16_t* kn = k_new + static_cast<int64_t>(b) * row_elems;
  const uint16_t* vn = v_new + static_cast<int64_t>(b) * row_elems;
  for (int v = threadIdx.x; v < row_vecs; v += blockDim.x) {
    const uint4 kv4 = *reinterpret_cast<const uint4*>(kn + v * 8);
    const uint4 vv4 = *reinterpret_cast<const uint4*>(vn + v * 8);
    *reinterpret_cast<uint4*>(kpage + row * row_elems + v * 8) = kv4;
    *reinterpret_cast<uint4*>(vpage + row * row_elems + v * 8) = vv4;
    if (kmin != nullptr) {
      float x[8];
      Stats8 st;
      unpack8(kv4, x);
      st.init(x);
      for (int t = 0; t < row; ++t) {
        unpack8(*reinterpret_cast<const uint4*>(kpage + t * row_elems + v * 8), x);
        st.add(x);
      }
      st.store(kmin, kmax, kmean, blk * row_elems + v * 8, row + 1);
    }
  }
  if (hh != nullptr)
    for (int h = threadIdx.x; h < H_kv; h += blockDim.x) hh[(blk * P + row) * H_kv + h] = 0;
}

}  // namespace

extern "C" int pagestats_update(uint16_t* kv_cache, int64_t num_blocks,
                                int page_size, int H_kv, int D,
                                uint16_t* k_min, uint16_t* k_max, float* k_mean,
                                const int32_t* block_table, int64_t bt_ld,
                                const int32_t* seq_lens, int B,
                                const uint16_t* k_new, const uint16_t* v_new,
                                uint16_t* hh_score, hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && num_blocks > 0 && bt_ld > 0,
              "pagestats_update: need B >= 0, H_kv > 0, num_blocks > 0, bt_ld > 0");
  SKV_REQUIRE(D == 64 || D == 128, "pagestats_update: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "pagestats_update: page_size must be 1, 2, 4, 8 or 16 (got %d)", page_size);
  SKV_REQUIRE(bt_ld <= 0x7fffffff, "pagestats_update: bt_ld too large");
  const bool any_stats = k_min || k_max || k_mean;
  const bool all_stats = k_min && k_max && k_mean;
  SKV_REQUIRE(any_stats == all_stats,
              "pagestats_update: k_min, k_max, k_mean must be all given or all NULL");
  SKV_REQUIRE((k_new == nullptr) == (v_new == nullptr),
              "pagestats_update: k_new and v_new must be both given or both NULL");
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(kv_cache);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(seq_lens);
  const int row_vecs = H_kv * D / 8;
  const int threads = row_vecs >= 256 ? 256 : ((row_vecs + 63) / 64) * 64;
  if (k_new == nullptr) {
    SKV_REQUIRE(all_stats, "pagestats_update: rebuild mode needs the statistics buffers");
    dim3 grid(static_cast<unsigned>(bt_ld), static_cast<unsigned>(B));
    hipLaunchKernelGGL(pagestats_rebuild_kernel, grid, dim3(threads), 0, stream,
                       kv_cache, num_blocks, page_size, row_vecs, k_min, k_max,
                       k_mean, block_table, bt_ld, seq_lens);
  } else {
    hipLaunchKernelGGL(pagestats_append_kernel, dim3(B), dim3(threads), 0, stream,
                       kv_cache, num_blocks, page_size, H_kv, row_vecs, k_min,
                       k_max, k_mean, block_table, bt_ld, seq_lens, k_new, v_new,
                       hh_score);
  }
  SKV_CHECK_LAUNCH();
}
