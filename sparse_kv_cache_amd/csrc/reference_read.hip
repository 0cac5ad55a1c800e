// reference_read.hip -- bandwidth references (no method arithmetic): the
// streaming read of N bytes, and the read of a list of page-heads of the
// paged cache with the decode's load pattern and nothing else.
#include "skv_device.h"
#include "skv_host.h"
#include "../../include/skv_reference.h"

namespace {

constexpr uint32_t kNever = 0x5ca1ab1eu;
constexpr int kStreamBlocks = 1024;
constexpr int kStreamThreads = 512;
// many short waves, one page-head each: the read requests of waves that wait
// on their item and of waves that wait on data overlap across the CU, which
// keeps more of them in flight than fewer waves with deeper batches (256
// blocks with 4 page-heads per wave reached 4.0 TB/s at long_context where
// this reaches 4.7-5.1)
constexpr int kGatherBlocks = 4096;
constexpr int kGatherWaves = 4;
constexpr int kGatherDepth = 1;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(
    const uint4* __restrict__ p, int64_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kStreamThreads;
#pragma unroll 4
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kStreamThreads + threadIdx.x; i < n16;
       i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

// One wave per item; lane = (row slot, 16-byte piece of the row).  Items
// wave, wave + W, ... are taken kGatherDepth at a time, all loads first.
template <int D>
__global__ __launch_bounds__(kGatherWaves * 64) void gather_read_kernel(
    const uint16_t* __restrict__ kv, int64_t v_off, int H_kv,
    const int32_t* __restrict__ items, int64_t n, uint32_t* __restrict__ sink) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPL = 64 / LPR;       // rows per load
  constexpr int NL = 16 / RPL;        // loads per 16-row page
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int slot = lane / LPR, c = lane % LPR;
  const int64_t rs = static_cast<int64_t>(H_kv) * D;
  uint32_t acc = 0;
  for (int64_t it = wave; it < n; it += nwaves * kGatherDepth) {
    uint4 K[kGatherDepth][NL], V[kGatherDepth][NL];
#pragma unroll
    for (int d = 0; d < kGatherDepth; ++d) {
      int64_t j = it + d * nwaves;
      if (j >= n) j = it;
      const int blk = items[3 * j], h = items[3 * j + 1], nv = items[3 * j + 2];
      const uint16_t* base = kv + static_cast<int64_t>(blk) * 16 * rs + h * D + c * 8;
#pragma unroll
      for (int r = 0; r < NL; ++r) {
        const int t = slot + RPL * r;
        const int64_t off = (t < nv ? t : 0) * rs;
        K[d][r] = *reinterpret_cast<const uint4*>(base + off);
        V[d][r] = *reinterpret_cast<const uint4*>(base + v_off + off);
      }
    }
#pragma unroll
    for (int d = 0; d < kGatherDepth; ++d)
#pragma unroll
      for (int r = 0; r < NL; ++r)
        acc ^= K[d][r].x ^ K[d][r].y ^ K[d][r].z ^ K[d][r].w ^ V[d][r].x ^ V[d][r].y ^
               V[d][r].z ^ V[d][r].w;
  }
  // (the sink holds 256 words whatever the grid)
  if (acc == kNever) sink[blockIdx.x & 255u] = acc;
}

}  // namespace

extern "C" int skv_ref_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                                   hipStream_t stream) {
  SKV_REQUIRE(bytes > 0 && bytes % 16 == 0, "skv_ref_stream_read: bytes must be a positive "
              "multiple of 16 (got %lld)", (long long)bytes);
  SKV_REQUIRE_PTR(buf);
  SKV_REQUIRE_PTR(sink);
  SKV_REQUIRE((reinterpret_cast<uintptr_t>(buf) & 15) == 0,
              "skv_ref_stream_read: buf must be 16-byte aligned");
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  SKV_CHECK_LAUNCH();
}

extern "C" int skv_ref_gather_read(const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                                   int H_kv, int D, const int32_t* items, int64_t n,
                                   uint32_t* sink, hipStream_t stream) {
  SKV_REQUIRE(page_size == 16, "skv_ref_gather_read: page_size must be 16 (got %d)", page_size);
  SKV_REQUIRE(D == 64 || D == 128, "skv_ref_gather_read: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(num_blocks > 0 && H_kv > 0 && n >= 0,
              "skv_ref_gather_read: need num_blocks > 0, H_kv > 0, n >= 0");
  if (n == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(kv_cache);
  SKV_REQUIRE_PTR(items);
  SKV_REQUIRE_PTR(sink);
  const int64_t v_off = num_blocks * 16 * static_cast<int64_t>(H_kv) * D;
  const int64_t waves = (n + kGatherDepth - 1) / kGatherDepth;
  int64_t grid = (waves + kGatherWaves - 1) / kGatherWaves;
  if (grid > kGatherBlocks) grid = kGatherBlocks;
  if (D == 128)
    hipLaunchKernelGGL(gather_read_kernel<128>, dim3(static_cast<unsigned>(grid)),
                       dim3(kGatherWaves * 64), 0, stream, kv_cache, v_off, H_kv, items, n, sink);
  else
    hipLaunchKernelGGL(gather_read_kernel<64>, dim3(static_cast<unsigned>(grid)),
                       dim3(kGatherWaves * 64), 0, stream, kv_cache, v_off, H_kv, items, n, sink);
  SKV_CHECK_LAUNCH();
}
