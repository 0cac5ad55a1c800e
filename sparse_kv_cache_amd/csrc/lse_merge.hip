// lse_merge.hip -- N-way log-sum-exp merge of split-K partial attention
// outputs.
//
// Algebra and edge cases: vllm.cpp test_ops_mla_chunked_context.cpp,
// MergeAttnStates test (partials weighted by exp(lse - max); a +inf lse is
// read as -inf; when every lse is -inf the first partial is emitted with lse
// -inf instead of 0/0).
//
// Mapping.  One wave per output row; each lane owns D/64 dims, so every split's
// partial row is one coalesced 256- or 512-byte read.
#include "skv_device.h"
#include "skv_host.h"

namespace {

template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    int rows, int ns, float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int VPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* L = lse_part + row * ns;
  const float* O = o_part + row * ns * D;
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) {
    float l = L[s];
    if (isinf(l)) l = -INFINITY;
    M = fmaxf(M, l);
  }
  M = skv::wave_max(M);
  float* dst = out + row * D + lane * VPL;
  if (M == -INFINITY) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) dst[j] = O[lane * VPL + j];
    if (lse_out != nullptr && lane == 0) lse_out[row] = -INFINITY;
    return;
  }
  float acc[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) acc[j] = 0.0f;
  float W = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float l = L[s];
    if (isinf(l)) continue;
    const float w = __expf(l - M);
    W += w;
#pragma unroll
    for (int j = 0; j < VPL; ++j) acc[j] = fmaf(w, O[s * D + lane * VPL + j], acc[j]);
  }
  const float inv = 1.0f / W;
#pragma unroll
  for (int j = 0; j < VPL; ++j) dst[j] = acc[j] * inv;
  if (lse_out != nullptr && lane == 0) lse_out[row] = M + __logf(W);
}

}  // namespace

extern "C" int lse_merge(const float* o_part, const float* lse_part, int rows,
                         int num_splits, int D, float* out, float* lse_out,
                         hipStream_t stream) {
  SKV_REQUIRE(rows >= 0, "lse_merge: rows must be >= 0");
  SKV_REQUIRE(num_splits >= 1, "lse_merge: num_splits must be >= 1 (got %d)", num_splits);
  SKV_REQUIRE(D == 64 || D == 128, "lse_merge: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE_PTR(o_part);
  SKV_REQUIRE_PTR(lse_part);
  SKV_REQUIRE_PTR(out);
  if (rows == 0) { skv::clear_error(); return SKV_OK; }
  dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (D == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(256), 0, stream, o_part,
                       lse_part, rows, num_splits, out, lse_out);
  else
    hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(256), 0, stream, o_part,
                       lse_part, rows, num_splits, out, lse_out);
  SKV_CHECK_LAUNCH();
}
