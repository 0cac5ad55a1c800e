// lse_merge.hip -- N-way log-sum-exp merge of split-K partial attention
// outputs.
//
// Algebra and edge cases: vllm.cpp test_ops_mla_chunked_context.cpp,
// MergeAttnStates test (partials weighted by exp(lse - max); a +inf lse is
// read as -inf; when every lse is -inf the first partial is emitted with lse
// -inf instead of 0/0).
//
// Mapping.  One block per output row (see the kernels): up to 8 splits per
// thread are merged from registers after one round of loads, more in
// LDS-staged passes.
#include "skv_device.h"
#include "skv_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWChunk = 1024;          // split weights staged in LDS per pass

// One block per output row.  The block first reduces max(lse) over the
// splits, then stages the weights exp(lse_s - M) in LDS; threads are
// (split group g, dim d) pairs, so each split's partial row is one coalesced
// read and every thread keeps ns / (256 / D) independent loads in flight.
template <int D>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    int rows, int ns, float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int NGRP = kThreads / D;
  __shared__ float ws[kWChunk];
  __shared__ float red[kThreads / 64];
  __shared__ float accs[NGRP][D];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* L = lse_part + row * ns;
  const float* O = o_part + row * static_cast<int64_t>(ns) * D;

  float m = -INFINITY;
  for (int s = tid; s < ns; s += kThreads) {
    float l = L[s];
    if (isinf(l)) l = -INFINITY;
    m = fmaxf(m, l);
  }
  m = skv::wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  if (M == -INFINITY) {
    for (int d = tid; d < D; d += kThreads) out[row * D + d] = O[d];
    if (lse_out != nullptr && tid == 0) lse_out[row] = -INFINITY;
    return;
  }
  const int g = tid / D, d = tid % D;
  float acc = 0.0f, wsum = 0.0f;
  for (int c0 = 0; c0 < ns; c0 += kWChunk) {
    const int cend = min(ns, c0 + kWChunk);
    for (int s = c0 + tid; s < cend; s += kThreads) {
      const float l = L[s];
      const float w = isinf(l) ? 0.0f : __expf(l - M);
      ws[s - c0] = w;
      wsum += w;
    }
    __syncthreads();
#pragma unroll 8
    for (int s = c0 + g; s < cend; s += NGRP)
      acc = fmaf(ws[s - c0], O[static_cast<int64_t>(s) * D + d], acc);
    __syncthreads();
  }
  wsum = skv::wave_sum(wsum);
  if (lane == 0) red[wave] = wsum;
  accs[g][d] = acc;
  __syncthreads();
  if (tid < D) {
    float W = 0.0f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) W += red[w];
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < NGRP; ++k) a += accs[k][tid];
    out[row * D + tid] = a / W;
    if (lse_out != nullptr && tid == 0) lse_out[row] = M + __logf(W);
  }
}

// Up to K * (256 / D) splits (K <= 8): every thread loads its splits' partial values
// and lse values at once, so the block waits on memory once; the weights are
// formed in registers (the same splits, in the same order, as above).  The
// threads of split group g share g's weight sum; its d == 0 thread reports it.
template <int D, int K>
__global__ __launch_bounds__(kThreads) void lse_merge_small_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    int rows, int ns, float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int NGRP = kThreads / D;
  __shared__ float red[kThreads / 64];
  __shared__ float wg[NGRP];
  __shared__ float accs[NGRP][D];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = tid / D, d = tid % D;
  const float* L = lse_part + row * ns;
  const float* O = o_part + row * static_cast<int64_t>(ns) * D;
  float o[K], l[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = g + k * NGRP;
    o[k] = s < ns ? O[static_cast<int64_t>(s) * D + d] : 0.0f;
    const float v = s < ns ? L[s] : -INFINITY;
    l[k] = isinf(v) ? -INFINITY : v;
  }
  float m = l[0];
#pragma unroll
  for (int k = 1; k < K; ++k) m = fmaxf(m, l[k]);
  m = skv::wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red[w]);
  if (M == -INFINITY) {
    for (int i = tid; i < D; i += kThreads) out[row * D + i] = O[i];
    if (lse_out != nullptr && tid == 0) lse_out[row] = -INFINITY;
    return;
  }
  float acc = 0.0f, wsum = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float w = l[k] == -INFINITY ? 0.0f : __expf(l[k] - M);
    wsum += w;
    acc = fmaf(w, o[k], acc);
  }
  if (d == 0) wg[g] = wsum;
  accs[g][d] = acc;
  __syncthreads();
  if (tid < D) {
    float W = 0.0f, a = 0.0f;
#pragma unroll
    for (int k = 0; k < NGRP; ++k) { W += wg[k]; a += accs[k][tid]; }
    out[row * D + tid] = a / W;
    if (lse_out != nullptr && tid == 0) lse_out[row] = M + __logf(W);
  }
}

}  // namespace

extern "C" int lse_merge(const float* o_part, const float* lse_part, int rows,
                         int num_splits, int D, float* out, float* lse_out,
                         hipStream_t stream) {
  SKV_REQUIRE(rows >= 0, "lse_merge: rows must be >= 0");
  SKV_REQUIRE(num_splits >= 1, "lse_merge: num_splits must be >= 1 (got %d)", num_splits);
  SKV_REQUIRE(D == 64 || D == 128, "lse_merge: D must be 64 or 128 (got %d)", D);
  // no rows: nothing is read or written, so no pointer is needed
  if (rows == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(o_part);
  SKV_REQUIRE_PTR(lse_part);
  SKV_REQUIRE_PTR(out);
  dim3 grid(static_cast<unsigned>(rows));
  // up to 8 splits per thread: the register-resident form (faster for few
  // splits: 3.0 -> 2.5 us at 8 splits; with 32 per thread the lse loads it
  // repeats per thread made it slower, 3.5 -> 4.6 us at 64 splits)
  const int ngrp = kThreads / D;
  const int k_need = (num_splits + ngrp - 1) / ngrp;
#define SKV_SMALL(DD, KK)                                                              \
  hipLaunchKernelGGL((lse_merge_small_kernel<DD, KK>), grid, dim3(kThreads), 0, stream, \
                     o_part, lse_part, rows, num_splits, out, lse_out)
  if (k_need <= 8) {
    if (D == 128) {
      if (k_need <= 4) SKV_SMALL(128, 4); else SKV_SMALL(128, 8);
    } else {
      if (k_need <= 4) SKV_SMALL(64, 4); else SKV_SMALL(64, 8);
    }
  } else if (D == 128) {
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(kThreads), 0, stream, o_part,
                       lse_part, rows, num_splits, out, lse_out);
  } else {
    hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(kThreads), 0, stream, o_part,
                       lse_part, rows, num_splits, out, lse_out);
  }
#undef SKV_SMALL
  SKV_CHECK_LAUNCH();
}
