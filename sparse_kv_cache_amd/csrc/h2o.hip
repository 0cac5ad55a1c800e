// h2o.hip -- token-level heavy-hitter (H2O) accumulator step, page_size 1.
//
// vortex_torch pull request "flow: add H2O sparse attention",
// "Token-level variants": the accumulated quantity is the softmax attention
// probability over the request's scored tokens (scale D^-0.5 by default), the
// accumulator decays (0.984375 = 1 - 2^-6, exact in bf16) and is stored in
// bf16; the hardware follow-up's reference step: the softmax covers only the
// window [bos, S - eos); for a query group the group-mean query is used.
//
// Two launches over (token chunk, request):
//   1. logits l_t = scale * log2(e) * qbar . k_t for every kv head over
//      64-token chunks, one token row of H_kv * D bf16 read with 16-byte loads
//      (D/8 lanes per head row); the chunk's (max, sum 2^(l - max)) per head go
//      to scratch.
//   2. merge of the chunk partials into (M, Z) per head, then per token:
//      p = 2^(l - M) / Z, stored bf16(p), hh <- bf16(bf16(p) + decay * hh)
//      (one fp32 fma, then round-to-nearest-even), and the new hh value is
//      written as an fp32 score row in logical order for the selection.
// Scratch layout: logits [B, H_kv, bt_ld] then partials [B, H_kv, nchunk, 2].
#include "skv_device.h"
#include "skv_host.h"

namespace {

constexpr int kChunk = 64;      // tokens per block of the logits pass
constexpr int kUpd = 256;       // tokens per block of the update pass
constexpr int kUnroll = 8;      // row loads in flight per lane

__device__ __forceinline__ void window(int S, int64_t bt_ld, int bos, int eos,
                                       int* ntok, int* lo, int* hi) {
  int n = S;
  if (n > bt_ld) n = static_cast<int>(bt_ld);
  if (n < 0) n = 0;
  int l = bos < n ? bos : n;
  int h = n - eos > 0 ? n - eos : 0;
  if (h < l) h = l;
  *ntok = n; *lo = l; *hi = h;
}

template <int D>
__global__ __launch_bounds__(256) void h2o_logits_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ bt,
    int64_t bt_ld, const int32_t* __restrict__ seq_lens, int bos, int eos,
    float scale_log2, float* __restrict__ logits, float* __restrict__ part,
    int nchunk) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;                // head rows per wave load
  extern __shared__ float smem[];
  float* qs = smem;                            // [H_kv][D]
  float* lg = smem + H_kv * D;                 // [H_kv][kChunk]
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  int ntok, lo, hi;
  window(seq_lens[b], bt_ld, bos, eos, &ntok, &lo, &hi);
  const int t0 = c * kChunk;
  if (t0 >= ntok) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, cc = lane % LPR;

  const float inv_g = 1.0f / static_cast<float>(G);
  for (int i = tid; i < H_kv * D; i += blockDim.x) {
    const int h = i / D, d = i % D;
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += q[(static_cast<int64_t>(b) * H_q + h * G + g) * D + d];
    qs[i] = s * inv_g * scale_log2;
  }
  __syncthreads();

  const int rows = kChunk * H_kv;
  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;
  const int step = 4 * RPW;                    // rows per block load
  for (int r0 = wave * RPW; r0 < rows; r0 += step * kUnroll) {
    uint4 kr[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int r = r0 + u * step + sub;
      const int t = t0 + r / H_kv;
      ok[u] = r < rows && t >= lo && t < hi;
      if (ok[u]) {
        const int64_t blk = btr[t];
        kr[u] = *reinterpret_cast<const uint4*>(
            kv + (blk * H_kv + (r % H_kv)) * D + cc * 8);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int r = r0 + u * step + sub;
      const int h = r % H_kv;
      float x[8];
      skv::unpack8(kr[u], x);
      const float* qq = qs + h * D + cc * 8;
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(qq[i], x[i], dot);
      dot = skv::group_sum<LPR>(dot);
      if (r < rows && cc == 0) lg[h * kChunk + r / H_kv] = ok[u] ? dot : -INFINITY;
    }
  }
  __syncthreads();

  const int nt = min(kChunk, ntok - t0);
  for (int h = wave; h < H_kv; h += 4) {
    const float* row = lg + h * kChunk;
    float m = -INFINITY;
    for (int j = lane; j < nt; j += 64) m = fmaxf(m, row[j]);
    m = skv::wave_max(m);
    float s = 0.0f;
    if (m != -INFINITY)
      for (int j = lane; j < nt; j += 64) s += exp2f(row[j] - m);
    s = skv::wave_sum(s);
    float* dst = logits + (static_cast<int64_t>(b) * H_kv + h) * bt_ld + t0;
    for (int j = lane; j < nt; j += 64) dst[j] = row[j];
    if (lane == 0) {
      float* pp = part + ((static_cast<int64_t>(b) * H_kv + h) * nchunk + c) * 2;
      pp[0] = m;
      pp[1] = s;
    }
  }
}

__global__ __launch_bounds__(256) void h2o_update_kernel(
    int H_kv, const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens, int bos, int eos, float decay,
    uint16_t* __restrict__ hh, float* __restrict__ scores, int64_t score_ld,
    const float* __restrict__ logits, const float* __restrict__ part,
    int nchunk) {
  extern __shared__ float smem[];
  float* sM = smem;              // [H_kv]
  float* sZ = smem + H_kv;       // [H_kv]
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  int ntok, lo, hi;
  window(seq_lens[b], bt_ld, bos, eos, &ntok, &lo, &hi);
  const int t0 = c * kUpd;
  if (t0 >= ntok) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nch_b = (ntok + kChunk - 1) / kChunk;
  for (int h = wave; h < H_kv; h += 4) {
    const float* pp = part + (static_cast<int64_t>(b) * H_kv + h) * nchunk * 2;
    float m = -INFINITY;
    for (int j = lane; j < nch_b; j += 64) m = fmaxf(m, pp[2 * j]);
    m = skv::wave_max(m);
    float z = 0.0f;
    if (m != -INFINITY)
      for (int j = lane; j < nch_b; j += 64)
        if (pp[2 * j] != -INFINITY) z += pp[2 * j + 1] * exp2f(pp[2 * j] - m);
    z = skv::wave_sum(z);
    if (lane == 0) { sM[h] = m; sZ[h] = z; }
  }
  __syncthreads();
  const int t = t0 + tid;
  if (t >= ntok) return;
  const int64_t slot = bt[static_cast<int64_t>(b) * bt_ld + t];
  const bool in_w = t >= lo && t < hi;
  for (int h = 0; h < H_kv; ++h) {
    uint16_t* cell = hh + slot * H_kv + h;
    float v = skv::bf16_to_f32(*cell);
    if (in_w) {
      const float l = logits[(static_cast<int64_t>(b) * H_kv + h) * bt_ld + t];
      const float p = exp2f(l - sM[h]) / sZ[h];
      const float pb = skv::bf16_to_f32(skv::f32_to_bf16(p));
      const uint16_t nb = skv::f32_to_bf16(fmaf(decay, v, pb));
      *cell = nb;
      v = skv::bf16_to_f32(nb);
    }
    scores[(static_cast<int64_t>(b) * H_kv + h) * score_ld + t] = v;
  }
}

int64_t nchunks(int64_t max_tokens) { return (max_tokens + kChunk - 1) / kChunk; }

}  // namespace

extern "C" int64_t h2o_scratch_floats(int B, int H_kv, int64_t max_tokens) {
  if (B < 0 || H_kv <= 0 || max_tokens <= 0) return -1;
  const int64_t rows = static_cast<int64_t>(B) * H_kv;
  return rows * max_tokens + rows * nchunks(max_tokens) * 2;
}

extern "C" int h2o_accumulate(const float* q, int B, int H_q, int H_kv, int D,
                              const uint16_t* kv_cache, int64_t num_blocks,
                              int page_size, const int32_t* block_table,
                              int64_t bt_ld, const int32_t* seq_lens,
                              int reserved_bos, int reserved_eos, float scale,
                              float decay, uint16_t* hh_score, float* scores,
                              int64_t score_ld, float* scratch,
                              int64_t scratch_floats, hipStream_t stream) {
  SKV_REQUIRE(page_size == 1, "h2o_accumulate: page_size must be 1 (got %d)", page_size);
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "h2o_accumulate: need H_q a positive multiple of H_kv");
  SKV_REQUIRE(H_q / H_kv <= 16, "h2o_accumulate: group size > 16");
  SKV_REQUIRE(D == 64 || D == 128, "h2o_accumulate: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(H_kv <= 16, "h2o_accumulate: H_kv must be <= 16");
  SKV_REQUIRE(num_blocks > 0 && bt_ld > 0 && score_ld >= bt_ld,
              "h2o_accumulate: need num_blocks > 0, bt_ld > 0, score_ld >= bt_ld");
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "h2o_accumulate: reserved_bos / reserved_eos must be >= 0");
  SKV_REQUIRE(decay > 0.0f && decay <= 1.0f, "h2o_accumulate: decay must lie in (0, 1]");
  SKV_REQUIRE(scale > 0.0f, "h2o_accumulate: scale must be > 0");
  SKV_REQUIRE(B <= 65535 && nchunks(bt_ld) <= 0x7fffffff, "h2o_accumulate: grid too large");
  SKV_REQUIRE_PTR(q);
  SKV_REQUIRE_PTR(kv_cache);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(seq_lens);
  SKV_REQUIRE_PTR(hh_score);
  SKV_REQUIRE_PTR(scores);
  SKV_REQUIRE_PTR(scratch);
  const int64_t need = h2o_scratch_floats(B, H_kv, bt_ld);
  SKV_REQUIRE(scratch_floats >= need, "h2o_accumulate: scratch has %lld floats, needs %lld",
              (long long)scratch_floats, (long long)need);
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  const int nch = static_cast<int>(nchunks(bt_ld));
  const int nupd = static_cast<int>((bt_ld + kUpd - 1) / kUpd);
  float* logits = scratch;
  float* part = scratch + static_cast<int64_t>(B) * H_kv * bt_ld;
  // decay is applied as its bf16 value, which is exact for 0.984375
  const float decay_b = skv_host_round_bf16(decay);
  dim3 grid(static_cast<unsigned>(nch), static_cast<unsigned>(B));
  const size_t sm1 = sizeof(float) * (static_cast<size_t>(H_kv) * D + static_cast<size_t>(H_kv) * kChunk);
  const float scale_log2 = scale * skv::kLog2e;
  if (D == 128)
    hipLaunchKernelGGL(h2o_logits_kernel<128>, grid, dim3(256), sm1, stream, q, H_q,
                       H_kv, H_q / H_kv, kv_cache, block_table, bt_ld, seq_lens,
                       reserved_bos, reserved_eos, scale_log2, logits, part, nch);
  else
    hipLaunchKernelGGL(h2o_logits_kernel<64>, grid, dim3(256), sm1, stream, q, H_q,
                       H_kv, H_q / H_kv, kv_cache, block_table, bt_ld, seq_lens,
                       reserved_bos, reserved_eos, scale_log2, logits, part, nch);
  const size_t sm2 = sizeof(float) * 2 * static_cast<size_t>(H_kv);
  hipLaunchKernelGGL(h2o_update_kernel, dim3(static_cast<unsigned>(nupd), static_cast<unsigned>(B)),
                     dim3(kUpd), sm2, stream, H_kv,
                     block_table, bt_ld, seq_lens, reserved_bos, reserved_eos,
                     decay_b, hh_score, scores, score_ld, logits, part, nch);
  SKV_CHECK_LAUNCH();
}
