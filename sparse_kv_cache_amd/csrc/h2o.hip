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
//      64-token chunks (16 waves per chunk, every head row read once with
//      16-byte loads, D/8 lanes per row); the chunk's (max, sum 2^(l - max))
//      per head go to scratch.
//   2. merge of the chunk partials into (M, Z) per head, then per token:
//      p = 2^(l - M) / Z, stored bf16(p), hh <- bf16(bf16(p) + decay * hh)
//      (one fp32 fma, then round-to-nearest-even), and the new hh value is
//      written as an fp32 score row in logical order for the selection.
// Scratch layout: logits [B, H_kv, bt_ld] then partials [B, H_kv, nchunk, 2].
#include "skv_device.h"
#include "skv_host.h"

namespace {

constexpr int kChunk = 64;      // tokens per block of the logits pass
constexpr int kLWaves = 16;     // waves per block of the logits pass
constexpr int kUpd = 64;        // tokens per block of the update pass

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

// Logits of one 64-token chunk of one request for every kv head.  The chunk's
// H_kv * 64 head rows are dealt to 16 waves, 4 * H_kv rows each; a wave issues
// all its 16-byte row loads (NLD per lane) before any arithmetic, masked rows
// reading a placeholder so the loads stay unconditional.
template <int D, int NLD>
__global__ __launch_bounds__(kLWaves * 64) void h2o_logits_kernel(
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
  int* sblk = reinterpret_cast<int*>(lg + H_kv * kChunk);   // [kChunk]
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  int ntok, lo, hi;
  window(seq_lens[b], bt_ld, bos, eos, &ntok, &lo, &hi);
  const int t0 = c * kChunk;
  if (t0 >= ntok) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, cc = lane % LPR;
  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;

  if (tid < kChunk) sblk[tid] = t0 + tid < ntok ? btr[t0 + tid] : 0;
  const float inv_g = 1.0f / static_cast<float>(G);
  for (int i = tid; i < H_kv * D; i += blockDim.x) {
    const int h = i / D, d = i % D;
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += q[(static_cast<int64_t>(b) * H_q + h * G + g) * D + d];
    qs[i] = s * inv_g * scale_log2;
  }
  __syncthreads();

  const int R = (kChunk / kLWaves) * H_kv;     // head rows of this wave
  uint4 kr[NLD];
  bool ok[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int rl = u * RPW + sub;
    const int r = wave * R + rl;
    const int tt = r / H_kv, h = r % H_kv;
    const int t = t0 + tt;
    ok[u] = rl < R && t >= lo && t < hi;
    const int64_t off = ok[u] ? (static_cast<int64_t>(sblk[ok[u] ? tt : 0]) * H_kv + h) * D + cc * 8
                              : cc * 8;
    kr[u] = *reinterpret_cast<const uint4*>(kv + off);
  }
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int rl = u * RPW + sub;
    const int r = wave * R + rl;
    const int tt = r / H_kv, h = r % H_kv;
    float x[8];
    skv::unpack8(kr[u], x);
    const float4 qa = *reinterpret_cast<const float4*>(qs + (rl < R ? h : 0) * D + cc * 8);
    const float4 qb = *reinterpret_cast<const float4*>(qs + (rl < R ? h : 0) * D + cc * 8 + 4);
    float dot = qa.x * x[0];
    dot = fmaf(qa.y, x[1], dot); dot = fmaf(qa.z, x[2], dot); dot = fmaf(qa.w, x[3], dot);
    dot = fmaf(qb.x, x[4], dot); dot = fmaf(qb.y, x[5], dot); dot = fmaf(qb.z, x[6], dot);
    dot = fmaf(qb.w, x[7], dot);
    dot = skv::group_sum<LPR>(dot);
    if (rl < R && cc == 0) lg[h * kChunk + tt] = ok[u] ? dot : -INFINITY;
  }
  __syncthreads();

  const int nt = min(kChunk, ntok - t0);
  for (int h = wave; h < H_kv; h += kLWaves) {
    const float v = lane < nt ? lg[h * kChunk + lane] : -INFINITY;
    const float m = skv::wave_max(v);
    float e = (m != -INFINITY && lane < nt) ? exp2f(v - m) : 0.0f;
    const float s = skv::wave_sum(e);
    if (lane < nt) logits[(static_cast<int64_t>(b) * H_kv + h) * bt_ld + t0 + lane] = v;
    if (lane == 0) {
      float* pp = part + ((static_cast<int64_t>(b) * H_kv + h) * nchunk + c) * 2;
      pp[0] = m;
      pp[1] = s;
    }
  }
}

// Normalise and fold into hh: block of 256 threads = 64 tokens x 4 head lanes.
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
  const int t = t0 + lane;
  if (t >= ntok) return;
  const int64_t slot = bt[static_cast<int64_t>(b) * bt_ld + t];
  const bool in_w = t >= lo && t < hi;
  for (int h = wave; h < H_kv; h += 4) {
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
  const size_t sm1 = sizeof(float) * (static_cast<size_t>(H_kv) * D +
                                      static_cast<size_t>(H_kv) * kChunk + kChunk);
  const float scale_log2 = scale * skv::kLog2e;
  // 16-byte row loads per lane: 4 * H_kv rows per wave over 64 / (D / 8) rows per load
  const int rpw = 64 / (D / 8);
  const int nld = (4 * H_kv + rpw - 1) / rpw;
#define SKV_LOGITS(DD, NN)                                                         \
  hipLaunchKernelGGL((h2o_logits_kernel<DD, NN>), grid, dim3(kLWaves * 64), sm1,   \
                     stream, q, H_q, H_kv, H_q / H_kv, kv_cache, block_table,      \
                     bt_ld, seq_lens, reserved_bos, reserved_eos, scale_log2,      \
                     logits, part, nch)
  if (D == 128) {
    if (nld <= 2) SKV_LOGITS(128, 2); else if (nld <= 4) SKV_LOGITS(128, 4);
    else if (nld <= 8) SKV_LOGITS(128, 8); else SKV_LOGITS(128, 16);
  } else {
    if (nld <= 2) SKV_LOGITS(64, 2); else if (nld <= 4) SKV_LOGITS(64, 4);
    else SKV_LOGITS(64, 8);
  }
#undef SKV_LOGITS
  const size_t sm2 = sizeof(float) * 2 * static_cast<size_t>(H_kv);
  hipLaunchKernelGGL(h2o_update_kernel, dim3(static_cast<unsigned>(nupd), static_cast<unsigned>(B)),
                     dim3(256), sm2, stream, H_kv,
                     block_table, bt_ld, seq_lens, reserved_bos, reserved_eos,
                     decay_b, hh_score, scores, score_ld, logits, part, nch);
  SKV_CHECK_LAUNCH();
}
