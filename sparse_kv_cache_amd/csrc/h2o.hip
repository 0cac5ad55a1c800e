// h2o.hip -- token-level heavy-hitter (H2O) accumulator step, page_size 1.
//
// vortex_torch pull request "flow: add H2O sparse attention",
// "Token-level variants": the accumulated quantity is the softmax attention
// probability over the request's scored tokens (scale D^-0.5 by default), the
// accumulator decays (0.984375 = 1 - 2^-6, exact in bf16) and is stored in
// bf16; the hardware follow-up's reference step: the softmax covers only the
// window [bos, S - eos).  A query group is served in one of two readings:
// the group-mean query (the follow-up's reference step), or every query head's
// own softmax averaged over the group (the GQA flows keep the query-group axis
// through the product and the softmax).
//
// Two launches over (token chunk, request):
//   1. logits l_t = scale * log2(e) * q_r . k_t over 64-token chunks for every
//      logit row r: one per kv head (q_r = the group-mean query) or one per
//      query head (its own query).  16 waves per chunk, every kv-head row read
//      once with 16-byte loads, D/8 lanes per row, dotted with each of the
//      head's logit-row queries; the chunk's (max, sum 2^(l - max)) per logit
//      row go to scratch.
//   2. merge of the chunk partials into (M, Z) per logit row, then per token
//      and kv head: p = 2^(l - M) / Z (per-head reading: the mean of that over
//      the group's rows), hh <- bf16(bf16(p) + decay * hh) (one fp32 fma, then
//      round-to-nearest-even), and the new hh value is written as an fp32
//      score row in logical order for the selection.
// Scratch layout: logits [B, R, bt_ld] then partials [B, R, nchunk, 2], with
// R = H_kv logit rows per request (group mean) or H_q (per head).
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

// Logits of one 64-token chunk of one request for every logit row.  The
// chunk's H_kv * 64 kv-head rows are dealt to 16 waves, 4 * H_kv rows each; a
// wave issues all its 16-byte row loads (NLD per lane) before any arithmetic,
// masked rows reading a placeholder so the loads stay unconditional.  PH: GR =
// G logit rows per kv head (the group's own queries), else GR = 1 (the mean).
// HM (H_kv divides 16): the rows are dealt head-major, so every row of a wave
// belongs to one kv head and each lane reads that head's query slices from
// LDS once per four logit rows, not once per key row.
template <int D, int NLD, bool PH, bool HM>
__global__ __launch_bounds__(kLWaves * 64) void h2o_logits_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ bt,
    int64_t bt_ld, const int32_t* __restrict__ seq_lens, int bos, int eos,
    float scale_log2, float* __restrict__ logits, float* __restrict__ part,
    int nchunk) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;                // head rows per wave load
  const int GR = PH ? G : 1;                   // logit rows per kv head
  const int HR = H_kv * GR;                    // logit rows per request
  extern __shared__ float smem[];
  float* qs = smem;                            // [HR][D]
  float* lg = smem + HR * D;                   // [HR][kChunk]
  int* sblk = reinterpret_cast<int*>(lg + HR * kChunk);     // [kChunk]
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
  if constexpr (PH) {
    for (int i = tid; i < H_q * D; i += blockDim.x)
      qs[i] = q[static_cast<int64_t>(b) * H_q * D + i] * scale_log2;
  } else {
    const float inv_g = 1.0f / static_cast<float>(G);
    for (int i = tid; i < H_kv * D; i += blockDim.x) {
      const int h = i / D, d = i % D;
      float s = 0.0f;
      for (int g = 0; g < G; ++g) s += q[(static_cast<int64_t>(b) * H_q + h * G + g) * D + d];
      qs[i] = s * inv_g * scale_log2;
    }
  }
  __syncthreads();

  const int R = (kChunk / kLWaves) * H_kv;     // kv-head rows of this wave
  // row rl of this wave: token tt of the chunk, kv head h
  auto row_of = [&](int rl, int& tt, int& h) {
    const int r = wave * R + rl;
    if constexpr (HM) { h = r / kChunk; tt = r % kChunk; }
    else { tt = r / H_kv; h = r % H_kv; }
  };
  uint4 kr[NLD];
  bool ok[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int rl = u * RPW + sub;
    int tt, h;
    row_of(rl, tt, h);
    const int t = t0 + tt;
    ok[u] = rl < R && t >= lo && t < hi;
    const int64_t off = ok[u] ? (static_cast<int64_t>(sblk[ok[u] ? tt : 0]) * H_kv + h) * D + cc * 8
                              : cc * 8;
    kr[u] = *reinterpret_cast<const uint4*>(kv + off);
  }
  auto dot8 = [](const float* qr, const float (&x)[8]) {
    const float4 qa = *reinterpret_cast<const float4*>(qr);
    const float4 qb = *reinterpret_cast<const float4*>(qr + 4);
    float dot = qa.x * x[0];
    dot = fmaf(qa.y, x[1], dot); dot = fmaf(qa.z, x[2], dot); dot = fmaf(qa.w, x[3], dot);
    dot = fmaf(qb.x, x[4], dot); dot = fmaf(qb.y, x[5], dot); dot = fmaf(qb.z, x[6], dot);
    return fmaf(qb.w, x[7], dot);
  };
  if constexpr (HM) {
    // the wave's kv head; four of its logit rows' query slices in registers
    const int hw = (wave * R) / kChunk;
    for (int g0 = 0; g0 < GR; g0 += 4) {
      float qv[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = g0 + j < GR ? g0 + j : GR - 1;
        const float* qr = qs + (hw * GR + g) * D + cc * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[j][i] = qr[i];
      }
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const int rl = u * RPW + sub;
        int tt, h;
        row_of(rl, tt, h);
        float x[8];
        skv::unpack8(kr[u], x);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (g0 + j >= GR) break;
          float dot = qv[j][0] * x[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) dot = fmaf(qv[j][i], x[i], dot);
          dot = skv::group_sum<LPR>(dot);
          if (rl < R && cc == 0) lg[(hw * GR + g0 + j) * kChunk + tt] = ok[u] ? dot : -INFINITY;
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int rl = u * RPW + sub;
      int tt, h;
      row_of(rl, tt, h);
      float x[8];
      skv::unpack8(kr[u], x);
      for (int gi = 0; gi < GR; ++gi) {
        float dot = dot8(qs + (rl < R ? h * GR + gi : 0) * D + cc * 8, x);
        dot = skv::group_sum<LPR>(dot);
        if (rl < R && cc == 0) lg[(h * GR + gi) * kChunk + tt] = ok[u] ? dot : -INFINITY;
      }
    }
  }
  __syncthreads();

  const int nt = min(kChunk, ntok - t0);
  for (int h = wave; h < HR; h += kLWaves) {
    const float v = lane < nt ? lg[h * kChunk + lane] : -INFINITY;
    const float m = skv::wave_max(v);
    float e = (m != -INFINITY && lane < nt) ? exp2f(v - m) : 0.0f;
    const float s = skv::wave_sum(e);
    if (lane < nt) logits[(static_cast<int64_t>(b) * HR + h) * bt_ld + t0 + lane] = v;
    if (lane == 0) {
      float* pp = part + ((static_cast<int64_t>(b) * HR + h) * nchunk + c) * 2;
      pp[0] = m;
      pp[1] = s;
    }
  }
}

// (m, z) <- the pair describing both sets: z is a sum of 2^(l - m) terms.
__device__ __forceinline__ void fold_max_sum(float& m, float& z, float m2, float z2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; z = z2; return; }
  const float M = fmaxf(m, m2);
  z = z * exp2f(m - M) + z2 * exp2f(m2 - M);
  m = M;
}

// Normalise and fold into hh: block of 256 threads = 64 tokens x 4 head lanes.
// PH: the kv head's p is the mean over its G logit rows' probabilities.
template <bool PH>
__global__ __launch_bounds__(256) void h2o_update_kernel(
    int H_kv, int G, const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens, int bos, int eos, float decay,
    uint16_t* __restrict__ hh, float* __restrict__ scores, int64_t score_ld,
    const float* __restrict__ logits, const float* __restrict__ part,
    int nchunk) {
  const int GR = PH ? G : 1;
  const int HR = H_kv * GR;
  extern __shared__ float smem[];
  float* sM = smem;              // [HR]
  float* sZ = smem + HR;         // [HR]
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  int ntok, lo, hi;
  window(seq_lens[b], bt_ld, bos, eos, &ntok, &lo, &hi);
  const int t0 = c * kUpd;
  if (t0 >= ntok) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nch_b = (ntok + kChunk - 1) / kChunk;
  // Token-side loads first (this lane's token: its slot, then the hh cell and
  // up to kPre logits of each of the wave's kv heads): they do not depend on
  // the (M, Z) merge below, so their latency overlaps it.
  constexpr int kMaxHw = 4;      // kv heads per wave: H_kv <= 16 over 4 waves
  constexpr int kPre = 4;        // logit rows per kv head loaded ahead
  const int t = t0 + lane;
  const bool tv = t < ntok;
  const bool in_w = tv && t >= lo && t < hi;
  const int64_t slot = tv ? bt[static_cast<int64_t>(b) * bt_ld + t] : 0;
  float hv[kMaxHw], lv[kMaxHw][kPre];
#pragma unroll
  for (int k = 0; k < kMaxHw; ++k) {
    const int h = wave + 4 * k;
    hv[k] = (tv && h < H_kv) ? skv::bf16_to_f32(hh[slot * H_kv + h]) : 0.0f;
#pragma unroll
    for (int j = 0; j < kPre; ++j)
      lv[k][j] = (in_w && h < H_kv && j < GR)
                     ? logits[(static_cast<int64_t>(b) * HR + h * GR + j) * bt_ld + t]
                     : 0.0f;
  }
  // (M, Z) of every logit row at once: LR lanes per row (a power of two) fold
  // their chunks' (max, sum) pairs, then the row's lanes combine theirs
  int LR = 64;
  while (LR > 1 && LR * HR > static_cast<int>(blockDim.x)) LR >>= 1;
  {
    const int row = tid / LR, sl = tid % LR;
    float m = -INFINITY, z = 0.0f;
    if (row < HR) {
      const float2* pp = reinterpret_cast<const float2*>(
          part + (static_cast<int64_t>(b) * HR + row) * nchunk * 2);
#pragma unroll 4
      for (int j = sl; j < nch_b; j += LR) fold_max_sum(m, z, pp[j].x, pp[j].y);
    }
    for (int off = LR >> 1; off > 0; off >>= 1)
      fold_max_sum(m, z, __shfl_xor(m, off), __shfl_xor(z, off));
    if (row < HR && sl == 0) { sM[row] = m; sZ[row] = z; }
  }
  __syncthreads();
  if (!tv) return;
#pragma unroll
  for (int k = 0; k < kMaxHw; ++k) {
    const int h = wave + 4 * k;
    if (h >= H_kv) break;
    float v = hv[k];
    if (in_w) {
      float p;
      if constexpr (PH) {
        p = 0.0f;
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
          if (j >= GR) break;
          const int r = h * GR + j;
          p += exp2f(lv[k][j] - sM[r]) / sZ[r];
        }
        for (int gi = kPre; gi < GR; ++gi) {
          const int r = h * GR + gi;
          const float l = logits[(static_cast<int64_t>(b) * HR + r) * bt_ld + t];
          p += exp2f(l - sM[r]) / sZ[r];
        }
        p /= static_cast<float>(GR);
      } else {
        p = exp2f(lv[k][0] - sM[h]) / sZ[h];
      }
      const float pb = skv::bf16_to_f32(skv::f32_to_bf16(p));
      const uint16_t nb = skv::f32_to_bf16(fmaf(decay, v, pb));
      hh[slot * H_kv + h] = nb;
      v = skv::bf16_to_f32(nb);
    }
    scores[(static_cast<int64_t>(b) * H_kv + h) * score_ld + t] = v;
  }
}

int64_t nchunks(int64_t max_tokens) { return (max_tokens + kChunk - 1) / kChunk; }

int64_t scratch_floats(int B, int rows, int64_t max_tokens) {
  if (B < 0 || rows <= 0 || max_tokens <= 0) return -1;
  const int64_t r = static_cast<int64_t>(B) * rows;
  return r * max_tokens + r * nchunks(max_tokens) * 2;
}

// Logits pass LDS: the logit-row queries, their chunk logits and the chunk's
// block ids.
size_t logits_lds(int rows, int D) {
  return sizeof(float) * (static_cast<size_t>(rows) * D + static_cast<size_t>(rows) * kChunk +
                          kChunk);
}
constexpr size_t kMaxLogitsLds = 64 * 1024;

template <bool PH>
int accumulate(const char* fn, const float* q, int B, int H_q, int H_kv, int D,
               const uint16_t* kv_cache, int64_t num_blocks, int page_size,
               const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
               int reserved_bos, int reserved_eos, float scale, float decay,
               uint16_t* hh_score, float* scores, int64_t score_ld, float* scratch,
               int64_t scratch_floats_have, hipStream_t stream) {
  SKV_REQUIRE(page_size == 1, "%s: page_size must be 1 (got %d)", fn, page_size);
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", fn);
  SKV_REQUIRE(H_q / H_kv <= 16, "%s: group size > 16", fn);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", fn, D);
  SKV_REQUIRE(H_kv <= 16, "%s: H_kv must be <= 16", fn);
  const int rows = PH ? H_q : H_kv;
  // (the update pass merges every logit row's partials with at least one of
  // its 256 threads per row; the LDS bound below keeps rows under 128)
  SKV_REQUIRE(logits_lds(rows, D) <= kMaxLogitsLds,
              "%s: H_q * (D + 64) too large for one block's LDS (H_q %d, D %d)", fn, H_q, D);
  SKV_REQUIRE(num_blocks > 0 && bt_ld > 0 && score_ld >= bt_ld,
              "%s: need num_blocks > 0, bt_ld > 0, score_ld >= bt_ld", fn);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", fn);
  SKV_REQUIRE(decay > 0.0f && decay <= 1.0f, "%s: decay must lie in (0, 1]", fn);
  SKV_REQUIRE(scale > 0.0f, "%s: scale must be > 0", fn);
  SKV_REQUIRE(B <= 65535 && nchunks(bt_ld) <= 0x7fffffff, "%s: grid too large", fn);
  SKV_REQUIRE_PTR_W(fn, q);
  SKV_REQUIRE_PTR_W(fn, kv_cache);
  SKV_REQUIRE_PTR_W(fn, block_table);
  SKV_REQUIRE_PTR_W(fn, seq_lens);
  SKV_REQUIRE_PTR_W(fn, hh_score);
  SKV_REQUIRE_PTR_W(fn, scores);
  SKV_REQUIRE_PTR_W(fn, scratch);
  const int64_t need = scratch_floats(B, rows, bt_ld);
  SKV_REQUIRE(scratch_floats_have >= need, "%s: scratch has %lld floats, needs %lld", fn,
              (long long)scratch_floats_have, (long long)need);
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  const int G = H_q / H_kv;
  const int nch = static_cast<int>(nchunks(bt_ld));
  const int nupd = static_cast<int>((bt_ld + kUpd - 1) / kUpd);
  float* logits = scratch;
  float* part = scratch + static_cast<int64_t>(B) * rows * bt_ld;
  // decay is applied as its bf16 value, which is exact for 0.984375
  const float decay_b = skv_host_round_bf16(decay);
  dim3 grid(static_cast<unsigned>(nch), static_cast<unsigned>(B));
  const size_t sm1 = logits_lds(rows, D);
  const float scale_log2 = scale * skv::kLog2e;
  // 16-byte row loads per lane: 4 * H_kv rows per wave over 64 / (D / 8) rows per load
  const int rpw = 64 / (D / 8);
  const int nld = (4 * H_kv + rpw - 1) / rpw;
  // head-major rows when every wave's rows belong to one kv head (per-head
  // logits with 16 loads per lane would not fit their query slices beside
  // the loads in 128 VGPRs)
  const bool hm = 16 % H_kv == 0 && (!PH || nld <= 8);
#define SKV_LOGITS(DD, NN)                                                               \
  do {                                                                                   \
    if (hm)                                                                              \
      hipLaunchKernelGGL((h2o_logits_kernel<DD, NN, PH, true>), grid, dim3(kLWaves * 64), \
                         sm1, stream, q, H_q, H_kv, G, kv_cache, block_table, bt_ld,      \
                         seq_lens, reserved_bos, reserved_eos, scale_log2, logits, part,  \
                         nch);                                                           \
    else                                                                                 \
      hipLaunchKernelGGL((h2o_logits_kernel<DD, NN, PH, false>), grid, dim3(kLWaves * 64),\
                         sm1, stream, q, H_q, H_kv, G, kv_cache, block_table, bt_ld,      \
                         seq_lens, reserved_bos, reserved_eos, scale_log2, logits, part,  \
                         nch);                                                           \
  } while (0)
  if (D == 128) {
    if (nld <= 2) SKV_LOGITS(128, 2); else if (nld <= 4) SKV_LOGITS(128, 4);
    else if (nld <= 8) SKV_LOGITS(128, 8); else SKV_LOGITS(128, 16);
  } else {
    if (nld <= 2) SKV_LOGITS(64, 2); else if (nld <= 4) SKV_LOGITS(64, 4);
    else SKV_LOGITS(64, 8);
  }
#undef SKV_LOGITS
  const size_t sm2 = sizeof(float) * 2 * static_cast<size_t>(rows);
  hipLaunchKernelGGL(h2o_update_kernel<PH>,
                     dim3(static_cast<unsigned>(nupd), static_cast<unsigned>(B)), dim3(256), sm2,
                     stream, H_kv, G, block_table, bt_ld, seq_lens, reserved_bos,
                     reserved_eos, decay_b, hh_score, scores, score_ld, logits, part, nch);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    skv::set_error("%s: launch failed: %s", fn, hipGetErrorString(e));
    return SKV_EIO;
  }
  skv::clear_error();
  return SKV_OK;
}

}  // namespace

extern "C" int64_t h2o_scratch_floats(int B, int H_kv, int64_t max_tokens) {
  return scratch_floats(B, H_kv, max_tokens);
}

extern "C" int64_t h2o_heads_scratch_floats(int B, int H_q, int64_t max_tokens) {
  return scratch_floats(B, H_q, max_tokens);
}

extern "C" int h2o_accumulate(const float* q, int B, int H_q, int H_kv, int D,
                              const uint16_t* kv_cache, int64_t num_blocks,
                              int page_size, const int32_t* block_table,
                              int64_t bt_ld, const int32_t* seq_lens,
                              int reserved_bos, int reserved_eos, float scale,
                              float decay, uint16_t* hh_score, float* scores,
                              int64_t score_ld, float* scratch,
                              int64_t scratch_floats, hipStream_t stream) {
  return accumulate<false>("h2o_accumulate", q, B, H_q, H_kv, D, kv_cache, num_blocks,
                           page_size, block_table, bt_ld, seq_lens, reserved_bos,
                           reserved_eos, scale, decay, hh_score, scores, score_ld, scratch,
                           scratch_floats, stream);
}

extern "C" int h2o_accumulate_heads(const float* q, int B, int H_q, int H_kv, int D,
                                    const uint16_t* kv_cache, int64_t num_blocks,
                                    int page_size, const int32_t* block_table,
                                    int64_t bt_ld, const int32_t* seq_lens,
                                    int reserved_bos, int reserved_eos, float scale,
                                    float decay, uint16_t* hh_score, float* scores,
                                    int64_t score_ld, float* scratch,
                                    int64_t scratch_floats, hipStream_t stream) {
  return accumulate<true>("h2o_accumulate_heads", q, B, H_q, H_kv, D, kv_cache, num_blocks,
                          page_size, block_table, bt_ld, seq_lens, reserved_bos,
                          reserved_eos, scale, decay, hh_score, scores, score_ld, scratch,
                          scratch_floats, stream);
}
