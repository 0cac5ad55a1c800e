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
//      logit row r: one per kv head (q_r = the group-mean query: fp32 dot
//      products, D/8 lanes per row) or one per query head (its own query: the
//      group's rows at once on the matrix cores).  16 waves per chunk, every
//      kv-head row read once with 16-byte loads; the chunk's
//      (max, sum 2^(l - max)) per logit row go to scratch.
//   2. merge of the chunk partials into (M, Z) per logit row, then per token
//      and kv head: p = 2^(l - M) / Z (per-head reading: the mean of that over
//      the group's rows), hh <- bf16(bf16(p) + decay * hh) (one fp32 fma, then
//      round-to-nearest-even), and the new hh value is written as an fp32
//      score row in logical order for the selection.
// Scratch layout: logits [B, R, bt_ld] then partials [B, R, nchunk, 2], with
// R = H_kv logit rows per request (group mean) or H_q (per head).
#include <mutex>

#include "skv_device.h"
#include "skv_host.h"

namespace {

#ifndef SKV_H2O_CHUNK
#define SKV_H2O_CHUNK 64
#endif
// tokens per block of the logits pass (64 measured best against 32 and 16:
// the merge of more, smaller chunk partials costs more than the finer grid
// gains)
constexpr int kChunk = SKV_H2O_CHUNK;
constexpr int kLWaves = kChunk / 4;     // waves per block: 4 tokens' rows each
constexpr int kTiles = kChunk / 16;     // 16-token MFMA tiles per kv head
static_assert(kChunk % 16 == 0 && kChunk <= 64, "chunk of 16, 32, 48 or 64 tokens");
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

// Logits of one chunk of kChunk tokens of one request, one logit row per kv
// head (the group-mean query).  The chunk's H_kv * kChunk kv-head rows are
// dealt to kChunk / 4 waves, 4 * H_kv rows each; a wave issues all its 16-byte
// row loads (NLD per lane) before any arithmetic, masked rows reading a
// placeholder so the loads stay unconditional.  HM (4 * H_kv divides the
// chunk): the rows are dealt head-major, so every row of a wave belongs to one
// kv head and each lane reads that head's query slice from LDS once, not once
// per key row.
template <int D, int NLD, bool HM>
__global__ __launch_bounds__(kLWaves * 64) void h2o_logits_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ bt,
    int64_t bt_ld, const int32_t* __restrict__ seq_lens, int bos, int eos,
    float scale_log2, float* __restrict__ logits, float* __restrict__ part,
    int nchunk, const uint16_t* __restrict__ hh, uint16_t* __restrict__ hh_snap,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ kv_w, uint16_t* __restrict__ hh_w, int64_t v_off) {
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
  // With k_new given, this step's append (the cache's and the accumulator's
  // side of it) is done here: the block whose chunk holds token S - 1 writes
  // its K and V rows, zeroes its accumulator, and takes its logit from k_new.
  const int t_new = seq_lens[b] - 1;
  const bool app = k_new != nullptr && t_new >= t0 && t_new < ntok && t_new - t0 < kChunk;
  if (app && tid < H_kv * (D / 8)) {
    const int hd = tid / (D / 8), c8 = tid % (D / 8);
    const int64_t dst = (static_cast<int64_t>(btr[t_new]) * H_kv + hd) * D + c8 * 8;
    const int64_t src = (static_cast<int64_t>(b) * H_kv + hd) * D + c8 * 8;
    *reinterpret_cast<uint4*>(kv_w + dst) = *reinterpret_cast<const uint4*>(k_new + src);
    *reinterpret_cast<uint4*>(kv_w + v_off + dst) = *reinterpret_cast<const uint4*>(v_new + src);
    if (c8 == 0) hh_w[static_cast<int64_t>(btr[t_new]) * H_kv + hd] = 0;
  }
  if (hh_snap != nullptr && tid < kChunk * H_kv) {
    // the accumulator before this step, per kv head in logical order, for a
    // consumer that must not read hh_score while it is being rewritten
    const int tt = tid / H_kv, hd = tid % H_kv;
    if (t0 + tt < ntok)
      hh_snap[(static_cast<int64_t>(b) * H_kv + hd) * bt_ld + t0 + tt] =
          (app && t0 + tt == t_new) ? static_cast<uint16_t>(0)
                                    : hh[static_cast<int64_t>(btr[t0 + tt]) * H_kv + hd];
  }
  const float inv_g = 1.0f / static_cast<float>(G);
  for (int i = tid; i < H_kv * D; i += blockDim.x) {
    const int h = i / D, d = i % D;
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += q[(static_cast<int64_t>(b) * H_q + h * G + g) * D + d];
    qs[i] = s * inv_g * scale_log2;
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
    const uint16_t* src = (app && ok[u] && t == t_new)
        ? k_new + (static_cast<int64_t>(b) * H_kv + h) * D + cc * 8 : kv + off;
    kr[u] = *reinterpret_cast<const uint4*>(src);
  }
  // HM: the wave's kv head and its query slice in registers
  float qv[8];
  if constexpr (HM) {
    const float* qr = qs + ((wave * R) / kChunk) * D + cc * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qr[i];
  }
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int rl = u * RPW + sub;
    int tt, h;
    row_of(rl, tt, h);
    float x[8];
    skv::unpack8(kr[u], x);
    if constexpr (!HM) {
      const float* qr = qs + (rl < R ? h : 0) * D + cc * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = qr[i];
    }
    float dot = qv[0] * x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) dot = fmaf(qv[i], x[i], dot);
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

// Per-head logits on the matrix cores (the per-head reading).  A chunk's
// kv-head rows form kTiles * H_kv tiles of (kv head h, 16 tokens), dealt to
// the kLWaves waves (up to TPW each).  Per tile
//   S (16 tokens x 16 query heads) = K (16 x D) . Q^T (D x 16)
// with 16x16x32 bf16 MFMAs: the 16-byte row pieces a lane loads are exactly
// its A operand (row lane & 15, dims c*32 + 8*(lane >> 4) .. +8), the group's
// queries (scaled by scale * log2(e)) are the B operand as bf16 hi + lo
// halves (two MFMAs per 32 dims, about 16 significant bits), columns past G
// are zero, and lane (n, kq) ends with rows 4*kq .. 4*kq + 3 of column n.
// The query halves sit in LDS with rows padded by 8 bf16 so that the 16 rows
// a quarter-wave reads fall in different banks.
template <int D, int TPW>
__global__ __launch_bounds__(kLWaves * 64) void h2o_logits_heads_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ bt,
    int64_t bt_ld, const int32_t* __restrict__ seq_lens, int bos, int eos,
    float scale_log2, float* __restrict__ logits, float* __restrict__ part,
    int nchunk, const uint16_t* __restrict__ hh, uint16_t* __restrict__ hh_snap,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ kv_w, uint16_t* __restrict__ hh_w, int64_t v_off) {
  constexpr int NC = D / 32;                   // 32-dim steps of the MFMA
  constexpr int QS = D + 8;                    // padded query row (bf16)
  constexpr int LGS = kChunk + 4;              // padded logit row (floats)
  extern __shared__ float smem[];
  uint16_t* qh = reinterpret_cast<uint16_t*>(smem);          // [H_q][QS]
  uint16_t* ql = qh + H_q * QS;                              // [H_q][QS]
  float* lg = smem + H_q * QS;                               // [H_q][LGS]
  int* sblk = reinterpret_cast<int*>(lg + H_q * LGS);        // [kChunk]
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  int ntok, lo, hi;
  window(seq_lens[b], bt_ld, bos, eos, &ntok, &lo, &hi);
  const int t0 = c * kChunk;
  if (t0 >= ntok) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;

  if (tid < kChunk) sblk[tid] = t0 + tid < ntok ? btr[t0 + tid] : 0;
  // With k_new given, this step's append (the cache's and the accumulator's
  // side of it) is done here: the block whose chunk holds token S - 1 writes
  // its K and V rows, zeroes its accumulator, and takes its logit from k_new.
  const int t_new = seq_lens[b] - 1;
  const bool app = k_new != nullptr && t_new >= t0 && t_new < ntok && t_new - t0 < kChunk;
  if (app && tid < H_kv * (D / 8)) {
    const int hd = tid / (D / 8), c8 = tid % (D / 8);
    const int64_t dst = (static_cast<int64_t>(btr[t_new]) * H_kv + hd) * D + c8 * 8;
    const int64_t src = (static_cast<int64_t>(b) * H_kv + hd) * D + c8 * 8;
    *reinterpret_cast<uint4*>(kv_w + dst) = *reinterpret_cast<const uint4*>(k_new + src);
    *reinterpret_cast<uint4*>(kv_w + v_off + dst) = *reinterpret_cast<const uint4*>(v_new + src);
    if (c8 == 0) hh_w[static_cast<int64_t>(btr[t_new]) * H_kv + hd] = 0;
  }
  if (hh_snap != nullptr && tid < kChunk * H_kv) {
    // the accumulator before this step, per kv head in logical order, for a
    // consumer that must not read hh_score while it is being rewritten
    const int tt = tid / H_kv, hd = tid % H_kv;
    if (t0 + tt < ntok)
      hh_snap[(static_cast<int64_t>(b) * H_kv + hd) * bt_ld + t0 + tt] =
          (app && t0 + tt == t_new) ? static_cast<uint16_t>(0)
                                    : hh[static_cast<int64_t>(btr[t0 + tt]) * H_kv + hd];
  }
  for (int i = tid; i < H_q * D; i += blockDim.x) {
    const int r = i / D, d = i % D;
    const float x = q[static_cast<int64_t>(b) * H_q * D + i] * scale_log2;
    const uint16_t hb = skv::f32_to_bf16(x);
    qh[r * QS + d] = hb;
    ql[r * QS + d] = skv::f32_to_bf16(x - skv::bf16_to_f32(hb));
  }
  __syncthreads();

  const int ntile = kTiles * H_kv;
  uint4 kt[TPW][NC];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + kLWaves * j;
    const int h = t < ntile ? t / kTiles : 0;
    const int tt = (t % kTiles) * 16 + n;      // the row this lane loads
    const int tok = t0 + tt;
    const bool ok = t < ntile && tok >= lo && tok < hi;
    const int64_t off = (ok ? (static_cast<int64_t>(sblk[tt]) * H_kv + h) * D : 0) + 8 * kq;
    const uint16_t* src = (app && ok && tok == t_new)
        ? k_new + (static_cast<int64_t>(b) * H_kv + h) * D + 8 * kq : kv + off;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      kt[j][cc] = *reinterpret_cast<const uint4*>(src + cc * 32);
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + kLWaves * j;
    if (t >= ntile) break;
    const int h = t / kTiles, tb = (t % kTiles) * 16;
    const bool col = n < G;
    const int qr = (h * G + (col ? n : 0)) * QS + 8 * kq;
    skv_f32x4 sacc = skv_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      uint4 bh = *reinterpret_cast<const uint4*>(qh + qr + cc * 32);
      uint4 bl = *reinterpret_cast<const uint4*>(ql + qr + cc * 32);
      if (!col) { bh = make_uint4(0u, 0u, 0u, 0u); bl = bh; }
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(skv::as_bf16x8(kt[j][cc]),
                                                     skv::as_bf16x8(bh), sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(skv::as_bf16x8(kt[j][cc]),
                                                     skv::as_bf16x8(bl), sacc, 0, 0, 0);
    }
    if (col) {
      float4 v;
      float* vv = reinterpret_cast<float*>(&v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + tb + 4 * kq + i;
        vv[i] = (tok >= lo && tok < hi) ? sacc[i] : -INFINITY;
      }
      *reinterpret_cast<float4*>(lg + (h * G + n) * LGS + tb + 4 * kq) = v;
    }
  }
  __syncthreads();

  const int nt = min(kChunk, ntok - t0);
  for (int r = wave; r < H_q; r += kLWaves) {
    const float v = lane < nt ? lg[r * LGS + lane] : -INFINITY;
    const float m = skv::wave_max(v);
    float e = (m != -INFINITY && lane < nt) ? exp2f(v - m) : 0.0f;
    const float s = skv::wave_sum(e);
    if (lane < nt) logits[(static_cast<int64_t>(b) * H_q + r) * bt_ld + t0 + lane] = v;
    if (lane == 0) {
      float* pp = part + ((static_cast<int64_t>(b) * H_q + r) * nchunk + c) * 2;
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

// Logits pass LDS: the logit-row queries (fp32, or bf16 hi + lo with rows
// padded by 8 for the per-head pass), their chunk logits (rows padded by 4 for
// the per-head pass) and the chunk's block ids.
size_t logits_lds(bool per_head, int rows, int D) {
  const size_t r = static_cast<size_t>(rows);
  return per_head ? sizeof(float) * (r * (D + 8) + r * (kChunk + 4) + kChunk)
                  : sizeof(float) * (r * D + r * kChunk + kChunk);
}
constexpr size_t kMaxLogitsLds = 64 * 1024;

// Offset (floats) of the accumulator snapshot in the scratch of the pass that
// feeds a fused update: after the logits and partials, 16-byte aligned.
int64_t snap_offset(int B, int rows, int64_t max_tokens) {
  return (scratch_floats(B, rows, max_tokens) + 3) / 4 * 4;
}

// pass == nullptr: the whole step (logits pass, then the update pass).
// pass given: the logits pass only, with a snapshot of the accumulator for a
// consumer that applies the update itself; scores is not used then.
template <bool PH>
int accumulate(const char* fn, const float* q, int B, int H_q, int H_kv, int D,
               const uint16_t* kv_cache, int64_t num_blocks, int page_size,
               const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
               int reserved_bos, int reserved_eos, float scale, float decay,
               uint16_t* hh_score, float* scores, int64_t score_ld, float* scratch,
               int64_t scratch_floats_have, hipStream_t stream,
               skv::H2oPass* pass = nullptr, const uint16_t* k_new = nullptr,
               const uint16_t* v_new = nullptr, uint16_t* kv_w = nullptr) {
  SKV_REQUIRE(page_size == 1, "%s: page_size must be 1 (got %d)", fn, page_size);
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", fn);
  SKV_REQUIRE(H_q / H_kv <= 16, "%s: group size > 16", fn);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", fn, D);
  SKV_REQUIRE(H_kv <= 16, "%s: H_kv must be <= 16", fn);
  const int rows = PH ? H_q : H_kv;
  // (the update pass merges every logit row's partials with at least one of
  // its 256 threads per row; the LDS bound below keeps rows under 128)
  SKV_REQUIRE(logits_lds(PH, rows, D) <= kMaxLogitsLds,
              "%s: the request's query rows and chunk logits exceed one block's LDS "
              "(%d rows, D %d)", fn, rows, D);
  SKV_REQUIRE(num_blocks > 0 && bt_ld > 0 && score_ld >= bt_ld,
              "%s: need num_blocks > 0, bt_ld > 0, score_ld >= bt_ld", fn);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", fn);
  SKV_REQUIRE(decay > 0.0f && decay <= 1.0f, "%s: decay must lie in (0, 1]", fn);
  SKV_REQUIRE(scale > 0.0f, "%s: scale must be > 0", fn);
  SKV_REQUIRE(B <= 65535 && nchunks(bt_ld) <= 0x7fffffff, "%s: grid too large", fn);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(fn, q);
  SKV_REQUIRE_PTR_W(fn, kv_cache);
  SKV_REQUIRE_PTR_W(fn, block_table);
  SKV_REQUIRE_PTR_W(fn, seq_lens);
  SKV_REQUIRE_PTR_W(fn, hh_score);
  if (pass == nullptr) SKV_REQUIRE_PTR_W(fn, scores);
  SKV_REQUIRE_PTR_W(fn, scratch);
  const int64_t need = pass == nullptr ? scratch_floats(B, rows, bt_ld)
      : snap_offset(B, rows, bt_ld) + (static_cast<int64_t>(B) * H_kv * bt_ld + 1) / 2;
  SKV_REQUIRE(scratch_floats_have >= need, "%s: scratch has %lld floats, needs %lld", fn,
              (long long)scratch_floats_have, (long long)need);
  const int G = H_q / H_kv;
  const int nch = static_cast<int>(nchunks(bt_ld));
  const int nupd = static_cast<int>((bt_ld + kUpd - 1) / kUpd);
  float* logits = scratch;
  float* part = scratch + static_cast<int64_t>(B) * rows * bt_ld;
  uint16_t* hh_snap = pass == nullptr ? nullptr
      : reinterpret_cast<uint16_t*>(scratch + snap_offset(B, rows, bt_ld));
  // decay is applied as its bf16 value, which is exact for 0.984375
  const float decay_b = skv_host_round_bf16(decay);
  const int64_t v_off = num_blocks * page_size * static_cast<int64_t>(H_kv) * D;
  dim3 grid(static_cast<unsigned>(nch), static_cast<unsigned>(B));
  const size_t sm1 = logits_lds(PH, rows, D);
  const float scale_log2 = scale * skv::kLog2e;
  if constexpr (PH) {
    // tiles of (kv head, 16 tokens) per wave
    const int tpw = (kTiles * H_kv + kLWaves - 1) / kLWaves;
#define SKV_HEADS(DD, TT)                                                                \
  hipLaunchKernelGGL((h2o_logits_heads_kernel<DD, TT>), grid, dim3(kLWaves * 64), sm1,   \
                     stream, q, H_q, H_kv, G, kv_cache, block_table, bt_ld, seq_lens,     \
                     reserved_bos, reserved_eos, scale_log2, logits, part, nch, hh_score,   \
                     hh_snap, k_new, v_new, kv_w, hh_score, v_off)
    if (D == 128) {
      if (tpw <= 1) SKV_HEADS(128, 1); else if (tpw == 2) SKV_HEADS(128, 2);
      else if (tpw == 3) SKV_HEADS(128, 3); else SKV_HEADS(128, 4);
    } else {
      if (tpw <= 1) SKV_HEADS(64, 1); else if (tpw == 2) SKV_HEADS(64, 2);
      else if (tpw == 3) SKV_HEADS(64, 3); else SKV_HEADS(64, 4);
    }
#undef SKV_HEADS
  } else {
    // 16-byte row loads per lane: 4 * H_kv rows per wave over 64 / (D / 8) rows per load
    const int rpw = 64 / (D / 8);
    const int nld = (4 * H_kv + rpw - 1) / rpw;
    // head-major rows when every wave's rows belong to one kv head
    const bool hm = (kChunk / 4) % H_kv == 0;
#define SKV_LOGITS_HM(DD, NN, HM)                                                        \
  hipLaunchKernelGGL((h2o_logits_kernel<DD, NN, HM>), grid, dim3(kLWaves * 64), sm1,      \
                     stream, q, H_q, H_kv, G, kv_cache, block_table, bt_ld, seq_lens,     \
                     reserved_bos, reserved_eos, scale_log2, logits, part, nch, hh_score,   \
                     hh_snap, k_new, v_new, kv_w, hh_score, v_off)
#define SKV_LOGITS(DD, NN)                                                               \
  do {                                                                                   \
    if (hm) SKV_LOGITS_HM(DD, NN, true); else SKV_LOGITS_HM(DD, NN, false);              \
  } while (0)
    if (D == 128) {
      // (one or two kv heads: 2 loads, and H_kv divides 16, so head-major)
      if (nld <= 2) SKV_LOGITS_HM(128, 2, true); else if (nld <= 4) SKV_LOGITS(128, 4);
      else if (nld <= 8) SKV_LOGITS(128, 8); else SKV_LOGITS(128, 16);
    } else {
      if (nld <= 2) SKV_LOGITS(64, 2); else if (nld <= 4) SKV_LOGITS(64, 4);
      else SKV_LOGITS(64, 8);
    }
#undef SKV_LOGITS
#undef SKV_LOGITS_HM
  }
  if (pass != nullptr) {
    *pass = skv::H2oPass{logits, part, hh_snap, nch, kChunk, decay_b};
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      skv::set_error("%s: launch failed: %s", fn, hipGetErrorString(e));
      return SKV_EIO;
    }
    skv::clear_error();
    return SKV_OK;
  }
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

// ------------------------------------------------- no-allocation form
// The scratch of h2o_accumulate_noalloc: a fixed array in device memory.
// Every GPU the library runs on holds its own copy, at its own address, until
// the process ends.  In host code the array's name is only a host-side
// stand-in: kernels get the device address fetched once per device.
static __device__ __align__(256) float g_noalloc_scratch[SKV_NOALLOC_SCRATCH_FLOATS];

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
float* g_noalloc_ptr[kMaxDevices] = {};

// Device address of this device's copy of the array, fetched on the first
// call that runs on the device (with the device current) and kept.
int noalloc_scratch(const char* fn, hipStream_t stream, float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    skv::set_error("%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    return SKV_EIO;
  }
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) {
      skv::set_error("%s: hipStreamGetDevice failed: %s", fn, hipGetErrorString(e));
      return SKV_EIO;
    }
    SKV_REQUIRE(sdev == dev, "%s: the stream belongs to device %d, the current device is %d",
                fn, static_cast<int>(sdev), dev);
  }
  SKV_REQUIRE(dev >= 0 && dev < kMaxDevices, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_noalloc_scratch));
    if (e != hipSuccess || p == nullptr) {
      skv::set_error("%s: hipGetSymbolAddress failed on device %d: %s", fn, dev,
                     hipGetErrorString(e));
      return SKV_EIO;
    }
    g_noalloc_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_noalloc_ptr[dev];
  return SKV_OK;
}

}  // namespace

namespace skv {

int h2o_logits_pass(const char* fn, bool per_head, const float* q, int B, int H_q, int H_kv,
                    int D, const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                    const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                    int reserved_bos, int reserved_eos, float scale, float decay,
                    uint16_t* hh_score, float* scratch, int64_t scratch_floats,
                    hipStream_t stream, H2oPass* out, const uint16_t* k_new,
                    const uint16_t* v_new, uint16_t* kv_w) {
  if (per_head)
    return accumulate<true>(fn, q, B, H_q, H_kv, D, kv_cache, num_blocks, page_size,
                            block_table, bt_ld, seq_lens, reserved_bos, reserved_eos, scale,
                            decay, hh_score, nullptr, bt_ld, scratch, scratch_floats, stream,
                            out, k_new, v_new, kv_w);
  return accumulate<false>(fn, q, B, H_q, H_kv, D, kv_cache, num_blocks, page_size,
                           block_table, bt_ld, seq_lens, reserved_bos, reserved_eos, scale,
                           decay, hh_score, nullptr, bt_ld, scratch, scratch_floats, stream,
                           out, k_new, v_new, kv_w);
}

int64_t h2o_pass_scratch_floats(int B, int rows, int H_kv, int64_t max_tokens) {
  if (B < 0 || rows <= 0 || H_kv <= 0 || max_tokens <= 0) return -1;
  return snap_offset(B, rows, max_tokens) + (static_cast<int64_t>(B) * H_kv * max_tokens + 1) / 2;
}

}  // namespace skv

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

extern "C" int h2o_accumulate_noalloc(const float* q, int B, int H_q, int H_kv, int D,
                                      const uint16_t* kv_cache, int64_t num_blocks,
                                      int page_size, const int32_t* block_table,
                                      int64_t bt_ld, const int32_t* seq_lens,
                                      int reserved_bos, int reserved_eos, float scale,
                                      float decay, uint16_t* hh_score, float* scores,
                                      int64_t score_ld, hipStream_t stream) {
  const char* fn = "h2o_accumulate_noalloc";
  SKV_REQUIRE(B >= 0 && H_kv > 0 && bt_ld > 0, "%s: need B >= 0, H_kv > 0, bt_ld > 0", fn);
  const int64_t need = scratch_floats(B, H_kv, bt_ld);
  SKV_REQUIRE(need <= SKV_NOALLOC_SCRATCH_FLOATS,
              "%s: the step needs %lld scratch floats, the fixed buffer holds %lld "
              "(use h2o_accumulate with a caller buffer)", fn, (long long)need,
              (long long)SKV_NOALLOC_SCRATCH_FLOATS);
  float* scratch = nullptr;
  if (B > 0) {
    // (scalar checks first, so that a bad argument is reported as such)
    const int rc = accumulate<false>(fn, q, 0, H_q, H_kv, D, kv_cache, num_blocks,
                                     page_size, block_table, bt_ld, seq_lens, reserved_bos,
                                     reserved_eos, scale, decay, hh_score, scores, score_ld,
                                     nullptr, 0, stream);
    if (rc != SKV_OK) return rc;
    const int rs = noalloc_scratch(fn, stream, &scratch);
    if (rs != SKV_OK) return rs;
  }
  return accumulate<false>(fn, q, B, H_q, H_kv, D, kv_cache, num_blocks, page_size,
                           block_table, bt_ld, seq_lens, reserved_bos, reserved_eos, scale,
                           decay, hh_score, scores, score_ld, scratch,
                           SKV_NOALLOC_SCRATCH_FLOATS, stream);
}
