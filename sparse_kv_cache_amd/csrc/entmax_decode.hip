// entmax_decode.hip -- 1.5-entmax attention over the tokens of the selected
// pages (the attention EntmaxKV decodes with: README "Quick start", alpha=1.5).
//
// alpha-entmax with alpha = 1.5 maps logits z to
//   p_t = [ z_t / 2 - tau ]_+ ^ 2,  tau such that sum_t p_t = 1
// (the published closed form of Peters, Niculae and Martins, 2019).  Unlike
// softmax, tau depends on every selected logit, so the decode takes three
// launches over one selection:
//   1. logits: one wave per (request, query head, split chunk) reads the
//      chunk's K rows once and writes z = scale * q . k per row (selection
//      order, -inf for rows past a page's valid count) to scratch;
//   2. tau: one block per (request, query head) finds tau by Newton steps on
//      f(tau) = sum [u - tau]_+^2 - 1 (u = z / 2) from tau = max u - 1, where
//      f >= 0; f is convex and falling there, so the steps rise monotonically
//      to the root (the row held in registers when it fits);
//   3. values: one wave per chunk again folds p_t v_t over the rows with
//      p_t > 0 only (16-row groups with no such row load no V at all) and
//      writes the chunk's (o = sum p v / m, lse = ln m) with its mass m, so
//      lse_merge's algebra returns sum over chunks of p v (total mass 1).
// Scratch: logits [B, H_q, k_cap * P] then tau [B, H_q].
// ALiBi heads add slope * (pos - (S - 1)) to each logit in pass 1.
#include "skv_device.h"
#include "skv_host.h"

namespace {

constexpr int kWaves = 4;            // waves per block of passes 1 and 3
constexpr int kTauThreads = 256;

struct Sel {
  int64_t qrow;       // b * H_q + query head
  int srow;           // selection row
  int start, len;     // chunk entries [start, start + len)
  int S, b, h;
};

// Chunk of (request, query head, split) for wave index w of the grid.
__device__ __forceinline__ bool chunk_of(int64_t w, int H_q, int H_kv, int G, int H_sel,
                                         int num_splits, int k_cap, int B,
                                         const int32_t* seq_lens, const int32_t* sel_cnt,
                                         Sel& c) {
  const int s = static_cast<int>(w % num_splits);
  const int64_t qrow = w / num_splits;
  if (qrow >= static_cast<int64_t>(B) * H_q) return false;
  const int b = static_cast<int>(qrow / H_q);
  const int i = static_cast<int>(qrow % H_q);
  const int h = i / G;
  c.qrow = qrow;
  c.b = b;
  c.h = h;
  c.srow = H_sel == H_q ? static_cast<int>(qrow) : b * H_kv + h;
  c.S = seq_lens[b];
  int cnt = sel_cnt[c.srow];
  cnt = cnt < 0 ? 0 : (cnt > k_cap ? k_cap : cnt);
  // the row's actual entries split evenly (a selection of adaptive size
  // would leave the trailing splits of a k_cap-sized grid empty)
  const int cap = (cnt + num_splits - 1) / num_splits;
  c.start = s * cap;
  int len = cnt - c.start;
  c.len = len < 0 ? 0 : (len > cap ? cap : len);
  return true;
}

typedef __bf16 skv_bf16x2_e __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2e(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(skv_bf16x2_e, a),
                                         __builtin_bit_cast(skv_bf16x2_e, b), c, false);
}

// Pass 1.  Lane layout as the softmax decode: D/8 lanes per row, 64/(D/8)
// rows per load, 16-row groups of 16/P entries.
template <int D>
__global__ __launch_bounds__(kWaves * 64) void entmax_logits_kernel(
    const float* __restrict__ q, int B, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, int64_t num_blocks, int P,
    const int32_t* __restrict__ bt, int64_t bt_ld, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
    const int32_t* __restrict__ sel_blk, int k_cap, int H_sel, float scale,
    int num_splits, const float* __restrict__ alibi, float* __restrict__ logits) {
  constexpr int LPR = D / 8;
  constexpr int RPL = 64 / LPR;
  constexpr int NL = 16 / RPL;
  const int lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  Sel c;
  if (!chunk_of(w, H_q, H_kv, G, H_sel, num_splits, k_cap, B, seq_lens, sel_cnt, c)) return;
  const int slot = lane / LPR, cc = lane % LPR;
  int64_t Nb = (static_cast<int64_t>(c.S) + P - 1) / P;
  if (Nb > bt_ld) Nb = bt_ld;
  const float slope = alibi != nullptr ? alibi[c.qrow % H_q] : 0.0f;
  // q split into bf16 hi + lo halves: exact bf16 products on the packed keys
  uint32_t qh[4], ql[4];
  {
    const float* qr = q + c.qrow * D + cc * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = qr[2 * i] * scale, x1 = qr[2 * i + 1] * scale;
      const uint16_t h0 = skv::f32_to_bf16(x0), h1 = skv::f32_to_bf16(x1);
      const uint16_t l0 = skv::f32_to_bf16(x0 - skv::bf16_to_f32(h0));
      const uint16_t l1 = skv::f32_to_bf16(x1 - skv::bf16_to_f32(h1));
      qh[i] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
      ql[i] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
    }
  }
  const int32_t* selr = sel_idx + static_cast<int64_t>(c.srow) * k_cap;
  const int32_t* sblk = sel_blk != nullptr ? sel_blk + static_cast<int64_t>(c.srow) * k_cap
                                           : nullptr;
  const int32_t* btr = bt + static_cast<int64_t>(c.b) * bt_ld;
  const int64_t row_stride = static_cast<int64_t>(H_kv) * D;
  const int64_t head_off = static_cast<int64_t>(c.h) * D + cc * 8;
  float* lrow = logits + c.qrow * (static_cast<int64_t>(k_cap) * P);
  const int epg = 16 / P;
  for (int w0 = 0; w0 < c.len; w0 += 64) {
    const int nw = min(64, c.len - w0);
    int my_blk = 0, my_nv = 0, my_off = 0;
    if (lane < nw) {
      const int p = selr[c.start + w0 + lane];
      if (p >= 0 && p < Nb) {
        my_blk = sblk != nullptr ? sblk[c.start + w0 + lane] : btr[p];
        const int n = c.S - p * P;
        my_nv = n < P ? n : P;
        my_off = p * P - (c.S - 1);        // first row's offset from the query
      }
    }
    const int ngroups = (nw + epg - 1) / epg;
    for (int grp = 0; grp < ngroups; ++grp) {
      uint4 K[NL];
      bool ok[NL];
      int ent[NL], tt[NL], rel[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int rr = slot + RPL * j;
        const int e = grp * epg + rr / P;
        const int t = rr % P;
        const int ec = e < 64 ? e : 63;
        const int blk = __shfl(my_blk, ec);
        const int nv = __shfl(my_nv, ec);
        ok[j] = e < nw && t < nv;
        ent[j] = e;
        tt[j] = t;
        rel[j] = __shfl(my_off, ec) + t;
        const int64_t off = ok[j] ? (static_cast<int64_t>(blk) * P + t) * row_stride + head_off
                                  : head_off;
        K[j] = *reinterpret_cast<const uint4*>(kv + off);
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        float d = 0.0f;
        d = dot2e(K[j].x, qh[0], d); d = dot2e(K[j].x, ql[0], d);
        d = dot2e(K[j].y, qh[1], d); d = dot2e(K[j].y, ql[1], d);
        d = dot2e(K[j].z, qh[2], d); d = dot2e(K[j].z, ql[2], d);
        d = dot2e(K[j].w, qh[3], d); d = dot2e(K[j].w, ql[3], d);
        d = skv::group_sum<LPR>(d);
        // ALiBi: slope * (pos - (S - 1)), the integer offset exact in fp32
        if (alibi != nullptr) d = fmaf(slope, static_cast<float>(rel[j]), d);
        if (cc == 0 && ent[j] < nw)
          lrow[static_cast<int64_t>(c.start + w0 + ent[j]) * P + tt[j]] = ok[j] ? d : -INFINITY;
      }
    }
  }
}

// Pass 2: tau of one query row over its cnt * P logits.  With R > 0 the
// row (at most THREADS * R logits) is read once into registers, so the
// Newton steps cost no memory round trips; with R == 0 every step re-reads
// the row.
template <int THREADS, int R>
__global__ __launch_bounds__(THREADS) void entmax_tau_kernel(
    int B, int H_q, int H_kv, int G, int P, const int32_t* __restrict__ sel_cnt,
    int k_cap, int H_sel, const float* __restrict__ logits, float* __restrict__ tau) {
  constexpr int NW = THREADS / 64;
  __shared__ float red[2][NW];
  const int64_t qrow = blockIdx.x;
  const int b = static_cast<int>(qrow / H_q);
  const int i = static_cast<int>(qrow % H_q);
  const int srow = H_sel == H_q ? static_cast<int>(qrow) : b * H_kv + i / G;
  int cnt = sel_cnt[srow];
  cnt = cnt < 0 ? 0 : (cnt > k_cap ? k_cap : cnt);
  const int n = cnt * P;
  const float* z = logits + qrow * (static_cast<int64_t>(k_cap) * P);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  auto block_sum2 = [&](float& a, float& c2) {
    a = skv::wave_sum(a);
    c2 = skv::wave_sum(c2);
    if (lane == 0) { red[0][wave] = a; red[1][wave] = c2; }
    __syncthreads();
    a = 0.0f; c2 = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) { a += red[0][w]; c2 += red[1][w]; }
    __syncthreads();
  };

  // u = z / 2 of this thread's entries (-inf past the row)
  float u[R > 0 ? R : 1];
  float um = -INFINITY;
  if constexpr (R > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = tid + r * THREADS;
      u[r] = t < n ? 0.5f * z[t] : -INFINITY;
      um = fmaxf(um, u[r]);
    }
  } else {
    for (int t = tid; t < n; t += THREADS) um = fmaxf(um, 0.5f * z[t]);
  }
  um = skv::wave_max(um);
  if (lane == 0) red[0][wave] = um;
  __syncthreads();
  um = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) um = fmaxf(um, red[0][w]);
  __syncthreads();
  if (um == -INFINITY) {                         // no valid row selected
    if (tid == 0) tau[qrow] = -INFINITY;
    return;
  }
  // Newton on f(tau) = sum [u - tau]_+^2 - 1 from the left (f >= 0 at
  // max u - 1); steps shrink quadratically near the root.
  float t0 = um - 1.0f;
  for (int it = 0; it < 30; ++it) {
    float f = 0.0f, g = 0.0f;
    if constexpr (R > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float d = u[r] - t0;
        if (d > 0.0f) { f = fmaf(d, d, f); g += d; }
      }
    } else {
      for (int t = tid; t < n; t += THREADS) {
        const float d = 0.5f * z[t] - t0;
        if (d > 0.0f) { f = fmaf(d, d, f); g += d; }
      }
    }
    block_sum2(f, g);
    f -= 1.0f;
    const float step = f / (2.0f * g);
    if (!(step > 1e-7f * fmaxf(1.0f, fabsf(t0)))) {
      if (step > 0.0f) t0 += step;
      break;
    }
    t0 += step;
  }
  if (tid == 0) tau[qrow] = t0;
}

// Pass 3: the chunk's sum of p v over rows with p > 0, as (o, lse) partials.
template <int D>
__global__ __launch_bounds__(kWaves * 64) void entmax_values_kernel(
    int B, int H_q, int H_kv, int G, const uint16_t* __restrict__ kv,
    int64_t num_blocks, int P, const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, const int32_t* __restrict__ sel_blk, int k_cap,
    int H_sel, int num_splits, const float* __restrict__ logits,
    const float* __restrict__ tau, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  constexpr int LPR = D / 8;
  constexpr int RPL = 64 / LPR;
  constexpr int NL = 16 / RPL;
  const int lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  Sel c;
  if (!chunk_of(w, H_q, H_kv, G, H_sel, num_splits, k_cap, B, seq_lens, sel_cnt, c)) return;
  const int s = static_cast<int>(w % num_splits);
  const int slot = lane / LPR, cc = lane % LPR;
  int64_t Nb = (static_cast<int64_t>(c.S) + P - 1) / P;
  if (Nb > bt_ld) Nb = bt_ld;
  const float tq = tau[c.qrow];
  const int32_t* selr = sel_idx + static_cast<int64_t>(c.srow) * k_cap;
  const int32_t* sblk = sel_blk != nullptr ? sel_blk + static_cast<int64_t>(c.srow) * k_cap
                                           : nullptr;
  const int32_t* btr = bt + static_cast<int64_t>(c.b) * bt_ld;
  const int64_t row_stride = static_cast<int64_t>(H_kv) * D;
  const int64_t v_off = num_blocks * P * row_stride;
  const int64_t head_off = static_cast<int64_t>(c.h) * D + cc * 8;
  const float* lrow = logits + c.qrow * (static_cast<int64_t>(k_cap) * P);
  const int epg = 16 / P;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  float mass = 0.0f;                 // this lane's rows
  for (int w0 = 0; w0 < c.len && tq != -INFINITY; w0 += 64) {
    const int nw = min(64, c.len - w0);
    int my_blk = 0, my_nv = 0;
    if (lane < nw) {
      const int p = selr[c.start + w0 + lane];
      if (p >= 0 && p < Nb) {
        my_blk = sblk != nullptr ? sblk[c.start + w0 + lane] : btr[p];
        const int n = c.S - p * P;
        my_nv = n < P ? n : P;
      }
    }
    const int ngroups = (nw + epg - 1) / epg;
    for (int grp = 0; grp < ngroups; ++grp) {
      float pr[NL];
      int64_t off[NL];
      bool any = false;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int rr = slot + RPL * j;
        const int e = grp * epg + rr / P;
        const int t = rr % P;
        const int ec = e < 64 ? e : 63;
        const int blk = __shfl(my_blk, ec);
        const int nv = __shfl(my_nv, ec);
        const bool ok = e < nw && t < nv;
        float p = 0.0f;
        if (ok) {
          const float d = 0.5f * lrow[static_cast<int64_t>(c.start + w0 + e) * P + t] - tq;
          p = d > 0.0f ? d * d : 0.0f;
        }
        pr[j] = p;
        any |= p > 0.0f;
        off[j] = p > 0.0f ? (static_cast<int64_t>(blk) * P + t) * row_stride + head_off
                          : head_off;
      }
      // a 16-row group with no row in the support loads no values
      if (__ballot(any) == 0ull) continue;
      uint4 V[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) V[j] = *reinterpret_cast<const uint4*>(kv + v_off + off[j]);
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        if (pr[j] > 0.0f) {
          float v[8];
          skv::unpack8(V[j], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(pr[j], v[i], acc[i]);
          mass += pr[j];
        }
      }
    }
  }
  // sum the row slots' accumulators (lanes cc, cc + LPR, ...)
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], o);
    mass += __shfl_xor(mass, o);
  }
  const int64_t prow = c.qrow * num_splits + s;
  if (slot == 0) {
    float4* dst = reinterpret_cast<float4*>(o_part + prow * D + cc * 8);
    const float inv = mass > 0.0f ? 1.0f / mass : 0.0f;
    dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (lane == 0) lse_part[prow] = mass > 0.0f ? logf(mass) : -INFINITY;
}

// ------------------------------------------------------- one-launch form

// One block per query row does the three passes itself: its NW waves split
// the row's entries evenly for the logits (into LDS when the row fits, else
// into the row's scratch), the block finds tau over them (the same Newton
// steps), the waves fold p v over their entries again, and the block sums the
// waves' (sum p v, mass) and writes out = sum p v / mass and lse = ln mass.
// No partials, no logits round trip through memory for rows that fit, no
// merge launch.  Block ids are dealt so that the G query rows of one
// (request, kv head) run on one XCD (8, round-robin) and share its L2.
constexpr int kXcds = 8;
constexpr int kFusedLds = 8192;          // logits per row held in LDS (32 KiB)

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void entmax_fused_kernel(
    const float* __restrict__ q, int B, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, int64_t num_blocks, int P,
    const int32_t* __restrict__ bt, int64_t bt_ld, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
    const int32_t* __restrict__ sel_blk, int k_cap, int H_sel, float scale,
    const float* __restrict__ alibi, float* scratch, float* __restrict__ out,
    float* __restrict__ lse_out, float* __restrict__ tau_out) {
  constexpr int LPR = D / 8;
  constexpr int RPL = 64 / LPR;
  constexpr int NL = 16 / RPL;
  constexpr int BLOCK = NW * 64;
  __shared__ float z_lds[kFusedLds];
  __shared__ __align__(16) float part[NW][D];
  __shared__ float pmass[NW];
  __shared__ float red[2][NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int xcd = blockIdx.x % kXcds;
  const int64_t kk = blockIdx.x / kXcds;
  const int64_t grp = xcd + kXcds * (kk / G);
  if (grp >= static_cast<int64_t>(B) * H_kv) return;
  const int g = static_cast<int>(kk % G);
  const int h = static_cast<int>(grp % H_kv);
  const int b = static_cast<int>(grp / H_kv);
  const int i = h * G + g;
  const int64_t qrow = static_cast<int64_t>(b) * H_q + i;
  const int srow = H_sel == H_q ? static_cast<int>(qrow) : b * H_kv + h;
  const int S = seq_lens[b];
  int64_t Nb = (static_cast<int64_t>(S) + P - 1) / P;
  if (Nb > bt_ld) Nb = bt_ld;
  int cnt = sel_cnt[srow];
  cnt = cnt < 0 ? 0 : (cnt > k_cap ? k_cap : cnt);
  const int n = cnt * P;
  float* z = n <= kFusedLds ? z_lds : scratch + qrow * (static_cast<int64_t>(k_cap) * P);
  const float slope = alibi != nullptr ? alibi[i] : 0.0f;
  const int slot = lane / LPR, cc = lane % LPR;
  const int cap = (cnt + NW - 1) / NW;
  const int start = wave * cap;
  int len = cnt - start;
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int32_t* selr = sel_idx + static_cast<int64_t>(srow) * k_cap;
  const int32_t* sblk = sel_blk != nullptr ? sel_blk + static_cast<int64_t>(srow) * k_cap
                                           : nullptr;
  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;
  const int64_t row_stride = static_cast<int64_t>(H_kv) * D;
  const int64_t head_off = static_cast<int64_t>(h) * D + cc * 8;
  const int epg = 16 / P;

  // pass 1: logits of this wave's entries
  {
    uint32_t qh[4], ql[4];
    const float* qr = q + qrow * D + cc * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = qr[2 * j] * scale, x1 = qr[2 * j + 1] * scale;
      const uint16_t h0 = skv::f32_to_bf16(x0), h1 = skv::f32_to_bf16(x1);
      const uint16_t l0 = skv::f32_to_bf16(x0 - skv::bf16_to_f32(h0));
      const uint16_t l1 = skv::f32_to_bf16(x1 - skv::bf16_to_f32(h1));
      qh[j] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
      ql[j] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
    }
    for (int w0 = 0; w0 < len; w0 += 64) {
      const int nw = min(64, len - w0);
      int my_blk = 0, my_nv = 0, my_off = 0;
      if (lane < nw) {
        const int p = selr[start + w0 + lane];
        if (p >= 0 && p < Nb) {
          my_blk = sblk != nullptr ? sblk[start + w0 + lane] : btr[p];
          const int nr = S - p * P;
          my_nv = nr < P ? nr : P;
          my_off = p * P - (S - 1);
        }
      }
      const int ngroups = (nw + epg - 1) / epg;
      for (int grp16 = 0; grp16 < ngroups; ++grp16) {
        uint4 K[NL];
        bool ok[NL];
        int ent[NL], tt[NL], rel[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int rr = slot + RPL * j;
          const int e = grp16 * epg + rr / P;
          const int t = rr % P;
          const int ec = e < 64 ? e : 63;
          const int blk = __shfl(my_blk, ec);
          const int nv = __shfl(my_nv, ec);
          ok[j] = e < nw && t < nv;
          ent[j] = e;
          tt[j] = t;
          rel[j] = __shfl(my_off, ec) + t;
          const int64_t off = ok[j] ? (static_cast<int64_t>(blk) * P + t) * row_stride + head_off
                                    : head_off;
          K[j] = *reinterpret_cast<const uint4*>(kv + off);
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          float d = 0.0f;
          d = dot2e(K[j].x, qh[0], d); d = dot2e(K[j].x, ql[0], d);
          d = dot2e(K[j].y, qh[1], d); d = dot2e(K[j].y, ql[1], d);
          d = dot2e(K[j].z, qh[2], d); d = dot2e(K[j].z, ql[2], d);
          d = dot2e(K[j].w, qh[3], d); d = dot2e(K[j].w, ql[3], d);
          d = skv::group_sum<LPR>(d);
          if (alibi != nullptr) d = fmaf(slope, static_cast<float>(rel[j]), d);
          if (cc == 0 && ent[j] < nw)
            z[(start + w0 + ent[j]) * P + tt[j]] = ok[j] ? d : -INFINITY;
        }
      }
    }
  }
  __syncthreads();

  // pass 2: tau over the row's n logits (the separate tau pass's steps)
  float um = -INFINITY;
  for (int t = tid; t < n; t += BLOCK) um = fmaxf(um, 0.5f * z[t]);
  um = skv::wave_max(um);
  if (lane == 0) red[0][wave] = um;
  __syncthreads();
  um = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) um = fmaxf(um, red[0][w]);
  __syncthreads();
  float t0 = -INFINITY;
  if (um != -INFINITY) {
    t0 = um - 1.0f;
    for (int it = 0; it < 30; ++it) {
      float f = 0.0f, gg = 0.0f;
      for (int t = tid; t < n; t += BLOCK) {
        const float dd = 0.5f * z[t] - t0;
        if (dd > 0.0f) { f = fmaf(dd, dd, f); gg += dd; }
      }
      f = skv::wave_sum(f);
      gg = skv::wave_sum(gg);
      if (lane == 0) { red[0][wave] = f; red[1][wave] = gg; }
      __syncthreads();
      f = 0.0f; gg = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) { f += red[0][w]; gg += red[1][w]; }
      __syncthreads();
      f -= 1.0f;
      const float step = f / (2.0f * gg);
      if (!(step > 1e-7f * fmaxf(1.0f, fabsf(t0)))) {
        if (step > 0.0f) t0 += step;
        break;
      }
      t0 += step;
    }
  }

  // pass 3: sum p v over this wave's entries
  const int64_t v_off = num_blocks * P * row_stride;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  float mass = 0.0f;
  for (int w0 = 0; w0 < len && t0 != -INFINITY; w0 += 64) {
    const int nw = min(64, len - w0);
    int my_blk = 0, my_nv = 0;
    if (lane < nw) {
      const int p = selr[start + w0 + lane];
      if (p >= 0 && p < Nb) {
        my_blk = sblk != nullptr ? sblk[start + w0 + lane] : btr[p];
        const int nr = S - p * P;
        my_nv = nr < P ? nr : P;
      }
    }
    const int ngroups = (nw + epg - 1) / epg;
    for (int grp16 = 0; grp16 < ngroups; ++grp16) {
      float pr[NL];
      int64_t off[NL];
      bool any = false;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int rr = slot + RPL * j;
        const int e = grp16 * epg + rr / P;
        const int t = rr % P;
        const int ec = e < 64 ? e : 63;
        const int blk = __shfl(my_blk, ec);
        const int nv = __shfl(my_nv, ec);
        const bool ok = e < nw && t < nv;
        float pp = 0.0f;
        if (ok) {
          const float dd = 0.5f * z[(start + w0 + e) * P + t] - t0;
          pp = dd > 0.0f ? dd * dd : 0.0f;
        }
        pr[j] = pp;
        any |= pp > 0.0f;
        off[j] = pp > 0.0f ? (static_cast<int64_t>(blk) * P + t) * row_stride + head_off
                           : head_off;
      }
      if (__ballot(any) == 0ull) continue;
      uint4 V[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) V[j] = *reinterpret_cast<const uint4*>(kv + v_off + off[j]);
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        if (pr[j] > 0.0f) {
          float v[8];
          skv::unpack8(V[j], v);
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[c] = fmaf(pr[j], v[c], acc[c]);
          mass += pr[j];
        }
      }
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], o);
    mass += __shfl_xor(mass, o);
  }
  if (slot == 0) {
    float4* dst = reinterpret_cast<float4*>(&part[wave][cc * 8]);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (lane == 0) pmass[wave] = mass;
  __syncthreads();
  float m = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) m += pmass[w];
  const float inv = m > 0.0f ? 1.0f / m : 0.0f;
  for (int d = tid; d < D; d += BLOCK) {
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o += part[w][d];
    out[qrow * D + d] = o * inv;
  }
  if (tid == 0) {
    if (lse_out != nullptr) lse_out[qrow] = m > 0.0f ? logf(m) : -INFINITY;
    if (tau_out != nullptr) tau_out[qrow] = t0;
  }
}

}  // namespace

extern "C" int64_t entmax_scratch_floats(int B, int H_q, int k_cap, int page_size) {
  if (B < 0 || H_q <= 0 || k_cap <= 0 || page_size <= 0) return -1;
  const int64_t rows = static_cast<int64_t>(B) * H_q;
  return rows * k_cap * page_size + rows;
}

extern "C" int entmax15_paged_decode(const float* q, int B, int H_q, int H_kv, int D,
                                     const uint16_t* kv_cache, int64_t num_blocks,
                                     int page_size, const int32_t* block_table,
                                     int64_t bt_ld, const int32_t* seq_lens,
                                     const int32_t* sel_idx, const int32_t* sel_cnt,
                                     const int32_t* sel_blk, int k_cap, int H_sel,
                                     float scale, int num_splits,
                                     const float* alibi_slopes, float* o_part,
                                     float* lse_part, float* scratch,
                                     int64_t scratch_floats, hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "entmax15_paged_decode: need H_q a positive multiple of H_kv");
  const int G = H_q / H_kv;
  SKV_REQUIRE(D == 64 || D == 128, "entmax15_paged_decode: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "entmax15_paged_decode: page_size must be 1, 2, 4, 8 or 16 (got %d)", page_size);
  SKV_REQUIRE(H_sel == H_q || H_sel == H_kv,
              "entmax15_paged_decode: H_sel must be H_q or H_kv (got %d)", H_sel);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= 65535,
              "entmax15_paged_decode: num_splits must be in [1, 65535]");
  SKV_REQUIRE(k_cap >= 1 && num_blocks > 0 && bt_ld > 0,
              "entmax15_paged_decode: need k_cap >= 1, num_blocks > 0, bt_ld > 0");
  SKV_REQUIRE(scale > 0.0f, "entmax15_paged_decode: scale must be > 0");
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(q);
  SKV_REQUIRE_PTR(kv_cache);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(seq_lens);
  SKV_REQUIRE_PTR(sel_idx);
  SKV_REQUIRE_PTR(sel_cnt);
  SKV_REQUIRE_PTR(o_part);
  SKV_REQUIRE_PTR(lse_part);
  SKV_REQUIRE_PTR(scratch);
  const int64_t need = entmax_scratch_floats(B, H_q, k_cap, page_size);
  SKV_REQUIRE(scratch_floats >= need,
              "entmax15_paged_decode: scratch has %lld floats, needs %lld",
              (long long)scratch_floats, (long long)need);
  const int64_t rows = static_cast<int64_t>(B) * H_q;
  const int64_t waves = rows * num_splits;
  SKV_REQUIRE((waves + kWaves - 1) / kWaves <= 0x7fffffffLL && rows <= 0x7fffffffLL,
              "entmax15_paged_decode: grid too large");
  float* logits = scratch;
  float* tau = scratch + rows * k_cap * page_size;
  const dim3 g13(static_cast<unsigned>((waves + kWaves - 1) / kWaves));
  if (D == 128)
    hipLaunchKernelGGL(entmax_logits_kernel<128>, g13, dim3(kWaves * 64), 0, stream, q, B,
                       H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
                       seq_lens, sel_idx, sel_cnt, sel_blk, k_cap, H_sel, scale, num_splits,
                       alibi_slopes, logits);
  else
    hipLaunchKernelGGL(entmax_logits_kernel<64>, g13, dim3(kWaves * 64), 0, stream, q, B,
                       H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
                       seq_lens, sel_idx, sel_cnt, sel_blk, k_cap, H_sel, scale, num_splits,
                       alibi_slopes, logits);
  // few rows: wide blocks; rows of up to 8 logits a thread stay in registers
  const int64_t row_logits = static_cast<int64_t>(k_cap) * page_size;
  const bool wide = rows < 256;
  const int64_t in_regs = (wide ? 1024 : kTauThreads) * 8;
#define SKV_TAU(TH, RR)                                                                  \
  hipLaunchKernelGGL((entmax_tau_kernel<TH, RR>), dim3(static_cast<unsigned>(rows)),      \
                     dim3(TH), 0, stream, B, H_q, H_kv, G, page_size, sel_cnt, k_cap,    \
                     H_sel, logits, tau)
  if (wide) { if (row_logits <= in_regs) SKV_TAU(1024, 8); else SKV_TAU(1024, 0); }
  else { if (row_logits <= in_regs) SKV_TAU(kTauThreads, 8); else SKV_TAU(kTauThreads, 0); }
#undef SKV_TAU
  if (D == 128)
    hipLaunchKernelGGL(entmax_values_kernel<128>, g13, dim3(kWaves * 64), 0, stream, B, H_q,
                       H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
                       seq_lens, sel_idx, sel_cnt, sel_blk, k_cap, H_sel, num_splits,
                       logits, tau, o_part, lse_part);
  else
    hipLaunchKernelGGL(entmax_values_kernel<64>, g13, dim3(kWaves * 64), 0, stream, B, H_q,
                       H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
                       seq_lens, sel_idx, sel_cnt, sel_blk, k_cap, H_sel, num_splits,
                       logits, tau, o_part, lse_part);
  SKV_CHECK_LAUNCH();
}

extern "C" int entmax15_paged_decode_merged(
    const float* q, int B, int H_q, int H_kv, int D, const uint16_t* kv_cache,
    int64_t num_blocks, int page_size, const int32_t* block_table, int64_t bt_ld,
    const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
    const int32_t* sel_blk, int k_cap, int H_sel, float scale, const float* alibi_slopes,
    float* out, float* lse_out, float* tau_out, float* scratch, int64_t scratch_floats,
    hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "entmax15_paged_decode_merged: need H_q a positive multiple of H_kv");
  const int G = H_q / H_kv;
  SKV_REQUIRE(D == 64 || D == 128,
              "entmax15_paged_decode_merged: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "entmax15_paged_decode_merged: page_size must be 1, 2, 4, 8 or 16 (got %d)",
              page_size);
  SKV_REQUIRE(H_sel == H_q || H_sel == H_kv,
              "entmax15_paged_decode_merged: H_sel must be H_q or H_kv (got %d)", H_sel);
  SKV_REQUIRE(k_cap >= 1 && num_blocks > 0 && bt_ld > 0,
              "entmax15_paged_decode_merged: need k_cap >= 1, num_blocks > 0, bt_ld > 0");
  SKV_REQUIRE(scale > 0.0f, "entmax15_paged_decode_merged: scale must be > 0");
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(q);
  SKV_REQUIRE_PTR(kv_cache);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(seq_lens);
  SKV_REQUIRE_PTR(sel_idx);
  SKV_REQUIRE_PTR(sel_cnt);
  SKV_REQUIRE_PTR(out);
  const int64_t rows = static_cast<int64_t>(B) * H_q;
  const int64_t row_logits = static_cast<int64_t>(k_cap) * page_size;
  if (row_logits > kFusedLds) {
    SKV_REQUIRE(scratch != nullptr && scratch_floats >= rows * row_logits,
                "entmax15_paged_decode_merged: rows of %lld logits need a scratch of "
                "%lld floats", (long long)row_logits, (long long)(rows * row_logits));
  }
  const int64_t groups = static_cast<int64_t>(B) * H_kv;
  const int64_t blocks = (groups + kXcds - 1) / kXcds * kXcds * G;
  SKV_REQUIRE(blocks <= 0x7fffffffLL, "entmax15_paged_decode_merged: grid too large");
  // few rows: 16 waves per row keep more loads in flight
  const bool wide = rows * 8 < 2048;
#define SKV_EMF(DD, NWW)                                                                \
  hipLaunchKernelGGL((entmax_fused_kernel<DD, NWW>), dim3(static_cast<unsigned>(blocks)), \
                     dim3(NWW * 64), 0, stream, q, B, H_q, H_kv, G, kv_cache, num_blocks,  \
                     page_size, block_table, bt_ld, seq_lens, sel_idx, sel_cnt, sel_blk,   \
                     k_cap, H_sel, scale, alibi_slopes, scratch, out, lse_out, tau_out)
  if (D == 128) { if (wide) SKV_EMF(128, 16); else SKV_EMF(128, 8); }
  else { if (wide) SKV_EMF(64, 16); else SKV_EMF(64, 8); }
#undef SKV_EMF
  SKV_CHECK_LAUNCH();
}
