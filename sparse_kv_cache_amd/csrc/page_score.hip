// page_score.hip -- score every page of every request for every query head
// from the per-page statistics alone.
//
// Score: vortex_torch pull request "flow: add H2O sparse attention",
// "Page-level variants": average relevance q . mean(k) plus the peak bound
// sum_d max(q_d * max_d, q_d * min_d), combined as w_avg * avg + w_peak * peak.
// EntmaxKV README "How it works": pages are scored from their statistics,
// without touching the cached tokens.
//
// Arithmetic.  With mid = (max + min) / 2 and half = (max - min) / 2 >= 0,
//   max(q * max, q * min) = q * mid + |q| * half
// exactly, for either sign of q.  For bf16 envelopes mid and half are exact in
// fp32, so each dim contributes
//   q * (w_avg * mean + w_peak * mid) + |q| * (w_peak * half),
// two FMAs per (dim, query head) after a per-dim setup shared by the whole
// query group.
//
// Mapping.  One block per (tile of pages, kv head, request); a page-head's
// statistics (256 + 256 + 512 bytes at D = 128) are read by D/8 lanes with
// 16-byte loads, so a wave covers 64/(D/8) pages per load and every byte of
// statistics is read once for the whole query group, whose rows sit in LDS.
// Groups larger than 8 are split into slices of 8 (grid.x = kv head x slice).
#include "skv_device.h"
#include "skv_host.h"

namespace {

constexpr int kIter = 2;
// Waves per block: 4, or (per-head scores) 8 when the 4-wave grid is at most
// kWideGrid blocks (8 per CU: the whole grid resident at once), where fewer,
// larger blocks stage the query rows fewer times (long_context, 8,192 pages x
// 8 kv heads: 16.4 against 17.1-17.5 us; with ALiBi 16.9 against 18.5).
// Larger grids keep the finer 4-wave blocks (high_batch: 215.7 against 221.5
// us with 8), and so does the group score, whose one-row blocks have less to
// stage (long_context: 17.3 against 15.2 us with 8).
constexpr int kWideGrid = 2048;

template <int D, int GS, bool AGG, int NW>
__global__ __launch_bounds__(NW * 64) void page_score_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kmin, const uint16_t* __restrict__ kmax,
    const float* __restrict__ kmean, const int32_t* __restrict__ bt,
    int64_t bt_ld, const int32_t* __restrict__ seq_lens, int P, float w_avg,
    float w_peak, float* __restrict__ scores, int64_t score_ld,
    int64_t max_pages, const float* __restrict__ alibi) {
  constexpr int LPR = D / 8;          // lanes per page-head
  constexpr int PPW = 64 / LPR;       // page-heads per wave load
  constexpr int TILE = kIter * NW * PPW;
  // kv heads vary fastest in launch order: blocks dispatched together read
  // neighbouring statistics rows (all heads of a page are contiguous)
  const int b = blockIdx.z;
  const int nslices = AGG ? 1 : (G + GS - 1) / GS;
  const int h = blockIdx.x / nslices;
  const int g0 = (blockIdx.x % nslices) * GS;
  const int S = seq_lens[b];
  int64_t N = (static_cast<int64_t>(S) + P - 1) / P;
  if (N > max_pages) N = max_pages;
  const int64_t p0 = static_cast<int64_t>(blockIdx.y) * TILE;
  if (p0 >= N) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / LPR;
  const int c = lane % LPR;

  // ALiBi slope (score units) of the head this lane writes: the group's mean
  // for the group score
  float slope = 0.0f;
  if (alibi != nullptr) {
    if constexpr (AGG) {
      for (int g = 0; g < G; ++g) slope += alibi[h * G + g];
      slope /= static_cast<float>(G);
    } else {
      slope = c < GS && g0 + c < G ? alibi[h * G + g0 + c] : 0.0f;
    }
  }

  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;
  uint4 mn[kIter], mx[kIter];
  float4 me0[kIter], me1[kIter];
  int64_t pg[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    pg[it] = p0 + (it * NW + wave) * PPW + sub;
    // unconditional loads (pages past N read page p0's entry, whose result
    // is never stored) keep the count of loads in flight static
    const int64_t blk = btr[pg[it] < N ? pg[it] : p0];
    const int64_t off = (blk * H_kv + h) * D + c * 8;
    mn[it] = *reinterpret_cast<const uint4*>(kmin + off);
    mx[it] = *reinterpret_cast<const uint4*>(kmax + off);
    me0[it] = *reinterpret_cast<const float4*>(kmean + off);
    me1[it] = *reinterpret_cast<const float4*>(kmean + off + 4);
  }

  // while the statistics loads are in flight, the group's query rows go to
  // LDS, leaving the registers to those loads
  __shared__ __align__(16) float qs[AGG ? 2 : GS][D];
  if constexpr (AGG) {
    // The group's mean score is linear in (q, |q|) per dim:
    //   mean_g [q_g . mp + |q_g| . hp] = qbar . mp + mean_g|q_g| . hp
    // so one row of means and one of mean magnitudes replace the G rows.
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float sq = 0.0f, sa = 0.0f;
      for (int g = 0; g < G; ++g) {
        const float v = q[(static_cast<int64_t>(b) * H_q + h * G + g) * D + d];
        sq += v;
        sa += fabsf(v);
      }
      qs[0][d] = sq / static_cast<float>(G);
      qs[1][d] = sa / static_cast<float>(G);
    }
  } else {
    for (int i = threadIdx.x; i < GS * D; i += blockDim.x) {
      const int g = i / D, d = i % D;
      qs[g][d] = g0 + g < G ? q[(static_cast<int64_t>(b) * H_q + h * G + g0 + g) * D + d] : 0.0f;
    }
  }
  __syncthreads();

#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    float lo[8], hi[8];
    skv::unpack8(mn[it], lo);
    skv::unpack8(mx[it], hi);
    const float me[8] = {me0[it].x, me0[it].y, me0[it].z, me0[it].w,
                         me1[it].x, me1[it].y, me1[it].z, me1[it].w};
    // w_peak / 2 is exact, so folding it saves the two halvings
    const float wp2 = 0.5f * w_peak;
    float mp[8], hp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mp[i] = fmaf(wp2, hi[i] + lo[i], w_avg * me[i]);
      hp[i] = wp2 * (hi[i] - lo[i]);
    }
    // ALiBi at the page's last (peak term) and mean (mean term) valid
    // positions, relative to the query at S - 1
    float bias = 0.0f;
    if (alibi != nullptr) {
      const int64_t pp = pg[it] < N ? pg[it] : p0;
      const int64_t nn = static_cast<int64_t>(S) - pp * P;
      const float n = static_cast<float>(nn < P ? nn : P);
      const float first = static_cast<float>(pp * P - (S - 1));
      bias = slope * fmaf(w_avg, first + 0.5f * (n - 1.0f), w_peak * (first + n - 1.0f));
    }
    if constexpr (AGG) {
      const float4 qa = *reinterpret_cast<const float4*>(&qs[0][c * 8]);
      const float4 qb = *reinterpret_cast<const float4*>(&qs[0][c * 8 + 4]);
      const float4 aa = *reinterpret_cast<const float4*>(&qs[1][c * 8]);
      const float4 ab = *reinterpret_cast<const float4*>(&qs[1][c * 8 + 4]);
      const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      const float av[8] = {aa.x, aa.y, aa.z, aa.w, ab.x, ab.y, ab.z, ab.w};
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(qv[i], mp[i], fmaf(av[i], hp[i], s));
      s = skv::group_sum<LPR>(s);
      if (pg[it] < N && c == 0)
        scores[(static_cast<int64_t>(b) * H_kv + h) * score_ld + pg[it]] = s + bias;
    } else {
      float mine = 0.0f;
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const float4 qa = *reinterpret_cast<const float4*>(&qs[g][c * 8]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[g][c * 8 + 4]);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(qv[i], mp[i], fmaf(fabsf(qv[i]), hp[i], s));
        s = skv::group_sum<LPR>(s);
        if (c == g) mine = s;
      }
      if (pg[it] < N && c < GS && g0 + c < G)
        scores[(static_cast<int64_t>(b) * H_q + h * G + g0 + c) * score_ld + pg[it]] = mine + bias;
    }
  }
}

template <int D, int GS, bool AGG>
void launch_score(bool wide, dim3 grid, hipStream_t stream, const float* q, int H_q,
                  int H_kv, int G, const uint16_t* kmin, const uint16_t* kmax,
                  const float* kmean, const int32_t* bt, int64_t bt_ld,
                  const int32_t* seq_lens, int P, float w_avg, float w_peak,
                  float* scores, int64_t score_ld, int64_t max_pages,
                  const float* alibi) {
  if constexpr (!AGG) {
    if (wide) {
      hipLaunchKernelGGL((page_score_kernel<D, GS, AGG, 8>), grid, dim3(512), 0, stream, q,
                         H_q, H_kv, G, kmin, kmax, kmean, bt, bt_ld, seq_lens, P,
                         w_avg, w_peak, scores, score_ld, max_pages, alibi);
      return;
    }
  }
  hipLaunchKernelGGL((page_score_kernel<D, GS, AGG, 4>), grid, dim3(256), 0, stream, q,
                     H_q, H_kv, G, kmin, kmax, kmean, bt, bt_ld, seq_lens, P,
                     w_avg, w_peak, scores, score_ld, max_pages, alibi);
}

// Shared by both entry points: validation, grid, dispatch on (D, group size).
int score_pages(const char* who, bool group, const float* q, int B, int H_q,
                int H_kv, int D, const uint16_t* k_min, const uint16_t* k_max,
                const float* k_mean, const int32_t* block_table, int64_t bt_ld,
                const int32_t* seq_lens, int page_size, float w_avg, float w_peak,
                float* scores, int64_t score_ld, const float* alibi,
                hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv (H_q=%d, H_kv=%d)", who, H_q, H_kv);
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "%s: group size %d > 16", who, G);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", who, D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "%s: page_size must be 1, 2, 4, 8 or 16 (got %d)", who, page_size);
  SKV_REQUIRE(bt_ld > 0 && score_ld >= bt_ld,
              "%s: need bt_ld > 0 and score_ld >= bt_ld", who);
  SKV_REQUIRE(B <= 65535, "%s: grid too large", who);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(who, q);
  SKV_REQUIRE_PTR_W(who, k_min);
  SKV_REQUIRE_PTR_W(who, k_max);
  SKV_REQUIRE_PTR_W(who, k_mean);
  SKV_REQUIRE_PTR_W(who, block_table);
  SKV_REQUIRE_PTR_W(who, seq_lens);
  SKV_REQUIRE_PTR_W(who, scores);
  const int64_t max_pages = bt_ld;
  const int GS = group ? 1 : G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  const int slices = group ? 1 : (G + GS - 1) / GS;
  const int ppw = 64 / (D / 8);
  const int64_t tiles4 = (max_pages + kIter * 4 * ppw - 1) / (kIter * 4 * ppw);
  const bool wide = !group && static_cast<int64_t>(H_kv) * slices * tiles4 * B <= kWideGrid;
  const int tile = kIter * (wide ? 8 : 4) * ppw;
  const int64_t tiles = (max_pages + tile - 1) / tile;
  SKV_REQUIRE(tiles <= 65535, "%s: bt_ld %lld too long", who, (long long)bt_ld);
  dim3 grid(static_cast<unsigned>(H_kv * slices), static_cast<unsigned>(tiles),
            static_cast<unsigned>(B));
#define SKV_SCORE(DD, GG, AA)                                                    \
  launch_score<DD, GG, AA>(wide, grid, stream, q, H_q, H_kv, G, k_min, k_max,     \
                           k_mean, block_table, bt_ld, seq_lens, page_size,     \
                           w_avg, w_peak, scores, score_ld, max_pages, alibi)
  if (group) {
    if (D == 128) SKV_SCORE(128, 1, true); else SKV_SCORE(64, 1, true);
  } else if (D == 128) {
    if (GS == 1) SKV_SCORE(128, 1, false); else if (GS == 2) SKV_SCORE(128, 2, false);
    else if (GS == 4) SKV_SCORE(128, 4, false); else SKV_SCORE(128, 8, false);
  } else {
    if (GS == 1) SKV_SCORE(64, 1, false); else if (GS == 2) SKV_SCORE(64, 2, false);
    else if (GS == 4) SKV_SCORE(64, 4, false); else SKV_SCORE(64, 8, false);
  }
#undef SKV_SCORE
  SKV_CHECK_LAUNCH_W(who);
}

}  // namespace

extern "C" int page_score(const float* q, int B, int H_q, int H_kv, int D,
                          const uint16_t* k_min, const uint16_t* k_max,
                          const float* k_mean, const int32_t* block_table,
                          int64_t bt_ld, const int32_t* seq_lens, int page_size,
                          float w_avg, float w_peak, float* scores,
                          int64_t score_ld, hipStream_t stream) {
  return score_pages("page_score", false, q, B, H_q, H_kv, D, k_min, k_max, k_mean,
                     block_table, bt_ld, seq_lens, page_size, w_avg, w_peak, scores,
                     score_ld, nullptr, stream);
}

extern "C" int page_score_ex(const float* q, int B, int H_q, int H_kv, int D,
                             const uint16_t* k_min, const uint16_t* k_max,
                             const float* k_mean, const int32_t* block_table,
                             int64_t bt_ld, const int32_t* seq_lens, int page_size,
                             float w_avg, float w_peak, float* scores,
                             int64_t score_ld, const float* alibi, hipStream_t stream) {
  return score_pages("page_score_ex", false, q, B, H_q, H_kv, D, k_min, k_max, k_mean,
                     block_table, bt_ld, seq_lens, page_size, w_avg, w_peak, scores,
                     score_ld, alibi, stream);
}

extern "C" int page_score_group(const float* q, int B, int H_q, int H_kv, int D,
                                const uint16_t* k_min, const uint16_t* k_max,
                                const float* k_mean, const int32_t* block_table,
                                int64_t bt_ld, const int32_t* seq_lens,
                                int page_size, float w_avg, float w_peak,
                                float* scores, int64_t score_ld, const float* alibi,
                                hipStream_t stream) {
  return score_pages("page_score_group", true, q, B, H_q, H_kv, D, k_min, k_max,
                     k_mean, block_table, bt_ld, seq_lens, page_size, w_avg, w_peak,
                     scores, score_ld, alibi, stream);
}
