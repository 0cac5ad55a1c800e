// sparse_decode.hip -- split-K exact softmax attention over the tokens of the
// selected pages, gathered through the block table.
//
// EntmaxKV README "How it works": only the selected pages are attended to and
// the attention is exact over that selection.  vllm.cpp
// test_ops_mla_chunked_context.cpp: partial attention outputs with their
// log-sum-exps merge into the single-shot result (the merge is lse_merge).
//
// Mapping.  One block (4 waves) per (split, kv head, request).  A block owns
// split s of the selection row(s) of its kv head: with one selection per
// query head, the G rows of the group; with a selection shared by the group
// (token-level flow), one row.  Per round the block copies up to 256 entries
// of those rows into LDS and, for per-head rows, merges them: an entry is
// kept only at its first occurrence and carries a G-bit mask of the heads
// that selected it (binary search in the other heads' ascending rows).  So a
// page picked by several heads of the group is read from HBM once for all of
// them, and its block id is resolved once per round.
//
// Token rows are processed in groups of 16 (one page at page_size 16, or 16
// pages of fewer rows).  A token row of one kv head is D bf16 values = D/8
// lanes x 16 bytes, so a wave holds 64/(D/8) rows per load and each group
// takes 16/(64/(D/8)) 16-byte loads per lane for K and as many for V; the
// next group's loads are issued before the current one is computed.  The dot
// products reduce over the D/8 lanes of a row with DPP row moves; every lane
// keeps an online-softmax state (max, sum, 8-dim accumulator) per head of the
// group for its own rows, and the states are merged across row slots (lane
// shuffles) and across waves (LDS) only once, at the end.  Exponentials are
// base 2 with the scale pre-multiplied by log2(e).
#include "skv_device.h"
#include "skv_host.h"

namespace {

constexpr int kWaves = 4;
constexpr int kMaxEnt = 256;          // entries per round

struct RowLoad {
  uint4 k, v;
  uint32_t mask;                      // heads that attend this row
};

template <int D, int GMAX>
__global__ __launch_bounds__(256) void sparse_decode_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, int64_t num_blocks, int P,
    const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int k_cap, int shared_sel,
    float scale_log2, int num_splits, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  constexpr int LPR = D / 8;          // lanes per token row
  constexpr int RPL = 64 / LPR;       // rows per wave load
  constexpr int NL = 16 / RPL;        // loads per 16-row group
  constexpr int R = kMaxEnt / GMAX;   // entries per head per round

  __shared__ __align__(16) float qs[GMAX][D];
  __shared__ int32_t raw[GMAX][R];
  __shared__ int32_t e_blk[kMaxEnt];
  __shared__ int32_t e_nv[kMaxEnt];
  __shared__ uint32_t e_mask[kMaxEnt];
  __shared__ int scan_smem[kWaves + 1];
  __shared__ int s_len[GMAX], s_start[GMAX], s_rows[GMAX];
  __shared__ float red_m[kWaves][GMAX], red_l[kWaves][GMAX];
  __shared__ float red_acc[kWaves][GMAX][D];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPR, c = lane % LPR;
  const int S = seq_lens[b];
  int64_t Nb = (static_cast<int64_t>(S) + P - 1) / P;
  if (Nb > bt_ld) Nb = bt_ld;
  const int nrows = shared_sel ? 1 : G;      // selection rows of this block
  const uint32_t all_heads = (G >= 32) ? 0xffffffffu : ((1u << G) - 1u);

  for (int i = tid; i < GMAX * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    qs[g][d] = g < G ? q[(static_cast<int64_t>(b) * H_q + h * G + g) * D + d] * scale_log2
                     : 0.0f;
  }
  if (tid < GMAX) {
    int len = 0, start = 0, row = 0;
    if (tid < nrows) {
      row = shared_sel ? b * H_kv + h : b * H_q + h * G + tid;
      int cnt = sel_cnt[row];
      cnt = cnt < 0 ? 0 : (cnt > k_cap ? k_cap : cnt);
      const int chunk = (cnt + num_splits - 1) / num_splits;
      start = s * chunk;
      len = cnt - start;
      len = len < 0 ? 0 : (len > chunk ? chunk : len);
    }
    s_len[tid] = len;
    s_start[tid] = start;
    s_rows[tid] = row;
  }
  __syncthreads();
  int max_len = 0;
  for (int g = 0; g < nrows; ++g) max_len = max(max_len, s_len[g]);
  const int rounds = (max_len + R - 1) / R;

  // per-lane online softmax state, one per head of the group
  float m[GMAX], l[GMAX], acc[GMAX][8];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY; l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
  }

  const int64_t head_off = static_cast<int64_t>(h) * D + c * 8;
  const int64_t row_stride = static_cast<int64_t>(H_kv) * D;       // per token row
  const int64_t v_off = num_blocks * P * row_stride;               // V half

  for (int rd = 0; rd < rounds; ++rd) {
    // 1. copy this round's part of each row into LDS
    {
      const int g = tid / R, j = tid % R;
      if (g < GMAX) {
        int v = -1;
        if (g < nrows) {
          const int pos = rd * R + j;
          if (pos < s_len[g])
            v = sel_idx[static_cast<int64_t>(s_rows[g]) * k_cap + s_start[g] + pos];
        }
        raw[g][j] = v;
      }
    }
    __syncthreads();
    // 2. merge duplicates across the group, resolve block ids
    int keep = 0;
    int32_t my_blk = 0, my_nv = 0;
    uint32_t my_mask = 0;
    {
      const int g = tid / R, j = tid % R;
      int p = -1;
      if (g < nrows) p = raw[g][j];
      if (p >= 0 && p < Nb) {
        bool first = true;
        uint32_t mask = 1u << g;
        if (shared_sel) {
          mask = all_heads;
        } else {
          for (int g2 = 0; g2 < nrows; ++g2) {
            if (g2 == g) continue;
            int len2 = s_len[g2] - rd * R;
            len2 = len2 < 0 ? 0 : (len2 > R ? R : len2);
            int a = 0, z = len2;            // lower bound of p in raw[g2][0, len2)
            while (a < z) {
              const int mid = (a + z) >> 1;
              if (raw[g2][mid] < p) a = mid + 1; else z = mid;
            }
            if (a < len2 && raw[g2][a] == p) {
              mask |= 1u << g2;
              if (g2 < g) first = false;
            }
          }
        }
        if (first) {
          keep = 1;
          my_mask = mask;
          my_blk = bt[static_cast<int64_t>(b) * bt_ld + p];
          const int nv = S - p * P;
          my_nv = nv < P ? nv : P;
        }
      }
    }
    int nent;
    const int pos = skv::block_exclusive_scan(keep, &nent, scan_smem);
    if (keep) {
      e_blk[pos] = my_blk;
      e_nv[pos] = my_nv;
      e_mask[pos] = my_mask;
    }
    __syncthreads();

    // 3. attend: groups of 16 token rows
    const int epg = 16 / P;                       // entries per group
    const int ngroups = (nent + epg - 1) / epg;
    auto load = [&](int grp, RowLoad (&x)[NL]) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int rr = slot + RPL * j;            // row in group, 0..15
        const int e = grp * epg + rr / P;
        const int t = rr % P;
        x[j].mask = 0u;
        x[j].k = x[j].v = make_uint4(0, 0, 0, 0);
        if (grp < ngroups && e < nent && t < e_nv[e]) {
          const int64_t off = (static_cast<int64_t>(e_blk[e]) * P + t) * row_stride + head_off;
          x[j].mask = e_mask[e];
          x[j].k = *reinterpret_cast<const uint4*>(kv + off);
          x[j].v = *reinterpret_cast<const uint4*>(kv + v_off + off);
        }
      }
    };
    RowLoad cur[NL], nxt[NL];
    int grp = wave;
    load(grp, cur);
    while (grp < ngroups) {
      const int ngrp = grp + kWaves;
      load(ngrp, nxt);
      float kf[NL][8], vf[NL][8];
      uint32_t any_mask = 0u;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        skv::unpack8(cur[j].k, kf[j]);
        skv::unpack8(cur[j].v, vf[j]);
        any_mask |= cur[j].mask;
      }
      // heads attended by any row of the group, uniform across the wave
      uint32_t gm = any_mask;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) gm |= __shfl_xor(gm, o);
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g >= G || !((gm >> g) & 1u)) continue;
        const float4 qa = *reinterpret_cast<const float4*>(&qs[g][c * 8]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[g][c * 8 + 4]);
        const float qq[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        float lg[NL];
        float mx = m[g];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          float d = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) d = fmaf(qq[i], kf[j][i], d);
          d = skv::group_sum<LPR>(d);
          lg[j] = ((cur[j].mask >> g) & 1u) ? d : -INFINITY;
          mx = fmaxf(mx, lg[j]);
        }
        if (mx == -INFINITY) continue;            // none of my rows yet
        const float alpha = exp2f(m[g] - mx);     // 0 when m[g] == -inf
        float ps = 0.0f;
        float pj[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) { pj[j] = exp2f(lg[j] - mx); ps += pj[j]; }
        l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float a = acc[g][i] * alpha;
#pragma unroll
          for (int j = 0; j < NL; ++j) a = fmaf(pj[j], vf[j][i], a);
          acc[g][i] = a;
        }
        m[g] = mx;
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) cur[j] = nxt[j];
      grp = ngrp;
    }
    __syncthreads();                              // LDS lists reused next round
  }

  // 4. merge the row slots of the wave (lanes c, c+LPR, ...)
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) continue;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m[g], o);
      const float l2 = __shfl_xor(l[g], o);
      const float mx = fmaxf(m[g], m2);
      const float a = mx == -INFINITY ? 0.0f : exp2f(m[g] - mx);
      const float bb = mx == -INFINITY ? 0.0f : exp2f(m2 - mx);
      l[g] = l[g] * a + l2 * bb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a2 = __shfl_xor(acc[g][i], o);
        acc[g][i] = acc[g][i] * a + a2 * bb;
      }
      m[g] = mx;
    }
    if (slot == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red_acc[wave][g][c * 8 + i] = acc[g][i];
      if (c == 0) { red_m[wave][g] = m[g]; red_l[wave][g] = l[g]; }
    }
  }
  __syncthreads();

  // 5. merge the waves and write the split's partial
  for (int i = tid; i < G * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][g]);
    const int64_t prow = (static_cast<int64_t>(b) * H_q + h * G + g) * num_splits + s;
    if (M == -INFINITY) {
      o_part[prow * D + d] = 0.0f;
      if (d == 0) lse_part[prow] = -INFINITY;
      continue;
    }
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = exp2f(red_m[w][g] - M);
      L = fmaf(red_l[w][g], e, L);
      A = fmaf(red_acc[w][g][d], e, A);
    }
    o_part[prow * D + d] = A / L;
    if (d == 0) lse_part[prow] = (M + log2f(L)) * skv::kLn2;
  }
}

template <int D, int GMAX>
void launch_decode(dim3 grid, hipStream_t stream, const float* q, int H_q,
                   int H_kv, int G, const uint16_t* kv, int64_t num_blocks,
                   int P, const int32_t* bt, int64_t bt_ld,
                   const int32_t* seq_lens, const int32_t* sel_idx,
                   const int32_t* sel_cnt, int k_cap, int shared_sel,
                   float scale_log2, int num_splits, float* o_part,
                   float* lse_part) {
  hipLaunchKernelGGL((sparse_decode_kernel<D, GMAX>), grid, dim3(kWaves * 64), 0,
                     stream, q, H_q, H_kv, G, kv, num_blocks, P, bt, bt_ld,
                     seq_lens, sel_idx, sel_cnt, k_cap, shared_sel, scale_log2,
                     num_splits, o_part, lse_part);
}

}  // namespace

extern "C" int sparse_paged_decode(const float* q, int B, int H_q, int H_kv,
                                   int D, const uint16_t* kv_cache,
                                   int64_t num_blocks, int page_size,
                                   const int32_t* block_table, int64_t bt_ld,
                                   const int32_t* seq_lens,
                                   const int32_t* sel_idx,
                                   const int32_t* sel_cnt, int k_cap,
                                   int H_sel, float scale, int num_splits,
                                   float* o_part, float* lse_part,
                                   hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "sparse_paged_decode: need H_q a positive multiple of H_kv");
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "sparse_paged_decode: group size %d > 16", G);
  SKV_REQUIRE(D == 64 || D == 128, "sparse_paged_decode: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "sparse_paged_decode: page_size must be 1, 2, 4, 8 or 16 (got %d)", page_size);
  SKV_REQUIRE(H_sel == H_q || H_sel == H_kv,
              "sparse_paged_decode: H_sel must be H_q or H_kv (got %d)", H_sel);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= 65535,
              "sparse_paged_decode: num_splits must be in [1, 65535]");
  SKV_REQUIRE(k_cap >= 1 && num_blocks > 0 && bt_ld > 0,
              "sparse_paged_decode: need k_cap >= 1, num_blocks > 0, bt_ld > 0");
  SKV_REQUIRE(num_blocks <= 0x7fffffffLL,
              "sparse_paged_decode: pool too large for 32-bit block ids");
  SKV_REQUIRE(B <= 65535 && H_kv <= 65535, "sparse_paged_decode: grid too large");
  SKV_REQUIRE_PTR(q);
  SKV_REQUIRE_PTR(kv_cache);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(seq_lens);
  SKV_REQUIRE_PTR(sel_idx);
  SKV_REQUIRE_PTR(sel_cnt);
  SKV_REQUIRE_PTR(o_part);
  SKV_REQUIRE_PTR(lse_part);
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  const int shared_sel = (H_sel == H_kv && G > 1) ? 1 : 0;
  const int GM = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
  dim3 grid(static_cast<unsigned>(num_splits), static_cast<unsigned>(H_kv),
            static_cast<unsigned>(B));
  const float scale_log2 = scale * skv::kLog2e;
#define SKV_DEC(DD, GG)                                                         \
  launch_decode<DD, GG>(grid, stream, q, H_q, H_kv, G, kv_cache, num_blocks,     \
                        page_size, block_table, bt_ld, seq_lens, sel_idx,       \
                        sel_cnt, k_cap, shared_sel, scale_log2, num_splits,     \
                        o_part, lse_part)
  if (D == 128) {
    if (GM == 1) SKV_DEC(128, 1); else if (GM == 2) SKV_DEC(128, 2);
    else if (GM == 4) SKV_DEC(128, 4); else if (GM == 8) SKV_DEC(128, 8);
    else SKV_DEC(128, 16);
  } else {
    if (GM == 1) SKV_DEC(64, 1); else if (GM == 2) SKV_DEC(64, 2);
    else if (GM == 4) SKV_DEC(64, 4); else if (GM == 8) SKV_DEC(64, 8);
    else SKV_DEC(64, 16);
  }
#undef SKV_DEC
  SKV_CHECK_LAUNCH();
}
