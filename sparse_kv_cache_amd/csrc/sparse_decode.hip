// sparse_decode.hip -- split-K exact softmax attention over the tokens of the
// selected pages, gathered through the block table.
//
// EntmaxKV README "How it works": only the selected pages are attended to and
// the attention is exact over that selection.  vllm.cpp
// test_ops_mla_chunked_context.cpp: partial attention outputs with their
// log-sum-exps merge into the single-shot result (the merge is lse_merge).
//
// Common layout.  A token row of one kv head is D bf16 values = D/8 lanes x
// 16 bytes, so a wave holds 64/(D/8) rows per load and a group of 16 token
// rows (one page at page_size 16, or 16/P pages) takes NL = 16/(64/(D/8))
// 16-byte loads per lane for K and as many for V.  Dot products reduce over
// the D/8 lanes of a row with DPP row moves.  Every lane keeps an online
// softmax state (max, sum, 8-dim accumulator) for its own rows; states are
// merged across row slots (lane shuffles) and waves (LDS) once, at the end.
// Exponentials are base 2 with the scale pre-multiplied by log2(e).  Loads run
// one group ahead of the arithmetic (packed bf16 in registers, unpacked on
// use), so each wave keeps up to 2 x 2 x 4 KB of K/V in flight.
//
// Split s of a selection row holds its entries [s*c, min((s+1)*c, cnt)) with
// c = ceil(k_cap / num_splits), so a block can fetch its chunk without first
// reading the count.
//
// Two mappings:
//  * wave kernel (one selection per query head): one wave per (request,
//    query head, split); the per-lane state is one head's, which leaves the
//    registers to the load pipeline and 4 waves per SIMD.  A page that
//    several heads of a group selected is fetched by each of their waves at
//    about the same time on one CU and served by L2 after the first read.
//  * group kernel (one selection shared by the group: the token-level flow
//    and group-shared page selection): one block per (split, kv head,
//    request); each wave walks part of the shared chunk once and applies
//    every query head of the group to the rows it loaded, on the matrix
//    cores.
#include <stdlib.h>
#include <string.h>

#include "skv_device.h"
#include "skv_host.h"
#include "skv_topk.h"

namespace {

constexpr int kMaxEnt = 256;          // LDS entries per round (group kernel)
#ifndef SKV_SCORE_KI
#define SKV_SCORE_KI 2                // pages in flight per lane, in-block scoring
#endif
constexpr int kXcds = 8;              // accelerator complex dies of an MI355X
#ifndef SKV_DECODE_WPE
#define SKV_DECODE_WPE 3              // waves per SIMD the wave kernel is sized for
#endif
#ifndef SKV_DECODE_WPE16
#define SKV_DECODE_WPE16 3            // same, page_size 16 path
#endif
#ifndef SKV_DECODE_WPE_ALONE
#define SKV_DECODE_WPE_ALONE 6        // the standalone page_size 16 decode (one page in flight)
#endif

// One head, one group of 16 token rows: fold the rows' logits and values into
// the lane's online-softmax state.  The query is split into bf16 hi + lo
// halves (q ~= hi + lo to about 16 significant bits): each dot product runs on
// the packed bf16 key words with v_dot2c_f32_bf16 (fp32 accumulation, exact
// bf16 products), so keys are never unpacked.  Rows with ok == false were
// loaded from a placeholder address: their logits are replaced and their
// values never multiplied.  `full` (wave-uniform) says every row is valid.
typedef __bf16 skv_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(skv_bf16x2, a),
                                         __builtin_bit_cast(skv_bf16x2, b), c, false);
}

__device__ __forceinline__ void split_query(const float (&qq)[8], uint32_t (&qh)[4],
                                            uint32_t (&ql)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t h0 = skv::f32_to_bf16(qq[2 * i]), h1 = skv::f32_to_bf16(qq[2 * i + 1]);
    const uint16_t l0 = skv::f32_to_bf16(qq[2 * i] - skv::bf16_to_f32(h0));
    const uint16_t l1 = skv::f32_to_bf16(qq[2 * i + 1] - skv::bf16_to_f32(h1));
    qh[i] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
    ql[i] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
  }
}

// With AL, row j's logit also gets slope2 * pos[j] (ALiBi, base-2 units;
// pos = key position - query position <= 0).
template <int LPR, int NL, bool AL>
__device__ __forceinline__ void attend_rows_split(const uint32_t (&qh)[4],
                                                  const uint32_t (&ql)[4],
                                                  const uint4 (&K)[NL],
                                                  const uint4 (&V)[NL],
                                                  const bool (&ok)[NL], bool full,
                                                  const float (&pos)[NL], float slope2,
                                                  float& m, float& l,
                                                  float (&acc)[8]) {
  float lg[NL];
  float mx = m;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    float d = 0.0f;
    d = dot2(K[j].x, qh[0], d); d = dot2(K[j].x, ql[0], d);
    d = dot2(K[j].y, qh[1], d); d = dot2(K[j].y, ql[1], d);
    d = dot2(K[j].z, qh[2], d); d = dot2(K[j].z, ql[2], d);
    d = dot2(K[j].w, qh[3], d); d = dot2(K[j].w, ql[3], d);
    d = skv::group_sum<LPR>(d);
    if constexpr (AL) d = fmaf(slope2, pos[j], d);   // after the row sum
    lg[j] = ok[j] ? d : -INFINITY;
    mx = fmaxf(mx, lg[j]);
  }
  if (mx == -INFINITY) return;            // none of this lane's rows yet
  const float alpha = __builtin_amdgcn_exp2f(m - mx);   // 0 while m == -inf
  float pj[NL];
  float ps = 0.0f;
#pragma unroll
  for (int j = 0; j < NL; ++j) { pj[j] = __builtin_amdgcn_exp2f(lg[j] - mx); ps += pj[j]; }
  l = fmaf(l, alpha, ps);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] *= alpha;
  if (full) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      float v[8];
      skv::unpack8(V[j], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(pj[j], v[i], acc[i]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      // masked rows: zero the packed words (never multiply a placeholder row)
      const uint4 vw = ok[j] ? V[j] : make_uint4(0, 0, 0, 0);
      float v[8];
      skv::unpack8(vw, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(pj[j], v[i], acc[i]);
    }
  }
  m = mx;
}

// Merge the online-softmax states of the 64/LPR row slots of a wave (lanes
// c, c + LPR, ...); afterwards every lane holds the wave's state for its dims.
template <int LPR>
__device__ __forceinline__ void merge_slots(float& m, float& l, float (&acc)[8]) {
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(m, o);
    const float l2 = __shfl_xor(l, o);
    const float mx = fmaxf(m, m2);
    const float a = mx == -INFINITY ? 0.0f : exp2f(m - mx);
    const float b = mx == -INFINITY ? 0.0f : exp2f(m2 - mx);
    l = l * a + l2 * b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a2 = __shfl_xor(acc[i], o);
      acc[i] = acc[i] * a + a2 * b;
    }
    m = mx;
  }
}

struct Chunk {
  int start, len;
};

__device__ __forceinline__ Chunk split_chunk(int cnt, int k_cap, int num_splits, int s) {
  cnt = cnt < 0 ? 0 : (cnt > k_cap ? k_cap : cnt);
  const int c = (k_cap + num_splits - 1) / num_splits;
  const int start = s * c;
  int len = cnt - start;
  len = len < 0 ? 0 : (len > c ? c : len);
  return {start, len};
}

// ------------------------------------------------------------- wave kernel

// One wave per (request, query head, split) chunk.  Waves are independent: no
// LDS and no barriers.  Lane j of a wave holds entry j of the chunk (its block
// id and valid row count, fetched once); the rows of a 16-row group take
// their block ids from those lanes with a permute.  Within a (request, kv
// head) the chunks are numbered s * G + g, so the query heads of one split
// share a block, and all blocks of the (request, kv head) go to one XCD:
// pages several heads selected are fetched through one L2 at about the same
// time.
//
// FUSE: one block per query head, wave w = split w (num_splits <= WB); the
// block merges its splits' states through LDS and writes the merged output
// and lse itself (the lse_merge algebra), so no separate merge launch is
// needed.  Partials are still written when o_part / lse_part are given.
// In-block selection (TKI > 0, with FUSE): the block first runs the top-k of
// its query head's score row (TKI entries per thread) into LDS, then decodes
// from there; the selection is copied out only when asked.
// With SC as well, the block also scores its query head's pages from the page
// statistics first (the page score, into LDS; one query head per block, so
// the peak term picks each dim's envelope by the query's sign), so one launch
// runs the whole page-level step.
struct TopkArgs {
  const float* scores; int64_t score_ld; int topk_pages; double topk_frac;
  int bos, eos; int32_t* sel_idx; int32_t* sel_cnt; int32_t* sel_blk;
  // in-block scoring (SC)
  const uint16_t* kmin; const uint16_t* kmax; const float* kmean;
  float w_avg, w_peak, inv_scale; int sc_cap; float* scores_out;
  // in-block accumulator update (token level): the logits pass's output
  const float* h_logits; const float* h_part; const uint16_t* h_snap; uint16_t* h_hh;
  int h_nchunk, h_chunk; float h_decay;
  // split decode with in-block selection: nonzero merges each block's splits
  // and writes one partial per block instead of one per split
  int block_partials;
};

// Bits [0, x) set (x clipped to [0, 32]).
__device__ __forceinline__ uint32_t low_bits_u(int x) {
  return x <= 0 ? 0u : x >= 32 ? 0xffffffffu : ((1u << x) - 1u);
}

// (max, sum) fold of two softmax partials in base 2, as the accumulator's
// update pass folds them (same operations, same order).
__device__ __forceinline__ void fold_max_sum(float& m, float& z, float m2, float z2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; z = z2; return; }
  const float M = fmaxf(m, m2);
  z = z * exp2f(m - M) + z2 * exp2f(m2 - M);
  m = M;
}

template <int D, int WB, int PFIX, bool AL, bool FUSE, int TKI, bool SC = false>
__global__ __launch_bounds__(WB * 64)
__attribute__((amdgpu_waves_per_eu((!FUSE && TKI == 0 && PFIX == 16) ? SKV_DECODE_WPE_ALONE
                                   : PFIX == 16 ? SKV_DECODE_WPE16 : SKV_DECODE_WPE)))
void sparse_decode_wave_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, int64_t num_blocks, int P,
    const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, const int32_t* __restrict__ sel_blk,
    int k_cap, float scale_log2, int num_splits, float* __restrict__ o_part,
    float* __restrict__ lse_part, int64_t n_groups, int blocks_per_group,
    const float* __restrict__ alibi, float* __restrict__ out,
    float* __restrict__ lse_out, TopkArgs ta) {
  static_assert(!SC || (TKI > 0 && FUSE), "in-block scoring selects and merges in-block");
  constexpr int LPR = D / 8;
  constexpr int RPL = 64 / LPR;
  constexpr int NL = 16 / RPL;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Blocks are dealt to the 8 XCDs round-robin by id; block id -> (xcd, k)
  // -> (request/kv-head group, block within the group) so that every block of
  // one (request, kv head) runs on the same XCD and shares its L2.
  const int xcd = blockIdx.x % kXcds;
  const int64_t k = blockIdx.x / kXcds;
  const int64_t grp_bh = xcd + kXcds * (k / blocks_per_group);
  const int local = static_cast<int>(k % blocks_per_group) * WB + wave;
  // In-block selection (TKI > 0): a block serves one query head, its waves
  // consecutive splits; a head's splits take blocks_per_group / G blocks
  // (one with FUSE).  Whole blocks return together; waves past num_splits
  // stay for the selection's barriers (and FUSE's merge) with an empty chunk.
  if (grp_bh >= n_groups || (!FUSE && TKI == 0 && local >= num_splits * G)) return;
  const int nsg = TKI > 0 ? blocks_per_group / G : 1;   // blocks per query head
  const int kb = static_cast<int>(k % blocks_per_group);
  const int g = TKI > 0 ? kb / nsg : FUSE ? kb : local % G;
  const int s = TKI > 0 ? (kb % nsg) * WB + wave : FUSE ? wave : local / G;
  const int h = static_cast<int>(grp_bh % H_kv);
  const int b = static_cast<int>(grp_bh / H_kv);
  const int64_t qrow = static_cast<int64_t>(b) * H_q + h * G + g;
  const int slot = lane / LPR, c = lane % LPR;
  const int S = seq_lens[b];
  int64_t Nb = (static_cast<int64_t>(S) + P - 1) / P;
  if (Nb > bt_ld) Nb = bt_ld;
  // The chunk's place in the row depends only on k_cap, so its entries (and
  // block ids, when the selection carries them) are fetched together with the
  // count instead of after it.
  const int cap = (k_cap + num_splits - 1) / num_splits;
  const int start = s * cap;
  // entries of this chunk that exist in the row: the last chunks of a row
  // whose capacity is not a multiple of num_splits (or is below it) are
  // shorter or empty, and nothing past the row's k_cap entries is read
  int avail = k_cap - start;
  avail = avail < 0 ? 0 : (avail > cap ? cap : avail);
  const int32_t* selr;
  const int32_t* sblk;
  int cnt;
  if constexpr (TKI > 0) {
    // dynamic LDS: [SC: sc_cap scores, sc_cap block ids] [k_cap indices, k_cap blocks]
    extern __shared__ int32_t dyn_lds[];
    int32_t* sel_lds = SC ? dyn_lds + 2 * ta.sc_cap : dyn_lds;
    if constexpr (SC) {
      float* sc_lds = reinterpret_cast<float*>(dyn_lds);
      int32_t* bid_lds = dyn_lds + ta.sc_cap;
      int64_t Nt64 = (static_cast<int64_t>(S) + P - 1) / P;
      if (Nt64 > bt_ld) Nt64 = bt_ld;
      const int Nt = static_cast<int>(Nt64);
      const int32_t* btr0 = bt + static_cast<int64_t>(b) * bt_ld;
      for (int j = threadIdx.x; j < Nt; j += WB * 64) bid_lds[j] = btr0[j];
      float qv[8];
      {
        const float4 qa = *reinterpret_cast<const float4*>(q + qrow * D + c * 8);
        const float4 qb = *reinterpret_cast<const float4*>(q + qrow * D + c * 8 + 4);
        qv[0] = qa.x; qv[1] = qa.y; qv[2] = qa.z; qv[3] = qa.w;
        qv[4] = qb.x; qv[5] = qb.y; qv[6] = qb.z; qv[7] = qb.w;
      }
      // ALiBi in score units: slope / softmax scale
      const float sslope = AL ? alibi[h * G + g] * ta.inv_scale : 0.0f;
      // The peak term taken as written: dim d contributes q_d * max_d where
      // q_d >= 0 and q_d * min_d elsewhere.  This lane's dims are fixed, so
      // the choice is a bit mask per packed pair of bf16 envelope values (one
      // bitfield select per two dims), and the weights fold into the query.
      float qa[8], qp[8];
      uint32_t env_mask[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qa[i] = ta.w_avg * qv[i];
        qp[i] = ta.w_peak * qv[i];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        env_mask[k] = (qv[2 * k] >= 0.0f ? 0x0000ffffu : 0u) |
                      (qv[2 * k + 1] >= 0.0f ? 0xffff0000u : 0u);
      __syncthreads();
      constexpr int KI = SKV_SCORE_KI;            // page loads in flight per lane
      for (int p0 = 0; p0 < Nt; p0 += WB * RPL * KI) {
        uint4 mn[KI], mx[KI];
        float4 me0[KI], me1[KI];
        int pg[KI];
#pragma unroll
        for (int it = 0; it < KI; ++it) {
          pg[it] = p0 + (it * WB + wave) * RPL + slot;
          const int64_t blk = bid_lds[pg[it] < Nt ? pg[it] : 0];
          const int64_t off = (blk * H_kv + h) * D + c * 8;
          mn[it] = *reinterpret_cast<const uint4*>(ta.kmin + off);
          mx[it] = *reinterpret_cast<const uint4*>(ta.kmax + off);
          me0[it] = *reinterpret_cast<const float4*>(ta.kmean + off);
          me1[it] = *reinterpret_cast<const float4*>(ta.kmean + off + 4);
        }
#pragma unroll
        for (int it = 0; it < KI; ++it) {
          const float me[8] = {me0[it].x, me0[it].y, me0[it].z, me0[it].w,
                               me1[it].x, me1[it].y, me1[it].z, me1[it].w};
          const uint32_t mnw[4] = {mn[it].x, mn[it].y, mn[it].z, mn[it].w};
          const uint32_t mxw[4] = {mx[it].x, mx[it].y, mx[it].z, mx[it].w};
          float s_env = 0.0f, s_avg = 0.0f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t e = (mxw[k] & env_mask[k]) | (mnw[k] & ~env_mask[k]);
            s_env = fmaf(qp[2 * k], __uint_as_float(e << 16), s_env);
            s_env = fmaf(qp[2 * k + 1], __uint_as_float(e & 0xffff0000u), s_env);
            s_avg = fmaf(qa[2 * k], me[2 * k], s_avg);
            s_avg = fmaf(qa[2 * k + 1], me[2 * k + 1], s_avg);
          }
          float sc = skv::group_sum<LPR>(s_env + s_avg);
          if (AL) {
            const int pp = pg[it] < Nt ? pg[it] : 0;
            const int nn = S - pp * P;
            const float n = static_cast<float>(nn < P ? nn : P);
            const float first = static_cast<float>(pp * P - (S - 1));
            sc += sslope * fmaf(ta.w_avg, first + 0.5f * (n - 1.0f),
                                ta.w_peak * (first + n - 1.0f));
          }
          if (c == 0 && pg[it] < Nt) {
            sc_lds[pg[it]] = sc;
            if (ta.scores_out != nullptr) ta.scores_out[qrow * ta.score_ld + pg[it]] = sc;
          }
        }
      }
      __syncthreads();
      cnt = skv::topk_row<WB * 64, TKI>(sc_lds, true, Nt, ta.topk_pages, ta.topk_frac,
                                        ta.bos, ta.eos, bid_lds, ta.sc_cap, sel_lds,
                                        sel_lds + k_cap, k_cap);
    } else {
    int64_t Nt = (static_cast<int64_t>(S) + P - 1) / P;
    if (Nt > ta.score_ld) Nt = ta.score_ld;
    const bool aligned = ((ta.score_ld & 3) == 0) &&
                         ((reinterpret_cast<uintptr_t>(ta.scores) & 15) == 0);
    cnt = skv::topk_row<WB * 64, TKI>(
        ta.scores + qrow * ta.score_ld, aligned, static_cast<int>(Nt), ta.topk_pages,
        ta.topk_frac, ta.bos, ta.eos, bt + static_cast<int64_t>(b) * bt_ld, bt_ld,
        sel_lds, sel_lds + k_cap, k_cap);
    }
    if (ta.sel_idx != nullptr && kb % nsg == 0) {
      for (int j = threadIdx.x; j < k_cap; j += WB * 64) {
        ta.sel_idx[qrow * k_cap + j] = sel_lds[j];
        if (ta.sel_blk != nullptr) ta.sel_blk[qrow * k_cap + j] = sel_lds[k_cap + j];
      }
      if (threadIdx.x == 0) ta.sel_cnt[qrow] = cnt;
    }
    selr = sel_lds + start;
    sblk = sel_lds + k_cap + start;
  } else {
    selr = sel_idx + qrow * k_cap + start;
    sblk = sel_blk != nullptr ? sel_blk + qrow * k_cap + start : nullptr;
    cnt = sel_cnt[qrow];
    cnt = cnt < 0 ? 0 : (cnt > k_cap ? k_cap : cnt);
  }
  int clen = cnt - start;
  clen = clen < 0 ? 0 : (clen > cap ? cap : clen);

  float qq[8];
  {
    const float4 qa = *reinterpret_cast<const float4*>(q + qrow * D + c * 8);
    const float4 qb = *reinterpret_cast<const float4*>(q + qrow * D + c * 8 + 4);
    qq[0] = qa.x * scale_log2; qq[1] = qa.y * scale_log2;
    qq[2] = qa.z * scale_log2; qq[3] = qa.w * scale_log2;
    qq[4] = qb.x * scale_log2; qq[5] = qb.y * scale_log2;
    qq[6] = qb.z * scale_log2; qq[7] = qb.w * scale_log2;
  }
  uint32_t qh[4], ql[4];
  split_query(qq, qh, ql);
  // ALiBi slope of this head in base-2 logit units.  Biases are taken
  // relative to the chunk's last selected page (the largest bias, where the
  // weight concentrates), so the fold works with small, exact offsets; the
  // common offset returns in the split's lse.
  const float slope2 = AL ? alibi[h * G + g] * skv::kLog2e : 0.0f;
  int pref = 0;
  if (AL && clen > 0) pref = selr[clen - 1];
  float m = -INFINITY, l = 0.0f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;

  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;
  const int head_off = h * D + c * 8;   // < H_kv * D: 32 bits
  const int64_t row_stride = static_cast<int64_t>(H_kv) * D;
  const int64_t v_off = num_blocks * P * row_stride;
  const int epg = 16 / P;

  for (int w0 = 0; w0 < avail; w0 += 64) {
    int p = -1, sb = -1;
    if (w0 + lane < avail) {
      p = selr[w0 + lane];
      if (sblk != nullptr) sb = sblk[w0 + lane];
    }
    const int nw = min(64, clen - w0);
    if (nw <= 0) break;
    int my_blk = 0, my_nv = 0, my_pg = 0;
    if (lane < nw && p >= 0 && p < Nb) {
      my_pg = p;
      my_blk = sblk != nullptr ? sb : btr[p];
      const int n = S - p * P;
      my_nv = n < P ? n : P;
    }
    const int ngroups = (nw + epg - 1) / epg;
    // pos (ALiBi only): key position minus the query's (S - 1), per row
    auto load = [&](int grp, uint4 (&K)[NL], uint4 (&V)[NL], bool (&ok)[NL], bool& full,
                    float (&pos)[NL]) {
      if constexpr (PFIX == 16) {
        // one page per group: its block id and row count are wave-uniform
        // (read from lane grp), so the row addresses are a scalar page base
        // plus a per-lane constant
        const int gc = grp < nw ? grp : 0;
        const int blk = __builtin_amdgcn_readlane(my_blk, gc);
        const int nv = grp < nw ? __builtin_amdgcn_readlane(my_nv, gc) : 0;
        full = nv == 16;
        if constexpr (AL) {
          const int pg = __builtin_amdgcn_readlane(my_pg, gc);
#pragma unroll
          for (int j = 0; j < NL; ++j)
            pos[j] = static_cast<float>((pg - pref) * 16 + slot + RPL * j);
        }
        // masked rows read row 0 of the same page (every page listed has
        // one, and an invalid entry reads block 0): the base stays scalar
        const uint16_t* kp = kv + static_cast<int64_t>(blk) * 16 * row_stride;
        const uint16_t* vp = kp + v_off;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int t = slot + RPL * j;
          ok[j] = t < nv;
          const uint32_t off = static_cast<uint32_t>((ok[j] ? t * static_cast<int>(row_stride) : 0) + head_off);
          K[j] = *reinterpret_cast<const uint4*>(kp + off);
          V[j] = *reinterpret_cast<const uint4*>(vp + off);
        }
      } else {
      full = false;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int rr = slot + RPL * j;            // row in group, 0..15
        const int e = grp * epg + rr / P;
        const int t = rr % P;
        const int ec = e < 64 ? e : 63;
        const int blk = __shfl(my_blk, ec);
        const int nv = __shfl(my_nv, ec);
        if constexpr (AL) pos[j] = static_cast<float>((__shfl(my_pg, ec) - pref) * P + t);
        ok[j] = grp < ngroups && e < nw && t < nv;
        // masked rows read row 0 of block 0: the loads are unconditional so
        // the count in flight is static and the waits stay exact
        const int64_t off = ok[j] ? (static_cast<int64_t>(blk) * P + t) * row_stride + head_off
                                  : head_off;
        K[j] = *reinterpret_cast<const uint4*>(kv + off);
        V[j] = *reinterpret_cast<const uint4*>(kv + v_off + off);
      }
      }
    };
    // Two groups in flight: while one is folded in, the next one's loads
    // are outstanding; each refill is unconditional (past the end it reads
    // placeholders) so the number of loads in flight stays static.
    // The standalone page_size 16 decode keeps one page in flight per wave
    // and more waves per SIMD (6, at 74 VGPRs): 25.2 against 25.5 us at
    // long_context and 22.6 against 23.0 at gqa_ragged for the two-page ring
    // at 4 waves (the same pages in the same order, so the same bits).  The
    // fused forms keep the ring (their block shapes cap the waves per SIMD),
    // and so does the generic page size (its addressing spills at 6).
    if constexpr (!FUSE && TKI == 0 && PFIX == 16) {
      uint4 Ks[NL], Vs[NL];
      bool os[NL];
      float ps[NL];
      bool fs = false;
      for (int grp = 0; grp < ngroups; ++grp) {
        load(grp, Ks, Vs, os, fs, ps);
        attend_rows_split<LPR, NL, AL>(qh, ql, Ks, Vs, os, fs, ps, slope2, m, l, acc);
      }
      continue;
    }
    uint4 K0[NL], V0[NL], K1[NL], V1[NL];
    bool o0[NL], o1[NL];
    float p0[NL], p1[NL];
    bool f0 = false, f1 = false;
    int grp = 0;
    load(0, K0, V0, o0, f0, p0);
    load(1, K1, V1, o1, f1, p1);
    while (grp < ngroups) {
      attend_rows_split<LPR, NL, AL>(qh, ql, K0, V0, o0, f0, p0, slope2, m, l, acc);
      if (++grp >= ngroups) break;
      load(grp + 1, K0, V0, o0, f0, p0);
      attend_rows_split<LPR, NL, AL>(qh, ql, K1, V1, o1, f1, p1, slope2, m, l, acc);
      if (++grp >= ngroups) break;
      load(grp + 1, K1, V1, o1, f1, p1);
    }
  }

  merge_slots<LPR>(m, l, acc);
  if constexpr (TKI > 0 && !FUSE) {
    if (ta.block_partials) {
      // The block's splits merged through LDS with FUSE's algebra into one
      // partial of the row (normalised output, natural-log lse), block j of
      // the head writing partial j; lse_merge then combines a head's
      // ceil(num_splits / WB) partials instead of its num_splits.
      __shared__ float x_m[WB], x_l[WB];
      __shared__ __align__(16) float x_acc[WB][D];
      float mabs = m;
      if (AL && m != -INFINITY) mabs = fmaf(slope2, static_cast<float>(pref * P - (S - 1)), m);
      if (slot == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x_acc[wave][c * 8 + i] = acc[i];
      }
      if (lane == 0) { x_m[wave] = mabs; x_l[wave] = l; }
      __syncthreads();
      if (wave != 0) return;
      constexpr int DPL = D / 64;          // dims per lane
      const int64_t brow = qrow * nsg + kb % nsg;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WB; ++w) M = fmaxf(M, x_m[w]);
      if (M == -INFINITY) {
#pragma unroll
        for (int j = 0; j < DPL; ++j) o_part[brow * D + lane + 64 * j] = 0.0f;
        if (lane == 0) lse_part[brow] = -INFINITY;
        return;
      }
      float L = 0.0f, A[DPL];
#pragma unroll
      for (int j = 0; j < DPL; ++j) A[j] = 0.0f;
#pragma unroll
      for (int w = 0; w < WB; ++w) {
        if (x_m[w] == -INFINITY) continue;
        const float e = exp2f(x_m[w] - M);
        L = fmaf(x_l[w], e, L);
#pragma unroll
        for (int j = 0; j < DPL; ++j) A[j] = fmaf(x_acc[w][lane + 64 * j], e, A[j]);
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) o_part[brow * D + lane + 64 * j] = A[j] / L;
      if (lane == 0) lse_part[brow] = (M + log2f(L)) * skv::kLn2;
      return;
    }
  }
  if constexpr (FUSE) {
    // the split's state in absolute base-2 units, then the block merge
    __shared__ float f_m[WB], f_l[WB];
    __shared__ __align__(16) float f_acc[WB][D];
    float mabs = m;
    if (AL && m != -INFINITY) mabs = fmaf(slope2, static_cast<float>(pref * P - (S - 1)), m);
    if (slot == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f_acc[wave][c * 8 + i] = acc[i];
    }
    if (lane == 0) { f_m[wave] = mabs; f_l[wave] = l; }
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += WB * 64) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WB; ++w) M = fmaxf(M, f_m[w]);
      if (M == -INFINITY) {
        out[qrow * D + d] = 0.0f;
        if (d == 0 && lse_out != nullptr) lse_out[qrow] = -INFINITY;
        continue;
      }
      float L = 0.0f, A = 0.0f;
#pragma unroll
      for (int w = 0; w < WB; ++w) {
        if (f_m[w] == -INFINITY) continue;
        const float e = exp2f(f_m[w] - M);
        L = fmaf(f_l[w], e, L);
        A = fmaf(f_acc[w][d], e, A);
      }
      out[qrow * D + d] = A / L;
      if (d == 0 && lse_out != nullptr) lse_out[qrow] = (M + log2f(L)) * skv::kLn2;
    }
    if (o_part == nullptr || s >= num_splits) return;
  }
  if (TKI > 0 && s >= num_splits) return;
  const int64_t prow = qrow * num_splits + s;
  if (slot == 0) {
    float4* dst = reinterpret_cast<float4*>(o_part + prow * D + c * 8);
    if (m == -INFINITY) {
      dst[0] = make_float4(0, 0, 0, 0);
      dst[1] = make_float4(0, 0, 0, 0);
    } else {
      const float inv = 1.0f / l;
      dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
  }
  if (lane == 0) {
    float lse2 = m + log2f(l);
    if (AL) lse2 = fmaf(slope2, static_cast<float>(pref * P - (S - 1)), lse2);
    lse_part[prow] = m == -INFINITY ? -INFINITY : lse2 * skv::kLn2;
  }
}

// ------------------------------------------------------------ group kernel

using skv::as_bf16x8;

// One block per (split, kv head, request) when the whole query group shares
// one selection: every selected row is read once and serves all G heads.
// Per 16-row group a wave computes the G x 16 logit tile and the G x D output
// update on the matrix cores:
//   S (16 rows x 16 heads) = K (16 x D) . Q^T (D x 16), K as read (16-byte
//     row pieces are exactly the A operand of the 16x16x32 bf16 MFMA), Q as
//     bf16 hi + lo halves (two MFMAs per 32 dims; about 16 significant bits);
//   O (16 heads x D) += P (16 x 16 rows) . V (16 rows x D), P in the lanes
//     where S left it (the S tile's layout is the A operand of the 16x16x16
//     bf16 MFMA), split hi + lo like Q; V is staged through LDS to read it in
//     the B operand's row-interleaved order.
// Heads past G carry zero queries and are dropped at the end.  Online softmax
// state per head lives in the four lanes of its S column; the waves' states
// are merged through LDS at the end.
// In-block selection (TKI > 0): the block first selects its row from the
// row's scores (ta.scores, TKI entries per thread, the device top-k shared
// with page_topk) into LDS and takes its chunk from there; every split block
// of a row selects the same row, so the selection never leaves the chip
// (block 0 of the row copies it out when ta.sel_idx is given).
// Token level (H2O = 1 group-mean query, 2 per-head softmax): the row's
// scores are the accumulator after this step's update, which the block
// computes itself from the logits pass's logits and chunk (max, sum)
// partials and the accumulator as it was before the step (the pass's
// snapshot), with the update pass's arithmetic; the row's split blocks
// share the write of the new accumulator (and, if asked, its fp32 row) after
// their decode, so no block reads a value another block rewrites.
template <int D, bool AL, int TKI = 0, int H2O = 0, int NWV = 4>
__global__ __launch_bounds__(NWV * 64) void sparse_decode_group_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const uint16_t* __restrict__ kv, int64_t num_blocks, int P,
    const int32_t* __restrict__ bt, int64_t bt_ld,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, const int32_t* __restrict__ sel_blk,
    int k_cap, float scale_log2, int num_splits, float* __restrict__ o_part,
    float* __restrict__ lse_part, const float* __restrict__ alibi, TopkArgs ta) {
  constexpr int NC = D / 32;            // 32-dim steps of the logit MFMA
  constexpr int NB = D / 16;            // 16-column blocks of the output MFMA
  constexpr int WAVES = NWV;            // (in-block selection: more waves share it)
  constexpr int VST = D + 4;            // staged V row stride (bf16), skews banks

  __shared__ int32_t e_blk[kMaxEnt];
  __shared__ int32_t e_nv[kMaxEnt];
  __shared__ int32_t e_pg[AL ? kMaxEnt : 1];
  __shared__ int s_start, s_len, s_pref;
  __shared__ __align__(16) uint16_t vstage[WAVES][16 * VST];
  __shared__ float red_m[WAVES][16], red_l[WAVES][16];
  __shared__ __align__(16) float red_o[WAVES][16][D];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15;              // S column (head) / MFMA row of A
  const int kq = lane >> 4;             // quarter of the wave
  const int S = seq_lens[b];
  int64_t Nb = (static_cast<int64_t>(S) + P - 1) / P;
  if (Nb > bt_ld) Nb = bt_ld;
  const int row = b * H_kv + h;

  // The chunk's place in the row depends only on k_cap: its first entries
  // (index and block id) are fetched together with the count, not after it.
  const int cap = (k_cap + num_splits - 1) / num_splits;
  const int start = s * cap;
  int avail = k_cap - start;
  avail = avail < 0 ? 0 : (avail > cap ? cap : avail);
  int pre_p = -1, pre_b = -1;
  // with in-block selection: the row's selection in LDS (k_cap entries)
  extern __shared__ int32_t sel_lds[];
  // token level: the row's new accumulator values this thread computed, and
  // the physical slots it writes them to when it owns them (the row's write
  // is spread over its split blocks and issued after the decode)
  constexpr int WB = (TKI > 0 && H2O > 0) ? TKI : 1;
  float wb_v[WB];
  int32_t wb_slot[WB];
  uint32_t wb_win = 0u;                 // entries inside the accumulator window
  bool wb_own = false;
  if constexpr (TKI > 0) {
    int64_t Nt;
    uint32_t key[TKI];
    if constexpr (H2O > 0) {
      constexpr bool PH = H2O == 2;
      const int GR = PH ? G : 1;              // logit rows of this kv head
      const int HR = H_kv * GR;               // logit rows of the request
      int ntok = S < bt_ld ? S : static_cast<int>(bt_ld);
      if (ntok < 0) ntok = 0;
      const int lo = ta.bos < ntok ? ta.bos : ntok;
      int hi = ntok - ta.eos > 0 ? ntok - ta.eos : 0;
      if (hi < lo) hi = lo;
      Nt = ntok;
      const int base = tid * TKI;
      // (rows of bt_ld % 4 == 0 start 16-byte aligned in both buffers)
      const bool vec = (bt_ld & 3) == 0 && base + TKI <= bt_ld;
      // the old accumulator and the first logit row, issued before the
      // normaliser so their latency overlaps it
      const uint16_t* hrow = ta.h_snap + (static_cast<int64_t>(b) * H_kv + h) * bt_ld;
      const float* lrow = ta.h_logits + (static_cast<int64_t>(b) * HR + h * GR) * bt_ld;
      const int32_t* btr0 = bt + static_cast<int64_t>(b) * bt_ld;
      float hv[TKI], lg[TKI];
      int32_t* slot = wb_slot;
      wb_own = (tid % num_splits) == s;
      if (vec) {
#pragma unroll
        for (int i = 0; i < TKI; i += 4) {
          const uint2 w = *reinterpret_cast<const uint2*>(hrow + base + i);
          hv[i] = skv::bf16_lo(w.x); hv[i + 1] = skv::bf16_hi(w.x);
          hv[i + 2] = skv::bf16_lo(w.y); hv[i + 3] = skv::bf16_hi(w.y);
          const float4 l4 = *reinterpret_cast<const float4*>(lrow + base + i);
          lg[i] = l4.x; lg[i + 1] = l4.y; lg[i + 2] = l4.z; lg[i + 3] = l4.w;
        }
        if (wb_own) {
#pragma unroll
          for (int i = 0; i < TKI; i += 4) {
            const int4 v4 = *reinterpret_cast<const int4*>(btr0 + base + i);
            slot[i] = v4.x; slot[i + 1] = v4.y; slot[i + 2] = v4.z; slot[i + 3] = v4.w;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < TKI; ++i) {
          const int t = base + i;
          hv[i] = t < ntok ? skv::bf16_to_f32(hrow[t]) : 0.0f;
          lg[i] = t < ntok ? lrow[t] : 0.0f;
          slot[i] = (wb_own && t < ntok) ? btr0[t] : 0;
        }
      }
      // (max, sum) of each logit row over the row's chunks, in the update
      // pass's lane layout: LR lanes per row fold every LR-th chunk, then a
      // butterfly over the row's lanes
      __shared__ float hM[16], hZ[16];
      {
        int LR = 64;
        while (LR > 1 && LR * HR > 256) LR >>= 1;
        const int r = tid / LR, sl = tid % LR;
        const int nch_b = (ntok + ta.h_chunk - 1) / ta.h_chunk;
        float m = -INFINITY, z = 0.0f;
        if (r < GR) {
          const float2* pp = reinterpret_cast<const float2*>(
              ta.h_part + (static_cast<int64_t>(b) * HR + h * GR + r) * ta.h_nchunk * 2);
          for (int j = sl; j < nch_b; j += LR) fold_max_sum(m, z, pp[j].x, pp[j].y);
        }
        for (int off = LR >> 1; off > 0; off >>= 1)
          fold_max_sum(m, z, __shfl_xor(m, off), __shfl_xor(z, off));
        if (r < GR && sl == 0) { hM[r] = m; hZ[r] = z; }
      }
      __syncthreads();
      float pr[TKI];
      if constexpr (PH) {
#pragma unroll
        for (int i = 0; i < TKI; ++i) pr[i] = exp2f(lg[i] - hM[0]) / hZ[0];
        for (int g = 1; g < GR; ++g) {
          const float* lr2 = lrow + static_cast<int64_t>(g) * bt_ld;
#pragma unroll
          for (int i = 0; i < TKI; ++i) {
            const int t = base + i;
            const float l2 = t < ntok ? lr2[t] : 0.0f;
            pr[i] += exp2f(l2 - hM[g]) / hZ[g];
          }
        }
        const float inv = static_cast<float>(GR);
#pragma unroll
        for (int i = 0; i < TKI; ++i) pr[i] /= inv;
      } else {
#pragma unroll
        for (int i = 0; i < TKI; ++i) pr[i] = exp2f(lg[i] - hM[0]) / hZ[0];
      }
      wb_win = low_bits_u(hi - base) & ~low_bits_u(lo - base) & low_bits_u(TKI);
#pragma unroll
      for (int i = 0; i < TKI; ++i) {
        const int t = base + i;
        float v = hv[i];
        if ((wb_win >> i) & 1u) {
          const float pb = skv::bf16_to_f32(skv::f32_to_bf16(pr[i]));
          v = skv::bf16_to_f32(skv::f32_to_bf16(fmaf(ta.h_decay, v, pb)));
        }
        wb_v[i] = v;
        key[i] = t < ntok ? skv::order_key(v) : 0u;
      }
    } else {
    Nt = (static_cast<int64_t>(S) + P - 1) / P;
    if (Nt > ta.score_ld) Nt = ta.score_ld;
    const float* srow = ta.scores + static_cast<int64_t>(row) * ta.score_ld;
    const bool aligned = ((ta.score_ld & 3) == 0) &&
                         ((reinterpret_cast<uintptr_t>(ta.scores) & 15) == 0);
    // the whole stored row is loaded before its length is known; entries
    // outside [bos, N - eos) are ignored by the selection
    skv::load_row_keys<TKI>(srow, aligned, ta.score_ld, key);
    }
    const int cnt = skv::topk_row_keys<NWV * 64, TKI>(key, static_cast<int>(Nt), ta.topk_pages,
                                                 ta.topk_frac, ta.bos, ta.eos, nullptr, 0,
                                                 sel_lds, nullptr, k_cap);
    if (ta.sel_idx != nullptr && s == 0) {
      const int32_t* btr0 = bt + static_cast<int64_t>(b) * bt_ld;
      for (int j = tid; j < k_cap; j += NWV * 64) {
        const int p = sel_lds[j];
        ta.sel_idx[static_cast<int64_t>(row) * k_cap + j] = p;
        if (ta.sel_blk != nullptr)
          ta.sel_blk[static_cast<int64_t>(row) * k_cap + j] = (p >= 0 && p < bt_ld) ? btr0[p] : -1;
      }
      if (tid == 0) ta.sel_cnt[row] = cnt;
    }
    if (tid < kMaxEnt && tid < avail) pre_p = sel_lds[start + tid];
    if (tid == 0) {
      const Chunk ch = split_chunk(cnt, k_cap, num_splits, s);
      s_start = ch.start;
      s_len = ch.len;
      s_pref = (AL && ch.len > 0) ? sel_lds[ch.start + ch.len - 1] : 0;
    }
  } else {
  if (tid < kMaxEnt && tid < avail) {
    const int64_t at = static_cast<int64_t>(row) * k_cap + start + tid;
    pre_p = sel_idx[at];
    if (sel_blk != nullptr) pre_b = sel_blk[at];
  }
  if (tid == 0) {
    const Chunk ch = split_chunk(sel_cnt[row], k_cap, num_splits, s);
    s_start = ch.start;
    s_len = ch.len;
    // ALiBi offsets are taken from the chunk's last selected page (see the
    // per-head kernel); its bias returns in the lse
    s_pref = (AL && ch.len > 0) ? sel_idx[static_cast<int64_t>(row) * k_cap + ch.start + ch.len - 1] : 0;
  }
  }

  // Q^T as the B operand: lane holds head n, dims c*32 + 8*kq .. +8, scaled
  // by scale*log2(e) and split into bf16 hi + lo.
  uint4 qh[NC], ql[NC];
  {
    const bool hv = n < G;
    const float* qr = q + (static_cast<int64_t>(b) * H_q + h * G + (hv ? n : 0)) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4 xa = *reinterpret_cast<const float4*>(qr + c * 32 + 8 * kq);
      const float4 xb = *reinterpret_cast<const float4*>(qr + c * 32 + 8 * kq + 4);
      float x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = hv ? x[2 * i] * scale_log2 : 0.0f;
        const float x1 = hv ? x[2 * i + 1] * scale_log2 : 0.0f;
        const uint16_t h0 = skv::f32_to_bf16(x0), h1 = skv::f32_to_bf16(x1);
        const uint16_t l0 = skv::f32_to_bf16(x0 - skv::bf16_to_f32(h0));
        const uint16_t l1 = skv::f32_to_bf16(x1 - skv::bf16_to_f32(h1));
        hw[i] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        lw[i] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
      }
      qh[c] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      ql[c] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
  __syncthreads();
  const int rounds = (s_len + kMaxEnt - 1) / kMaxEnt;

  // ALiBi slope of head n in base-2 logit units
  const float slope2 = (AL && n < G) ? alibi[h * G + n] * skv::kLog2e : 0.0f;
  float m = -INFINITY, l = 0.0f;       // state of head n
  skv_f32x4 O[NB];                     // O[head 4*kq + i][blk*16 + n]
#pragma unroll
  for (int bk = 0; bk < NB; ++bk) O[bk] = skv_f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t row_stride = static_cast<int64_t>(H_kv) * D;
  const int64_t v_off = num_blocks * P * row_stride;
  const int64_t head_off = static_cast<int64_t>(h) * D;
  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;
  const int epg = 16 / P;
  const int rr = lane & 15;            // row this lane loads (A operand row)
  uint16_t* vw = vstage[wave];

  for (int rd = 0; rd < rounds; ++rd) {
    for (int j = tid; j < kMaxEnt; j += blockDim.x) {
      const int pos = rd * kMaxEnt + j;
      int blk = -1, nv = 0;
      if (pos < s_len) {
        int p, pb;
        if (rd == 0) {
          p = pre_p;                       // fetched above (256 threads: j == tid)
          pb = pre_b;
        } else if constexpr (TKI > 0) {
          p = sel_lds[s_start + pos];
          pb = -1;
        } else {
          const int64_t at = static_cast<int64_t>(row) * k_cap + s_start + pos;
          p = sel_idx[at];
          pb = sel_blk != nullptr ? sel_blk[at] : -1;
        }
        if (p >= 0 && p < Nb) {
          blk = (TKI == 0 && sel_blk != nullptr) ? pb : btr[p];
          const int nn = S - p * P;
          nv = nn < P ? nn : P;
        }
        if constexpr (AL) e_pg[j] = p;
      }
      e_blk[j] = blk;
      e_nv[j] = nv;
    }
    __syncthreads();
    int n_here = s_len - rd * kMaxEnt;
    n_here = n_here > kMaxEnt ? kMaxEnt : n_here;
    const int ngroups = (n_here + epg - 1) / epg;

    // 16-byte pieces of row rr: dims c*32 + 8*kq .. +8 (the A operand layout);
    // masked rows read row 0 of block 0 so the loads stay unconditional
    // rpos (ALiBi only): this lane's row position minus the query's (S - 1)
    auto load = [&](int grp, uint4 (&Kc)[NC], uint4 (&Vc)[NC], bool& ok, float& rpos) {
      const int e = grp * epg + rr / P;
      const int t = rr % P;
      const int ec = e < kMaxEnt ? e : kMaxEnt - 1;
      ok = grp < ngroups && e < n_here && t < e_nv[ec];
      if constexpr (AL) rpos = ok ? static_cast<float>((e_pg[ec] - s_pref) * P + t) : 0.0f;
      const int64_t off = (ok ? (static_cast<int64_t>(e_blk[ec]) * P + t) * row_stride : 0) +
                          head_off + 8 * kq;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Kc[c] = *reinterpret_cast<const uint4*>(kv + off + c * 32);
        Vc[c] = *reinterpret_cast<const uint4*>(kv + v_off + off + c * 32);
      }
    };
    auto apply = [&](const uint4 (&Kc)[NC], const uint4 (&Vc)[NC], bool ok, float rpos) {
      // masked rows stage zeros: a placeholder row is never multiplied
#pragma unroll
      for (int c = 0; c < NC; ++c)
        *reinterpret_cast<uint4*>(vw + rr * VST + c * 32 + 8 * kq) =
            ok ? Vc[c] : make_uint4(0u, 0u, 0u, 0u);
      skv_f32x4 sacc = skv_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Kc[c]), as_bf16x8(qh[c]),
                                                       sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Kc[c]), as_bf16x8(ql[c]),
                                                       sacc, 0, 0, 0);
      }
      if constexpr (AL) {
        // row 4*kq + i's position sits in lane 4*kq + i (the A-operand row)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[i] = fmaf(slope2, __shfl(rpos, 4 * kq + i), sacc[i]);
      }
      // rows 4*kq + i of column n; invalid rows (bit clear) drop out
      const uint64_t okm = __ballot(ok);
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sv[i] = ((okm >> (4 * kq + i)) & 1ull) ? sacc[i] : -INFINITY;
      float tm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      tm = fmaxf(tm, __shfl_xor(tm, 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float mn = fmaxf(m, tm);
      float alpha = 1.0f;
      float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (mn != -INFINITY) {
        alpha = __builtin_amdgcn_exp2f(m - mn);          // 0 while m == -inf
#pragma unroll
        for (int i = 0; i < 4; ++i) ps[i] = __builtin_amdgcn_exp2f(sv[i] - mn);
        m = mn;
      }
      float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l = fmaf(l, alpha, psum);
      // output rows are heads 4*kq + i: their factors sit in lanes 4*kq + i
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kq + i);
      skv_short4 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t hb = skv::f32_to_bf16(ps[i]);
        ph[i] = static_cast<short>(hb);
        pl[i] = static_cast<short>(skv::f32_to_bf16(ps[i] - skv::bf16_to_f32(hb)));
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int bk = 0; bk < NB; ++bk) {
        skv_short4 vb;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vb[i] = static_cast<short>(vw[(4 * kq + i) * VST + bk * 16 + n]);
        skv_f32x4 o = O[bk];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= al[i];
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vb, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, o, 0, 0, 0);
        O[bk] = o;
      }
      __builtin_amdgcn_wave_barrier();
    };
    uint4 K0[NC], V0[NC], K1[NC], V1[NC];
    bool o0, o1;
    float r0 = 0.0f, r1 = 0.0f;
    int grp = wave;
    load(grp, K0, V0, o0, r0);
    while (grp < ngroups) {
      load(grp + WAVES, K1, V1, o1, r1);
      apply(K0, V0, o0, r0);
      grp += WAVES;
      if (grp >= ngroups) break;
      load(grp + WAVES, K0, V0, o0, r0);
      apply(K1, V1, o1, r1);
      grp += WAVES;
    }
    __syncthreads();
  }

  if (lane < 16) { red_m[wave][lane] = m; red_l[wave][lane] = l; }
#pragma unroll
  for (int bk = 0; bk < NB; ++bk)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[wave][4 * kq + i][bk * 16 + n] = O[bk][i];
  __syncthreads();
  for (int i = tid; i < G * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, red_m[w][g]);
    const int64_t prow = (static_cast<int64_t>(b) * H_q + h * G + g) * num_splits + s;
    if (M == -INFINITY) {
      o_part[prow * D + d] = 0.0f;
      if (d == 0) lse_part[prow] = -INFINITY;
      continue;
    }
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      if (red_m[w][g] == -INFINITY) continue;
      const float e = exp2f(red_m[w][g] - M);
      L = fmaf(red_l[w][g], e, L);
      A = fmaf(red_o[w][g][d], e, A);
    }
    o_part[prow * D + d] = A / L;
    if (d == 0) {
      float lse2 = M + log2f(L);
      if (AL) lse2 = fmaf(alibi[h * G + g] * skv::kLog2e,
                          static_cast<float>(s_pref * P - (S - 1)), lse2);
      lse_part[prow] = lse2 * skv::kLn2;
    }
  }
  if constexpr (TKI > 0 && H2O > 0) {
    // the new accumulator (and its fp32 row) of the entries this thread owns
    if (wb_own) {
      int ntok = S < bt_ld ? S : static_cast<int>(bt_ld);
      float* srow_out = ta.scores_out != nullptr
          ? ta.scores_out + static_cast<int64_t>(row) * ta.score_ld : nullptr;
#pragma unroll
      for (int i = 0; i < TKI; ++i) {
        const int t = tid * TKI + i;
        if ((wb_win >> i) & 1u)
          ta.h_hh[static_cast<int64_t>(wb_slot[i]) * H_kv + h] = skv::f32_to_bf16(wb_v[i]);
        if (srow_out != nullptr && t < ntok) srow_out[t] = wb_v[i];
      }
    }
  }
}

struct Args {
  const float* q; int H_q, H_kv, G; const uint16_t* kv; int64_t num_blocks; int P;
  const int32_t* bt; int64_t bt_ld; const int32_t* seq_lens; const int32_t* sel_idx;
  const int32_t* sel_cnt; const int32_t* sel_blk; int k_cap; float scale_log2; int num_splits;
  float* o_part; float* lse_part; const float* alibi;
};

constexpr int kWaveBlock = 4;          // waves per block of the wave kernel

template <int D, int PFIX, bool AL>
void launch_wave(hipStream_t st, const Args& a, int64_t n_groups) {
  const int per_group = (a.num_splits * a.G + kWaveBlock - 1) / kWaveBlock;
  const int64_t blocks = kXcds * per_group * ((n_groups + kXcds - 1) / kXcds);
  hipLaunchKernelGGL((sparse_decode_wave_kernel<D, kWaveBlock, PFIX, AL, false, 0>),
                     dim3(static_cast<unsigned>(blocks)), dim3(kWaveBlock * 64), 0, st,
                     a.q, a.H_q, a.H_kv, a.G, a.kv, a.num_blocks, a.P, a.bt, a.bt_ld,
                     a.seq_lens, a.sel_idx, a.sel_cnt, a.sel_blk, a.k_cap, a.scale_log2,
                     a.num_splits, a.o_part, a.lse_part, n_groups, per_group, a.alibi,
                     nullptr, nullptr, TopkArgs{});
}

// One block per query head, kFuseWaves waves = splits, merged in the block.
constexpr int kFuseWaves = 8;

template <int D, int PFIX, bool AL, int TKI, bool SC = false>
void launch_wave_fused(hipStream_t st, const Args& a, int64_t n_groups, float* out,
                       float* lse_out, const TopkArgs& ta) {
  const int per_group = a.G;
  const int64_t blocks = kXcds * per_group * ((n_groups + kXcds - 1) / kXcds);
  const size_t lds = TKI > 0 ? sizeof(int32_t) * (2 * static_cast<size_t>(a.k_cap) +
                                                  (SC ? 2 * static_cast<size_t>(ta.sc_cap) : 0))
                             : 0;
  hipLaunchKernelGGL((sparse_decode_wave_kernel<D, kFuseWaves, PFIX, AL, true, TKI, SC>),
                     dim3(static_cast<unsigned>(blocks)), dim3(kFuseWaves * 64), lds, st,
                     a.q, a.H_q, a.H_kv, a.G, a.kv, a.num_blocks, a.P, a.bt, a.bt_ld,
                     a.seq_lens, a.sel_idx, a.sel_cnt, a.sel_blk, a.k_cap, a.scale_log2,
                     a.num_splits, a.o_part, a.lse_part, n_groups, per_group, a.alibi,
                     out, lse_out, ta);
}

// In-block selection with split partials: one block per (query head, group
// of as many splits as the block has waves), each selecting its head's row.
// 16 waves at page_size 16; 8 for the generic page size, whose addressing
// would spill within the 128 registers a 16-wave block allows.
constexpr int kSplitWaves = 16;

constexpr int split_waves(int pfix) { return pfix == 16 ? kSplitWaves : kSplitWaves / 2; }

template <int D, int PFIX, bool AL, int TKI>
void launch_wave_split(hipStream_t st, const Args& a, int64_t n_groups, const TopkArgs& ta) {
  constexpr int WB = split_waves(PFIX);
  const int nsg = (a.num_splits + WB - 1) / WB;
  const int per_group = a.G * nsg;
  const int64_t blocks = kXcds * per_group * ((n_groups + kXcds - 1) / kXcds);
  const size_t lds = sizeof(int32_t) * 2 * static_cast<size_t>(a.k_cap);
  hipLaunchKernelGGL((sparse_decode_wave_kernel<D, WB, PFIX, AL, false, TKI>),
                     dim3(static_cast<unsigned>(blocks)), dim3(WB * 64), lds, st,
                     a.q, a.H_q, a.H_kv, a.G, a.kv, a.num_blocks, a.P, a.bt, a.bt_ld,
                     a.seq_lens, a.sel_idx, a.sel_cnt, a.sel_blk, a.k_cap, a.scale_log2,
                     a.num_splits, a.o_part, a.lse_part, n_groups, per_group, a.alibi,
                     nullptr, nullptr, ta);
}

template <int D, bool AL, int TKI = 0, int H2O = 0, int NWV = 4>
void launch_group(dim3 grid, hipStream_t st, const Args& a, const TopkArgs& ta = TopkArgs{}) {
  const size_t lds = TKI > 0 ? sizeof(int32_t) * static_cast<size_t>(a.k_cap) : 0;
  hipLaunchKernelGGL((sparse_decode_group_kernel<D, AL, TKI, H2O, NWV>), grid, dim3(NWV * 64),
                     lds, st,
                     a.q, a.H_q, a.H_kv, a.G, a.kv, a.num_blocks, a.P, a.bt, a.bt_ld,
                     a.seq_lens, a.sel_idx, a.sel_cnt, a.sel_blk, a.k_cap, a.scale_log2,
                     a.num_splits, a.o_part, a.lse_part, a.alibi, ta);
}

}  // namespace

namespace {

// Validation and dispatch shared by both entry points.  out == nullptr: the
// split partials only; otherwise the in-block merge as well (per-head
// selection with num_splits <= kFuseWaves, checked by the caller).
int decode_impl(const char* who, const float* q, int B, int H_q, int H_kv, int D,
                const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                const int32_t* sel_idx, const int32_t* sel_cnt, const int32_t* sel_blk,
                int k_cap, int H_sel, float scale, int num_splits, float* o_part,
                float* lse_part, const float* alibi_slopes, float* out, float* lse_out,
                hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", who);
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "%s: group size %d > 16", who, G);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", who, D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "%s: page_size must be 1, 2, 4, 8 or 16 (got %d)", who, page_size);
  SKV_REQUIRE(H_sel == H_q || H_sel == H_kv,
              "%s: H_sel must be H_q or H_kv (got %d)", who, H_sel);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= 65535,
              "%s: num_splits must be in [1, 65535]", who);
  SKV_REQUIRE(k_cap >= 1 && num_blocks > 0 && bt_ld > 0,
              "%s: need k_cap >= 1, num_blocks > 0, bt_ld > 0", who);
  SKV_REQUIRE(num_blocks <= 0x7fffffffLL, "%s: pool too large for 32-bit block ids", who);
  SKV_REQUIRE(B <= 65535 && H_kv <= 65535, "%s: grid too large", who);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(who, q);
  SKV_REQUIRE_PTR_W(who, kv_cache);
  SKV_REQUIRE_PTR_W(who, block_table);
  SKV_REQUIRE_PTR_W(who, seq_lens);
  SKV_REQUIRE_PTR_W(who, sel_idx);
  SKV_REQUIRE_PTR_W(who, sel_cnt);
  const bool shared_sel = (H_sel == H_kv && G > 1);
  if (out == nullptr) {
    SKV_REQUIRE_PTR_W(who, o_part);
    SKV_REQUIRE_PTR_W(who, lse_part);
  } else {
    SKV_REQUIRE(!shared_sel, "%s: the merged output needs one selection per query head", who);
    SKV_REQUIRE(num_splits <= kFuseWaves, "%s: num_splits must be <= %d (got %d)", who,
                kFuseWaves, num_splits);
    SKV_REQUIRE((o_part == nullptr) == (lse_part == nullptr),
                "%s: o_part and lse_part must both be given or both be NULL", who);
  }
  const int64_t n_groups = static_cast<int64_t>(B) * H_kv;
  const int64_t per_group = out != nullptr
      ? G : (static_cast<int64_t>(num_splits) * G + kWaveBlock - 1) / kWaveBlock;
  SKV_REQUIRE(shared_sel || per_group * (n_groups + kXcds) < 0x7fffffffLL,
              "%s: grid too large", who);
  dim3 grid(static_cast<unsigned>(num_splits), static_cast<unsigned>(H_kv),
            static_cast<unsigned>(B));
  const Args a{q, H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
               seq_lens, sel_idx, sel_cnt, sel_blk, k_cap, scale * skv::kLog2e, num_splits,
               o_part, lse_part, alibi_slopes};
  const bool al = alibi_slopes != nullptr;
  if (shared_sel) {
    if (D == 128) { if (al) launch_group<128, true>(grid, stream, a); else launch_group<128, false>(grid, stream, a); }
    else { if (al) launch_group<64, true>(grid, stream, a); else launch_group<64, false>(grid, stream, a); }
  } else if (out != nullptr) {
#define SKV_FUSED(DD, PP)                                                          \
  do {                                                                             \
    if (al) launch_wave_fused<DD, PP, true, 0>(stream, a, n_groups, out, lse_out,  \
                                               TopkArgs{});                      \
    else launch_wave_fused<DD, PP, false, 0>(stream, a, n_groups, out, lse_out,    \
                                             TopkArgs{});                        \
  } while (0)
    if (page_size == 16) {
      if (D == 128) SKV_FUSED(128, 16); else SKV_FUSED(64, 16);
    } else {
      if (D == 128) SKV_FUSED(128, 0); else SKV_FUSED(64, 0);
    }
#undef SKV_FUSED
  } else {
#define SKV_WAVE(DD, PP)                                                   \
  do {                                                                     \
    if (al) launch_wave<DD, PP, true>(stream, a, n_groups);                \
    else launch_wave<DD, PP, false>(stream, a, n_groups);                  \
  } while (0)
    if (page_size == 16) {
      if (D == 128) SKV_WAVE(128, 16); else SKV_WAVE(64, 16);
    } else {
      if (D == 128) SKV_WAVE(128, 0); else SKV_WAVE(64, 0);
    }
#undef SKV_WAVE
  }
  SKV_CHECK_LAUNCH_W(who);
}

}  // namespace

extern "C" int sparse_paged_decode(const float* q, int B, int H_q, int H_kv, int D,
                                   const uint16_t* kv_cache, int64_t num_blocks,
                                   int page_size, const int32_t* block_table,
                                   int64_t bt_ld, const int32_t* seq_lens,
                                   const int32_t* sel_idx, const int32_t* sel_cnt,
                                   int k_cap, int H_sel, float scale, int num_splits,
                                   float* o_part, float* lse_part, hipStream_t stream) {
  return decode_impl("sparse_paged_decode", q, B, H_q, H_kv, D, kv_cache, num_blocks,
                     page_size, block_table, bt_ld, seq_lens, sel_idx, sel_cnt, nullptr,
                     k_cap, H_sel, scale, num_splits, o_part, lse_part, nullptr, nullptr,
                     nullptr, stream);
}

extern "C" int sparse_paged_decode_ex(const float* q, int B, int H_q, int H_kv, int D,
                                      const uint16_t* kv_cache, int64_t num_blocks,
                                      int page_size, const int32_t* block_table,
                                      int64_t bt_ld, const int32_t* seq_lens,
                                      const int32_t* sel_idx, const int32_t* sel_cnt,
                                      const int32_t* sel_blk, int k_cap, int H_sel,
                                      float scale, int num_splits, float* o_part,
                                      float* lse_part, const float* alibi_slopes,
                                      hipStream_t stream) {
  return decode_impl("sparse_paged_decode_ex", q, B, H_q, H_kv, D, kv_cache, num_blocks,
                     page_size, block_table, bt_ld, seq_lens, sel_idx, sel_cnt, sel_blk,
                     k_cap, H_sel, scale, num_splits, o_part, lse_part, alibi_slopes,
                     nullptr, nullptr, stream);
}

extern "C" int sparse_paged_decode_merged(const float* q, int B, int H_q, int H_kv,
                                          int D, const uint16_t* kv_cache,
                                          int64_t num_blocks, int page_size,
                                          const int32_t* block_table, int64_t bt_ld,
                                          const int32_t* seq_lens,
                                          const int32_t* sel_idx,
                                          const int32_t* sel_cnt,
                                          const int32_t* sel_blk, int k_cap,
                                          float scale, int num_splits, float* o_part,
                                          float* lse_part, const float* alibi_slopes,
                                          float* out, float* lse_out,
                                          hipStream_t stream) {
  SKV_REQUIRE_PTR(out);
  return decode_impl("sparse_paged_decode_merged", q, B, H_q, H_kv, D, kv_cache,
                     num_blocks, page_size, block_table, bt_ld, seq_lens, sel_idx, sel_cnt,
                     sel_blk, k_cap, H_q, scale, num_splits, o_part, lse_part, alibi_slopes,
                     out, lse_out, stream);
}

extern "C" int sparse_select_decode(const float* scores, int64_t score_ld, int topk_pages,
                                    float topk_frac, int reserved_bos, int reserved_eos,
                                    const float* q, int B, int H_q, int H_kv, int D,
                                    const uint16_t* kv_cache, int64_t num_blocks,
                                    int page_size, const int32_t* block_table,
                                    int64_t bt_ld, const int32_t* seq_lens, int k_cap,
                                    float scale, int num_splits, const float* alibi_slopes,
                                    float* out, float* lse_out, int32_t* sel_idx,
                                    int32_t* sel_cnt, int32_t* sel_blk,
                                    hipStream_t stream) {
  const char* who = "sparse_select_decode";
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", who);
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "%s: group size %d > 16", who, G);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", who, D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "%s: page_size must be 1, 2, 4, 8 or 16 (got %d)", who, page_size);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= kFuseWaves,
              "%s: num_splits must be in [1, %d] (got %d)", who, kFuseWaves, num_splits);
  SKV_REQUIRE(score_ld > 0 && score_ld <= 8 * kFuseWaves * 64,
              "%s: score_ld must be in [1, %d] (got %lld)", who, 8 * kFuseWaves * 64,
              (long long)score_ld);
  SKV_REQUIRE(topk_pages >= 1, "%s: topk_pages must be >= 1 (got %d)", who, topk_pages);
  SKV_REQUIRE(topk_frac >= 0.0f && topk_frac <= 1.0f, "%s: topk_frac must be in [0, 1]", who);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", who);
  SKV_REQUIRE(num_blocks > 0 && num_blocks <= 0x7fffffffLL && bt_ld > 0,
              "%s: need 0 < num_blocks < 2^31 and bt_ld > 0", who);
  const double frac = static_cast<double>(topk_frac);
  int64_t need = topk_pages;
  const int64_t fk = static_cast<int64_t>(floor(frac * static_cast<double>(score_ld)));
  if (fk > need) need = fk;
  if (static_cast<int64_t>(reserved_bos) + reserved_eos > need)
    need = static_cast<int64_t>(reserved_bos) + reserved_eos;
  if (need > score_ld) need = score_ld;
  SKV_REQUIRE(k_cap >= need && k_cap <= 4096,
              "%s: k_cap %d must cover the largest selection %lld (and be <= 4096)", who,
              k_cap, (long long)need);
  SKV_REQUIRE(B <= 65535, "%s: grid too large", who);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(who, scores);
  SKV_REQUIRE_PTR_W(who, q);
  SKV_REQUIRE_PTR_W(who, kv_cache);
  SKV_REQUIRE_PTR_W(who, block_table);
  SKV_REQUIRE_PTR_W(who, seq_lens);
  SKV_REQUIRE_PTR_W(who, out);
  SKV_REQUIRE((sel_idx == nullptr) == (sel_cnt == nullptr),
              "%s: sel_idx and sel_cnt must both be given or both be NULL", who);
  SKV_REQUIRE(sel_blk == nullptr || sel_idx != nullptr,
              "%s: sel_blk needs sel_idx", who);
  const int64_t n_groups = static_cast<int64_t>(B) * H_kv;
  const Args a{q, H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
               seq_lens, nullptr, nullptr, nullptr, k_cap, scale * skv::kLog2e, num_splits,
               nullptr, nullptr, alibi_slopes};
  const TopkArgs ta{scores, score_ld, topk_pages, frac, reserved_bos, reserved_eos,
                    sel_idx, sel_cnt, sel_blk};
  const bool al = alibi_slopes != nullptr;
  const int tki = score_ld <= 512 ? 1 : score_ld <= 2048 ? 4 : 8;
#define SKV_SEL(DD, PP, TT)                                                            \
  do {                                                                                 \
    if (al) launch_wave_fused<DD, PP, true, TT>(stream, a, n_groups, out, lse_out, ta); \
    else launch_wave_fused<DD, PP, false, TT>(stream, a, n_groups, out, lse_out, ta);   \
  } while (0)
#define SKV_SEL_T(DD, PP)                                                              \
  do {                                                                                 \
    if (tki == 1) SKV_SEL(DD, PP, 1);                                                  \
    else if (tki == 4) SKV_SEL(DD, PP, 4);                                             \
    else SKV_SEL(DD, PP, 8);                                                           \
  } while (0)
  if (page_size == 16) {
    if (D == 128) SKV_SEL_T(128, 16); else SKV_SEL_T(64, 16);
  } else {
    if (D == 128) SKV_SEL_T(128, 0); else SKV_SEL_T(64, 0);
  }
#undef SKV_SEL_T
#undef SKV_SEL
  SKV_CHECK_LAUNCH();
}

extern "C" int sparse_page_decode(const float* q, int B, int H_q, int H_kv, int D,
                                  const uint16_t* kv_cache, int64_t num_blocks,
                                  int page_size, const uint16_t* k_min,
                                  const uint16_t* k_max, const float* k_mean,
                                  const int32_t* block_table, int64_t bt_ld,
                                  const int32_t* seq_lens, float w_avg, float w_peak,
                                  int topk_pages, float topk_frac, int reserved_bos,
                                  int reserved_eos, int k_cap, float scale,
                                  int num_splits, const float* alibi_slopes, float* out,
                                  float* lse_out, float* scores, int32_t* sel_idx,
                                  int32_t* sel_cnt, int32_t* sel_blk, hipStream_t stream) {
  const char* who = "sparse_page_decode";
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", who);
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "%s: group size %d > 16", who, G);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", who, D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "%s: page_size must be 1, 2, 4, 8 or 16 (got %d)", who, page_size);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= kFuseWaves,
              "%s: num_splits must be in [1, %d] (got %d)", who, kFuseWaves, num_splits);
  SKV_REQUIRE(bt_ld > 0 && bt_ld <= 8 * kFuseWaves * 64,
              "%s: bt_ld must be in [1, %d] (got %lld)", who, 8 * kFuseWaves * 64,
              (long long)bt_ld);
  SKV_REQUIRE(topk_pages >= 1, "%s: topk_pages must be >= 1 (got %d)", who, topk_pages);
  SKV_REQUIRE(topk_frac >= 0.0f && topk_frac <= 1.0f, "%s: topk_frac must be in [0, 1]", who);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", who);
  SKV_REQUIRE(num_blocks > 0 && num_blocks <= 0x7fffffffLL,
              "%s: need 0 < num_blocks < 2^31", who);
  SKV_REQUIRE(scale > 0.0f, "%s: scale must be > 0", who);
  const double frac = static_cast<double>(topk_frac);
  int64_t need = topk_pages;
  const int64_t fk = static_cast<int64_t>(floor(frac * static_cast<double>(bt_ld)));
  if (fk > need) need = fk;
  if (static_cast<int64_t>(reserved_bos) + reserved_eos > need)
    need = static_cast<int64_t>(reserved_bos) + reserved_eos;
  if (need > bt_ld) need = bt_ld;
  const int sc_cap = static_cast<int>((bt_ld + 3) / 4 * 4);
  SKV_REQUIRE(k_cap >= need && (2LL * sc_cap + 2LL * k_cap) * 4 <= 48 * 1024,
              "%s: k_cap %d must cover the largest selection %lld, and the block's "
              "scores and selection must fit 48 KiB of LDS", who, k_cap, (long long)need);
  SKV_REQUIRE(B <= 65535, "%s: grid too large", who);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(who, q);
  SKV_REQUIRE_PTR_W(who, kv_cache);
  SKV_REQUIRE_PTR_W(who, k_min);
  SKV_REQUIRE_PTR_W(who, k_max);
  SKV_REQUIRE_PTR_W(who, k_mean);
  SKV_REQUIRE_PTR_W(who, block_table);
  SKV_REQUIRE_PTR_W(who, seq_lens);
  SKV_REQUIRE_PTR_W(who, out);
  SKV_REQUIRE((sel_idx == nullptr) == (sel_cnt == nullptr),
              "%s: sel_idx and sel_cnt must both be given or both be NULL", who);
  SKV_REQUIRE(sel_blk == nullptr || sel_idx != nullptr, "%s: sel_blk needs sel_idx", who);
  const int64_t n_groups = static_cast<int64_t>(B) * H_kv;
  const Args a{q, H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
               seq_lens, nullptr, nullptr, nullptr, k_cap, scale * skv::kLog2e, num_splits,
               nullptr, nullptr, alibi_slopes};
  const TopkArgs ta{nullptr, bt_ld, topk_pages, frac, reserved_bos, reserved_eos,
                    sel_idx, sel_cnt, sel_blk, k_min, k_max, k_mean, w_avg, w_peak,
                    1.0f / scale, sc_cap, scores};
  const bool al = alibi_slopes != nullptr;
  const int tki = bt_ld <= 512 ? 1 : bt_ld <= 2048 ? 4 : 8;
#define SKV_SC(DD, PP, TT)                                                                   \
  do {                                                                                       \
    if (al) launch_wave_fused<DD, PP, true, TT, true>(stream, a, n_groups, out, lse_out, ta); \
    else launch_wave_fused<DD, PP, false, TT, true>(stream, a, n_groups, out, lse_out, ta);   \
  } while (0)
#define SKV_SC_T(DD, PP)                                                                     \
  do {                                                                                       \
    if (tki == 1) SKV_SC(DD, PP, 1);                                                         \
    else if (tki == 4) SKV_SC(DD, PP, 4);                                                    \
    else SKV_SC(DD, PP, 8);                                                                  \
  } while (0)
  if (page_size == 16) {
    if (D == 128) SKV_SC_T(128, 16); else SKV_SC_T(64, 16);
  } else {
    if (D == 128) SKV_SC_T(128, 0); else SKV_SC_T(64, 0);
  }
#undef SKV_SC_T
#undef SKV_SC
  SKV_CHECK_LAUNCH();
}

namespace {

// Split selection + decode, one partial per split, or (blocks) one per block
// of split_waves splits.
int split_select_decode(const char* who, bool blocks, const float* scores, int64_t score_ld,
                        int topk_pages, float topk_frac, int reserved_bos, int reserved_eos,
                        const float* q, int B, int H_q, int H_kv, int D,
                        const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                        const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                        int k_cap, float scale, int num_splits, const float* alibi_slopes,
                        float* o_part, float* lse_part, int32_t* sel_idx, int32_t* sel_cnt,
                        int32_t* sel_blk, hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", who);
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "%s: group size %d > 16", who, G);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", who, D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "%s: page_size must be 1, 2, 4, 8 or 16 (got %d)", who, page_size);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= 4096,
              "%s: num_splits must be in [1, 4096] (got %d)", who, num_splits);
  SKV_REQUIRE(score_ld > 0 && score_ld <= 8 * kSplitWaves * 64,
              "%s: score_ld must be in [1, %d] (got %lld)", who, 8 * kSplitWaves * 64,
              (long long)score_ld);
  SKV_REQUIRE(topk_pages >= 1, "%s: topk_pages must be >= 1 (got %d)", who, topk_pages);
  SKV_REQUIRE(topk_frac >= 0.0f && topk_frac <= 1.0f, "%s: topk_frac must be in [0, 1]", who);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", who);
  SKV_REQUIRE(num_blocks > 0 && num_blocks <= 0x7fffffffLL && bt_ld > 0,
              "%s: need 0 < num_blocks < 2^31 and bt_ld > 0", who);
  const double frac = static_cast<double>(topk_frac);
  int64_t need = topk_pages;
  const int64_t fk = static_cast<int64_t>(floor(frac * static_cast<double>(score_ld)));
  if (fk > need) need = fk;
  if (static_cast<int64_t>(reserved_bos) + reserved_eos > need)
    need = static_cast<int64_t>(reserved_bos) + reserved_eos;
  if (need > score_ld) need = score_ld;
  SKV_REQUIRE(k_cap >= need && k_cap <= 4096,
              "%s: k_cap %d must cover the largest selection %lld (and be <= 4096)", who,
              k_cap, (long long)need);
  const int64_t n_groups = static_cast<int64_t>(B) * H_kv;
  const int wb = split_waves(page_size == 16 ? 16 : 0);
  const int64_t nsg = (num_splits + wb - 1) / wb;
  SKV_REQUIRE(B <= 65535 && G * nsg * (n_groups + kXcds) < 0x7fffffffLL,
              "%s: grid too large", who);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(who, scores);
  SKV_REQUIRE_PTR_W(who, q);
  SKV_REQUIRE_PTR_W(who, kv_cache);
  SKV_REQUIRE_PTR_W(who, block_table);
  SKV_REQUIRE_PTR_W(who, seq_lens);
  SKV_REQUIRE_PTR_W(who, o_part);
  SKV_REQUIRE_PTR_W(who, lse_part);
  SKV_REQUIRE((sel_idx == nullptr) == (sel_cnt == nullptr),
              "%s: sel_idx and sel_cnt must both be given or both be NULL", who);
  SKV_REQUIRE(sel_blk == nullptr || sel_idx != nullptr, "%s: sel_blk needs sel_idx", who);
  const Args a{q, H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
               seq_lens, nullptr, nullptr, nullptr, k_cap, scale * skv::kLog2e, num_splits,
               o_part, lse_part, alibi_slopes};
  TopkArgs ta{scores, score_ld, topk_pages, frac, reserved_bos, reserved_eos,
              sel_idx, sel_cnt, sel_blk};
  ta.block_partials = blocks ? 1 : 0;
  const bool al = alibi_slopes != nullptr;
  // entries per thread of the block's selection (wb * 64 threads)
  const int64_t per_thread = (score_ld + wb * 64 - 1) / (wb * 64);
  const int tki = per_thread <= 1 ? 1 : per_thread <= 2 ? 2 : per_thread <= 4 ? 4
                  : per_thread <= 8 ? 8 : 16;
#define SKV_SPL(DD, PP, TT)                                                          \
  do {                                                                               \
    if (al) launch_wave_split<DD, PP, true, TT>(stream, a, n_groups, ta);            \
    else launch_wave_split<DD, PP, false, TT>(stream, a, n_groups, ta);              \
  } while (0)
#define SKV_SPL_T(DD, PP)                                                            \
  do {                                                                               \
    if (tki == 1) SKV_SPL(DD, PP, 1);                                                \
    else if (tki == 2) SKV_SPL(DD, PP, 2);                                           \
    else if (tki == 4) SKV_SPL(DD, PP, 4);                                           \
    else if (tki == 8) SKV_SPL(DD, PP, 8);                                           \
    else if constexpr (PP != 16) SKV_SPL(DD, PP, 16);                                \
  } while (0)
  if (page_size == 16) {
    if (D == 128) SKV_SPL_T(128, 16); else SKV_SPL_T(64, 16);
  } else {
    if (D == 128) SKV_SPL_T(128, 0); else SKV_SPL_T(64, 0);
  }
#undef SKV_SPL_T
#undef SKV_SPL
  SKV_CHECK_LAUNCH_W(who);
}

}  // namespace

extern "C" int sparse_select_decode_split(const float* scores, int64_t score_ld,
                                          int topk_pages, float topk_frac, int reserved_bos,
                                          int reserved_eos, const float* q, int B, int H_q,
                                          int H_kv, int D, const uint16_t* kv_cache,
                                          int64_t num_blocks, int page_size,
                                          const int32_t* block_table, int64_t bt_ld,
                                          const int32_t* seq_lens, int k_cap, float scale,
                                          int num_splits, const float* alibi_slopes,
                                          float* o_part, float* lse_part, int32_t* sel_idx,
                                          int32_t* sel_cnt, int32_t* sel_blk,
                                          hipStream_t stream) {
  return split_select_decode("sparse_select_decode_split", false, scores, score_ld, topk_pages,
                             topk_frac, reserved_bos, reserved_eos, q, B, H_q, H_kv, D,
                             kv_cache, num_blocks, page_size, block_table, bt_ld, seq_lens,
                             k_cap, scale, num_splits, alibi_slopes, o_part, lse_part,
                             sel_idx, sel_cnt, sel_blk, stream);
}

extern "C" int sparse_select_decode_split_blocks_count(int num_splits, int page_size) {
  if (num_splits < 1 || num_splits > 4096 || !skv_supported_page_size(page_size)) return -1;
  const int wb = split_waves(page_size == 16 ? 16 : 0);
  return (num_splits + wb - 1) / wb;
}

extern "C" int sparse_select_decode_split_blocks(
    const float* scores, int64_t score_ld, int topk_pages, float topk_frac, int reserved_bos,
    int reserved_eos, const float* q, int B, int H_q, int H_kv, int D, const uint16_t* kv_cache,
    int64_t num_blocks, int page_size, const int32_t* block_table, int64_t bt_ld,
    const int32_t* seq_lens, int k_cap, float scale, int num_splits, const float* alibi_slopes,
    float* o_part, float* lse_part, int32_t* sel_idx, int32_t* sel_cnt, int32_t* sel_blk,
    hipStream_t stream) {
  return split_select_decode("sparse_select_decode_split_blocks", true, scores, score_ld,
                             topk_pages, topk_frac, reserved_bos, reserved_eos, q, B, H_q,
                             H_kv, D, kv_cache, num_blocks, page_size, block_table, bt_ld,
                             seq_lens, k_cap, scale, num_splits, alibi_slopes, o_part,
                             lse_part, sel_idx, sel_cnt, sel_blk, stream);
}

extern "C" int sparse_select_decode_group(const float* scores, int64_t score_ld,
                                          int topk_pages, float topk_frac, int reserved_bos,
                                          int reserved_eos, const float* q, int B, int H_q,
                                          int H_kv, int D, const uint16_t* kv_cache,
                                          int64_t num_blocks, int page_size,
                                          const int32_t* block_table, int64_t bt_ld,
                                          const int32_t* seq_lens, int k_cap, float scale,
                                          int num_splits, const float* alibi_slopes,
                                          float* o_part, float* lse_part, int32_t* sel_idx,
                                          int32_t* sel_cnt, int32_t* sel_blk,
                                          hipStream_t stream) {
  const char* who = "sparse_select_decode_group";
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", who);
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "%s: group size %d > 16", who, G);
  SKV_REQUIRE(D == 64 || D == 128, "%s: D must be 64 or 128 (got %d)", who, D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "%s: page_size must be 1, 2, 4, 8 or 16 (got %d)", who, page_size);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= 65535,
              "%s: num_splits must be in [1, 65535] (got %d)", who, num_splits);
  SKV_REQUIRE(score_ld > 0 && score_ld <= 8192,
              "%s: score_ld must be in [1, 8192] (got %lld)", who, (long long)score_ld);
  SKV_REQUIRE(topk_pages >= 1, "%s: topk_pages must be >= 1 (got %d)", who, topk_pages);
  SKV_REQUIRE(topk_frac >= 0.0f && topk_frac <= 1.0f, "%s: topk_frac must be in [0, 1]", who);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", who);
  SKV_REQUIRE(num_blocks > 0 && num_blocks <= 0x7fffffffLL && bt_ld > 0,
              "%s: need 0 < num_blocks < 2^31 and bt_ld > 0", who);
  const double frac = static_cast<double>(topk_frac);
  int64_t need = topk_pages;
  const int64_t fk = static_cast<int64_t>(floor(frac * static_cast<double>(score_ld)));
  if (fk > need) need = fk;
  if (static_cast<int64_t>(reserved_bos) + reserved_eos > need)
    need = static_cast<int64_t>(reserved_bos) + reserved_eos;
  if (need > score_ld) need = score_ld;
  SKV_REQUIRE(k_cap >= need && k_cap <= 4096,
              "%s: k_cap %d must cover the largest selection %lld (and be <= 4096)", who,
              k_cap, (long long)need);
  SKV_REQUIRE(B <= 65535 && H_kv <= 65535, "%s: grid too large", who);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR_W(who, scores);
  SKV_REQUIRE_PTR_W(who, q);
  SKV_REQUIRE_PTR_W(who, kv_cache);
  SKV_REQUIRE_PTR_W(who, block_table);
  SKV_REQUIRE_PTR_W(who, seq_lens);
  SKV_REQUIRE_PTR_W(who, o_part);
  SKV_REQUIRE_PTR_W(who, lse_part);
  SKV_REQUIRE((sel_idx == nullptr) == (sel_cnt == nullptr),
              "%s: sel_idx and sel_cnt must both be given or both be NULL", who);
  SKV_REQUIRE(sel_blk == nullptr || sel_idx != nullptr, "%s: sel_blk needs sel_idx", who);
  const Args a{q, H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
               seq_lens, nullptr, nullptr, nullptr, k_cap, scale * skv::kLog2e, num_splits,
               o_part, lse_part, alibi_slopes};
  const TopkArgs ta{scores, score_ld, topk_pages, frac, reserved_bos, reserved_eos,
                    sel_idx, sel_cnt, sel_blk};
  dim3 grid(static_cast<unsigned>(num_splits), static_cast<unsigned>(H_kv),
            static_cast<unsigned>(B));
  const bool al = alibi_slopes != nullptr;
  // 8 waves: the selection's entries spread over 512 threads
  const int tki = score_ld <= 2048 ? 4 : score_ld <= 4096 ? 8 : score_ld <= 6144 ? 12 : 16;
#define SKV_GSEL(DD, TT)                                                     \
  do {                                                                       \
    if (al) launch_group<DD, true, TT, 0, 8>(grid, stream, a, ta);           \
    else launch_group<DD, false, TT, 0, 8>(grid, stream, a, ta);             \
  } while (0)
#define SKV_GSEL_T(DD)                                                       \
  do {                                                                       \
    if (tki == 4) SKV_GSEL(DD, 4);                                           \
    else if (tki == 8) SKV_GSEL(DD, 8);                                      \
    else if (tki == 12) SKV_GSEL(DD, 12);                                    \
    else SKV_GSEL(DD, 16);                                                   \
  } while (0)
  if (D == 128) SKV_GSEL_T(128); else SKV_GSEL_T(64);
#undef SKV_GSEL_T
#undef SKV_GSEL
  SKV_CHECK_LAUNCH();
}

extern "C" int64_t h2o_select_decode_scratch_floats(int B, int H_q, int H_kv,
                                                    int64_t max_tokens, int per_head) {
  if (B < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 || max_tokens <= 0) return -1;
  return skv::h2o_pass_scratch_floats(B, per_head ? H_q : H_kv, H_kv, max_tokens);
}

extern "C" int h2o_select_decode(const float* q, int B, int H_q, int H_kv, int D,
                                 uint16_t* kv_cache, int64_t num_blocks, int page_size,
                                 const int32_t* block_table, int64_t bt_ld,
                                 const int32_t* seq_lens, int reserved_bos, int reserved_eos,
                                 float scale, float decay, int per_head, uint16_t* hh_score,
                                 float* scores, int64_t score_ld, int topk_pages,
                                 float topk_frac, int k_cap, int num_splits, float* o_part,
                                 float* lse_part, int32_t* sel_idx, int32_t* sel_cnt,
                                 int32_t* sel_blk, const uint16_t* k_new,
                                 const uint16_t* v_new, float* scratch,
                                 int64_t scratch_floats, hipStream_t stream) {
  const char* who = "h2o_select_decode";
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "%s: need H_q a positive multiple of H_kv", who);
  SKV_REQUIRE(H_q / H_kv <= 16, "%s: group size > 16", who);
  SKV_REQUIRE(page_size == 1, "%s: page_size must be 1 (got %d)", who, page_size);
  SKV_REQUIRE(bt_ld > 0 && bt_ld <= 8192, "%s: bt_ld must be in [1, 8192] (got %lld)", who,
              (long long)bt_ld);
  SKV_REQUIRE(scores == nullptr || score_ld >= bt_ld,
              "%s: score_ld must be >= bt_ld when scores are written", who);
  SKV_REQUIRE(num_splits >= 1 && num_splits <= 65535,
              "%s: num_splits must be in [1, 65535] (got %d)", who, num_splits);
  SKV_REQUIRE(topk_pages >= 1, "%s: topk_pages must be >= 1 (got %d)", who, topk_pages);
  SKV_REQUIRE(topk_frac >= 0.0f && topk_frac <= 1.0f, "%s: topk_frac must be in [0, 1]", who);
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "%s: reserved_bos / reserved_eos must be >= 0", who);
  SKV_REQUIRE(num_blocks > 0 && num_blocks <= 0x7fffffffLL,
              "%s: need 0 < num_blocks < 2^31", who);
  const double frac = static_cast<double>(topk_frac);
  int64_t need = topk_pages;
  const int64_t fk = static_cast<int64_t>(floor(frac * static_cast<double>(bt_ld)));
  if (fk > need) need = fk;
  if (static_cast<int64_t>(reserved_bos) + reserved_eos > need)
    need = static_cast<int64_t>(reserved_bos) + reserved_eos;
  if (need > bt_ld) need = bt_ld;
  SKV_REQUIRE(k_cap >= need && k_cap <= 4096,
              "%s: k_cap %d must cover the largest selection %lld (and be <= 4096)", who,
              k_cap, (long long)need);
  SKV_REQUIRE(B <= 65535 && H_kv <= 65535, "%s: grid too large", who);
  SKV_REQUIRE((sel_idx == nullptr) == (sel_cnt == nullptr),
              "%s: sel_idx and sel_cnt must both be given or both be NULL", who);
  SKV_REQUIRE(sel_blk == nullptr || sel_idx != nullptr, "%s: sel_blk needs sel_idx", who);
  SKV_REQUIRE((k_new == nullptr) == (v_new == nullptr),
              "%s: k_new and v_new must both be given or both be NULL", who);
  // the logits pass validates the rest (D, window, decay, scale, scratch size)
  skv::H2oPass pass{};
  const int rc = skv::h2o_logits_pass(who, per_head != 0, q, B, H_q, H_kv, D, kv_cache,
                                      num_blocks, page_size, block_table, bt_ld, seq_lens,
                                      reserved_bos, reserved_eos, scale, decay, hh_score,
                                      scratch, scratch_floats, stream, &pass, k_new, v_new,
                                      kv_cache);
  if (rc != SKV_OK || B == 0) return rc;
  SKV_REQUIRE_PTR_W(who, o_part);
  SKV_REQUIRE_PTR_W(who, lse_part);
  const int G = H_q / H_kv;
  const Args a{q, H_q, H_kv, G, kv_cache, num_blocks, page_size, block_table, bt_ld,
               seq_lens, nullptr, nullptr, nullptr, k_cap, scale * skv::kLog2e, num_splits,
               o_part, lse_part, nullptr};
  TopkArgs ta{};
  ta.scores = nullptr; ta.score_ld = score_ld; ta.topk_pages = topk_pages; ta.topk_frac = frac;
  ta.bos = reserved_bos; ta.eos = reserved_eos;
  ta.sel_idx = sel_idx; ta.sel_cnt = sel_cnt; ta.sel_blk = sel_blk;
  ta.scores_out = scores;
  ta.h_logits = pass.logits; ta.h_part = pass.part; ta.h_snap = pass.snap; ta.h_hh = hh_score;
  ta.h_nchunk = pass.nchunk; ta.h_chunk = pass.chunk; ta.h_decay = pass.decay;
  dim3 grid(static_cast<unsigned>(num_splits), static_cast<unsigned>(H_kv),
            static_cast<unsigned>(B));
  // 8 waves: the row's update and selection spread over 512 threads
  const int tki = bt_ld <= 2048 ? 4 : bt_ld <= 4096 ? 8 : bt_ld <= 6144 ? 12 : 16;
#define SKV_H2OSEL(DD, TT)                                                   \
  do {                                                                       \
    if (per_head) launch_group<DD, false, TT, 2, 8>(grid, stream, a, ta);    \
    else launch_group<DD, false, TT, 1, 8>(grid, stream, a, ta);             \
  } while (0)
#define SKV_H2OSEL_T(DD)                                                     \
  do {                                                                       \
    if (tki == 4) SKV_H2OSEL(DD, 4);                                         \
    else if (tki == 8) SKV_H2OSEL(DD, 8);                                    \
    else if (tki == 12) SKV_H2OSEL(DD, 12);                                  \
    else SKV_H2OSEL(DD, 16);                                                 \
  } while (0)
  if (D == 128) SKV_H2OSEL_T(128); else SKV_H2OSEL_T(64);
#undef SKV_H2OSEL_T
#undef SKV_H2OSEL
  SKV_CHECK_LAUNCH_W(who);
}
