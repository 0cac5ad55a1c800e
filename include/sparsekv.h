/*
 * sparsekv.h -- C ABI of libsparsekv.so: decode-time page-scored sparse
 * attention over a paged bf16 KV cache, hand-written HIP for gfx950 (MI355X).
 *
 * Sources (cited by page title and section):
 *   [VTX] vortex_torch pull request "flow: add H2O sparse attention
 *         (page-level and token-level, MHA + GQA)": "Page-level variants"
 *         (page score), "Token-level variants" (accumulator, reset on write,
 *         decay), the follow-up's oracle harness (reserved bos/eos window).
 *   [EKV] EntmaxKV README, "How it works" and "Quick start": the cache layout
 *         [2, num_blocks, page_size, H_kv, D] plus a block table, per-page key
 *         statistics, top-k pages per query head with the tail page in the
 *         budget, exact attention over the selection, append of k_new/v_new.
 *   [MLA] vllm.cpp test_ops_mla_chunked_context.cpp: chunked attention merged
 *         by log-sum-exp, MergeAttnStates and its -inf / +inf rules.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or synchronises; each call only enqueues work on
 *     `stream` and returns.  Outputs are caller buffers; the cache, the page
 *     statistics and hh_score are updated in place.
 *   - Tensors are dense row-major, except for the explicit leading dimensions
 *     bt_ld (block table row length) and score_ld (score row length).
 *   - bf16 values travel as their uint16_t bit patterns.
 *   - seq_lens[b] is the token count of request b INCLUDING the token appended
 *     this step.  Request b has N_b = ceil(seq_lens[b] / page_size) logical
 *     pages; logical page p is physical block block_table[b * bt_ld + p].
 *     Kernels clamp N_b to bt_ld (and to score_ld where scores are indexed) so
 *     that a bad length cannot index outside the caller's tables.
 *   - Query head i reads kv head i / G with G = H_q / H_kv (consecutive
 *     groups); H_q must be a multiple of H_kv and G <= 16.
 *   - Supported shapes: D in {64, 128}; page_size in {1, 2, 4, 8, 16};
 *     h2o_accumulate also needs H_kv <= 16.
 *   - Device-side contents (block ids, lengths, selections) are trusted: they
 *     must lie inside the caller's buffers.
 *   - A call with no rows (B = 0, or rows = 0 for lse_merge) checks its scalar
 *     arguments and returns SKV_OK without reading or writing anything, so its
 *     pointers may be NULL then (an empty batch is a no-op).
 *
 * Return value of every int entry point
 *   SKV_OK (0) on success.  SKV_EINVAL (-22) for a bad scalar argument,
 *   SKV_EFAULT (-14) for a required NULL pointer: both are detected before
 *   anything is enqueued.  SKV_EIO (-5) if the launch itself failed
 *   (hipGetLastError).  sparsekv_last_error() returns a message for the most
 *   recent failure on the calling thread.
 */
#ifndef SPARSEKV_H
#define SPARSEKV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKV_OK 0
#define SKV_EIO (-5)
#define SKV_EFAULT (-14)
#define SKV_EINVAL (-22)

/* Message for the latest non-zero return on this thread ("" if none). */
const char *sparsekv_last_error(void);

/* Build id: the SHA-1 (hex) over the names and bytes of the sources the
 * library was built from (these headers and the kernel sources), so that a
 * binding can refuse a library whose entry points may differ from the
 * declarations it marshals for.  Static string; no device work. */
const char *sparsekv_build_id(void);

/*
 * pagestats_update -- per-page key statistics, optionally fused with the KV
 * append of one decode step.   [VTX "Page-level variants": element-wise
 * min / max envelope and mean of the keys; EKV "How it works" and
 * "Quick start": statistics kept per page, k_new / v_new appended by the
 * decode call; VTX "Token-level variants" point 2: the score slot of a freshly
 * written token is zeroed.]
 *
 *   kv_cache   bf16 [2, num_blocks, page_size, H_kv, D]   in/out
 *   k_min,
 *   k_max      bf16 [num_blocks, H_kv, D]                 out (exact)
 *   k_mean     fp32 [num_blocks, H_kv, D]                 out (fp32 sum / n)
 *              The three may all be NULL (page_size 1 needs no statistics).
 *   block_table int32 [B, bt_ld], seq_lens int32 [B]
 *   k_new, v_new bf16 [B, H_kv, D] or both NULL.
 *     Both NULL  = rebuild: statistics of every page p < N_b of every request,
 *                  over its n = min(P, S_b - p*P) valid rows.
 *     Both given = append: token S_b - 1 is written (block
 *                  bt[b][(S_b-1)/P], row (S_b-1)%P), then the statistics of
 *                  that tail page are recomputed over its valid rows.
 *   hh_score   bf16 [num_blocks * page_size, H_kv] or NULL; in append mode the
 *              written slot is set to 0 for every kv head.
 */
int pagestats_update(uint16_t *kv_cache, int64_t num_blocks, int page_size,
                     int H_kv, int D, uint16_t *k_min, uint16_t *k_max,
                     float *k_mean, const int32_t *block_table, int64_t bt_ld,
                     const int32_t *seq_lens, int B, const uint16_t *k_new,
                     const uint16_t *v_new, uint16_t *hh_score,
                     hipStream_t stream);

/*
 * page_score -- score of every page p < N_b for every query head.
 * [VTX "Page-level variants": average relevance q . mean(k), peak relevance
 * sum_d max(q_d * max_d, q_d * min_d) (an upper bound of max_t q . k_t that
 * needs both envelopes because q is signed), combined as
 * w_avg * avg + w_peak * peak; EKV "How it works": pages are scored from the
 * statistics alone, without touching the cached tokens.]
 *
 *   q        fp32 [B, H_q, D]
 *   k_min, k_max bf16 / k_mean fp32 [num_blocks, H_kv, D] (from pagestats_update)
 *   block_table int32 [B, bt_ld], seq_lens int32 [B]
 *   scores   fp32 [B, H_q, score_ld], logical page order; entries p >= N_b
 *            are not written.  score_ld >= bt_ld.
 * The softmax scale is not applied (a positive factor does not change ranks).
 */
int page_score(const float *q, int B, int H_q, int H_kv, int D,
               const uint16_t *k_min, const uint16_t *k_max, const float *k_mean,
               const int32_t *block_table, int64_t bt_ld, const int32_t *seq_lens, int page_size,
               float w_avg, float w_peak, float *scores, int64_t score_ld, hipStream_t stream);

/*
 * page_score_ex -- page_score with ALiBi heads.  [EKV "How it works": the page
 * bound includes ALiBi at each page's best logical position.]
 *
 *   Arguments as page_score, plus
 *   alibi    fp32 [H_q] or NULL: the slope of each query head DIVIDED BY the
 *            softmax scale (the score is in q.k units).  A key at position t
 *            of a request of S tokens has logit bias slope * (t - (S - 1)); the
 *            peak term takes the bias of the page's last valid position (its
 *            best), the mean term that of the mean of its valid positions.
 *            NULL: no bias, the same result as page_score.
 */
int page_score_ex(const float *q, int B, int H_q, int H_kv, int D,
                  const uint16_t *k_min, const uint16_t *k_max,
                  const float *k_mean, const int32_t *block_table, int64_t bt_ld,
                  const int32_t *seq_lens, int page_size, float w_avg,
                  float w_peak, float *scores, int64_t score_ld,
                  const float *alibi, hipStream_t stream);

/*
 * page_score_group -- one score per (request, kv head, page): the mean, over
 * the G = H_q / H_kv query heads that read kv head h, of page_score_ex's value.
 * [VTX: the GQA variants of the page-level flow reduce over the query-group
 * axis; the reduction is read as the plain mean of the group's scores, which
 * ranks pages as their sum does.  Selecting once per kv head (page_topk with
 * H_sel = H_kv) lets sparse_paged_decode read each selected page once for the
 * whole group.]
 *
 *   Arguments and layouts as page_score_ex, except
 *   scores   fp32 [B, H_kv, score_ld]; entries p >= N_b are not written.
 *   alibi    as page_score_ex; the group's mean slope applies (the mean of the
 *            group's biased scores).
 * The mean is formed per dim from the group's mean query and mean |q|
 * (mean_g max(q_g max, q_g min) summed over d equals the mean of the
 * per-head peaks exactly), so its cost does not grow with G.
 */
int page_score_group(const float *q, int B, int H_q, int H_kv, int D,
                     const uint16_t *k_min, const uint16_t *k_max,
                     const float *k_mean, const int32_t *block_table,
                     int64_t bt_ld, const int32_t *seq_lens, int page_size,
                     float w_avg, float w_peak, float *scores, int64_t score_ld,
                     const float *alibi, hipStream_t stream);

/*
 * page_topk -- top-k selection per row (b, h), h < H_sel.
 * [EKV "How it works": keep topk_pages per query head, the budget counts
 * pages and includes the always-attended tail page; VTX follow-up: the
 * reserved leading bos and trailing eos entries are kept unconditionally and
 * only the window between them is ranked.]
 *
 *   scores   fp32 [B, H_sel, score_ld] (page_score, page_score_group or
 *            h2o_accumulate output)
 *   N = min(ceil(seq_lens[b] / page_size), score_ld) candidates per row.
 *   k = min(N, max(topk_pages, floor(topk_frac * N))), floor taken in double
 *       of the fp32 topk_frac.
 *   R = [0, bos) u [N - eos, N) clipped to [0, N) is always selected; the
 *   other max(0, k - |R|) entries are the highest scores of [bos, N - eos),
 *   ties going to the lower index (-0.0 equals +0.0; scores must not be NaN).
 *   sel_idx  int32 [B, H_sel, k_cap]: ascending indices, padded with -1.
 *   sel_cnt  int32 [B, H_sel]: number selected (= max(|R|, k)).
 *   Requires k_cap >= max(topk_pages, floor(topk_frac * score_ld), bos + eos)
 *   and score_ld <= 32768.
 */
int page_topk(const float *scores, int64_t score_ld, int B, int H_sel,
              const int32_t *seq_lens, int page_size,
              int topk_pages, float topk_frac, int reserved_bos, int reserved_eos,
              int32_t *sel_idx, int32_t *sel_cnt, int k_cap, hipStream_t stream);

/*
 * page_topk_blk -- page_topk that also writes the physical block of every
 * selected page, so the decode needs no block-table lookup.  [Sources of
 * page_topk; EKV "How it works": the block table maps logical pages to blocks.]
 *
 *   Arguments as page_topk, plus
 *   block_table int32 [B, bt_ld] and bt_ld: read only when sel_blk is given.
 *   sel_blk  int32 [B, H_sel, k_cap] or NULL: block_table[b * bt_ld + p] of
 *            every selected page p (-1 padded, -1 for p >= bt_ld).  NULL: the
 *            same result as page_topk.
 */
int page_topk_blk(const float *scores, int64_t score_ld, int B, int H_sel,
                  const int32_t *seq_lens, int page_size, int topk_pages,
                  float topk_frac, int reserved_bos, int reserved_eos,
                  int32_t *sel_idx, int32_t *sel_cnt, int k_cap,
                  const int32_t *block_table, int64_t bt_ld, int32_t *sel_blk,
                  hipStream_t stream);

/*
 * sparse_paged_decode -- split-K exact softmax attention over the tokens of
 * the selected pages.  [EKV "How it works": only the selected pages are
 * attended and the attention is exact over that selection; MLA: chunked
 * partials merged by log-sum-exp equal single-shot attention.]
 *
 *   q        fp32 [B, H_q, D];  kv_cache bf16 [2, num_blocks, page_size, H_kv, D]
 *   block_table int32 [B, bt_ld], seq_lens int32 [B]
 *   sel_idx  int32 [B, H_sel, k_cap], sel_cnt int32 [B, H_sel] (page_topk's)
 *   H_sel == H_q : row (b, i) of sel_idx is query head i's own selection.
 *   H_sel == H_kv: the G query heads of kv head h share row (b, h) (the
 *                  token-level flow selects per kv head).
 *   Each selection row (cnt entries, ascending, -1 padded) is cut into
 *   num_splits contiguous groups of c = ceil(k_cap / num_splits) entries;
 *   split s holds entries [s*c, min((s+1)*c, cnt)).  Tokens are
 *   {p*P + t : t < n_p} with n_p = min(P, S_b - p*P); l = scale * q . k.
 *   Per (b, i, s):
 *     o_part   fp32 [B, H_q, num_splits, D]  = sum softmax(l) v over the split
 *     lse_part fp32 [B, H_q, num_splits]     = ln sum exp(l)  (-inf if empty,
 *                                               with o_part = 0)
 *   With H_sel == H_kv every row a block loads serves all G query heads of
 *   the group; with H_sel == H_q each query head's chunk is walked by its own
 *   wave(s), and pages shared by heads of a group are served by the caches
 *   after their first read.
 */
int sparse_paged_decode(const float *q, int B, int H_q, int H_kv, int D,
                        const uint16_t *kv_cache, int64_t num_blocks, int page_size,
                        const int32_t *block_table, int64_t bt_ld, const int32_t *seq_lens,
                        const int32_t *sel_idx, const int32_t *sel_cnt, int k_cap, int H_sel,
                        float scale, int num_splits, float *o_part, float *lse_part,
                        hipStream_t stream);

/*
 * sparse_paged_decode_ex -- sparse_paged_decode with block ids from
 * page_topk_blk and ALiBi heads.  [Sources of sparse_paged_decode; EKV
 * "How it works": ALiBi heads.]
 *
 *   Arguments as sparse_paged_decode, plus
 *   sel_blk  int32 [B, H_sel, k_cap] or NULL: page_topk_blk's block ids for
 *            the same rows; when given, the block table is not read.
 *   alibi_slopes fp32 [H_q] or NULL: per query head ALiBi slope; the logit
 *            of the key at position t becomes
 *            l = scale * q . k + slope * (t - (S_b - 1)).
 *   Both NULL: the same result as sparse_paged_decode.
 */
int sparse_paged_decode_ex(const float *q, int B, int H_q, int H_kv, int D,
                           const uint16_t *kv_cache, int64_t num_blocks,
                           int page_size, const int32_t *block_table,
                           int64_t bt_ld, const int32_t *seq_lens,
                           const int32_t *sel_idx, const int32_t *sel_cnt,
                           const int32_t *sel_blk, int k_cap, int H_sel,
                           float scale, int num_splits, float *o_part,
                           float *lse_part, const float *alibi_slopes,
                           hipStream_t stream);

/*
 * sparse_paged_decode_merged -- sparse_paged_decode_ex for one selection per
 * query head (H_sel = H_q) with the split merge done in the same launch: one
 * block per query head, one wave per split, merged in LDS by lse_merge's
 * algebra.  [Same sources as sparse_paged_decode and lse_merge.]
 *
 *   Arguments as sparse_paged_decode_ex (H_sel is H_q), plus
 *   out      fp32 [B, H_q, D]   merged attention output (required)
 *   lse_out  fp32 [B, H_q] or NULL
 *   o_part, lse_part  both NULL, or both given to also receive the partials.
 *   Requires num_splits <= 8 (-EINVAL otherwise).
 * The result equals sparse_paged_decode followed by lse_merge up to fp32
 * rounding order.
 */
int sparse_paged_decode_merged(const float *q, int B, int H_q, int H_kv, int D,
                               const uint16_t *kv_cache, int64_t num_blocks,
                               int page_size, const int32_t *block_table,
                               int64_t bt_ld, const int32_t *seq_lens,
                               const int32_t *sel_idx, const int32_t *sel_cnt,
                               const int32_t *sel_blk, int k_cap, float scale,
                               int num_splits, float *o_part, float *lse_part,
                               const float *alibi_slopes, float *out,
                               float *lse_out, hipStream_t stream);

/*
 * sparse_select_decode -- page_topk and sparse_paged_decode_merged in one
 * launch, for one selection per query head: one block per query head first
 * selects from its score row into LDS, then its waves (one per split) attend
 * over the selection and merge.  [Same sources as page_topk and
 * sparse_paged_decode_merged.]
 *
 *   scores   fp32 [B, H_q, score_ld] (page_score's output), score_ld <= 4096
 *   topk_pages, topk_frac, reserved_bos, reserved_eos, k_cap: as page_topk
 *            (k_cap <= 4096)
 *   q ... seq_lens, scale, num_splits (<= 8), alibi_slopes: as
 *            sparse_paged_decode (H_sel = H_q)
 *   out      fp32 [B, H_q, D];  lse_out fp32 [B, H_q] or NULL
 *   sel_idx, sel_cnt (both or neither), sel_blk (needs sel_idx): when given,
 *            receive the selection exactly as page_topk writes it.
 * The result equals page_topk followed by sparse_paged_decode and lse_merge
 * up to fp32 rounding order.
 */
int sparse_select_decode(const float *scores, int64_t score_ld, int topk_pages,
                         float topk_frac, int reserved_bos, int reserved_eos,
                         const float *q, int B, int H_q, int H_kv, int D,
                         const uint16_t *kv_cache, int64_t num_blocks, int page_size,
                         const int32_t *block_table, int64_t bt_ld,
                         const int32_t *seq_lens, int k_cap, float scale,
                         int num_splits, const float *alibi_slopes, float *out,
                         float *lse_out, int32_t *sel_idx, int32_t *sel_cnt,
                         int32_t *sel_blk, hipStream_t stream);

/*
 * sparse_select_decode_split -- page_topk and sparse_paged_decode in one
 * launch for one selection per query head (H_sel = H_q) at any split count:
 * the split partials go to lse_merge.  One 16-wave block per (query head,
 * group of 16 splits; 8-wave blocks of 8 splits below page size 16) first
 * selects its head's row from the scores into LDS (the top-k of page_topk;
 * the blocks of a head derive the same selection),
 * then each wave attends over one split's chunk of it.  This is
 * sparse_select_decode without its in-block merge, for rows with more than
 * 8 splits or up to 8192 entries.  [Same sources as page_topk and
 * sparse_paged_decode; EKV "How it works": top-k pages per query head.]
 *
 *   scores   fp32 [B, H_q, score_ld] (page_score's output), score_ld <= 8192
 *   topk_pages, topk_frac, reserved_bos, reserved_eos, k_cap: as page_topk
 *            (k_cap <= 4096)
 *   q ... seq_lens, scale, num_splits (<= 4096), alibi_slopes: as
 *            sparse_paged_decode_ex with H_sel = H_q (split s of a row holds
 *            the selected entries [s c, min((s + 1) c, cnt)),
 *            c = ceil(k_cap / num_splits))
 *   o_part   fp32 [B, H_q, num_splits, D], lse_part fp32 [B, H_q, num_splits]:
 *            exactly what sparse_paged_decode writes for that selection
 *   sel_idx, sel_cnt (both or neither), sel_blk (needs sel_idx):
 *            [B, H_q, k_cap] / [B, H_q]; when given, receive the selection
 *            exactly as page_topk_blk writes it.
 *   Errors as sparse_paged_decode.
 */
int sparse_select_decode_split(const float *scores, int64_t score_ld, int topk_pages,
                               float topk_frac, int reserved_bos, int reserved_eos,
                               const float *q, int B, int H_q, int H_kv, int D,
                               const uint16_t *kv_cache, int64_t num_blocks,
                               int page_size, const int32_t *block_table,
                               int64_t bt_ld, const int32_t *seq_lens, int k_cap,
                               float scale, int num_splits,
                               const float *alibi_slopes, float *o_part,
                               float *lse_part, int32_t *sel_idx, int32_t *sel_cnt,
                               int32_t *sel_blk, hipStream_t stream);

/*
 * sparse_select_decode_split_blocks -- sparse_select_decode_split whose
 * blocks also merge their splits: each block folds its waves' split states
 * with lse_merge's algebra (in LDS) and writes one partial, so lse_merge
 * then combines nb = sparse_select_decode_split_blocks_count(num_splits,
 * page_size) partials per query head instead of num_splits.  The merged
 * output equals that of sparse_select_decode_split + lse_merge up to the
 * order of its fp32 sums.  [Same sources as sparse_select_decode_split and
 * lse_merge.]
 *
 *   Arguments as sparse_select_decode_split, except
 *   o_part   fp32 [B, H_q, nb, D], lse_part fp32 [B, H_q, nb]: block j of a
 *            head's partial (its splits j*w .. j*w + w - 1, w = 16 at page
 *            size 16, else 8; splits past num_splits are empty), normalised
 *            output and natural-log lse; a block with no selected entry
 *            writes zeros and -inf.
 *   Errors as sparse_select_decode_split.
 */
int sparse_select_decode_split_blocks(const float *scores, int64_t score_ld, int topk_pages,
                                      float topk_frac, int reserved_bos, int reserved_eos,
                                      const float *q, int B, int H_q, int H_kv, int D,
                                      const uint16_t *kv_cache, int64_t num_blocks,
                                      int page_size, const int32_t *block_table,
                                      int64_t bt_ld, const int32_t *seq_lens, int k_cap,
                                      float scale, int num_splits,
                                      const float *alibi_slopes, float *o_part,
                                      float *lse_part, int32_t *sel_idx, int32_t *sel_cnt,
                                      int32_t *sel_blk, hipStream_t stream);

/* Partials per query head sparse_select_decode_split_blocks writes (nb);
 * no device work; -1 on bad arguments (num_splits outside [1, 4096], an
 * unsupported page size). */
int sparse_select_decode_split_blocks_count(int num_splits, int page_size);

/*
 * sparse_select_decode_group -- page_topk and sparse_paged_decode in one
 * launch for a selection shared by each kv head's query group (H_sel = H_kv:
 * the token-level flow, page_score_group).  One block per (split, kv head,
 * request) first selects its row from the scores into LDS (the top-k of
 * page_topk; every split block of a row derives the same selection), then
 * attends over its chunk of it for the G query heads of the group.  [Same
 * sources as page_topk and sparse_paged_decode; VTX "Token-level variants":
 * the token flow selects once per kv head.]
 *
 *   scores   fp32 [B, H_kv, score_ld] (h2o_accumulate's or page_score_group's
 *            output), score_ld <= 8192
 *   topk_pages, topk_frac, reserved_bos, reserved_eos, k_cap: as page_topk
 *            (k_cap <= 4096)
 *   q ... seq_lens, scale, num_splits, alibi_slopes: as sparse_paged_decode_ex
 *            with H_sel = H_kv (split s of a row holds the selected entries
 *            [s c, min((s + 1) c, cnt)), c = ceil(k_cap / num_splits))
 *   o_part   fp32 [B, H_q, num_splits, D], lse_part fp32 [B, H_q, num_splits]:
 *            what sparse_paged_decode writes for that selection (lse_merge
 *            combines them): bit for bit while a split holds at most 4
 *            groups of 16 rows (16 / page_size entries each); past that the
 *            8 waves of this form fold a split's groups in another order
 *            than the standalone kernel's 4, which moves values by about
 *            1e-5 of their magnitude (the online softmax rescales by other
 *            running maxima)
 *   sel_idx, sel_cnt (both or neither), sel_blk (needs sel_idx):
 *            [B, H_kv, k_cap] / [B, H_kv]; when given, receive the selection
 *            exactly as page_topk_blk writes it.
 */
int sparse_select_decode_group(const float *scores, int64_t score_ld, int topk_pages,
                               float topk_frac, int reserved_bos, int reserved_eos,
                               const float *q, int B, int H_q, int H_kv, int D,
                               const uint16_t *kv_cache, int64_t num_blocks,
                               int page_size, const int32_t *block_table,
                               int64_t bt_ld, const int32_t *seq_lens, int k_cap,
                               float scale, int num_splits,
                               const float *alibi_slopes, float *o_part,
                               float *lse_part, int32_t *sel_idx, int32_t *sel_cnt,
                               int32_t *sel_blk, hipStream_t stream);

/*
 * sparse_page_decode -- the whole page-level step in one launch: page_score,
 * page_topk, sparse_paged_decode and lse_merge for one selection per query
 * head.  One block per query head scores its pages from the statistics into
 * LDS (page_score's arithmetic, ALiBi included), selects, attends (one wave
 * per split) and merges.  [Sources of the four steps.]
 *
 *   q, kv_cache ... seq_lens, k_min / k_max / k_mean, w_avg, w_peak: as
 *            page_score and sparse_paged_decode; bt_ld <= 4096 (the score row
 *            is bt_ld long)
 *   topk_pages, topk_frac, reserved_bos, reserved_eos, k_cap: as page_topk
 *   scale, num_splits (<= 8), alibi_slopes (logit units, NULL = none): as
 *            sparse_paged_decode; the score takes slope / scale (R30 reading)
 *   out fp32 [B, H_q, D]; lse_out fp32 [B, H_q] or NULL
 *   scores fp32 [B, H_q, bt_ld] or NULL; sel_idx / sel_cnt (both or neither)
 *            and sel_blk: optional copies of the intermediate results.
 *   Requires (2 * ceil4(bt_ld) + 2 * k_cap) * 4 bytes <= 48 KiB.
 */
int sparse_page_decode(const float *q, int B, int H_q, int H_kv, int D,
                       const uint16_t *kv_cache, int64_t num_blocks, int page_size,
                       const uint16_t *k_min, const uint16_t *k_max,
                       const float *k_mean, const int32_t *block_table,
                       int64_t bt_ld, const int32_t *seq_lens, float w_avg,
                       float w_peak, int topk_pages, float topk_frac,
                       int reserved_bos, int reserved_eos, int k_cap, float scale,
                       int num_splits, const float *alibi_slopes, float *out,
                       float *lse_out, float *scores, int32_t *sel_idx,
                       int32_t *sel_cnt, int32_t *sel_blk, hipStream_t stream);

/*
 * entmax15_paged_decode -- 1.5-entmax attention over the tokens of the
 * selected pages, as split partials for lse_merge.  [EKV "Quick start"
 * (alpha=1.5) and the component list (decode over selected pages, alpha 1.5);
 * the mapping is the published 1.5-entmax: p_t = [z_t / 2 - tau]_+^2 with
 * z_t = scale * q . k_t and tau such that sum p_t = 1.]
 *
 *   Arguments as sparse_paged_decode (same selection rows and H_sel), except
 *   that split s takes the entries [s c, (s + 1) c) of the row's sel_cnt
 *   entries with c = ceil(sel_cnt / num_splits); plus
 *   alibi_slopes fp32 [H_q] or NULL: ALiBi slope of each query head in
 *            logit units; a key at position t gets z_t += slope * (t - (S - 1)).
 *   scratch  fp32 device buffer of at least entmax_scratch_floats(B, H_q,
 *            k_cap, page_size) floats (logits, then tau per query head).
 *   Per (b, i, s):  m = sum of p over the split's rows,
 *     o_part = sum p v / m,  lse_part = ln m   (o = 0, lse = -inf if m = 0),
 *   so lse_merge over the splits returns sum_t p_t v_t (total mass 1).
 *   Three launches: logits (K read once), tau (Newton from below), values
 *   (V read only for 16-row groups holding a row with p > 0).
 */
int64_t entmax_scratch_floats(int B, int H_q, int k_cap, int page_size);
int entmax15_paged_decode(const float *q, int B, int H_q, int H_kv, int D,
                          const uint16_t *kv_cache, int64_t num_blocks,
                          int page_size, const int32_t *block_table,
                          int64_t bt_ld, const int32_t *seq_lens,
                          const int32_t *sel_idx, const int32_t *sel_cnt,
                          const int32_t *sel_blk, int k_cap, int H_sel,
                          float scale, int num_splits,
                          const float *alibi_slopes, float *o_part,
                          float *lse_part, float *scratch,
                          int64_t scratch_floats, hipStream_t stream);

/*
 * entmax15_paged_decode_merged -- the same attention in one launch, merged:
 * one block per query row computes the logits of its selected rows (kept in
 * LDS when k_cap * page_size <= 8192, else in scratch), tau, and
 * out = sum_t p_t v_t / sum_t p_t, with lse_out = ln sum_t p_t (about 0).
 *   Arguments as entmax15_paged_decode, without the partials and splits;
 *   out      fp32 [B, H_q, D];  lse_out fp32 [B, H_q] or NULL;
 *   tau_out  fp32 [B, H_q] or NULL (tau of each row, -inf with no valid row);
 *   scratch  fp32 device buffer of >= B * H_q * k_cap * page_size floats when
 *            k_cap * page_size > 8192, else ignored (may be NULL).
 */
int entmax15_paged_decode_merged(const float *q, int B, int H_q, int H_kv, int D,
                                 const uint16_t *kv_cache, int64_t num_blocks,
                                 int page_size, const int32_t *block_table,
                                 int64_t bt_ld, const int32_t *seq_lens,
                                 const int32_t *sel_idx, const int32_t *sel_cnt,
                                 const int32_t *sel_blk, int k_cap, int H_sel,
                                 float scale, const float *alibi_slopes, float *out,
                                 float *lse_out, float *tau_out, float *scratch,
                                 int64_t scratch_floats, hipStream_t stream);

/*
 * Gaussian-aware adaptive selection.  [EKV "How it works": pages keep mean /
 * std key statistics; each page's scores are modelled as a Gaussian; the
 * distributional entmax constraint gives the threshold tau-hat (a page
 * mixture for ALiBi heads, one Gaussian for NoPE heads); every page whose
 * estimated maximum can cross tau-hat is selected, so the number of pages
 * adapts.  EKV "Quick start": the Gaussian-aware decode runs alpha = 1.5.]
 * A step: pagestats_update, page_var_update, gauss_moments, gauss_select,
 * entmax15_paged_decode_merged over the selection (H_sel = H_q) (or
 * entmax15_paged_decode, then lse_merge).
 *
 * page_var_update -- population variance of the keys of a page per (kv head,
 * dim), over its n = min(P, S_b - p P) valid rows, around k_mean.
 *   k_mean   fp32 [num_blocks, H_kv, D] in (from pagestats_update, which must
 *            have run first on the same stream)
 *   k_var    fp32 [num_blocks, H_kv, D] out
 *   tail_only 0: every page p < N_b of every request (rebuild);
 *            nonzero: only the page holding token S_b - 1 (after an append).
 */
int page_var_update(const uint16_t *kv_cache, int64_t num_blocks, int page_size,
                    int H_kv, int D, const float *k_mean, float *k_var,
                    const int32_t *block_table, int64_t bt_ld,
                    const int32_t *seq_lens, int B, int tail_only,
                    hipStream_t stream);

/*
 * gauss_moments -- mean and variance of each page's logits z = scale q . k
 * for every query head (key dimensions, and the position, taken as
 * independent):
 *   mu  = scale q . k_mean + slope * (mean valid position - (S_b - 1)),
 *   var = scale^2 sum_d q_d^2 k_var_d + slope^2 (n^2 - 1) / 12.
 *   q            fp32 [B, H_q, D];  k_mean, k_var fp32 [num_blocks, H_kv, D]
 *   alibi_slopes fp32 [H_q] (logit units) or NULL (no bias terms)
 *   mu, var      fp32 [B, H_q, ld], ld >= bt_ld; entries p >= N_b untouched.
 */
int gauss_moments(const float *q, int B, int H_q, int H_kv, int D,
                  const float *k_mean, const float *k_var,
                  const int32_t *block_table, int64_t bt_ld,
                  const int32_t *seq_lens, int page_size, float scale,
                  const float *alibi_slopes, float *mu, float *var, int64_t ld,
                  hipStream_t stream);

/*
 * gauss_select -- tau-hat and the adaptive selection of every (request,
 * query head) row.
 *   With u = z / 2 and n_p valid rows per page, tau-hat solves
 *     mixture != 0:  sum_p n_p E[(X_p - tau)_+^2] = 1, X_p ~ N(mu_p/2, var_p/4);
 *     mixture == 0:  S E[(X - tau)_+^2] = 1, X ~ N(m/2, v/4) with m, v the
 *                    pooled mean and variance of the S tokens of the pages;
 *   (safeguarded Newton steps on log F in fp64).
 *   est_p = mu_p + sqrt(var_p) sqrt(2 ln n_p) (mu_p for n_p = 1), fp32.  Selected: the reserved first reserved_bos and
 *   last reserved_eos pages, and every other page with est_p / 2 > tau-hat
 *   (fp32 comparison); at most k_cap pages (largest estimates, ties to the
 *   lower index), at least one.
 *   mu, var  fp32 [B, H_q, ld] (from gauss_moments); bt_ld <= 32768.
 *   tau      fp32 [B * H_q] out, or NULL;  est fp32 [B, H_q, ld] out
 *            (required: the selection reads it back).
 *   sel_idx  int32 [B * H_q, k_cap] out, ascending, padded with -1;
 *   sel_cnt  int32 [B * H_q] out;  sel_blk int32 [B * H_q, k_cap] out or NULL
 *            (block_table[b][p] of each selected page).
 *   k_cap must hold the reserved pages (>= min(bt_ld, bos + eos)).
 */
int gauss_select(const float *mu, const float *var, int64_t ld, int B, int H_q,
                 const int32_t *seq_lens, int page_size,
                 const int32_t *block_table, int64_t bt_ld, int mixture,
                 int reserved_bos, int reserved_eos, int k_cap, float *tau,
                 float *est, int32_t *sel_idx, int32_t *sel_cnt, int32_t *sel_blk,
                 hipStream_t stream);

/*
 * lse_merge -- N-way log-sum-exp merge of split partials.  [MLA:
 * MergeAttnStates algebra; a +inf lse is read as -inf; if every partial is
 * -inf the first partial is emitted with lse -inf.]
 *
 *   o_part [rows, num_splits, D], lse_part [rows, num_splits] (fp32)
 *   out    fp32 [rows, D];  lse_out fp32 [rows] or NULL.
 *   With M = max lse_s, w_s = exp(lse_s - M):
 *     out = sum w_s o_s / sum w_s,  lse = M + ln sum w_s.
 */
int lse_merge(const float *o_part, const float *lse_part, int rows,
              int num_splits, int D, float *out, float *lse_out,
              hipStream_t stream);

/*
 * h2o_accumulate -- token-level heavy-hitter accumulator step (page_size 1).
 * [VTX "Token-level variants": the accumulated quantity is the softmax
 * attention probability over the request's scored tokens, scale defaults to
 * D^-0.5, the accumulator decays (0.984375 = 1 - 2^-6, exact in bf16) and is
 * stored in bf16; the follow-up's reference step: softmax over the window
 * [bos, S - eos) only.]
 *
 *   Per (b, kv head h): qbar = mean of the G query rows of the group,
 *   l_t = scale * qbar . k_t for t in W = [bos, S_b - eos), p = softmax_W(l),
 *   hh_t <- bf16( bf16(p_t) + bf16(decay) * hh_t ) for t in W (fp32 math,
 *   round-to-nearest-even stores); entries outside W are not touched.
 *   hh_score bf16 [num_blocks, H_kv] (token slot = physical block), in place.
 *   scores   fp32 [B, H_kv, score_ld]: the new hh value of every t < S_b, in
 *            logical order (input of page_topk with H_sel = H_kv).
 *   scratch  fp32 device buffer of at least
 *            h2o_scratch_floats(B, H_kv, bt_ld) floats (its contents on entry
 *            are ignored).
 *   decay must lie in (0, 1].
 */
int h2o_accumulate(const float *q, int B, int H_q, int H_kv, int D,
                   const uint16_t *kv_cache, int64_t num_blocks, int page_size,
                   const int32_t *block_table, int64_t bt_ld,
                   const int32_t *seq_lens, int reserved_bos, int reserved_eos,
                   float scale, float decay, uint16_t *hh_score, float *scores,
                   int64_t score_ld, float *scratch, int64_t scratch_floats,
                   hipStream_t stream);

/* Scratch size (floats) h2o_accumulate needs for B requests, H_kv heads and
 * rows of at most max_tokens tokens.  No device work; -1 on bad arguments. */
int64_t h2o_scratch_floats(int B, int H_kv, int64_t max_tokens);

/*
 * h2o_accumulate_noalloc -- h2o_accumulate for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same step, the same kernels and the same result,
 * with the scratch taken from a fixed buffer inside the library instead of a
 * caller argument.  The call itself allocates and frees nothing.
 *
 *   Arguments, layouts and errors as h2o_accumulate, without scratch and
 *   scratch_floats.  Additionally
 *     - h2o_scratch_floats(B, H_kv, bt_ld) must not exceed
 *       SKV_NOALLOC_SCRATCH_FLOATS (SKV_EINVAL otherwise);
 *     - stream must belong to the current device (SKV_EINVAL otherwise);
 *       NULL is the current device's null stream.
 *   The buffer is a device array of SKV_NOALLOC_SCRATCH_FLOATS floats (8 MiB)
 *   that each GPU the library runs on holds until the process ends; its
 *   address is looked up once per device, on the first call there.  Every
 *   call on one GPU uses that GPU's single buffer: calls whose work overlaps
 *   on one GPU (other streams, other threads) race and must be serialised by
 *   the caller.  Nothing in the buffer needs to start at zero: each call
 *   writes what it reads.
 */
#define SKV_NOALLOC_SCRATCH_FLOATS (2 * 1024 * 1024)
int h2o_accumulate_noalloc(const float *q, int B, int H_q, int H_kv, int D,
                           const uint16_t *kv_cache, int64_t num_blocks,
                           int page_size, const int32_t *block_table,
                           int64_t bt_ld, const int32_t *seq_lens,
                           int reserved_bos, int reserved_eos, float scale,
                           float decay, uint16_t *hh_score, float *scores,
                           int64_t score_ld, hipStream_t stream);

/*
 * h2o_select_decode -- the token-level step, up to the split partials, in two
 * launches: (optionally the append), h2o_accumulate (either reading), then
 * page_topk with H_sel = H_kv and sparse_paged_decode.  [VTX "Token-level variants":
 * accumulate, select per kv head, attend over the selected tokens; the
 * sources of the three steps.]
 *   Launch 1 is the accumulator's logits pass, which also copies the
 *   accumulator of every token it covers into the scratch.  Launch 2 runs one
 *   block per (split, kv head, request): it applies the accumulator update to
 *   its row from the logits and that copy (the arithmetic of h2o_accumulate's
 *   update), selects the row's tokens in-block (page_topk's selection), and
 *   attends over its chunk of the selection for the G query heads; the
 *   row's split blocks then share writing the new hh values (and the fp32
 *   row, when scores is given).  The accumulator, the score rows and the
 *   selection equal h2o_accumulate (per_head: h2o_accumulate_heads) +
 *   page_topk_blk bit for bit, and the partials equal sparse_paged_decode's
 *   as sparse_select_decode_group's do (bit for bit while a split holds at
 *   most 64 tokens).
 *
 *   q ... seq_lens, reserved_bos, reserved_eos, scale, decay, hh_score: as
 *            h2o_accumulate (page_size 1); bt_ld <= 8192.
 *   per_head 0: group-mean query (h2o_accumulate); nonzero: every query
 *            head's own softmax averaged over the group (h2o_accumulate_heads).
 *   scores   fp32 [B, H_kv, score_ld] or NULL: the new hh row, as
 *            h2o_accumulate writes it (score_ld >= bt_ld).
 *   topk_pages, topk_frac, k_cap: as page_topk (k_cap <= 4096); the reserved
 *            window is reserved_bos / reserved_eos, as for the accumulator.
 *   num_splits, o_part [B, H_q, num_splits, D], lse_part [B, H_q, num_splits]:
 *            as sparse_paged_decode with H_sel = H_kv; lse_merge combines them.
 *   sel_idx, sel_cnt (both or neither), sel_blk (needs sel_idx):
 *            [B, H_kv, k_cap] / [B, H_kv] or NULL, as page_topk_blk writes them.
 *   k_new, v_new  bf16 [B, H_kv, D] (both or neither) or NULL: this step's
 *            new token; given, launch 1 also does pagestats_update's append
 *            with no statistics (K and V written at position S_b - 1, its hh
 *            slot zeroed; nothing when S_b - 1 >= bt_ld) and takes that
 *            token's key from k_new, so the results equal pagestats_update
 *            (append, hh_score given, no statistics) followed by the call
 *            without them.  kv_cache is written only then.
 *   scratch  fp32, at least h2o_select_decode_scratch_floats(B, H_q, H_kv,
 *            bt_ld, per_head) floats; contents on entry are ignored.
 */
int h2o_select_decode(const float *q, int B, int H_q, int H_kv, int D,
                      uint16_t *kv_cache, int64_t num_blocks, int page_size,
                      const int32_t *block_table, int64_t bt_ld,
                      const int32_t *seq_lens, int reserved_bos, int reserved_eos,
                      float scale, float decay, int per_head, uint16_t *hh_score,
                      float *scores, int64_t score_ld, int topk_pages,
                      float topk_frac, int k_cap, int num_splits, float *o_part,
                      float *lse_part, int32_t *sel_idx, int32_t *sel_cnt,
                      int32_t *sel_blk, const uint16_t *k_new,
                      const uint16_t *v_new, float *scratch, int64_t scratch_floats,
                      hipStream_t stream);

/* Scratch size (floats) h2o_select_decode needs; no device work; -1 on bad
 * arguments. */
int64_t h2o_select_decode_scratch_floats(int B, int H_q, int H_kv,
                                         int64_t max_tokens, int per_head);

/*
 * h2o_accumulate_heads -- the same step with the query-group axis kept through
 * the softmax.  [VTX description: the GQA variants compute the product and
 * the softmax over the query-group axis; VTX "Token-level variants" for the
 * accumulator.]
 *
 *   Per (b, kv head h): every query head g of the group takes its own
 *   p_g = softmax_W(scale * q_g . k_t) over W = [bos, S_b - eos), and
 *   p = (1/G) sum_g p_g (still one unit of mass per step) feeds the same
 *   recurrence, hh_t <- bf16( bf16(p_t) + bf16(decay) * hh_t ) for t in W.
 *   Arguments, layouts and errors as h2o_accumulate, except that the scratch
 *   holds h2o_heads_scratch_floats(B, H_q, bt_ld) floats and
 *   H_q * (D + 72) + 64 must stay within 16384 (a request's query rows as
 *   bf16 halves and one 64-token chunk's logits sit in one block's 64 KiB of
 *   LDS; SKV_EINVAL otherwise).  The logits run on the matrix cores with the
 *   query as bf16 hi + lo halves (about 16 significant bits).
 */
int h2o_accumulate_heads(const float *q, int B, int H_q, int H_kv, int D,
                         const uint16_t *kv_cache, int64_t num_blocks,
                         int page_size, const int32_t *block_table,
                         int64_t bt_ld, const int32_t *seq_lens,
                         int reserved_bos, int reserved_eos, float scale,
                         float decay, uint16_t *hh_score, float *scores,
                         int64_t score_ld, float *scratch,
                         int64_t scratch_floats, hipStream_t stream);

/* Scratch size (floats) h2o_accumulate_heads needs for B requests, H_q query
 * heads and rows of at most max_tokens tokens.  No device work; -1 on bad
 * arguments. */
int64_t h2o_heads_scratch_floats(int B, int H_q, int64_t max_tokens);

#ifdef __cplusplus
}
#endif

#endif /* SPARSEKV_H */
