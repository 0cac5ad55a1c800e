/*
 * sparsekv_oracle.c -- plain, slow, float64 CPU oracle for decode-time
 * page-scored sparse attention over a paged bf16 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; it reads the same input bytes and nothing else.
 *
 * Sources (cited by page title and section):
 *   [VTX]  vortex_torch pull request "flow: add H2O sparse attention
 *          (page-level and token-level, MHA + GQA)": sections "Page-level
 *          variants", "Token-level variants", "Verification" and the
 *          follow-up's reference recurrence ("reference_step").
 *   [EKV]  EntmaxKV README: "How it works" (paged layout, per-page key
 *          statistics, top-k per query head with the tail page in the budget).
 *   [MLA]  vllm.cpp test_ops_mla_chunked_context.cpp: the float64 two-pass
 *          attention oracle and the MergeAttnStates log-sum-exp algebra with
 *          its -inf / +inf edge cases.
 *
 * Conventions (plain readings where the pages are silent):
 *   - cache layout [2, num_blocks, page_size, H_kv, D], bf16 bit patterns,
 *     index 0 = K, 1 = V [EKV "How it works"];
 *   - seq_lens[b] counts the token appended this step; request b has
 *     N_b = ceil(S_b / P) logical pages, logical page p lives in physical block
 *     block_table[b * bt_ld + p];
 *   - query head i reads kv head i / G (consecutive groups);
 *   - everything is float64; bf16 values are decoded exactly.
 *
 * Parity pins: every function below is pinned by a test against closed forms,
 * invariants, brute force or printed values, with one exception in kind:
 * the Gaussian-aware selection's estimated-maximum rule (est = mu +
 * sigma * sqrt(2 ln n), a page kept when est / 2 > tau-hat) is a reading of
 * [EKV "How it works"], which names an estimated maximum but prints no
 * formula.  Its tests (brute force, limit cases) pin this code to that
 * reading; against the pages the rule is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */

/* A bf16 value is the upper half of an IEEE binary32 pattern, so widening is
 * exact: shift the 16 bits up and reinterpret. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in one step (no
 * intermediate binary32 rounding).  bf16 keeps 8 significant bits and the
 * binary32 exponent range: the spacing in [2^e, 2^(e+1)) is 2^(e-7), and below
 * 2^-126 the subnormal spacing 2^-133 applies.  Values that round to 2^128 or
 * beyond become infinity. */
uint16_t oracle_double_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e2;
    frexp(a, &e2);              /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;             /* a in [2^e, 2^(e+1)) */
    if (e < -126)
        e = -126;
    double spacing = ldexp(1.0, e - 7);
    double m = nearbyint(a / spacing);  /* exact division; ties to even */
    double r = m * spacing;
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;
    float rf = (float)r;        /* exact: r is a bf16 value */
    uint32_t w;
    memcpy(&w, &rf, sizeof w);
    return sign | (uint16_t)((w >> 16) & 0x7FFF);
}

/* ------------------------------------------------------------ helpers */

static int64_t cache_index(int kv, int64_t blk, int t, int h, int d,
                           int64_t num_blocks, int P, int H_kv, int D)
{
    return ((((int64_t)kv * num_blocks + blk) * P + t) * H_kv + h) * D + d;
}

static int pages_of(int S, int P)
{
    return (S + P - 1) / P;
}

/* -------------------------------------------------- page statistics (O2) */

/* Per-page key statistics [VTX "Page-level variants": element-wise max / min
 * envelope and mean of the keys; EKV "How it works": min/max per page].
 * For every request b and logical page p < N_b, over the n valid rows of the
 * page (n = min(P, S_b - p*P)), for every kv head and dim:
 *   kmin = min_t k, kmax = max_t k, kmean = (1/n) sum_t k.
 * Outputs are indexed by physical block: [num_blocks, H_kv, D]; blocks not
 * referenced by any request are left untouched. */
void oracle_page_stats(const uint16_t *kv_cache, int64_t num_blocks, int P,
                       int H_kv, int D, const int32_t *block_table,
                       int64_t bt_ld, const int32_t *seq_lens, int B,
                       double *kmin, double *kmax, double *kmean)
{
    for (int b = 0; b < B; ++b) {
        int S = seq_lens[b];
        int N = pages_of(S, P);
        for (int p = 0; p < N; ++p) {
            int64_t blk = block_table[(int64_t)b * bt_ld + p];
            int n = S - p * P < P ? S - p * P : P;
            for (int h = 0; h < H_kv; ++h) {
                for (int d = 0; d < D; ++d) {
                    double lo = INFINITY, hi = -INFINITY, sum = 0.0;
                    for (int t = 0; t < n; ++t) {
                        double k = oracle_bf16_to_double(kv_cache[cache_index(
                            0, blk, t, h, d, num_blocks, P, H_kv, D)]);
                        if (k < lo) lo = k;
                        if (k > hi) hi = k;
                        sum += k;
                    }
                    int64_t o = (blk * H_kv + h) * D + d;
                    kmin[o] = lo;
                    kmax[o] = hi;
                    kmean[o] = sum / n;
                }
            }
        }
    }
}

/* ------------------------------------------------------ page score (O3) */

/* Page score [VTX "Page-level variants"]:
 *   average relevance  a = sum_d q_d * kmean_d        (= page mean of q.k)
 *   peak relevance     u = sum_d max(q_d*kmax_d, q_d*kmin_d)
 *                          (upper bound of max_t q.k_t; both envelopes are
 *                           needed because q is signed)
 *   score = w_avg * a + w_peak * u            (the Add(alpha, beta) combine)
 * The softmax scale is not applied: a positive factor does not change the
 * ranking.  scores is [B, H_q, ld] in logical page order; only p < N_b is
 * written. */
void oracle_page_score(const double *q, int B, int H_q, int H_kv, int D,
                       const double *kmin, const double *kmax,
                       const double *kmean, const int32_t *block_table,
                       int64_t bt_ld, const int32_t *seq_lens, int P,
                       double w_avg, double w_peak, double *scores,
                       int64_t ld)
{
    int G = H_q / H_kv;
    for (int b = 0; b < B; ++b) {
        int N = pages_of(seq_lens[b], P);
        for (int i = 0; i < H_q; ++i) {
            int h = i / G;
            const double *qi = q + ((int64_t)b * H_q + i) * D;
            for (int p = 0; p < N; ++p) {
                int64_t blk = block_table[(int64_t)b * bt_ld + p];
                const double *mn = kmin + (blk * H_kv + h) * D;
                const double *mx = kmax + (blk * H_kv + h) * D;
                const double *me = kmean + (blk * H_kv + h) * D;
                double avg = 0.0, peak = 0.0;
                for (int d = 0; d < D; ++d) {
                    avg += qi[d] * me[d];
                    double up = qi[d] * mx[d], lo = qi[d] * mn[d];
                    peak += up > lo ? up : lo;
                }
                scores[((int64_t)b * H_q + i) * ld + p] =
                    w_avg * avg + w_peak * peak;
            }
        }
    }
}

/* Group-shared page score, for a selection made once per kv head: the mean,
 * over the G query heads that read kv head h, of the per-head score above.
 * The vortex_torch pull request names GQA variants of the page-level flow
 * that reduce over the query-group axis; the reduction is read here as the
 * plain mean of the group's scores (its ranking equals that of the sum).
 * Output [B, H_kv, ld]. */
void oracle_page_score_group(const double *q, int B, int H_q, int H_kv, int D,
                             const double *kmin, const double *kmax,
                             const double *kmean, const int32_t *block_table,
                             int64_t bt_ld, const int32_t *seq_lens, int P,
                             double w_avg, double w_peak, double *scores,
                             int64_t ld)
{
    int G = H_q / H_kv;
    for (int b = 0; b < B; ++b) {
        int N = pages_of(seq_lens[b], P);
        for (int h = 0; h < H_kv; ++h) {
            for (int p = 0; p < N; ++p) {
                int64_t blk = block_table[(int64_t)b * bt_ld + p];
                const double *mn = kmin + (blk * H_kv + h) * D;
                const double *mx = kmax + (blk * H_kv + h) * D;
                const double *me = kmean + (blk * H_kv + h) * D;
                double total = 0.0;
                for (int g = 0; g < G; ++g) {
                    const double *qi = q + ((int64_t)b * H_q + h * G + g) * D;
                    double avg = 0.0, peak = 0.0;
                    for (int d = 0; d < D; ++d) {
                        avg += qi[d] * me[d];
                        double up = qi[d] * mx[d], lo = qi[d] * mn[d];
                        peak += up > lo ? up : lo;
                    }
                    total += w_avg * avg + w_peak * peak;
                }
                scores[((int64_t)b * H_kv + h) * ld + p] = total / G;
            }
        }
    }
}

/* ALiBi-aware page score.  EntmaxKV README "How it works": the page bound
 * includes the ALiBi bias at the page's best logical position.  A key at
 * position t of a request with S tokens gets the logit bias
 * slope_i * (t - (S - 1)) <= 0 (the query sits at S - 1), so in the score's
 * q.k units each term takes alibi_i = slope_i / scale times the offset of the
 * position it describes: the peak term (a bound on the page's best logit) at
 * the page's last valid position, the mean term (the page's mean logit) at
 * the mean of its valid positions.
 *   alibi     [H_q] per query head, score units (slope / softmax scale)
 *   aggregate 0: scores [B, H_q, ld]; 1: scores [B, H_kv, ld] = the mean over
 *             each kv head's query group (as oracle_page_score_group). */
void oracle_page_score_alibi(const double *q, int B, int H_q, int H_kv, int D,
                             const double *kmin, const double *kmax,
                             const double *kmean, const int32_t *block_table,
                             int64_t bt_ld, const int32_t *seq_lens, int P,
                             double w_avg, double w_peak, const double *alibi,
                             int aggregate, double *scores, int64_t ld)
{
    int G = H_q / H_kv;
    for (int b = 0; b < B; ++b) {
        int S = seq_lens[b];
        int N = pages_of(S, P);
        for (int h = 0; h < H_kv; ++h) {
            for (int p = 0; p < N; ++p) {
                int64_t blk = block_table[(int64_t)b * bt_ld + p];
                const double *mn = kmin + (blk * H_kv + h) * D;
                const double *mx = kmax + (blk * H_kv + h) * D;
                const double *me = kmean + (blk * H_kv + h) * D;
                int n = S - p * P < P ? S - p * P : P;
                double last = (double)p * P + (n - 1) - (double)(S - 1);
                double mid = (double)p * P + 0.5 * (n - 1) - (double)(S - 1);
                double total = 0.0;
                for (int g = 0; g < G; ++g) {
                    int i = h * G + g;
                    const double *qi = q + ((int64_t)b * H_q + i) * D;
                    double avg = 0.0, peak = 0.0;
                    for (int d = 0; d < D; ++d) {
                        avg += qi[d] * me[d];
                        double up = qi[d] * mx[d], lo = qi[d] * mn[d];
                        peak += up > lo ? up : lo;
                    }
                    double s = w_avg * (avg + alibi[i] * mid) +
                               w_peak * (peak + alibi[i] * last);
                    if (aggregate)
                        total += s;
                    else
                        scores[((int64_t)b * H_q + i) * ld + p] = s;
                }
                if (aggregate)
                    scores[((int64_t)b * H_kv + h) * ld + p] = total / G;
            }
        }
    }
}

/* --------------------------------------------------------- selection (O4) */

struct ranked {
    double score;
    int32_t index;
};

/* Total order: higher score first, then lower index first. */
static int by_score_desc_index_asc(const void *pa, const void *pb)
{
    const struct ranked *a = pa, *b = pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->index > b->index) - (a->index < b->index);
}

static int by_int_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Budget of a row with N candidates [EKV "How it works": the budget counts
 * pages and includes the always-attended tail page]:
 *   k = min(N, max(topk_pages, floor(topk_frac * N))). */
int oracle_budget(int N, int topk_pages, double topk_frac)
{
    double f = floor(topk_frac * (double)N);
    int k = topk_pages;
    if (f > (double)k) k = (int)f;
    return k < N ? k : N;
}

/* Top-k selection of one row of N scores [EKV "How it works"; VTX follow-up:
 * the reserved leading bos and trailing eos entries are kept unconditionally
 * and only the window between them is ranked].
 *   R = [0, bos) u [N - eos, N), clipped to [0, N);
 *   rank the other entries by (score desc, index asc) and take the first
 *   max(0, k - |R|); the result is R u taken, ascending.
 * Writes the indices to out (capacity >= max(k, |R|)) and returns the count. */
int oracle_select(const double *scores, int N, int topk_pages,
                  double topk_frac, int bos, int eos, int32_t *out)
{
    int k = oracle_budget(N, topk_pages, topk_frac);
    int lo = bos < N ? bos : N;              /* window [lo, hi) */
    int hi = N - eos > 0 ? N - eos : 0;
    if (hi < lo) hi = lo;
    int count = 0;
    for (int p = 0; p < N; ++p)
        if (p < lo || p >= hi)
            out[count++] = p;
    int want = k - count;
    if (want > 0) {
        int n = hi - lo;
        struct ranked *r = malloc(sizeof *r * (n > 0 ? n : 1));
        for (int j = 0; j < n; ++j) {
            r[j].score = scores[lo + j];
            r[j].index = lo + j;
        }
        qsort(r, n, sizeof *r, by_score_desc_index_asc);
        for (int j = 0; j < want && j < n; ++j)
            out[count++] = r[j].index;
        free(r);
    }
    qsort(out, count, sizeof *out, by_int_asc);
    return count;
}

/* ------------------------------------------------------ attention (O5) */

/* Exact softmax attention of one query row over the tokens of a list of
 * logical pages [EKV "How it works": only the selected pages are attended,
 * exactly; MLA: the float64 two-pass oracle].  Tokens are {p*P + t : p in
 * pages, t < n_p} with n_p = min(P, S - p*P).  With l = scale * q.k:
 *   m = max l,  Z = sum exp(l - m),  o = sum exp(l - m) v / Z,
 *   lse = m + ln Z.
 * An empty token set gives o = 0 and lse = -inf. */
void oracle_attend(const double *q, int D, const uint16_t *kv_cache,
                   int64_t num_blocks, int P, int H_kv, int kv_head,
                   const int32_t *bt_row, int S, const int32_t *pages,
                   int npages, double scale, double *o, double *lse)
{
    int ntok = 0;
    for (int j = 0; j < npages; ++j) {
        int n = S - pages[j] * P < P ? S - pages[j] * P : P;
        ntok += n > 0 ? n : 0;
    }
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (ntok == 0) {
        *lse = -INFINITY;
        return;
    }
    double *logit = malloc(sizeof *logit * ntok);
    int64_t *blk = malloc(sizeof *blk * ntok);
    int *row = malloc(sizeof *row * ntok);
    int t = 0;
    for (int j = 0; j < npages; ++j) {
        int n = S - pages[j] * P < P ? S - pages[j] * P : P;
        for (int r = 0; r < n; ++r, ++t) {
            blk[t] = bt_row[pages[j]];
            row[t] = r;
        }
    }
    /* pass 1: logits and their maximum */
    double m = -INFINITY;
    for (t = 0; t < ntok; ++t) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += q[d] * oracle_bf16_to_double(kv_cache[cache_index(
                       0, blk[t], row[t], kv_head, d, num_blocks, P, H_kv, D)]);
        logit[t] = scale * dot;
        if (logit[t] > m) m = logit[t];
    }
    /* pass 2: normaliser and weighted sum of values */
    double Z = 0.0;
    for (t = 0; t < ntok; ++t) {
        double w = exp(logit[t] - m);
        Z += w;
        for (int d = 0; d < D; ++d)
            o[d] += w * oracle_bf16_to_double(kv_cache[cache_index(
                        1, blk[t], row[t], kv_head, d, num_blocks, P, H_kv, D)]);
    }
    for (int d = 0; d < D; ++d)
        o[d] /= Z;
    *lse = m + log(Z);
    free(logit);
    free(blk);
    free(row);
}

/* The same attention with an ALiBi bias: logit_t = scale * q.k_t +
 * slope * (t - (S - 1)) for a key at logical position t (EntmaxKV README "How
 * it works" names ALiBi heads; the bias is the standard linear one, zero at
 * the query's own position). */
void oracle_attend_alibi(const double *q, int D, const uint16_t *kv_cache,
                         int64_t num_blocks, int P, int H_kv, int kv_head,
                         const int32_t *bt_row, int S, const int32_t *pages,
                         int npages, double scale, double slope, double *o,
                         double *lse)
{
    int ntok = 0;
    for (int j = 0; j < npages; ++j) {
        int n = S - pages[j] * P < P ? S - pages[j] * P : P;
        ntok += n > 0 ? n : 0;
    }
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (ntok == 0) {
        *lse = -INFINITY;
        return;
    }
    double *logit = malloc(sizeof *logit * ntok);
    int64_t *blk = malloc(sizeof *blk * ntok);
    int *row = malloc(sizeof *row * ntok);
    int t = 0;
    double m = -INFINITY;
    for (int j = 0; j < npages; ++j) {
        int n = S - pages[j] * P < P ? S - pages[j] * P : P;
        for (int r = 0; r < n; ++r, ++t) {
            blk[t] = bt_row[pages[j]];
            row[t] = r;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += q[d] * oracle_bf16_to_double(kv_cache[cache_index(
                           0, blk[t], r, kv_head, d, num_blocks, P, H_kv, D)]);
            double pos = (double)pages[j] * P + r;
            logit[t] = scale * dot + slope * (pos - (double)(S - 1));
            if (logit[t] > m) m = logit[t];
        }
    }
    double Z = 0.0;
    for (t = 0; t < ntok; ++t) {
        double w = exp(logit[t] - m);
        Z += w;
        for (int d = 0; d < D; ++d)
            o[d] += w * oracle_bf16_to_double(kv_cache[cache_index(
                        1, blk[t], row[t], kv_head, d, num_blocks, P, H_kv, D)]);
    }
    for (int d = 0; d < D; ++d)
        o[d] /= Z;
    *lse = m + log(Z);
    free(logit);
    free(blk);
    free(row);
}

/* ------------------------------------------------- 1.5-entmax (NEXT row) */

/* alpha-entmax with alpha = 1.5 (EntmaxKV README, "Quick start": alpha=1.5;
 * the mapping is the published one of Peters, Niculae and Martins, 2019):
 *   p_t = [ (alpha - 1) z_t - tau ]_+ ^ (1 / (alpha - 1)) = [ z_t / 2 - tau ]_+ ^ 2
 * with tau the unique value making sum_t p_t = 1.  f(tau) = sum [u - tau]_+^2
 * - 1 (u = z / 2) falls strictly from f(max u - 1) >= 0 to f(max u) = -1, so
 * tau is found by bisection on [max u - 1, max u] (200 halvings: the bracket
 * ends far below one ulp of the double). */
double oracle_entmax15_tau(const double *z, int n)
{
    double umax = -INFINITY;
    for (int t = 0; t < n; ++t)
        if (z[t] / 2.0 > umax) umax = z[t] / 2.0;
    double lo = umax - 1.0, hi = umax;
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi);
        double f = -1.0;
        for (int t = 0; t < n; ++t) {
            double d = z[t] / 2.0 - mid;
            if (d > 0.0) f += d * d;
        }
        if (f >= 0.0) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/* 1.5-entmax attention of one query row over the tokens of the selected
 * pages: z_t = scale * q.k_t, p = entmax15(z), o = sum_t p_t v_t.  Writes o
 * [D] and tau; an empty selection gives o = 0 and tau = -inf. */
void oracle_attend_entmax15_alibi(const double *q, int D, const uint16_t *kv_cache,
                                  int64_t num_blocks, int P, int H_kv, int kv_head,
                                  const int32_t *bt_row, int S, const int32_t *pages,
                                  int npages, double scale, double slope, double *o,
                                  double *tau)
{
    int ntok = 0;
    for (int j = 0; j < npages; ++j) {
        int n = S - pages[j] * P < P ? S - pages[j] * P : P;
        ntok += n > 0 ? n : 0;
    }
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (ntok == 0) {
        *tau = -INFINITY;
        return;
    }
    double *z = malloc(sizeof *z * ntok);
    int64_t *blk = malloc(sizeof *blk * ntok);
    int *row = malloc(sizeof *row * ntok);
    int t = 0;
    for (int j = 0; j < npages; ++j) {
        int n = S - pages[j] * P < P ? S - pages[j] * P : P;
        for (int r = 0; r < n; ++r, ++t) {
            blk[t] = bt_row[pages[j]];
            row[t] = r;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += q[d] * oracle_bf16_to_double(kv_cache[cache_index(
                           0, blk[t], r, kv_head, d, num_blocks, P, H_kv, D)]);
            /* ALiBi bias of a key at position pos: slope * (pos - (S - 1)) */
            z[t] = scale * dot + slope * ((double)pages[j] * P + r - (double)(S - 1));
        }
    }
    double tu = oracle_entmax15_tau(z, ntok);
    for (t = 0; t < ntok; ++t) {
        double d = z[t] / 2.0 - tu;
        if (d <= 0.0)
            continue;
        double p = d * d;
        for (int c = 0; c < D; ++c)
            o[c] += p * oracle_bf16_to_double(kv_cache[cache_index(
                        1, blk[t], row[t], kv_head, c, num_blocks, P, H_kv, D)]);
    }
    *tau = tu;
    free(z);
    free(blk);
    free(row);
}

void oracle_attend_entmax15(const double *q, int D, const uint16_t *kv_cache,
                            int64_t num_blocks, int P, int H_kv, int kv_head,
                            const int32_t *bt_row, int S, const int32_t *pages,
                            int npages, double scale, double *o, double *tau)
{
    oracle_attend_entmax15_alibi(q, D, kv_cache, num_blocks, P, H_kv, kv_head, bt_row,
                                 S, pages, npages, scale, 0.0, o, tau);
}

/* ------------------------------------- Gaussian-aware selection (NEXT row) */

/* EntmaxKV README "How it works": for the Gaussian-aware strategy pages keep
 * mean and std key statistics, each page's scores are modelled as a Gaussian,
 * the distributional entmax constraint gives a threshold tau-hat (a page
 * mixture for ALiBi heads, a single Gaussian otherwise), and every page whose
 * estimated maximum can cross tau-hat is selected, so the page count adapts.
 * The pages give no formulas; the plain readings taken here:
 *   page statistic  population variance per dim over the page's valid rows;
 *   page moments    z = scale q.k (+ the ALiBi bias): mu_p = scale q.mean_p
 *                   (+ the bias at the page's mean position), var_p =
 *                   scale^2 sum_d q_d^2 var_pd (+ slope^2 (n_p^2 - 1) / 12,
 *                   the variance of the bias over n_p consecutive positions):
 *                   key dimensions and position taken as independent;
 *   constraint      with u = z / 2 (alpha = 1.5), sum over the request's
 *                   tokens of E[(u - tau)_+^2] = 1: each page contributes
 *                   n_p E[(X - tau)_+^2], X ~ N(mu_p / 2, var_p / 4)
 *                   (mixture), or all S tokens share N(mu, var) with the
 *                   pooled mean and variance (single);
 *   estimated max   mu_p + sqrt(var_p) sqrt(2 ln n_p) (the usual estimate of
 *                   the largest of n_p Gaussian draws);
 *   selection       reserved pages, plus every other page with est_max / 2 >
 *                   tau-hat; above k_cap entries the largest estimates win,
 *                   ties to the lower index.  The qualifying pages are the
 *                   ones of largest estimate, so this is the top-k selection
 *                   over the estimates with the budget (reserved + qualifying,
 *                   at most k_cap, at least one page). */

void oracle_page_var(const uint16_t *kv_cache, int64_t num_blocks, int P, int H_kv,
                     int D, const int32_t *block_table, int64_t bt_ld,
                     const int32_t *seq_lens, int B, double *kvar)
{
    for (int b = 0; b < B; ++b) {
        int S = seq_lens[b];
        int N = pages_of(S, P);
        for (int p = 0; p < N; ++p) {
            int64_t blk = block_table[(int64_t)b * bt_ld + p];
            int n = S - p * P < P ? S - p * P : P;
            for (int h = 0; h < H_kv; ++h)
                for (int d = 0; d < D; ++d) {
                    double mean = 0.0, ss = 0.0;
                    for (int t = 0; t < n; ++t)
                        mean += oracle_bf16_to_double(kv_cache[cache_index(
                            0, blk, t, h, d, num_blocks, P, H_kv, D)]);
                    mean /= n;
                    for (int t = 0; t < n; ++t) {
                        double k = oracle_bf16_to_double(kv_cache[cache_index(
                            0, blk, t, h, d, num_blocks, P, H_kv, D)]);
                        ss += (k - mean) * (k - mean);
                    }
                    kvar[(blk * H_kv + h) * D + d] = ss / n;
                }
        }
    }
}

/* mu, var [B, H_q, ld] for p < N_b.  alibi [H_q] (logit units) or NULL. */
void oracle_gauss_moments(const double *q, int B, int H_q, int H_kv, int D,
                          const double *kmean, const double *kvar,
                          const int32_t *block_table, int64_t bt_ld,
                          const int32_t *seq_lens, int P, double scale,
                          const double *alibi, double *mu, double *var, int64_t ld)
{
    int G = H_q / H_kv;
    for (int b = 0; b < B; ++b) {
        int S = seq_lens[b];
        int N = pages_of(S, P);
        for (int i = 0; i < H_q; ++i) {
            const double *qi = q + ((int64_t)b * H_q + i) * D;
            for (int p = 0; p < N; ++p) {
                int64_t blk = block_table[(int64_t)b * bt_ld + p];
                const double *me = kmean + (blk * H_kv + i / G) * D;
                const double *va = kvar + (blk * H_kv + i / G) * D;
                double m = 0.0, v = 0.0;
                for (int d = 0; d < D; ++d) {
                    m += qi[d] * me[d];
                    v += qi[d] * qi[d] * va[d];
                }
                m *= scale;
                v *= scale * scale;
                if (alibi != NULL) {
                    int n = S - p * P < P ? S - p * P : P;
                    m += alibi[i] * ((double)p * P + 0.5 * (n - 1) - (double)(S - 1));
                    v += alibi[i] * alibi[i] * ((double)n * n - 1.0) / 12.0;
                }
                mu[((int64_t)b * H_q + i) * ld + p] = m;
                var[((int64_t)b * H_q + i) * ld + p] = v;
            }
        }
    }
}

/* E[(X - tau)_+^2] for X ~ N(m, s^2). */
static double gauss_excess2(double m, double s, double tau)
{
    double d = m - tau;
    if (s <= 0.0)
        return d > 0.0 ? d * d : 0.0;
    double a = d / s;
    double Phi = 0.5 * erfc(-a / sqrt(2.0));
    double phi = exp(-0.5 * a * a) / 2.5066282746310002;   /* sqrt(2 pi) */
    return (d * d + s * s) * Phi + d * s * phi;
}

/* tau-hat of one row: mu, var, n over N pages; mixture != 0 sums the page
 * Gaussians, else the pooled single Gaussian.  Bisection on [max m - 2,
 * max (m + 12 s)] where the constraint is >= 2 and ~0 respectively. */
double oracle_gauss_tau(const double *mu, const double *var, const int *n, int N,
                        int mixture)
{
    double S = 0.0, sm = 0.0, sq = 0.0;
    for (int p = 0; p < N; ++p) {
        S += n[p];
        sm += n[p] * mu[p];
        sq += n[p] * (var[p] + mu[p] * mu[p]);
    }
    double gm = sm / S, gv = sq / S - gm * gm;
    if (gv < 0.0) gv = 0.0;
    double mmax = -INFINITY, hi = -INFINITY;
    for (int p = 0; p < N; ++p) {
        double m = mixture ? mu[p] / 2.0 : gm / 2.0;
        double s = sqrt(mixture ? var[p] : gv) / 2.0;
        if (m > mmax) mmax = m;
        if (m + 12.0 * s > hi) hi = m + 12.0 * s;
    }
    double lo = mmax - 2.0;
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi), f = 0.0;
        if (mixture) {
            for (int p = 0; p < N; ++p)
                f += n[p] * gauss_excess2(mu[p] / 2.0, sqrt(var[p]) / 2.0, mid);
        } else {
            f = S * gauss_excess2(gm / 2.0, sqrt(gv) / 2.0, mid);
        }
        if (f >= 1.0) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/* Pages of one row whose estimated max can cross tau (see above); writes the
 * ascending selection to sel and returns its size. */
int oracle_gauss_select(const double *mu, const double *var, const int *n, int N,
                        double tau, int bos, int eos, int k_cap, int32_t *sel)
{
    double *est = malloc(sizeof *est * (N > 0 ? N : 1));
    int lo = bos < N ? bos : N;
    int hi = N - eos > 0 ? N - eos : 0;
    if (hi < lo) hi = lo;
    int qual = 0;
    for (int p = 0; p < N; ++p) {
        double e = mu[p] + (n[p] > 1 ? sqrt(var[p]) * sqrt(2.0 * log((double)n[p])) : 0.0);
        est[p] = e;
        if (e / 2.0 > tau && p >= lo && p < hi) ++qual;
    }
    int nres = N - (hi - lo);
    int budget = qual + nres;
    if (budget > k_cap) budget = k_cap;
    if (budget < 1) budget = 1;
    int cnt = oracle_select(est, N, budget, 0.0, bos, eos, sel);
    free(est);
    return cnt;
}

/* ------------------------------------------------------ LSE merge (O6) */

/* N-way merge of normalised partial outputs by their log-sum-exps [MLA:
 * MergeAttnStates algebra and edge cases].  A +inf lse is treated as -inf.
 * M = max lse_i; if M = -inf the first partial is returned with lse -inf;
 * otherwise w_i = exp(lse_i - M), out = sum w_i o_i / sum w_i,
 * lse = M + ln sum w_i. */
void oracle_lse_merge(const double *o_parts, const double *lses, int n, int D,
                      double *out, double *lse_out)
{
    double M = -INFINITY;
    for (int i = 0; i < n; ++i) {
        double l = isinf(lses[i]) ? -INFINITY : lses[i];
        if (l > M) M = l;
    }
    if (M == -INFINITY) {
        for (int d = 0; d < D; ++d)
            out[d] = n > 0 ? o_parts[d] : 0.0;
        *lse_out = -INFINITY;
        return;
    }
    double W = 0.0;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    for (int i = 0; i < n; ++i) {
        double l = isinf(lses[i]) ? -INFINITY : lses[i];
        double w = exp(l - M);
        W += w;
        for (int d = 0; d < D; ++d)
            out[d] += w * o_parts[(int64_t)i * D + d];
    }
    for (int d = 0; d < D; ++d)
        out[d] /= W;
    *lse_out = M + log(W);
}

/* ------------------------------------------------------------ append (O7) */

/* KV append with reset-on-write [EKV quick start: the decode call appends
 * k_new / v_new; VTX "Token-level variants" point 2: the accumulated score of
 * a freshly written slot is zeroed so a recycled page does not inherit it].
 * Token S_b - 1 of request b is written: block bt[b][(S_b-1)/P], row
 * (S_b-1)%P.  k_new, v_new are [B, H_kv, D]; hh (nullable) is
 * [num_blocks*P, H_kv] and its written slot is set to zero for every kv head. */
void oracle_append(uint16_t *kv_cache, int64_t num_blocks, int P, int H_kv,
                   int D, const int32_t *block_table, int64_t bt_ld,
                   const int32_t *seq_lens, int B, const uint16_t *k_new,
                   const uint16_t *v_new, uint16_t *hh)
{
    for (int b = 0; b < B; ++b) {
        int pos = seq_lens[b] - 1;
        int64_t blk = block_table[(int64_t)b * bt_ld + pos / P];
        int row = pos % P;
        for (int h = 0; h < H_kv; ++h) {
            for (int d = 0; d < D; ++d) {
                int64_t src = ((int64_t)b * H_kv + h) * D + d;
                kv_cache[cache_index(0, blk, row, h, d, num_blocks, P, H_kv, D)] =
                    k_new[src];
                kv_cache[cache_index(1, blk, row, h, d, num_blocks, P, H_kv, D)] =
                    v_new[src];
            }
            if (hh)
                hh[(blk * P + row) * H_kv + h] = 0;
        }
    }
}

/* ------------------------------------------------ H2O accumulator (O8) */

/* One step of the decayed heavy-hitter accumulator over n entries [VTX
 * "Token-level variants" point 3 and the execute-mode Add + Save recurrence]:
 * the probability is stored in bf16 first, then
 *   hh <- bf16( bf16(p) + bf16(decay) * hh )
 * with the sum formed in float64 and rounded once. */
void oracle_h2o_recurrence(const double *p, uint16_t *hh, int n, double decay)
{
    double dd = oracle_bf16_to_double(oracle_double_to_bf16(decay));
    for (int t = 0; t < n; ++t) {
        double pb = oracle_bf16_to_double(oracle_double_to_bf16(p[t]));
        double old = oracle_bf16_to_double(hh[t]);
        hh[t] = oracle_double_to_bf16(pb + dd * old);
    }
}

/* Token-level H2O scoring step (page_size 1) [VTX "Token-level variants"
 * point 1 and the follow-up's reference step]: per request b and kv head h,
 *   qbar = mean of the G query rows of the group,
 *   over the window W = [bos, S_b - eos): l_t = scale * qbar . k_t,
 *   p = softmax_W(l), and every t in W gets the recurrence above.
 * Entries outside W are not touched.  hh is [num_blocks, H_kv] (bf16, in
 * place, physical token slots); scores [B, H_kv, ld] receives the value of hh
 * after the step for every t < S_b, in logical order. */
void oracle_h2o_step(const double *q, int B, int H_q, int H_kv, int D,
                     const uint16_t *kv_cache, int64_t num_blocks,
                     const int32_t *block_table, int64_t bt_ld,
                     const int32_t *seq_lens, int bos, int eos, double scale,
                     double decay, uint16_t *hh, double *scores, int64_t ld)
{
    int G = H_q / H_kv;
    double *qbar = malloc(sizeof *qbar * D);
    for (int b = 0; b < B; ++b) {
        int S = seq_lens[b];
        int lo = bos < S ? bos : S;
        int hi = S - eos > 0 ? S - eos : 0;
        if (hi < lo) hi = lo;
        int n = hi - lo;
        const int32_t *bt = block_table + (int64_t)b * bt_ld;
        double *l = malloc(sizeof *l * (n > 0 ? n : 1));
        double *pr = malloc(sizeof *pr * (n > 0 ? n : 1));
        uint16_t *slot = malloc(sizeof *slot * (n > 0 ? n : 1));
        for (int h = 0; h < H_kv; ++h) {
            for (int d = 0; d < D; ++d) {
                double s = 0.0;
                for (int g = 0; g < G; ++g)
                    s += q[((int64_t)b * H_q + h * G + g) * D + d];
                qbar[d] = s / G;
            }
            double m = -INFINITY;
            for (int j = 0; j < n; ++j) {
                int64_t blk = bt[lo + j];
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += qbar[d] * oracle_bf16_to_double(kv_cache[cache_index(
                               0, blk, 0, h, d, num_blocks, 1, H_kv, D)]);
                l[j] = scale * dot;
                if (l[j] > m) m = l[j];
            }
            double Z = 0.0;
            for (int j = 0; j < n; ++j) {
                pr[j] = exp(l[j] - m);
                Z += pr[j];
            }
            for (int j = 0; j < n; ++j) {
                pr[j] /= Z;
                slot[j] = hh[(int64_t)bt[lo + j] * H_kv + h];
            }
            oracle_h2o_recurrence(pr, slot, n, decay);
            for (int j = 0; j < n; ++j)
                hh[(int64_t)bt[lo + j] * H_kv + h] = slot[j];
            for (int t = 0; t < S; ++t)
                scores[((int64_t)b * H_kv + h) * ld + t] =
                    oracle_bf16_to_double(hh[(int64_t)bt[t] * H_kv + h]);
        }
        free(l);
        free(pr);
        free(slot);
    }
    free(qbar);
}

/* Per-head reading of the GQA token flow [VTX description: the GQA variants
 * run the product and the softmax with the query-group axis kept]: per request
 * b and kv head h, every query head g of the group takes its own softmax over
 * the window W = [bos, S_b - eos),
 *   p_g = softmax_W(scale * q_g . k_t),
 * the group's probabilities are averaged, p = (1/G) sum_g p_g (one unit of
 * mass per step, as in the group-mean reading), and every t in W gets the
 * recurrence above.  Layouts and untouched entries as oracle_h2o_step. */
void oracle_h2o_step_heads(const double *q, int B, int H_q, int H_kv, int D,
                           const uint16_t *kv_cache, int64_t num_blocks,
                           const int32_t *block_table, int64_t bt_ld,
                           const int32_t *seq_lens, int bos, int eos,
                           double scale, double decay, uint16_t *hh,
                           double *scores, int64_t ld)
{
    int G = H_q / H_kv;
    for (int b = 0; b < B; ++b) {
        int S = seq_lens[b];
        int lo = bos < S ? bos : S;
        int hi = S - eos > 0 ? S - eos : 0;
        if (hi < lo) hi = lo;
        int n = hi - lo;
        int nn = n > 0 ? n : 1;
        const int32_t *bt = block_table + (int64_t)b * bt_ld;
        double *l = malloc(sizeof *l * nn);
        double *pr = malloc(sizeof *pr * nn);
        uint16_t *slot = malloc(sizeof *slot * nn);
        for (int h = 0; h < H_kv; ++h) {
            for (int j = 0; j < n; ++j)
                pr[j] = 0.0;
            for (int g = 0; g < G; ++g) {
                const double *qg = q + ((int64_t)b * H_q + h * G + g) * D;
                double m = -INFINITY;
                for (int j = 0; j < n; ++j) {
                    int64_t blk = bt[lo + j];
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += qg[d] * oracle_bf16_to_double(kv_cache[cache_index(
                                   0, blk, 0, h, d, num_blocks, 1, H_kv, D)]);
                    l[j] = scale * dot;
                    if (l[j] > m) m = l[j];
                }
                double Z = 0.0;
                for (int j = 0; j < n; ++j) {
                    l[j] = exp(l[j] - m);
                    Z += l[j];
                }
                for (int j = 0; j < n; ++j)
                    pr[j] += l[j] / Z / G;
            }
            for (int j = 0; j < n; ++j)
                slot[j] = hh[(int64_t)bt[lo + j] * H_kv + h];
            oracle_h2o_recurrence(pr, slot, n, decay);
            for (int j = 0; j < n; ++j)
                hh[(int64_t)bt[lo + j] * H_kv + h] = slot[j];
            for (int t = 0; t < S; ++t)
                scores[((int64_t)b * H_kv + h) * ld + t] =
                    oracle_bf16_to_double(hh[(int64_t)bt[t] * H_kv + h]);
        }
        free(l);
        free(pr);
        free(slot);
    }
}

/* ------------------------------------------------ whole decode step */

/* One page-level decode step for the whole batch, used as the CPU baseline
 * and as the end-to-end reference: scores (O3) from the given statistics,
 * selection (O4) per query head, exact attention (O5) over the selection.
 * sel_idx is [B, H_q, k_cap] (-1 padded), sel_cnt [B, H_q], out [B, H_q, D],
 * lse [B, H_q]; scores is caller scratch [B, H_q, ld]. */
void oracle_decode_step(const double *q, int B, int H_q, int H_kv, int D,
                        const uint16_t *kv_cache, int64_t num_blocks, int P,
                        const int32_t *block_table, int64_t bt_ld,
                        const int32_t *seq_lens, const double *kmin,
                        const double *kmax, const double *kmean,
                        double w_avg, double w_peak, int topk_pages,
                        double topk_frac, int bos, int eos, double scale,
                        double *scores, int64_t ld, int32_t *sel_idx,
                        int32_t *sel_cnt, int k_cap, double *out, double *lse)
{
    int G = H_q / H_kv;
    oracle_page_score(q, B, H_q, H_kv, D, kmin, kmax, kmean, block_table,
                      bt_ld, seq_lens, P, w_avg, w_peak, scores, ld);
    for (int b = 0; b < B; ++b) {
        int N = pages_of(seq_lens[b], P);
        for (int i = 0; i < H_q; ++i) {
            int64_t r = (int64_t)b * H_q + i;
            int32_t *sel = sel_idx + r * k_cap;
            for (int j = 0; j < k_cap; ++j)
                sel[j] = -1;
            sel_cnt[r] = oracle_select(scores + r * ld, N, topk_pages,
                                       topk_frac, bos, eos, sel);
            oracle_attend(q + r * D, D, kv_cache, num_blocks, P, H_kv, i / G,
                          block_table + (int64_t)b * bt_ld, seq_lens[b], sel,
                          sel_cnt[r], scale, out + r * D, lse + r);
        }
    }
}
