/* Drives every function of oracle/sparsekv_oracle.c once or more on small,
 * ragged and degenerate inputs, with every buffer sized exactly, so that a
 * build with -fsanitize=address,undefined reports any out-of-bounds access,
 * use after free, leak or undefined operation.  Values are not checked here
 * (the pytest pins do that); the exit status carries the sanitizers' findings.
 * Test infrastructure: built and run by tests/test_oracle_sanitized.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_bf16_to_double(uint16_t bits);
uint16_t oracle_double_to_bf16(double x);
void oracle_page_stats(const uint16_t *kv_cache, int64_t num_blocks, int P, int H_kv,
                       int D, const int32_t *block_table, int64_t bt_ld,
                       const int32_t *seq_lens, int B, double *kmin, double *kmax,
                       double *kmean);
void oracle_page_score(const double *q, int B, int H_q, int H_kv, int D,
                       const double *kmin, const double *kmax, const double *kmean,
                       const int32_t *block_table, int64_t bt_ld, const int32_t *seq_lens,
                       int P, double w_avg, double w_peak, double *scores, int64_t ld);
void oracle_page_score_group(const double *q, int B, int H_q, int H_kv, int D,
                             const double *kmin, const double *kmax, const double *kmean,
                             const int32_t *block_table, int64_t bt_ld,
                             const int32_t *seq_lens, int P, double w_avg, double w_peak,
                             double *scores, int64_t ld);
void oracle_page_score_alibi(const double *q, int B, int H_q, int H_kv, int D,
                             const double *kmin, const double *kmax, const double *kmean,
                             const int32_t *block_table, int64_t bt_ld,
                             const int32_t *seq_lens, int P, double w_avg, double w_peak,
                             const double *alibi, int aggregate, double *scores,
                             int64_t ld);
int oracle_budget(int N, int topk_pages, double topk_frac);
int oracle_select(const double *scores, int N, int topk_pages, double topk_frac, int bos,
                  int eos, int32_t *out);
void oracle_attend(const double *q, int D, const uint16_t *kv_cache, int64_t num_blocks,
                   int P, int H_kv, int kv_head, const int32_t *bt_row, int S,
                   const int32_t *pages, int npages, double scale, double *o, double *lse);
void oracle_attend_alibi(const double *q, int D, const uint16_t *kv_cache,
                         int64_t num_blocks, int P, int H_kv, int kv_head,
                         const int32_t *bt_row, int S, const int32_t *pages, int npages,
                         double scale, double slope, double *o, double *lse);
double oracle_entmax15_tau(const double *z, int n);
void oracle_attend_entmax15_alibi(const double *q, int D, const uint16_t *kv_cache,
                                  int64_t num_blocks, int P, int H_kv, int kv_head,
                                  const int32_t *bt_row, int S, const int32_t *pages,
                                  int npages, double scale, double slope, double *o,
                                  double *tau);
void oracle_attend_entmax15(const double *q, int D, const uint16_t *kv_cache,
                            int64_t num_blocks, int P, int H_kv, int kv_head,
                            const int32_t *bt_row, int S, const int32_t *pages, int npages,
                            double scale, double *o, double *tau);
void oracle_page_var(const uint16_t *kv_cache, int64_t num_blocks, int P, int H_kv, int D,
                     const int32_t *block_table, int64_t bt_ld, const int32_t *seq_lens,
                     int B, double *kvar);
void oracle_gauss_moments(const double *q, int B, int H_q, int H_kv, int D,
                          const double *kmean, const double *kvar,
                          const int32_t *block_table, int64_t bt_ld,
                          const int32_t *seq_lens, int P, double scale,
                          const double *alibi, double *mu, double *var, int64_t ld);
double oracle_gauss_tau(const double *mu, const double *var, const int *n, int N,
                        int mixture);
int oracle_gauss_select(const double *mu, const double *var, const int *n, int N,
                        double tau, int bos, int eos, int k_cap, int32_t *sel);
void oracle_lse_merge(const double *o_parts, const double *lses, int n, int D, double *out,
                      double *lse_out);
void oracle_append(uint16_t *kv_cache, int64_t num_blocks, int P, int H_kv, int D,
                   const int32_t *block_table, int64_t bt_ld, const int32_t *seq_lens,
                   int B, const uint16_t *k_new, const uint16_t *v_new, uint16_t *hh);
void oracle_h2o_recurrence(const double *p, uint16_t *hh, int n, double decay);
void oracle_h2o_step(const double *q, int B, int H_q, int H_kv, int D,
                     const uint16_t *kv_cache, int64_t num_blocks,
                     const int32_t *block_table, int64_t bt_ld, const int32_t *seq_lens,
                     int bos, int eos, double scale, double decay, uint16_t *hh,
                     double *scores, int64_t ld);
void oracle_h2o_step_heads(const double *q, int B, int H_q, int H_kv, int D,
                           const uint16_t *kv_cache, int64_t num_blocks,
                           const int32_t *block_table, int64_t bt_ld,
                           const int32_t *seq_lens, int bos, int eos, double scale,
                           double decay, uint16_t *hh, double *scores, int64_t ld);
void oracle_decode_step(const double *q, int B, int H_q, int H_kv, int D,
                        const uint16_t *kv_cache, int64_t num_blocks, int P,
                        const int32_t *block_table, int64_t bt_ld, const int32_t *seq_lens,
                        const double *kmin, const double *kmax, const double *kmean,
                        double w_avg, double w_peak, int topk_pages, double topk_frac,
                        int bos, int eos, double scale, double *scores, int64_t ld,
                        int32_t *sel_idx, int32_t *sel_cnt, int k_cap, double *out,
                        double *lse);

static uint64_t lcg = 12345u;
static double uniform(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg >> 11) * (1.0 / 9007199254740992.0);
}
static double normal(void)
{
    double u = uniform(), v = uniform();
    return sqrt(-2.0 * log(u + 1e-300)) * cos(6.283185307179586 * v);
}
static void *alloc(size_t n) { return calloc(n > 0 ? n : 1, 1); }

enum { B = 3, H_Q = 8, H_KV = 2, D = 16, P = 4, LD = 10, NB = B * LD };

int main(void)
{
    /* bf16 round trips, including the special values */
    const double specials[] = {0.0, -0.0, 1.0, -2.5, 1e-40, 3.4e38, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i)
        (void)oracle_bf16_to_double(oracle_double_to_bf16(specials[i]));

    /* a paged cache with ragged requests: empty, one token, two and a half
     * pages, completely full */
    const int32_t seq_lens[B] = {0, 10, LD * P};
    const size_t ncache = (size_t)2 * NB * P * H_KV * D;
    uint16_t *cache = alloc(sizeof *cache * ncache);
    for (size_t i = 0; i < ncache; ++i) cache[i] = oracle_double_to_bf16(normal());
    int32_t *bt = alloc(sizeof *bt * B * LD);
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < LD; ++p) bt[b * LD + p] = NB - 1 - (p * B + b);   /* reversed */
    const size_t nstat = (size_t)NB * H_KV * D;
    double *kmin = alloc(sizeof *kmin * nstat), *kmax = alloc(sizeof *kmax * nstat);
    double *kmean = alloc(sizeof *kmean * nstat), *kvar = alloc(sizeof *kvar * nstat);
    oracle_page_stats(cache, NB, P, H_KV, D, bt, LD, seq_lens, B, kmin, kmax, kmean);
    oracle_page_var(cache, NB, P, H_KV, D, bt, LD, seq_lens, B, kvar);

    double *q = alloc(sizeof *q * B * H_Q * D);
    for (int i = 0; i < B * H_Q * D; ++i) q[i] = normal();
    double alibi[H_Q];
    for (int h = 0; h < H_Q; ++h) alibi[h] = pow(2.0, -8.0 * (h + 1) / H_Q);
    double *scores = alloc(sizeof *scores * B * H_Q * LD);
    double *gscores = alloc(sizeof *gscores * B * H_KV * LD);
    oracle_page_score(q, B, H_Q, H_KV, D, kmin, kmax, kmean, bt, LD, seq_lens, P, 1.0, 0.5,
                      scores, LD);
    oracle_page_score_group(q, B, H_Q, H_KV, D, kmin, kmax, kmean, bt, LD, seq_lens, P, 1.0,
                            0.5, gscores, LD);
    oracle_page_score_alibi(q, B, H_Q, H_KV, D, kmin, kmax, kmean, bt, LD, seq_lens, P, 1.0,
                            1.0, alibi, 0, scores, LD);
    oracle_page_score_alibi(q, B, H_Q, H_KV, D, kmin, kmax, kmean, bt, LD, seq_lens, P, 1.0,
                            1.0, alibi, 1, gscores, LD);

    /* selection: empty rows, budgets above N, reserved windows, ties */
    int32_t sel[LD];
    double ties[LD];
    for (int i = 0; i < LD; ++i) ties[i] = 1.0;
    for (int N = 0; N <= LD; ++N) {
        (void)oracle_budget(N, 3, 0.25);
        (void)oracle_select(scores, N, 3, 0.0, 0, 1, sel);
        (void)oracle_select(scores, N, 20, 0.0, 2, 3, sel);
        (void)oracle_select(ties, N, 1, 0.5, 1, 1, sel);
    }

    /* attention over none, one and all pages of each request */
    double o[D], lse, tau;
    for (int b = 0; b < B; ++b) {
        const int S = seq_lens[b];
        const int N = (S + P - 1) / P;
        int32_t pages[LD];
        for (int p = 0; p < N; ++p) pages[p] = p;
        for (int np = 0; np <= N; np = np == 0 ? 1 : (np == N ? N + 1 : N)) {
            oracle_attend(q + b * H_Q * D, D, cache, NB, P, H_KV, 1, bt + b * LD, S, pages,
                          np, 0.25, o, &lse);
            oracle_attend_alibi(q + b * H_Q * D, D, cache, NB, P, H_KV, 0, bt + b * LD, S,
                                pages, np, 0.25, 0.5, o, &lse);
            oracle_attend_entmax15(q + b * H_Q * D, D, cache, NB, P, H_KV, 1, bt + b * LD, S,
                                   pages, np, 0.25, o, &tau);
            oracle_attend_entmax15_alibi(q + b * H_Q * D, D, cache, NB, P, H_KV, 0,
                                         bt + b * LD, S, pages, np, 0.25, 0.5, o, &tau);
        }
    }
    const double z1[1] = {0.3}, z4[4] = {1.0, 1.0, -2.0, 5.0};
    (void)oracle_entmax15_tau(z1, 1);
    (void)oracle_entmax15_tau(z4, 4);

    /* Gaussian moments, tau-hat and the adaptive selection */
    double *mu = alloc(sizeof *mu * B * H_Q * LD), *var = alloc(sizeof *var * B * H_Q * LD);
    oracle_gauss_moments(q, B, H_Q, H_KV, D, kmean, kvar, bt, LD, seq_lens, P, 0.25, NULL, mu,
                         var, LD);
    oracle_gauss_moments(q, B, H_Q, H_KV, D, kmean, kvar, bt, LD, seq_lens, P, 0.25, alibi,
                         mu, var, LD);
    for (int b = 1; b < B; ++b) {
        const int S = seq_lens[b];
        const int N = (S + P - 1) / P;
        int n[LD];
        for (int p = 0; p < N; ++p) n[p] = S - p * P < P ? S - p * P : P;
        for (int mix = 0; mix <= 1; ++mix) {
            const double t = oracle_gauss_tau(mu + b * H_Q * LD, var + b * H_Q * LD, n, N, mix);
            int32_t gsel[LD];
            (void)oracle_gauss_select(mu + b * H_Q * LD, var + b * H_Q * LD, n, N, t, 0, 1, N,
                                      gsel);
            (void)oracle_gauss_select(mu + b * H_Q * LD, var + b * H_Q * LD, n, N, t, 1, 1, 2,
                                      gsel);
        }
    }

    /* N-way merge with empty and +inf partials */
    double parts[4 * D], lses[4] = {-INFINITY, 0.5, INFINITY, -1.0}, mo[D], ml;
    for (int i = 0; i < 4 * D; ++i) parts[i] = normal();
    oracle_lse_merge(parts, lses, 4, D, mo, &ml);
    const double all_empty[2] = {-INFINITY, -INFINITY};
    oracle_lse_merge(parts, all_empty, 2, D, mo, &ml);

    /* a whole page-level step */
    const int k_cap = LD;
    int32_t *sel_idx = alloc(sizeof *sel_idx * B * H_Q * k_cap);
    int32_t *sel_cnt = alloc(sizeof *sel_cnt * B * H_Q);
    double *out = alloc(sizeof *out * B * H_Q * D), *lse_out = alloc(sizeof *lse_out * B * H_Q);
    oracle_decode_step(q, B, H_Q, H_KV, D, cache, NB, P, bt, LD, seq_lens, kmin, kmax, kmean,
                       1.0, 1.0, 3, 0.0, 0, 1, 0.25, scores, LD, sel_idx, sel_cnt, k_cap, out,
                       lse_out);

    /* token level: append with reset, the accumulator in both readings */
    enum { LD1 = 24, NB1 = B * LD1 };
    const int32_t sl1[B] = {1, 9, LD1};
    const size_t nc1 = (size_t)2 * NB1 * H_KV * D;
    uint16_t *cache1 = alloc(sizeof *cache1 * nc1);
    for (size_t i = 0; i < nc1; ++i) cache1[i] = oracle_double_to_bf16(normal());
    int32_t *bt1 = alloc(sizeof *bt1 * B * LD1);
    for (int i = 0; i < B * LD1; ++i) bt1[i] = i;
    uint16_t *hh = alloc(sizeof *hh * NB1 * H_KV);
    uint16_t knew[B * H_KV * D], vnew[B * H_KV * D];
    for (int i = 0; i < B * H_KV * D; ++i) {
        knew[i] = oracle_double_to_bf16(normal());
        vnew[i] = oracle_double_to_bf16(normal());
    }
    oracle_append(cache1, NB1, 1, H_KV, D, bt1, LD1, sl1, B, knew, vnew, hh);
    oracle_append(cache, NB, P, H_KV, D, bt, LD, seq_lens + 1, B - 1, knew, vnew, NULL);
    double *sc1 = alloc(sizeof *sc1 * B * H_KV * LD1);
    oracle_h2o_step(q, B, H_Q, H_KV, D, cache1, NB1, bt1, LD1, sl1, 0, 1, 0.25, 0.984375, hh,
                    sc1, LD1);
    oracle_h2o_step(q, B, H_Q, H_KV, D, cache1, NB1, bt1, LD1, sl1, 4, 8, 0.25, 0.984375, hh,
                    sc1, LD1);
    oracle_h2o_step_heads(q, B, H_Q, H_KV, D, cache1, NB1, bt1, LD1, sl1, 0, 1, 0.25, 1.0, hh,
                          sc1, LD1);
    double pr[5] = {0.1, 0.2, 0.3, 0.4, 0.0};
    oracle_h2o_recurrence(pr, hh, 5, 0.984375);

    free(cache); free(bt); free(kmin); free(kmax); free(kmean); free(kvar); free(q);
    free(scores); free(gscores); free(mu); free(var); free(sel_idx); free(sel_cnt);
    free(out); free(lse_out); free(cache1); free(bt1); free(hh); free(sc1);
    puts("oracle sanitizer run: ok");
    return 0;
}
