/*
 * The boundary contract: the seven C entry points the decode step is cut
 * into, with the argument names of the pages' problem statement (EntmaxKV
 * README "Quick start": the cache [2, num_blocks, page_size, H_kv, D], the
 * block table, seq_lens, topk_pages; vortex_torch "Page-level variants" and
 * "Token-level variants": w_avg, w_peak, scale, decay).  include/sparsekv.h
 * must declare each of them with exactly these tokens (comments aside);
 * tests/test_abi.py compares them.  Extensions live in separately named
 * entry points.
 */
int pagestats_update(uint16_t* kv_cache, int64_t num_blocks, int page_size, int H_kv, int D,
                     uint16_t* k_min, uint16_t* k_max, float* k_mean,
                     const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens, int B,
                     const uint16_t* k_new, const uint16_t* v_new,
                     uint16_t* hh_score,
                     hipStream_t stream);
int page_score(const float* q, int B, int H_q, int H_kv, int D,
               const uint16_t* k_min, const uint16_t* k_max, const float* k_mean,
               const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens, int page_size,
               float w_avg, float w_peak, float* scores, int64_t score_ld, hipStream_t stream);
int page_topk(const float* scores, int64_t score_ld, int B, int H_sel,
              const int32_t* seq_lens, int page_size,
              int topk_pages, float topk_frac, int reserved_bos, int reserved_eos,
              int32_t* sel_idx, int32_t* sel_cnt, int k_cap, hipStream_t stream);
int sparse_paged_decode(const float* q, int B, int H_q, int H_kv, int D,
                        const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                        const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                        const int32_t* sel_idx, const int32_t* sel_cnt, int k_cap, int H_sel,
                        float scale, int num_splits, float* o_part, float* lse_part,
                        hipStream_t stream);
int lse_merge(const float* o_part, const float* lse_part, int rows, int num_splits, int D,
              float* out, float* lse_out, hipStream_t stream);
int h2o_accumulate(const float* q, int B, int H_q, int H_kv, int D,
                   const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                   const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                   int reserved_bos, int reserved_eos, float scale, float decay,
                   uint16_t* hh_score, float* scores, int64_t score_ld,
                   float* scratch, int64_t scratch_floats, hipStream_t stream);
int64_t h2o_scratch_floats(int B, int H_kv, int64_t max_tokens);
