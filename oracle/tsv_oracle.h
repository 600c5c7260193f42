/*
 * tsv_oracle.h -- plain CPU oracle for query-aware page selection with sparse
 * paged-attention decode.
 *
 * TEST INFRASTRUCTURE.  This library exists only to check the HIP path: it is
 * called from the tests, from the package smoke check and from the CPU
 * baseline leg of the benchmark, never from the product path.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Source of the method: TinyServe, "Query-Aware Cache Selection for Efficient
 * LLM Serving" (arXiv 2509.12211), abstract and method-details section (key
 * design: every KV block carries a bounding box, the query is scored against
 * each box and the highest-scoring blocks are loaded; masked attention runs
 * over the loaded blocks only).  The box is the per-channel [min, max] of a
 * page's keys and the score is the largest q.k any point of that box reaches,
 * sum_d max(q_d*kmin_d, q_d*kmax_d).
 *
 * All pointers are host pointers.  Layouts match the HIP library's:
 *   k_pool, v_pool [NP][Hkv][P][D]   KV dtype
 *   meta           [NP][Hkv][2][D]   KV dtype, row 0 = min, row 1 = max
 *   q              [B][Hq][D]        fp32
 *   block_table    [B][MP]           int32 (physical page of logical page p)
 *   seq_lens       [B]               int32, counts the token being decoded
 *   scores         [B][Hkv][MP]      fp32 (entries p >= n_b untouched)
 *   sel            [B][Hkv][k_max]   int32 ascending logical pages, -1 padded
 *   sel_count      [B][Hkv]          int32
 *   out            [B][Hq][D]        fp32
 * Return 0 on success, -1 on an invalid argument or an out-of-range
 * block-table / selection entry.
 */
#ifndef TSV_ORACLE_H
#define TSV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* KV storage formats: IEEE binary32, IEEE binary16, bfloat16, OCP FP8
 * E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities, 0x7F / 0xFF are NaN, largest finite 448) and OCP FP8 E5M2
 * (1 sign, 5 exponent bits with bias 15, 2 mantissa bits; exponent field 31
 * holds infinities and NaNs as in IEEE, largest finite 57344). */
enum { TSVO_F32 = 0, TSVO_F16 = 1, TSVO_BF16 = 2, TSVO_FP8 = 3, TSVO_FP8_E5M2 = 4 };

typedef struct {
  int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size,
      max_pages_per_seq, num_phys_pages;
  int32_t kv_dtype;
} tsvo_shape;

/* How the G query heads of a KV head combine their box bounds into the page
 * score: the largest (TSVO_AGG_MAX) or their fp32 sum in increasing head
 * order (TSVO_AGG_SUM). */
enum { TSVO_AGG_MAX = 0, TSVO_AGG_SUM = 1 };

/* Selection: with keff = min(K_b, n_b), the first f = min(n_sink, keff)
 * pages (attention sinks) and the last r = min(n_recent, keff - f) pages
 * (local window) are always kept; the remaining keff - f - r slots go to the
 * highest-scoring pages in between (ties: lower logical page).
 * n_sink + n_recent must not exceed k_max. */

int tsvo_meta_build(const tsvo_shape* s, const void* k_pool, void* meta,
                    const int32_t* block_table, const int32_t* seq_lens);

int tsvo_meta_append(const tsvo_shape* s, const void* k_new, const void* v_new,
                     void* k_pool, void* v_pool, void* meta,
                     const int32_t* block_table, const int32_t* seq_lens);

int tsvo_page_scores(const tsvo_shape* s, const float* q, const void* meta,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int32_t group_agg, float* scores);

int tsvo_select_from_scores(const tsvo_shape* s, const float* scores,
                            const int32_t* seq_lens, int32_t k_max,
                            const int32_t* k_per_seq, int32_t n_sink,
                            int32_t n_recent, int32_t* sel, int32_t* sel_count);

int tsvo_select_pages(const tsvo_shape* s, const float* q, const void* meta,
                      const int32_t* block_table, const int32_t* seq_lens,
                      int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                      int32_t n_recent, int32_t group_agg, int32_t* sel,
                      int32_t* sel_count, float* scores_out);

int tsvo_sparse_decode(const tsvo_shape* s, const float* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table,
                       const int32_t* seq_lens, const int32_t* sel,
                       const int32_t* sel_count, int32_t k_max, float scale,
                       float* out);

int tsvo_decode_step(const tsvo_shape* s, const float* q, const void* k_new,
                     const void* v_new, void* k_pool, void* v_pool, void* meta,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                     int32_t n_recent, int32_t group_agg, float scale,
                     int32_t* sel, int32_t* sel_count, float* scores_out,
                     float* out);

#ifdef __cplusplus
}
#endif
#endif
