/*
 * tsv.h -- query-aware page selection with sparse paged-attention decode on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is TinyServe's ("Query-Aware Cache Selection for Efficient LLM
 * Serving", arXiv 2509.12211): every page (block) of the paged KV cache
 * carries a bounding box of its keys; at each decode step the query is scored
 * against every box, only the highest-scoring pages are kept, and masked
 * softmax attention runs over the tokens of those pages alone (abstract;
 * method details, key design).  The box is the per-channel [min, max] of the
 * page's keys; the score of a page for one query head is
 *     s = sum_d max(q_d * kmin_d, q_d * kmax_d),
 * the largest q.k any point of the box reaches, so it bounds the true q.k of
 * every token in the page.
 *
 * Conventions for every call
 * --------------------------
 *  B = batch, Hq / Hkv = query / KV heads, G = Hq / Hkv (query head hq reads
 *  KV head hq / G), D = head_dim, P = page_size, MP = max_pages_per_seq,
 *  NP = num_phys_pages.  len_b = seq_lens[b] counts the token being decoded;
 *  n_b = ceil(len_b / P) pages; page p holds min(P, len_b - p*P) valid tokens.
 *
 *  Layouts (row-major, all device pointers on the current HIP device):
 *    k_pool, v_pool  [NP][Hkv][P][D]   KV dtype
 *    meta            [NP][Hkv][2][D]   KV dtype; row 0 = per-channel min,
 *                                      row 1 = per-channel max of the page's
 *                                      valid keys
 *    q               [B][Hq][D]        fp32
 *    out             [B][Hq][D]        fp32
 *    block_table     [B][MP]           int32 physical page of logical page p
 *    seq_lens        [B]               int32
 *    sel             [B][Hkv][k_max]   int32 logical pages, ascending, -1 pad
 *    sel_count       [B][Hkv]          int32
 *    scores_out      [B][Hkv][MP]      fp32 (only p < n_b written)
 *  q, out, pools, meta, k_new, v_new: 16-byte aligned; int32 arrays 4-byte.
 *
 *  Ownership: the caller allocates and owns every buffer.  The library
 *  allocates nothing, keeps no state between calls and is thread-safe; calls
 *  on one stream run in order, calls on different streams that write the same
 *  buffers race.
 *
 *  Streams: `stream` is a hipStream_t (NULL = the default stream).  Every call
 *  only enqueues work on it and returns without synchronising.
 *
 *  Data contents are not checked on the host.  The device clamps len_b into
 *  [0, MP*P] and block-table entries into [0, NP) so that no access leaves
 *  the buffers; a block-table entry outside [0, NP) gives undefined results.
 *  A sequence with len_b = 0 selects nothing and its output rows are zero.
 *  Pages shared by several sequences must be full wherever they are shared.
 *
 *  Return value: TSV_OK, or an error code.  Argument checks run before any
 *  HIP call, so an error return has enqueued nothing.
 */
#ifndef TSV_H
#define TSV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: TSV_WORKSPACE_ZERO_BYTES grew from 16384 to 2113536 (the split rows'
   page-key slots joined their counters); a workspace zeroed for version 1
   must be zeroed again over the new prefix. */
#define TSV_VERSION 2

/* KV storage types.  TSV_FP8_E4M3 is the OCP 8-bit float E4M3 ("FN"): sign,
   4 exponent bits (bias 7), 3 mantissa bits, no infinities, NaN only at
   magnitude 0x7F, largest finite value 448.  TSV_FP8_E5M2 is the OCP E5M2:
   sign, 5 exponent bits (bias 15), 2 mantissa bits, infinities and NaNs at
   exponent field 31 as in IEEE, largest finite value 57344.  Values are used
   as stored (no scale factor); every one of them is exact in fp32 and bf16,
   so the page boxes and scores are exact functions of the stored codes as
   for the other types.  Box metadata is kept in the KV type. */
typedef enum {
  TSV_F32 = 0,
  TSV_F16 = 1,
  TSV_BF16 = 2,
  TSV_FP8_E4M3 = 3,
  TSV_FP8_E5M2 = 4
} tsv_dtype;

typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_phys_pages;
  int32_t kv_dtype; /* tsv_dtype */
} tsv_shape;

enum {
  TSV_OK = 0,
  /* null pointer, non-positive size, Hq % Hkv != 0, k_max < 1,
     n_sink outside [0, k_max], misaligned pointer, workspace too small or
     not 256-byte aligned */
  TSV_ERR_INVALID_ARG = -1,
  /* head_dim not 64/128, page_size not 8/16/32/64, G not 1/2/4/8/16,
     unknown dtype, max_pages_per_seq > 4096 */
  TSV_ERR_UNSUPPORTED = -2,
  /* a kernel launch failed (hipGetLastError after the launch) */
  TSV_ERR_HIP = -3
};

/* Library version (TSV_VERSION). */
int tsv_version(void);

/* Static description of a status code. */
const char* tsv_status_string(int status);

/* Bytes of the metadata array for `shape`: NP*Hkv*2*D*sizeof(KV dtype);
   0 when the shape is invalid or unsupported. */
size_t tsv_meta_bytes(const tsv_shape* shape);

/* Bytes of the caller-owned scratch that tsv_select_pages,
   tsv_sparse_decode and tsv_decode_step need for rows of k_max selected
   pages; 0 when the shape is invalid or unsupported.  The workspace holds the
   page-score keys, the selected pages' physical indices and the split
   decode's partial softmax states.  It must be 256-byte aligned.  Its first
   TSV_WORKSPACE_ZERO_BYTES bytes hold the counters and page-key slots
   through which the workgroups of one row synchronise: they must be zero
   before the workspace is first used (for example hipMemsetAsync once after
   allocation), and every call leaves them zero, whatever the shape; the rest
   needs no initialisation.  Calls that may run at the same time (different
   streams) need separate workspaces. */
#define TSV_WORKSPACE_ZERO_BYTES 2113536
size_t tsv_workspace_bytes(const tsv_shape* shape, int32_t k_max);

/* Kernel launches one tsv_decode_step makes for `shape` (with_append != 0:
   with k_new / v_new).  1 when the whole step of a (sequence, KV head) runs
   in workgroups of its own, which needs the block-table row and the decode
   staging to fit 64 KiB of local memory (when B*Hkv <= 128 each row may be
   spread over several workgroups, which share the scoring and merge their
   shares in the same kernel).  Otherwise 3 or 4 (append,
   score and select, split decode, merge).  0 when the shape is invalid or
   unsupported.  Informational only. */
int tsv_decode_step_launches(const tsv_shape* shape, int32_t k_max, int32_t with_append);

/* Rebuild the bounding box of every page p < n_b of every sequence from the
   keys in k_pool (method details, key design: each block's box covers the
   keys it contains).  Only valid slots are read.  Also the recovery path
   after the pool is restored. */
int tsv_meta_build(const tsv_shape* shape, const void* k_pool, void* meta,
                   const int32_t* block_table, const int32_t* seq_lens,
                   void* stream);

/* Append one token per sequence and keep its page's box current (method
   details, key design: every block keeps the bounding box of the keys it
   holds, so the box of the block receiving a decoded token widens as the
   token lands; the token also joins the cache that attention reads).
   seq_lens already counts the new token; k_new / v_new [B][Hkv][D] (KV dtype)
   go to slot (len_b-1) % P of physical page block_table[b][(len_b-1)/P],
   which the caller must have allocated.  Slot 0 resets the box to the new
   key; any other slot widens it (min/max per channel).  Sequences with
   len_b < 1 are skipped.  The page being written must not be shared. */
int tsv_meta_append(const tsv_shape* shape, const void* k_new,
                    const void* v_new, void* k_pool, void* v_pool, void* meta,
                    const int32_t* block_table, const int32_t* seq_lens,
                    void* stream);

/* Score every page of every (sequence, KV head) against the query and keep
   the top pages (method details, key design: compute the similarity of the
   query to each block's box and load the most similar blocks).
   Page score: fp32, each product q_d*kmin_d / q_d*kmax_d rounded once, the D
   per-channel maxima summed as a balanced pairwise tree over contiguous
   channels, the maximum taken over the G query heads of the KV head, -0
   stored as +0.  Budget K_b = clamp(k_per_seq[b], 1, k_max) (k_per_seq may
   be NULL: K_b = k_max); the first min(n_sink, K_b, n_b) pages are always
   kept (attention-sink pages, counted inside the budget); the remaining
   min(K_b, n_b) - that slots go to the highest scores, equal scores to the
   lower logical page.  sel gets the chosen logical pages in ascending order,
   -1 padded to k_max; sel_count the number chosen.  scores_out may be NULL.
   `workspace` of at least tsv_workspace_bytes(shape, k_max) bytes. */
int tsv_select_pages(const tsv_shape* shape, const float* q, const void* meta,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                     int32_t* sel, int32_t* sel_count, float* scores_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Masked softmax attention of every query head over the valid tokens of its
   KV head's selected pages only (abstract: masked attention over the loaded
   pages): out = sum_t softmax(scale * q.k_t) v_t.  Tokens at or past len_b
   are never read.  Entries of sel must be pages < n_b; with sel = every page
   this is dense paged decode.  fp32 arithmetic; `workspace` of at least
   tsv_workspace_bytes(shape, k_max) bytes.  The result does not depend on
   how the work is split: every output element is bitwise reproducible. */
int tsv_sparse_decode(const tsv_shape* shape, const float* q,
                      const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* sel, const int32_t* sel_count,
                      int32_t k_max, float scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* One decode step: optional append (k_new and v_new both non-NULL, or both
   NULL to skip it), page selection and sparse attention, enqueued on one
   stream (abstract: page scoring, sparse memory access and masked attention
   in one pass over the cache).  Arguments and results as in the three calls
   above: sel, sel_count and scores_out are identical to tsv_select_pages';
   out agrees with tsv_sparse_decode within the rounding of a different
   summation order.  Where tsv_decode_step_launches() is 1 or 2, each
   (sequence, KV head) is handled by workgroups of its own that append,
   score, select and attend in one kernel.  As for tsv_meta_append, the page receiving the new token
   must belong to one sequence only. */
int tsv_decode_step(const tsv_shape* shape, const float* q, const void* k_new,
                    const void* v_new, void* k_pool, void* v_pool, void* meta,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                    float scale, int32_t* sel, int32_t* sel_count,
                    float* scores_out, float* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Selection variants (the pages fix neither how the G query heads of a KV
   head are combined nor which pages besides the highest-scoring ones are
   kept; attention-sink pages are cited under "Builds on").
     group_agg  TSV_AGG_MAX: page score = the largest of the G heads' box
                bounds (the default); TSV_AGG_SUM: their fp32 sum, heads in
                increasing order, each addition rounded once (the bound of the
                group's summed logit).
     n_recent   >= 0: the last min(n_recent, K_b') pages of every sequence are
                always kept as a local window, where K_b' = min(K_b, n_b) minus
                the sink pages kept; counted inside the budget.  Sinks are
                served first, then the window, then the highest scores among
                the pages in between.  n_sink + n_recent must not exceed
                k_max.
   Per-layer budgets need no option: each call is one layer's step and takes
   its own k_max / k_per_seq. */
typedef enum { TSV_AGG_MAX = 0, TSV_AGG_SUM = 1 } tsv_group_agg;

typedef struct {
  int32_t n_recent;
  int32_t group_agg; /* tsv_group_agg */
} tsv_select_opts;

/* tsv_select_pages with selection variants; opts = NULL is
   {n_recent = 0, group_agg = TSV_AGG_MAX}, i.e. tsv_select_pages.
   TSV_ERR_INVALID_ARG also for n_recent < 0, n_sink + n_recent > k_max or an
   unknown group_agg. */
int tsv_select_pages_ex(const tsv_shape* shape, const float* q, const void* meta,
                        const int32_t* block_table, const int32_t* seq_lens,
                        int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                        const tsv_select_opts* opts, int32_t* sel,
                        int32_t* sel_count, float* scores_out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* tsv_decode_step with selection variants (opts as for
   tsv_select_pages_ex; NULL gives tsv_decode_step). */
int tsv_decode_step_ex(const tsv_shape* shape, const float* q, const void* k_new,
                       const void* v_new, void* k_pool, void* v_pool, void* meta,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                       const tsv_select_opts* opts, float scale, int32_t* sel,
                       int32_t* sel_count, float* scores_out, float* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Longest-first row schedule of the one-launch step (abstract: scoring,
   sparse memory access and masked attention fused into one pass; method
   details, key design: the sparse accesses are organised around what the
   hardware does well).  The step's rows ((sequence, KV head) pairs) differ
   in work by the number of pages they score and keep; a serving loop knows
   every sequence's length on the host, and from those lengths this call
   ranks the rows by the bytes their step reads (every page box, the keys and
   values of a full budget of full pages, the block-table row) and writes the
   order in which the workgroups of tsv_decode_step_scheduled take them.
   The GPU starts workgroups in index order, which makes the order a
   longest-processing-time-first queue: the first num_cus * per_cu
   workgroups are resident together (workgroup j*num_cus + c on the same CU
   as workgroup c), and the heaviest rows fill them, each going to the CU
   with the least weight so far among those with fewer than per_cu rows (so
   heavy rows share a CU with light ones, or keep it to themselves while
   light ones share); entries of -1 are idle workgroups in the slots a CU
   does not use.  Rows after those follow heaviest first and start as
   earlier workgroups finish.
   seq_lens [B] (len_b as for the step), k_per_seq [B] (nullable, as for the
   step) and row_order are HOST arrays; the call makes no HIP call.  num_cus
   and per_cu as tsv_step_residency reports them (>= 1).  *order_len
   receives the order's length, at most max(B*Hkv, num_cus*per_cu); with
   row_order NULL only the length is computed, otherwise `capacity` entries
   must hold it (TSV_ERR_INVALID_ARG if they do not).  The order only decides which
   workgroup runs which row and when: the step's results do not depend on
   it.  Rows of equal weight keep index order, so equal lengths and budgets
   give 0 .. B*Hkv-1, the plain step's own order, which the plain step runs
   without the order's load. */
int tsv_schedule_rows(const tsv_shape* shape, int32_t k_max, const int32_t* seq_lens,
                      const int32_t* k_per_seq, int32_t num_cus, int32_t per_cu,
                      int32_t* row_order, int32_t capacity, int32_t* order_len);

/* The current device's CU count, and how many workgroups of this shape's
   one-launch step one CU holds at once.  *per_cu = 0 when the step of this
   shape takes no row order (it needs several launches, or it spreads each
   row over several workgroups, which happens when B*Hkv <= 128).  Queries
   the HIP runtime; enqueues nothing.  TSV_ERR_HIP when the queries fail. */
int tsv_step_residency(const tsv_shape* shape, int32_t k_max, int32_t* num_cus,
                       int32_t* per_cu);

/* tsv_decode_step_ex whose workgroups take their rows from row_order: a
   DEVICE array of order_len int32 (4-byte aligned), order_len in
   [B*Hkv, 2^24]; workgroup w handles row row_order[w] = b*Hkv + h, and
   entries outside [0, B*Hkv) are idle workgroups.  The order must list every
   row exactly once, as tsv_schedule_rows writes it: a row left out is not
   computed (its outputs keep their old contents), a row listed twice is
   computed twice.  It is used where tsv_step_residency reports per_cu > 0
   and ignored otherwise; row_order = NULL is tsv_decode_step_ex.  Results
   are bitwise those of tsv_decode_step_ex. */
int tsv_decode_step_scheduled(const tsv_shape* shape, const float* q, const void* k_new,
                              const void* v_new, void* k_pool, void* v_pool, void* meta,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                              const tsv_select_opts* opts, const int32_t* row_order,
                              int32_t order_len, float scale, int32_t* sel,
                              int32_t* sel_count, float* scores_out, float* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* tsv_decode_step_ex for callers that cannot allocate device memory: code
   under HIP graph capture that may not call hipMalloc, tight serving loops,
   harnesses that forbid allocation.  There is no workspace argument: the
   step's scratch (split-row counters and key slots, page-score keys,
   partial softmax states) lives in a device array owned by the library,
   TSV_NOALLOC_SCRATCH_BYTES on each GPU, which exists from the loading of the
   library's device code on that GPU until the process ends.  The call
   allocates nothing (no hipMalloc, no allocating library routine).  The
   first call on a GPU also enqueues one small kernel on `stream` that clears
   the array's first TSV_WORKSPACE_ZERO_BYTES; every call leaves them zero.
   All calls on one GPU share its array: calls that may run at the same time
   on one GPU (different streams, or a graph replay overlapping another call)
   race on it and must not be made.  TSV_ERR_UNSUPPORTED when tsv_workspace_bytes(shape,
   k_max) exceeds TSV_NOALLOC_SCRATCH_BYTES; TSV_ERR_HIP when the array's
   device address cannot be obtained; otherwise arguments, results and errors
   as for tsv_decode_step_ex. */
#define TSV_NOALLOC_SCRATCH_BYTES 33554432
int tsv_decode_step_noalloc(const tsv_shape* shape, const float* q, const void* k_new,
                            const void* v_new, void* k_pool, void* v_pool, void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                            const tsv_select_opts* opts, float scale, int32_t* sel,
                            int32_t* sel_count, float* scores_out, float* out,
                            void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TSV_H */
