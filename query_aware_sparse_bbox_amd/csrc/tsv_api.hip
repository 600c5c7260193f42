// C-ABI host layer of libtsv: argument validation, workspace carving and
// kernel launches.  Every check runs before the first HIP call, so a rejected
// call has touched neither the device nor the runtime.
//
// Built twice: the library proper, which keeps no state between calls, and a
// testing library (TSV_TEST_HOOKS) that also exports the hook declared in
// tsv_testing.h.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "../../include/tsv.h"
#include "tsv_launch.h"
#ifdef TSV_TEST_HOOKS
#include "../../include/tsv_testing.h"
#endif

static_assert(tsv::kZeroBytes == TSV_WORKSPACE_ZERO_BYTES, "zeroed workspace prefix");
static_assert(tsv::kNoAllocScratchBytes == TSV_NOALLOC_SCRATCH_BYTES, "no-allocation scratch");

namespace {

using tsv::Dims;

bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Shape check shared by every entry point; fills `d` on success.
int check_shape(const tsv_shape* s, Dims* d) {
  if (!s) return TSV_ERR_INVALID_ARG;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 ||
      s->head_dim < 1 || s->page_size < 1 || s->max_pages_per_seq < 1 ||
      s->num_phys_pages < 1)
    return TSV_ERR_INVALID_ARG;
  if (s->num_q_heads % s->num_kv_heads) return TSV_ERR_INVALID_ARG;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (s->kv_dtype != TSV_F32 && s->kv_dtype != TSV_F16 && s->kv_dtype != TSV_BF16 &&
      s->kv_dtype != TSV_FP8_E4M3 && s->kv_dtype != TSV_FP8_E5M2)
    return TSV_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return TSV_ERR_UNSUPPORTED;
  if (s->page_size != 8 && s->page_size != 16 && s->page_size != 32 &&
      s->page_size != 64)
    return TSV_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return TSV_ERR_UNSUPPORTED;
  if (s->max_pages_per_seq > tsv::kMaxPagesPerSeq) return TSV_ERR_UNSUPPORTED;
  // element offsets are computed in 64 bits; token positions in 32 bits
  if ((int64_t)s->max_pages_per_seq * s->page_size > INT32_MAX / 2)
    return TSV_ERR_UNSUPPORTED;
  d->B = s->batch;
  d->Hq = s->num_q_heads;
  d->Hkv = s->num_kv_heads;
  d->D = s->head_dim;
  d->P = s->page_size;
  d->MP = s->max_pages_per_seq;
  d->NP = s->num_phys_pages;
  d->dt = s->kv_dtype;
  d->G = G;
  return TSV_OK;
}

size_t elem_bytes(const Dims& d) { return (size_t)tsv::kv_bytes(d.dt); }

int check_workspace(const Dims& d, int32_t k_max, const void* ws, size_t ws_bytes) {
  if (!ws || !aligned(ws, 256)) return TSV_ERR_INVALID_ARG;
  if (ws_bytes < tsv::workspace_layout(d, k_max, nullptr, nullptr)) return TSV_ERR_INVALID_ARG;
  return TSV_OK;
}

// Selection policy of a call; opts may be NULL (no window, max over heads).
int make_policy(int32_t k_max, int32_t n_sink, const tsv_select_opts* opts,
                tsv::SelectPolicy* pol) {
  const int32_t n_recent = opts ? opts->n_recent : 0;
  const int32_t agg = opts ? opts->group_agg : TSV_AGG_MAX;
  if (n_sink < 0 || n_recent < 0 || n_sink > k_max || n_recent > k_max - n_sink)
    return TSV_ERR_INVALID_ARG;
  if (agg != TSV_AGG_MAX && agg != TSV_AGG_SUM) return TSV_ERR_INVALID_ARG;
  pol->n_sink = n_sink;
  pol->n_recent = n_recent;
  pol->group_sum = agg == TSV_AGG_SUM;
  return TSV_OK;
}

int check_select_args(const Dims& d, const float* q, const void* meta,
                      const int32_t* bt, const int32_t* seq_lens, int32_t k_max,
                      const int32_t* sel, const int32_t* sel_count,
                      const void* ws, size_t ws_bytes) {
  if (!q || !meta || !bt || !seq_lens || !sel || !sel_count)
    return TSV_ERR_INVALID_ARG;
  if (k_max < 1) return TSV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(meta, 16)) return TSV_ERR_INVALID_ARG;
  return check_workspace(d, k_max, ws, ws_bytes);
}

int check_decode_args(const Dims& d, const float* q, const void* k_pool,
                      const void* v_pool, const int32_t* bt,
                      const int32_t* seq_lens, const int32_t* sel,
                      const int32_t* sel_count, int32_t k_max, const float* out,
                      const void* ws, size_t ws_bytes) {
  if (!q || !k_pool || !v_pool || !bt || !seq_lens || !sel || !sel_count || !out)
    return TSV_ERR_INVALID_ARG;
  if (k_max < 1) return TSV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(out, 16))
    return TSV_ERR_INVALID_ARG;
  return check_workspace(d, k_max, ws, ws_bytes);
}

int hip_status(hipError_t e) { return e == hipSuccess ? TSV_OK : TSV_ERR_HIP; }

// Longest row order tsv_decode_step_scheduled accepts (workgroups per launch).
constexpr int32_t kMaxOrderLen = 1 << 24;

#ifdef TSV_TEST_HOOKS
// Polls of a split row's score exchange, settable by tsv_debug_exchange_polls.
std::atomic<int> g_exchange_polls{tsv::kDefaultExchangePolls};
int exchange_polls() { return g_exchange_polls.load(std::memory_order_relaxed); }
#else
constexpr int exchange_polls() { return tsv::kDefaultExchangePolls; }
#endif

}  // namespace

extern "C" {

int tsv_version(void) { return TSV_VERSION; }

#ifdef TSV_TEST_HOOKS
int tsv_debug_exchange_polls(int32_t polls) {
  return polls < 0 ? g_exchange_polls.load() : g_exchange_polls.exchange(polls);
}

int tsv_debug_phase_stamps(int32_t kv_dtype, void* host, size_t bytes) {
  if (host == nullptr) return TSV_ERR_INVALID_ARG;
  hipError_t e;
  switch (kv_dtype) {
    case TSV_F32: e = tsv::read_phase_stamps_t<tsv::DT_F32>(host, bytes); break;
    case TSV_F16: e = tsv::read_phase_stamps_t<tsv::DT_F16>(host, bytes); break;
    case TSV_BF16: e = tsv::read_phase_stamps_t<tsv::DT_BF16>(host, bytes); break;
    case TSV_FP8_E4M3: e = tsv::read_phase_stamps_t<tsv::DT_F8>(host, bytes); break;
    case TSV_FP8_E5M2: e = tsv::read_phase_stamps_t<tsv::DT_F8E5>(host, bytes); break;
    default: return TSV_ERR_INVALID_ARG;
  }
  return e == hipSuccess ? TSV_OK : TSV_ERR_HIP;
}
#endif

const char* tsv_status_string(int status) {
  switch (status) {
    case TSV_OK: return "ok";
    case TSV_ERR_INVALID_ARG: return "invalid argument";
    case TSV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TSV_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t tsv_meta_bytes(const tsv_shape* shape) {
  Dims d;
  if (check_shape(shape, &d) != TSV_OK) return 0;
  return (size_t)d.NP * d.Hkv * 2 * d.D * elem_bytes(d);
}

size_t tsv_workspace_bytes(const tsv_shape* shape, int32_t k_max) {
  Dims d;
  if (check_shape(shape, &d) != TSV_OK || k_max < 1) return 0;
  return tsv::workspace_layout(d, k_max, nullptr, nullptr);
}

int tsv_decode_step_launches(const tsv_shape* shape, int32_t k_max, int32_t with_append) {
  Dims d;
  if (check_shape(shape, &d) != TSV_OK || k_max < 1) return 0;
  if (tsv::step_fits(d)) return 1;
  return (with_append ? 1 : 0) + 1 + 1 + (tsv::decode_splits(d, k_max) > 1 ? 1 : 0);
}

int tsv_meta_build(const tsv_shape* shape, const void* k_pool, void* meta,
                   const int32_t* block_table, const int32_t* seq_lens,
                   void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!k_pool || !meta || !block_table || !seq_lens) return TSV_ERR_INVALID_ARG;
  return hip_status(tsv::launch_meta_build(d, k_pool, meta, block_table, seq_lens,
                                           (hipStream_t)stream));
}

int tsv_meta_append(const tsv_shape* shape, const void* k_new, const void* v_new,
                    void* k_pool, void* v_pool, void* meta,
                    const int32_t* block_table, const int32_t* seq_lens,
                    void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!k_new || !v_new || !k_pool || !v_pool || !meta || !block_table || !seq_lens)
    return TSV_ERR_INVALID_ARG;
  return hip_status(tsv::launch_meta_append(d, k_new, v_new, k_pool, v_pool, meta,
                                            block_table, seq_lens,
                                            (hipStream_t)stream));
}

int tsv_select_pages_ex(const tsv_shape* shape, const float* q, const void* meta,
                        const int32_t* block_table, const int32_t* seq_lens,
                        int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                        const tsv_select_opts* opts, int32_t* sel, int32_t* sel_count,
                        float* scores_out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  rc = check_select_args(d, q, meta, block_table, seq_lens, k_max, sel, sel_count,
                         workspace, workspace_bytes);
  if (rc) return rc;
  tsv::SelectPolicy pol;
  rc = make_policy(k_max, n_sink, opts, &pol);
  if (rc) return rc;
  tsv::Workspace ws;
  tsv::workspace_layout(d, k_max, workspace, &ws);
  return hip_status(tsv::launch_score_select(d, q, meta, block_table, seq_lens, k_max,
                                             k_per_seq, pol, sel, sel_count, scores_out,
                                             ws, (hipStream_t)stream));
}

int tsv_select_pages(const tsv_shape* shape, const float* q, const void* meta,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                     int32_t* sel, int32_t* sel_count, float* scores_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return tsv_select_pages_ex(shape, q, meta, block_table, seq_lens, k_max, k_per_seq,
                             n_sink, nullptr, sel, sel_count, scores_out, workspace,
                             workspace_bytes, stream);
}

int tsv_sparse_decode(const tsv_shape* shape, const float* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* sel,
                      const int32_t* sel_count, int32_t k_max, float scale,
                      float* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  rc = check_decode_args(d, q, k_pool, v_pool, block_table, seq_lens, sel,
                         sel_count, k_max, out, workspace, workspace_bytes);
  if (rc) return rc;
  tsv::Workspace ws;
  tsv::workspace_layout(d, k_max, workspace, &ws);
  return hip_status(tsv::launch_decode(d, q, k_pool, v_pool, block_table, seq_lens,
                                       sel, nullptr, sel_count, k_max, scale, ws, out,
                                       (hipStream_t)stream));
}

namespace {

// Checks of tsv_decode_step_ex / tsv_decode_step_noalloc other than the
// workspace's; fills d and pol.
int check_step(const tsv_shape* shape, const float* q, const void* k_new, const void* v_new,
               const void* k_pool, const void* v_pool, const void* meta,
               const int32_t* block_table, const int32_t* seq_lens, int32_t k_max,
               int32_t n_sink, const tsv_select_opts* opts, const int32_t* sel,
               const int32_t* sel_count, const float* out, Dims* d, tsv::SelectPolicy* pol) {
  int rc = check_shape(shape, d);
  if (rc) return rc;
  if ((k_new == nullptr) != (v_new == nullptr)) return TSV_ERR_INVALID_ARG;
  if (!q || !meta || !block_table || !seq_lens || !sel || !sel_count || !k_pool || !v_pool ||
      !out)
    return TSV_ERR_INVALID_ARG;
  if (k_max < 1) return TSV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(meta, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(out, 16))
    return TSV_ERR_INVALID_ARG;
  return make_policy(k_max, n_sink, opts, pol);
}

// The step on a checked call, with its workspace at `workspace`.
int run_step(const Dims& d, const tsv::SelectPolicy& pol, const float* q, const void* k_new,
             const void* v_new, void* k_pool, void* v_pool, void* meta,
             const int32_t* block_table, const int32_t* seq_lens, int32_t k_max,
             const int32_t* k_per_seq, float scale, int32_t* sel, int32_t* sel_count,
             float* scores_out, float* out, void* workspace, hipStream_t s,
             const int32_t* row_order = nullptr, int32_t order_len = 0) {
  tsv::Workspace ws;
  tsv::workspace_layout(d, k_max, workspace, &ws);
  if (tsv::step_fits(d))  // every row's whole step in its own workgroup(s)
    return hip_status(tsv::launch_step(d, exchange_polls(), q, k_new, v_new, k_pool, v_pool,
                                       meta, block_table, seq_lens, k_max, k_per_seq, pol,
                                       scale, row_order, order_len, sel, sel_count,
                                       scores_out, ws, out, s));
  int rc;
  if (k_new) {
    rc = hip_status(tsv::launch_meta_append(d, k_new, v_new, k_pool, v_pool, meta,
                                            block_table, seq_lens, s));
    if (rc) return rc;
  }
  rc = hip_status(tsv::launch_score_select(d, q, meta, block_table, seq_lens, k_max,
                                           k_per_seq, pol, sel, sel_count, scores_out,
                                           ws, s));
  if (rc) return rc;
  return hip_status(tsv::launch_decode(d, q, k_pool, v_pool, block_table, seq_lens,
                                       sel, ws.sel_phys, sel_count, k_max, scale, ws,
                                       out, s));
}

}  // namespace

int tsv_decode_step_ex(const tsv_shape* shape, const float* q, const void* k_new,
                       const void* v_new, void* k_pool, void* v_pool, void* meta,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                       const tsv_select_opts* opts, float scale, int32_t* sel,
                       int32_t* sel_count, float* scores_out, float* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  tsv::SelectPolicy pol;
  int rc = check_step(shape, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens,
                      k_max, n_sink, opts, sel, sel_count, out, &d, &pol);
  if (rc) return rc;
  rc = check_workspace(d, k_max, workspace, workspace_bytes);
  if (rc) return rc;
  return run_step(d, pol, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens, k_max,
                  k_per_seq, scale, sel, sel_count, scores_out, out, workspace,
                  (hipStream_t)stream);
}

int tsv_decode_step_noalloc(const tsv_shape* shape, const float* q, const void* k_new,
                            const void* v_new, void* k_pool, void* v_pool, void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                            const tsv_select_opts* opts, float scale, int32_t* sel,
                            int32_t* sel_count, float* scores_out, float* out,
                            void* stream) {
  Dims d;
  tsv::SelectPolicy pol;
  int rc = check_step(shape, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens,
                      k_max, n_sink, opts, sel, sel_count, out, &d, &pol);
  if (rc) return rc;
  if (tsv::workspace_layout(d, k_max, nullptr, nullptr) > tsv::kNoAllocScratchBytes)
    return TSV_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  void* scratch = nullptr;
  rc = hip_status(tsv::noalloc_scratch(s, &scratch));
  if (rc) return rc;
  return run_step(d, pol, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens, k_max,
                  k_per_seq, scale, sel, sel_count, scores_out, out, scratch, s);
}

int tsv_step_residency(const tsv_shape* shape, int32_t k_max, int32_t* num_cus,
                       int32_t* per_cu) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (k_max < 1 || !num_cus || !per_cu) return TSV_ERR_INVALID_ARG;
  int dev = 0, cus = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return TSV_ERR_HIP;
  if (tsv::step_fits(d) && tsv::step_splits_for(d, k_max) == 1 &&
      tsv::step_per_cu(d, k_max, &n) != hipSuccess)
    return TSV_ERR_HIP;
  *num_cus = cus;
  *per_cu = n;
  return TSV_OK;
}

int tsv_schedule_rows(const tsv_shape* shape, int32_t k_max, const int32_t* seq_lens,
                      const int32_t* k_per_seq, int32_t num_cus, int32_t per_cu,
                      int32_t* row_order, int32_t capacity, int32_t* order_len) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (k_max < 1 || !seq_lens || !order_len || num_cus < 1 || per_cu < 1 || capacity < 0 ||
      (capacity > 0 && !row_order))
    return TSV_ERR_INVALID_ARG;
  if ((int64_t)d.B * d.Hkv > INT32_MAX / 2) return TSV_ERR_UNSUPPORTED;
  // weight of a row: the bytes its step reads -- every page box, the kept
  // pages' keys and values (a full budget of full pages), the block-table row
  const double e = tsv::kv_bytes(d.dt), box = 2.0 * d.D * e, page = 2.0 * d.D * e * d.P;
  std::vector<double> w(d.B);  // per sequence: each of its Hkv rows weighs the same
  for (int b = 0; b < d.B; ++b) {
    const long len_b = std::min<long>(std::max(seq_lens[b], 0), (long)d.MP * d.P);
    const long n = (len_b + d.P - 1) / d.P;
    const long kb = std::min<long>(
        n, std::max(1, std::min(k_per_seq ? k_per_seq[b] : k_max, k_max)));
    w[b] = box * n + page * kb + 4.0 * n;
  }
  // one planning pass: it reports the length, and fills row_order when
  // given and large enough
  long len = 0;
  const bool filled = tsv::schedule_rows(w.data(), d.B, d.Hkv, num_cus, per_cu, row_order,
                                         capacity, &len);
  if (len > INT32_MAX) return TSV_ERR_UNSUPPORTED;
  *order_len = (int32_t)len;
  if (row_order == nullptr) return TSV_OK;  // length query
  return filled ? TSV_OK : TSV_ERR_INVALID_ARG;
}

int tsv_decode_step_scheduled(const tsv_shape* shape, const float* q, const void* k_new,
                              const void* v_new, void* k_pool, void* v_pool, void* meta,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                              const tsv_select_opts* opts, const int32_t* row_order,
                              int32_t order_len, float scale, int32_t* sel,
                              int32_t* sel_count, float* scores_out, float* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  tsv::SelectPolicy pol;
  int rc = check_step(shape, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens,
                      k_max, n_sink, opts, sel, sel_count, out, &d, &pol);
  if (rc) return rc;
  rc = check_workspace(d, k_max, workspace, workspace_bytes);
  if (rc) return rc;
  if (row_order != nullptr &&
      (!aligned(row_order, 4) || order_len < (int64_t)d.B * d.Hkv || order_len > kMaxOrderLen))
    return TSV_ERR_INVALID_ARG;
  return run_step(d, pol, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens, k_max,
                  k_per_seq, scale, sel, sel_count, scores_out, out, workspace,
                  (hipStream_t)stream, row_order, row_order ? order_len : 0);
}

int tsv_decode_step(const tsv_shape* shape, const float* q, const void* k_new,
                    const void* v_new, void* k_pool, void* v_pool, void* meta,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int32_t k_max, const int32_t* k_per_seq, int32_t n_sink,
                    float scale, int32_t* sel, int32_t* sel_count,
                    float* scores_out, float* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return tsv_decode_step_ex(shape, q, k_new, v_new, k_pool, v_pool, meta, block_table,
                            seq_lens, k_max, k_per_seq, n_sink, nullptr, scale, sel,
                            sel_count, scores_out, out, workspace, workspace_bytes, stream);
}

}  // extern "C"
