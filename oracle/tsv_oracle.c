/*
 * tsv_oracle.c -- plain, slow CPU oracle for query-aware page selection with
 * sparse paged-attention decode.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code with the
 * HIP library.  Built with gcc -O2 -ffp-contract=off (no fused multiply-add,
 * no fast-math), single-threaded, every step in the order the method states it.
 *
 * Method: TinyServe, "Query-Aware Cache Selection for Efficient LLM Serving".
 *   - method details, key design: each KV block has a bounding box; the query
 *     is compared with every box and the most similar blocks are loaded;
 *   - abstract: selection uses bounding-box metadata, then masked attention
 *     runs over the selected pages only.
 * Readings taken where the pages are silent (each is listed with its reason in
 * the design notes of the repository):
 *   box      per-channel [min, max] over the page's valid tokens, stored in the
 *            KV dtype (min/max of representable values is representable);
 *   score    s_g = sum_d max(fl(q_d*mn_d), fl(q_d*mx_d)), the largest q.k any
 *            point of the box reaches; summed in fp32 as a balanced pairwise
 *            tree over contiguous channels; page score = max over the G query
 *            heads sharing the KV head; -0 is stored as +0;
 *   select   the first min(n_sink, K) pages are always kept, the rest of the
 *            budget K_b = clamp(k_per_seq[b], 1, k_max) goes to the highest
 *            scores, equal scores to the lower logical page; the chosen pages
 *            are emitted in ascending order, -1 padded;
 *   attend   softmax(scale * q.k) over the tokens of the chosen pages, tokens
 *            at or past the sequence length excluded; computed in double.
 *   lengths  clamped to [0, MP*P]; a length of 0 selects nothing and gives an
 *            all-zero output.
 */
#include "tsv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* storage formats                                                            */
/* ------------------------------------------------------------------------- */

static size_t elem_bytes(int dtype) {
  return dtype == TSVO_F32 ? 4u : (dtype == TSVO_FP8 || dtype == TSVO_FP8_E5M2) ? 1u : 2u;
}

/* IEEE 754 binary16 -> float, from the format's definition. */
static float half_bits_to_float(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return (float)(sign ? -v : v);
}

/* bfloat16 -> float: the top half of an IEEE binary32. */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* OCP FP8 E4M3 -> float, from the format's definition: exponent field e
 * (bias 7), mantissa m; e = 0 is subnormal (m/8 * 2^-6); e = 15 with m = 7 is
 * NaN; there are no infinities. */
static float fp8_bits_to_float(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xf;
  int m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return (float)(sign ? -v : v);
}

/* every binary16 pattern decoded once by half_bits_to_float */
static float half_table[65536];
static int half_table_ready = 0;

static float half_lookup(uint16_t h) {
  if (!half_table_ready) {
    for (uint32_t i = 0; i < 65536; ++i) half_table[i] = half_bits_to_float((uint16_t)i);
    half_table_ready = 1;
  }
  return half_table[h];
}

/* OCP FP8 E5M2 -> float, from the format's definition: exponent field e
 * (bias 15), mantissa m; e = 0 is subnormal (m/4 * 2^-14); e = 31 is infinity
 * (m = 0) or NaN. */
static float e5m2_bits_to_float(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 2) & 0x1f;
  int m = b & 3;
  double v;
  if (e == 31)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -16); /* m/4 * 2^-14 */
  else
    v = ldexp((double)(4 + m), e - 17); /* (1 + m/4) * 2^(e-15) */
  return (float)(sign ? -v : v);
}

/* every E4M3 / E5M2 code decoded once */
static float fp8_table[256], e5m2_table[256];
static int fp8_tables_ready = 0;

static float fp8_lookup(uint8_t b, int dtype) {
  if (!fp8_tables_ready) {
    for (uint32_t i = 0; i < 256; ++i) {
      fp8_table[i] = fp8_bits_to_float((uint8_t)i);
      e5m2_table[i] = e5m2_bits_to_float((uint8_t)i);
    }
    fp8_tables_ready = 1;
  }
  return dtype == TSVO_FP8 ? fp8_table[b] : e5m2_table[b];
}

/* Element i of a KV-dtype array as float.  Inlined into every loop that
 * reads the pools (a call per element would double the oracle's run time). */
static inline __attribute__((always_inline)) float kv_get(const void* base, int64_t i,
                                                          int dtype) {
  if (dtype == TSVO_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * i, 4);
    return f;
  }
  if (dtype == TSVO_FP8 || dtype == TSVO_FP8_E5M2)
    return fp8_lookup(((const uint8_t*)base)[i], dtype);
  uint16_t h;
  memcpy(&h, (const char*)base + 2 * i, 2);
  return dtype == TSVO_F16 ? half_lookup(h) : bf16_bits_to_float(h);
}

static void kv_copy(void* dst, int64_t di, const void* src, int64_t si,
                    int dtype) {
  size_t e = elem_bytes(dtype);
  memcpy((char*)dst + e * di, (const char*)src + e * si, e);
}

/* ------------------------------------------------------------------------- */
/* shape helpers                                                              */
/* ------------------------------------------------------------------------- */

static int shape_ok(const tsvo_shape* s) {
  if (!s) return 0;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 ||
      s->head_dim < 1 || s->page_size < 1 || s->max_pages_per_seq < 1 ||
      s->num_phys_pages < 1)
    return 0;
  if (s->num_q_heads % s->num_kv_heads) return 0;
  if (s->head_dim & (s->head_dim - 1)) return 0; /* tree needs a power of 2 */
  if (s->kv_dtype < TSVO_F32 || s->kv_dtype > TSVO_FP8_E5M2) return 0;
  return 1;
}

static int64_t seq_len(const tsvo_shape* s, const int32_t* seq_lens, int b) {
  int64_t L = seq_lens[b];
  int64_t cap = (int64_t)s->max_pages_per_seq * s->page_size;
  if (L < 0) L = 0;
  if (L > cap) L = cap;
  return L;
}

static int64_t n_pages(const tsvo_shape* s, int64_t len) {
  return (len + s->page_size - 1) / s->page_size;
}

/* valid tokens of logical page p of a sequence of length len */
static int64_t page_valid(const tsvo_shape* s, int64_t len, int64_t p) {
  int64_t v = len - p * s->page_size;
  return v < s->page_size ? v : s->page_size;
}

static int phys_of(const tsvo_shape* s, const int32_t* bt, int b, int64_t p,
                   int64_t* phys) {
  int32_t e = bt[(int64_t)b * s->max_pages_per_seq + p];
  if (e < 0 || e >= s->num_phys_pages) return 0;
  *phys = e;
  return 1;
}

/* element index of k/v pool entry (phys, h, slot, d) */
static int64_t pool_idx(const tsvo_shape* s, int64_t phys, int h, int64_t slot,
                        int d) {
  return ((phys * s->num_kv_heads + h) * s->page_size + slot) * s->head_dim + d;
}

/* element index of metadata entry (phys, h, row, d); row 0 = min, 1 = max */
static int64_t meta_idx(const tsvo_shape* s, int64_t phys, int h, int row,
                        int d) {
  return ((phys * s->num_kv_heads + h) * 2 + row) * s->head_dim + d;
}

/* ------------------------------------------------------------------------- */
/* metadata: per-channel bounding box of each page's keys                     */
/* ------------------------------------------------------------------------- */

int tsvo_meta_build(const tsvo_shape* s, const void* k_pool, void* meta,
                    const int32_t* bt, const int32_t* seq_lens) {
  if (!shape_ok(s) || !k_pool || !meta || !bt || !seq_lens) return -1;
  for (int b = 0; b < s->batch; ++b) {
    int64_t len = seq_len(s, seq_lens, b);
    int64_t n = n_pages(s, len);
    for (int64_t p = 0; p < n; ++p) {
      int64_t phys;
      if (!phys_of(s, bt, b, p, &phys)) return -1;
      int64_t v = page_valid(s, len, p);
      for (int h = 0; h < s->num_kv_heads; ++h)
        for (int d = 0; d < s->head_dim; ++d) {
          /* the valid token holding the smallest / largest value */
          int64_t imin = 0, imax = 0;
          float vmin = kv_get(k_pool, pool_idx(s, phys, h, 0, d), s->kv_dtype);
          float vmax = vmin;
          for (int64_t t = 1; t < v; ++t) {
            float x = kv_get(k_pool, pool_idx(s, phys, h, t, d), s->kv_dtype);
            if (x < vmin) { vmin = x; imin = t; }
            if (x > vmax) { vmax = x; imax = t; }
          }
          kv_copy(meta, meta_idx(s, phys, h, 0, d), k_pool,
                  pool_idx(s, phys, h, imin, d), s->kv_dtype);
          kv_copy(meta, meta_idx(s, phys, h, 1, d), k_pool,
                  pool_idx(s, phys, h, imax, d), s->kv_dtype);
        }
    }
  }
  return 0;
}

/* Append the token being decoded (position len-1) and widen its page's box. */
int tsvo_meta_append(const tsvo_shape* s, const void* k_new, const void* v_new,
                     void* k_pool, void* v_pool, void* meta, const int32_t* bt,
                     const int32_t* seq_lens) {
  if (!shape_ok(s) || !k_new || !v_new || !k_pool || !v_pool || !meta || !bt ||
      !seq_lens)
    return -1;
  for (int b = 0; b < s->batch; ++b) {
    int64_t len = seq_len(s, seq_lens, b);
    if (len < 1) continue; /* nothing to append */
    int64_t pos = len - 1;
    int64_t p = pos / s->page_size, slot = pos % s->page_size;
    int64_t phys;
    if (!phys_of(s, bt, b, p, &phys)) return -1;
    for (int h = 0; h < s->num_kv_heads; ++h)
      for (int d = 0; d < s->head_dim; ++d) {
        int64_t src = ((int64_t)b * s->num_kv_heads + h) * s->head_dim + d;
        int64_t dst = pool_idx(s, phys, h, slot, d);
        kv_copy(k_pool, dst, k_new, src, s->kv_dtype);
        kv_copy(v_pool, dst, v_new, src, s->kv_dtype);
        float k = kv_get(k_new, src, s->kv_dtype);
        int64_t mi = meta_idx(s, phys, h, 0, d), ma = meta_idx(s, phys, h, 1, d);
        if (slot == 0) { /* first token of a fresh page: the box is the point */
          kv_copy(meta, mi, k_new, src, s->kv_dtype);
          kv_copy(meta, ma, k_new, src, s->kv_dtype);
        } else {
          if (k < kv_get(meta, mi, s->kv_dtype)) kv_copy(meta, mi, k_new, src, s->kv_dtype);
          if (k > kv_get(meta, ma, s->kv_dtype)) kv_copy(meta, ma, k_new, src, s->kv_dtype);
        }
      }
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* page score: upper bound of q.k over the page's box                         */
/* ------------------------------------------------------------------------- */

/* Balanced pairwise fp32 sum over t[0..n), n a power of two:
 * T(lo,hi) = T(lo,mid) + T(mid,hi). */
static float tree_sum(const float* t, int n) {
  if (n == 1) return t[0];
  int h = n / 2;
  float a = tree_sum(t, h);
  float b = tree_sum(t + h, h);
  return a + b;
}

int tsvo_page_scores(const tsvo_shape* s, const float* q, const void* meta,
                     const int32_t* bt, const int32_t* seq_lens,
                     int32_t group_agg, float* scores) {
  if (!shape_ok(s) || !q || !meta || !bt || !seq_lens || !scores) return -1;
  if (group_agg != TSVO_AGG_MAX && group_agg != TSVO_AGG_SUM) return -1;
  const int D = s->head_dim, G = s->num_q_heads / s->num_kv_heads;
  float* t = (float*)malloc(sizeof(float) * (size_t)D);
  if (!t) return -1;
  for (int b = 0; b < s->batch; ++b) {
    int64_t n = n_pages(s, seq_len(s, seq_lens, b));
    for (int h = 0; h < s->num_kv_heads; ++h)
      for (int64_t p = 0; p < n; ++p) {
        int64_t phys;
        if (!phys_of(s, bt, b, p, &phys)) { free(t); return -1; }
        float best = 0.0f;
        for (int gi = 0; gi < G; ++gi) {
          const int g = gi; /* query heads in increasing order */
          const float* qv = q + ((int64_t)b * s->num_q_heads + h * G + g) * D;
          for (int d = 0; d < D; ++d) {
            float mn = kv_get(meta, meta_idx(s, phys, h, 0, d), s->kv_dtype);
            float mx = kv_get(meta, meta_idx(s, phys, h, 1, d), s->kv_dtype);
            float a = qv[d] * mn; /* each product rounded to fp32 */
            float c = qv[d] * mx;
            t[d] = a > c ? a : c;
          }
          float sg = tree_sum(t, D);
          if (group_agg == TSVO_AGG_SUM)
            best = gi == 0 ? sg : best + sg; /* fp32, one rounding per head */
          else if (gi == 0 || sg > best)
            best = sg;
        }
        if (best == 0.0f) best = 0.0f; /* -0 -> +0 */
        scores[((int64_t)b * s->num_kv_heads + h) * s->max_pages_per_seq + p] =
            best;
      }
  }
  free(t);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* top-K selection                                                            */
/* ------------------------------------------------------------------------- */

typedef struct {
  float score;
  int32_t page;
} cand_t;

/* higher score first; on equal scores the lower logical page first */
static int cand_cmp(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->page > b->page) - (a->page < b->page);
}

int tsvo_select_from_scores(const tsvo_shape* s, const float* scores,
                            const int32_t* seq_lens, int32_t k_max,
                            const int32_t* k_per_seq, int32_t n_sink,
                            int32_t n_recent, int32_t* sel, int32_t* sel_count) {
  if (!shape_ok(s) || !scores || !seq_lens || !sel || !sel_count) return -1;
  if (k_max < 1 || n_sink < 0 || n_recent < 0 || n_sink > k_max ||
      n_recent > k_max - n_sink)
    return -1;
  const int64_t MP = s->max_pages_per_seq;
  cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)MP);
  char* chosen = (char*)malloc((size_t)MP);
  if (!cand || !chosen) { free(cand); free(chosen); return -1; }
  for (int b = 0; b < s->batch; ++b) {
    int64_t n = n_pages(s, seq_len(s, seq_lens, b));
    int64_t kb = k_per_seq ? k_per_seq[b] : k_max;
    if (kb < 1) kb = 1;
    if (kb > k_max) kb = k_max;
    int64_t keff = kb < n ? kb : n;
    int64_t f = n_sink < keff ? n_sink : keff;
    int64_t r = n_recent < keff - f ? n_recent : keff - f;
    for (int h = 0; h < s->num_kv_heads; ++h) {
      const float* row = scores + ((int64_t)b * s->num_kv_heads + h) * MP;
      memset(chosen, 0, (size_t)MP);
      for (int64_t p = 0; p < f; ++p) chosen[p] = 1; /* forced sink pages */
      for (int64_t p = n - r; p < n; ++p) chosen[p] = 1; /* forced recent pages */
      int64_t nc = 0;
      for (int64_t p = f; p < n - r; ++p) {
        cand[nc].score = row[p];
        cand[nc].page = (int32_t)p;
        ++nc;
      }
      qsort(cand, (size_t)nc, sizeof(cand_t), cand_cmp);
      for (int64_t i = 0; i < keff - f - r; ++i) chosen[cand[i].page] = 1;
      int32_t* out = sel + ((int64_t)b * s->num_kv_heads + h) * k_max;
      int32_t c = 0;
      for (int64_t p = 0; p < n; ++p)
        if (chosen[p]) out[c++] = (int32_t)p;
      sel_count[(int64_t)b * s->num_kv_heads + h] = c;
      for (int64_t i = c; i < k_max; ++i) out[i] = -1;
    }
  }
  free(cand);
  free(chosen);
  return 0;
}

int tsvo_select_pages(const tsvo_shape* s, const float* q, const void* meta,
                      const int32_t* bt, const int32_t* seq_lens, int32_t k_max,
                      const int32_t* k_per_seq, int32_t n_sink, int32_t n_recent,
                      int32_t group_agg, int32_t* sel, int32_t* sel_count,
                      float* scores_out) {
  if (!shape_ok(s)) return -1;
  size_t ns = (size_t)s->batch * s->num_kv_heads * s->max_pages_per_seq;
  float* sc = scores_out ? scores_out : (float*)malloc(sizeof(float) * ns);
  if (!sc) return -1;
  int rc = tsvo_page_scores(s, q, meta, bt, seq_lens, group_agg, sc);
  if (rc == 0)
    rc = tsvo_select_from_scores(s, sc, seq_lens, k_max, k_per_seq, n_sink,
                                 n_recent, sel, sel_count);
  if (!scores_out) free(sc);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* masked softmax attention over the selected pages, in double                */
/* ------------------------------------------------------------------------- */

int tsvo_sparse_decode(const tsvo_shape* s, const float* q, const void* k_pool,
                       const void* v_pool, const int32_t* bt,
                       const int32_t* seq_lens, const int32_t* sel,
                       const int32_t* sel_count, int32_t k_max, float scale,
                       float* out) {
  if (!shape_ok(s) || !q || !k_pool || !v_pool || !bt || !seq_lens || !sel ||
      !sel_count || !out || k_max < 1)
    return -1;
  const int D = s->head_dim, G = s->num_q_heads / s->num_kv_heads;
  const int64_t P = s->page_size;
  int64_t cap = (int64_t)k_max * P;
  double* z = (double*)malloc(sizeof(double) * (size_t)cap);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap); /* pool row */
  double* acc = (double*)malloc(sizeof(double) * (size_t)D);
  if (!z || !tok || !acc) { free(z); free(tok); free(acc); return -1; }
  int rc = 0;
  for (int b = 0; b < s->batch && rc == 0; ++b) {
    int64_t len = seq_len(s, seq_lens, b);
    int64_t n = n_pages(s, len);
    for (int hq = 0; hq < s->num_q_heads && rc == 0; ++hq) {
      int h = hq / G;
      int64_t u = (int64_t)b * s->num_kv_heads + h;
      int32_t cnt = sel_count[u];
      if (cnt < 0 || cnt > k_max) { rc = -1; break; }
      /* the token set: valid slots of every selected page */
      int64_t nt = 0;
      for (int32_t i = 0; i < cnt; ++i) {
        int64_t p = sel[u * k_max + i], phys;
        if (p < 0 || p >= n || !phys_of(s, bt, b, p, &phys)) { rc = -1; break; }
        int64_t v = page_valid(s, len, p);
        for (int64_t t = 0; t < v; ++t) tok[nt++] = phys * s->num_kv_heads * P + h * P + t;
      }
      if (rc) break;
      float* o = out + ((int64_t)b * s->num_q_heads + hq) * D;
      if (nt == 0) {
        for (int d = 0; d < D; ++d) o[d] = 0.0f;
        continue;
      }
      const float* qv = q + ((int64_t)b * s->num_q_heads + hq) * D;
      double m = -INFINITY;
      for (int64_t i = 0; i < nt; ++i) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += (double)qv[d] * (double)kv_get(k_pool, tok[i] * D + d, s->kv_dtype);
        z[i] = (double)scale * dot;
        if (z[i] > m) m = z[i];
      }
      double l = 0.0;
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (int64_t i = 0; i < nt; ++i) {
        double w = exp(z[i] - m);
        l += w;
        for (int d = 0; d < D; ++d)
          acc[d] += w * (double)kv_get(v_pool, tok[i] * D + d, s->kv_dtype);
      }
      for (int d = 0; d < D; ++d) o[d] = (float)(acc[d] / l);
    }
  }
  free(z);
  free(tok);
  free(acc);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* one decode step: append, score, select, attend                            */
/* ------------------------------------------------------------------------- */

int tsvo_decode_step(const tsvo_shape* s, const float* q, const void* k_new,
                     const void* v_new, void* k_pool, void* v_pool, void* meta,
                     const int32_t* bt, const int32_t* seq_lens, int32_t k_max,
                     const int32_t* k_per_seq, int32_t n_sink, int32_t n_recent,
                     int32_t group_agg, float scale, int32_t* sel,
                     int32_t* sel_count, float* scores_out, float* out) {
  int rc = 0;
  if (k_new || v_new) {
    rc = tsvo_meta_append(s, k_new, v_new, k_pool, v_pool, meta, bt, seq_lens);
    if (rc) return rc;
  }
  rc = tsvo_select_pages(s, q, meta, bt, seq_lens, k_max, k_per_seq, n_sink,
                         n_recent, group_agg, sel, sel_count, scores_out);
  if (rc) return rc;
  return tsvo_sparse_decode(s, q, k_pool, v_pool, bt, seq_lens, sel, sel_count,
                            k_max, scale, out);
}
