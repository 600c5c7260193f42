// Internal interface between the C-ABI host layer (tsv_api.hip) and the
// gfx950 kernels (tsv_kernels.hip).  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tsv {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Validated sizes of one call.
struct Dims {
  int B, Hq, Hkv, D, P, MP, NP, dt, G;
};

constexpr int kMaxPagesPerSeq = 4096;

// Tokens of the selected-token stream one decode workgroup covers.
int decode_tile_tokens(const Dims& d);
// Number of split slots per (sequence, KV head) for rows of k_max pages.
int decode_splits(const Dims& d, int k_max);
// Partial-state floats per (sequence, query head, split).
inline int partial_stride(const Dims& d) { return d.D + 2; }

hipError_t launch_meta_build(const Dims& d, const void* k_pool, void* meta,
                             const int32_t* bt, const int32_t* seq_lens,
                             hipStream_t s);

hipError_t launch_meta_append(const Dims& d, const void* k_new,
                              const void* v_new, void* k_pool, void* v_pool,
                              void* meta, const int32_t* bt,
                              const int32_t* seq_lens, hipStream_t s);

// sel_phys (nullable): physical page of every selected entry, consumed by
// the decode so it skips the block-table lookup.
hipError_t launch_score_select(const Dims& d, const float* q, const void* meta,
                               const int32_t* bt, const int32_t* seq_lens,
                               int k_max, const int32_t* k_per_seq,
                               int n_sink, int32_t* sel, int32_t* sel_count,
                               int32_t* sel_phys, float* scores_out,
                               hipStream_t s);

// Split decode (partials into `partials`) followed by the merge into `out`.
hipError_t launch_decode(const Dims& d, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* bt,
                         const int32_t* seq_lens, const int32_t* sel,
                         const int32_t* sel_phys, const int32_t* sel_count,
                         int k_max, float scale, float* partials, float* out,
                         hipStream_t s);

}  // namespace tsv
