// Internal interface between the C-ABI host layer (tsv_api.hip), the host-side
// launch planning (tsv_host.hip) and the gfx950 kernels (tsv_kernels.hip,
// built once per KV type and kernel family).  Not installed; not part of the
// ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tsv {

// KV types; DT_F8 is OCP E4M3, DT_F8E5 OCP E5M2.
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_F8 = 3, DT_F8E5 = 4 };

constexpr bool is_fp8(int dt) { return dt == DT_F8 || dt == DT_F8E5; }

// Bytes of one KV element.
constexpr int kv_bytes(int dt) { return dt == DT_F32 ? 4 : is_fp8(dt) ? 1 : 2; }
// Consecutive channels of one row a lane loads at once: one 16-byte load, or
// 8 bytes for fp8 (so a lane holds as many channels as for 16-bit data).
constexpr int kv_vec(int dt) { return is_fp8(dt) ? 8 : 16 / kv_bytes(dt); }

// Selection policy of one call: forced sink pages, forced most recent pages,
// and whether the G query heads' box bounds are summed (else maxed).
struct SelectPolicy {
  int n_sink, n_recent, group_sum;
};

// Validated sizes of one call.
struct Dims {
  int B, Hq, Hkv, D, P, MP, NP, dt, G;
};

constexpr int kMaxPagesPerSeq = 4096;
// Decode tiles one workgroup of the phased decode streams at most.
constexpr int kMaxTilesPerSplit = 8;
// Threads of a phased (VALU) decode workgroup.
constexpr int kDecodeThreads = 256;
// Most workgroups a row of the one-launch step is spread over.
constexpr int kStepMaxSplits = 8;
// A split of a row covers at least this many 16-token steps per wave.
constexpr int kStepMinSpanSteps = 2;

// Tokens of the selected-token stream one decode workgroup covers.
int decode_tile_tokens(const Dims& d);
// Number of split slots per (sequence, KV head) for rows of k_max pages.
int decode_splits(const Dims& d, int k_max);
// Partial-state floats per (sequence, query head, split).
inline int partial_stride(const Dims& d) { return d.D + 2; }

// Rows whose step is spread over several workgroups synchronise through the
// start of the workspace, zero before the first call and left zero by every
// call: one 128-byte line of counters per row (rows are split only when
// B*Hkv <= 128), then the slots through which the row's workgroups exchange
// page keys, [B*Hkv][MP] of the current shape, at most kSyncRows rows of
// kMaxPagesPerSeq pages.  A slot reads 0 until its key is written (an order
// key is never 0) and the row's last workgroup to finish clears the slots it
// used.  The prefix does not depend on the shape, so a workspace reused for
// other shapes keeps it intact.
constexpr int kSyncRows = 128;
constexpr int kSyncWordsPerRow = 32;
constexpr size_t kSyncBytes = (size_t)kSyncRows * kSyncWordsPerRow * sizeof(uint32_t);
constexpr size_t kXchgWords = (size_t)kSyncRows * kMaxPagesPerSeq;
constexpr size_t kZeroBytes = kSyncBytes + kXchgWords * sizeof(uint32_t);

// Regions of the caller's workspace (only `sync` and `xkeys` need
// initialisation).
struct Workspace {
  uint32_t* sync;      // [kSyncRows][kSyncWordsPerRow] split-row counters
  uint32_t* xkeys;     // [B*Hkv][MP] split-row key slots (kXchgWords at most)
  uint32_t* keys;      // [B*Hkv][MP] order keys of the page scores (phased path)
  int32_t* sel_phys;   // [B*Hkv][k_max] physical page of each selection
  float* partials;     // [B*Hq][splits][D+2] tile softmax states
};
// Total workspace bytes; with `base` non-null also fills `ws`.
size_t workspace_layout(const Dims& d, int k_max, void* base, Workspace* ws);

// Scratch of tsv_decode_step_noalloc: a library-owned device array of this
// many bytes per GPU (tsv_scratch.hip).  noalloc_scratch returns its device
// address on the current device; the first call on a device also enqueues,
// on stream s, the clearing of its split-row prefix (kZeroBytes).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(hipStream_t s, void** out);

// Phased decode: S_max split slots per row, TPW tiles per split.
struct DecodePlan {
  int S_max, TPW, tile_tokens;
};
DecodePlan plan_decode(const Dims& d, int k_max);

// One-launch step: nt threads per workgroup, S workgroups per row, lds bytes
// of dynamic local memory, `polls` reads of a row's key slots before a split
// stops waiting for the row's other splits' page keys.
struct StepPlan {
  int nt, S, polls;
  size_t lds;
};
// Polls when no testing hook overrides them (several milliseconds: only
// reached if a row's workgroups are not resident at the same time).
constexpr int kDefaultExchangePolls = 1 << 14;
constexpr size_t kStepMaxLds = 64 * 1024;
StepPlan plan_step(const Dims& d, int k_max, int polls);
// The whole step of a (sequence, KV head) fits the one-launch kernel: its
// local memory, which grows with max_pages_per_seq, stays within kStepMaxLds.
bool step_fits(const Dims& d);

// Launchers, one instantiation per KV type (defined in tsv_kernels.hip).
template <int DT>
hipError_t meta_build_t(const Dims& d, const void* k_pool, void* meta, const int32_t* bt,
                        const int32_t* seq_lens, hipStream_t s);
template <int DT>
hipError_t meta_append_t(const Dims& d, const void* k_new, const void* v_new, void* k_pool,
                         void* v_pool, void* meta, const int32_t* bt, const int32_t* seq_lens,
                         hipStream_t s);
template <int DT>
hipError_t score_select_t(const Dims& d, const float* q, const void* meta, const int32_t* bt,
                          const int32_t* seq_lens, int k_max, const int32_t* k_per_seq,
                          const SelectPolicy& pol, int32_t* sel, int32_t* sel_count,
                          float* scores_out, const Workspace& ws, hipStream_t s);
template <int DT>
hipError_t decode_t(const Dims& d, const DecodePlan& plan, const float* q, const void* k_pool,
                    const void* v_pool, const int32_t* bt, const int32_t* seq_lens,
                    const int32_t* sel, const int32_t* sel_phys, const int32_t* sel_count,
                    int k_max, float scale, const Workspace& ws, float* out, hipStream_t s);
// Testing build only: copies the last step launch's phase stamps of KV type
// DT (kStampWorkgroups x 8 words of 64 bits, tsv_device.h) to host memory.
template <int DT>
hipError_t read_phase_stamps_t(void* host, size_t bytes);
// order (nullable, device): row of each workgroup of a launch with one
// workgroup per row (plan.S == 1), order_len workgroups; unused otherwise.
template <int DT>
hipError_t step_t(const Dims& d, const StepPlan& plan, const float* q, const void* k_new,
                  const void* v_new, void* k_pool, void* v_pool, void* meta, const int32_t* bt,
                  const int32_t* seq_lens, int k_max, const int32_t* k_per_seq,
                  const SelectPolicy& pol, float scale, const int32_t* order, int order_len,
                  int32_t* sel, int32_t* sel_count, float* scores_out, const Workspace& ws,
                  float* out, hipStream_t s);
// Workgroups of the step kernel for d / plan that one CU holds at once.
template <int DT>
hipError_t step_per_cu_t(const Dims& d, const StepPlan& plan, int* per_cu);

// Dispatch by KV type (tsv_host.hip).
hipError_t launch_meta_build(const Dims& d, const void* k_pool, void* meta,
                             const int32_t* bt, const int32_t* seq_lens, hipStream_t s);
hipError_t launch_meta_append(const Dims& d, const void* k_new, const void* v_new,
                              void* k_pool, void* v_pool, void* meta, const int32_t* bt,
                              const int32_t* seq_lens, hipStream_t s);
// Scores every page, keeps the top pages; also fills ws.sel_phys.
hipError_t launch_score_select(const Dims& d, const float* q, const void* meta,
                               const int32_t* bt, const int32_t* seq_lens, int k_max,
                               const int32_t* k_per_seq, const SelectPolicy& pol,
                               int32_t* sel, int32_t* sel_count, float* scores_out,
                               const Workspace& ws, hipStream_t s);
// Split decode; units with several tiles are merged by a second kernel.
// sel_phys (nullable): physical page of every selected entry, so the decode
// skips the block-table lookup.
hipError_t launch_decode(const Dims& d, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* bt, const int32_t* seq_lens,
                         const int32_t* sel, const int32_t* sel_phys,
                         const int32_t* sel_count, int k_max, float scale,
                         const Workspace& ws, float* out, hipStream_t s);
// The whole step of one (sequence, KV head) in one workgroup (or in plan.S
// workgroups that share the row's scoring, each select the whole row and
// decode a share of it; the last one to finish merges the shares): [append]
// -> score -> top-K -> decode, one launch.  Usable when step_fits(d).
// With `order` non-null and plan.S == 1, workgroup w of order_len handles
// row order[w] (entries outside [0, B*Hkv) idle).
hipError_t launch_step(const Dims& d, int polls, const float* q, const void* k_new,
                       const void* v_new, void* k_pool, void* v_pool, void* meta,
                       const int32_t* bt, const int32_t* seq_lens, int k_max,
                       const int32_t* k_per_seq, const SelectPolicy& pol, float scale,
                       const int32_t* order, int order_len, int32_t* sel,
                       int32_t* sel_count, float* scores_out, const Workspace& ws,
                       float* out, hipStream_t s);
// Workgroups per row of the one-launch step (1: a row order applies).
int step_splits_for(const Dims& d, int k_max);
// Workgroups of the one-launch step one CU holds at once.
hipError_t step_per_cu(const Dims& d, int k_max, int* per_cu);

// Longest-first row order for the one-launch step (host only, no HIP call).
// w[b] is the weight of each of sequence b's Hkv rows; num_cus CUs hold
// per_cu workgroups each.  Writes the order's length to *len and, when
// order != null and *len <= cap, the order itself (-1 = an idle workgroup).
// Returns false when cap is too small.
bool schedule_rows(const double* w, int B, int Hkv, int num_cus, int per_cu, int32_t* order,
                   long cap, long* len);

}  // namespace tsv
