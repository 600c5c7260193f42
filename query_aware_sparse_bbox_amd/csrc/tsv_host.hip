// Host-side launch planning of libtsv: workspace carving, decode split sizes,
// the one-launch step's workgroup shape, and dispatch to the launchers of the
// call's KV type.  No device code.
#include <algorithm>
#include <numeric>
#include <queue>
#include <type_traits>
#include <vector>

#include "tsv_launch.h"

namespace tsv {
namespace {

constexpr int kWave = 64;

template <int V>
using IC = std::integral_constant<int, V>;

template <class Fn>
hipError_t by_dtype(int dt, Fn&& fn) {
  switch (dt) {
    case DT_F32: return fn(IC<DT_F32>{});
    case DT_F16: return fn(IC<DT_F16>{});
    case DT_BF16: return fn(IC<DT_BF16>{});
    case DT_F8: return fn(IC<DT_F8>{});
    case DT_F8E5: return fn(IC<DT_F8E5>{});
  }
  return hipErrorInvalidValue;
}

size_t round_up(size_t x) { return (x + 255) / 256 * 256; }

// A launch is checked with hipGetLastError, which also reports (and clears)
// an error some earlier runtime call of the caller's thread left behind;
// clearing it first makes the check see this call's launches only.
void clear_stale_error() { (void)hipGetLastError(); }

// Grouped-query heads (groups of 4, 8 or 16) on 16-bit or fp8 KV take the
// MFMA decode (64-token steps); everything else the VALU decode.
bool use_mfma_decode(const Dims& d) {
  return d.dt != DT_F32 && (d.G == 4 || d.G == 8 || d.G == 16);
}

// Tiles per workgroup: enough workgroups to fill the chip several times
// over, each streaming as many tiles as that allows.
int decode_tiles_per_split(const Dims& d, int k_max) {
  const long tile = decode_tile_tokens(d);
  const long tiles_per_row = ((long)k_max * d.P + tile - 1) / tile;
  const long total = tiles_per_row * d.B * d.Hkv;
  return (int)std::max(1L, std::min((long)kMaxTilesPerSplit, total / 1024));
}

// Threads of a k_step workgroup.  Rows that fill the chip twice over get 4
// waves each, so two rows share a CU and one row's select / combine phases
// overlap the other's streaming; fewer rows get 8 waves.  16-wave workgroups
// for single-head groups measured slower than 8 (46.8 against 45.7 us on
// 256 rows of 1024 pages, 9.5 against 8.5 us on 4 rows of 64).
int step_threads(const Dims& d) {
  const long units = (long)d.B * d.Hkv;
  return units >= 512 ? 256 : 512;
}

// Dynamic LDS of k_step: block-table row and keys (MP words each, rounded to
// 4), then every wave's combine area (G rows of D + 1 floats).
size_t step_lds_bytes(const Dims& d) {
  const int nw = step_threads(d) / kWave;
  const size_t dec = (size_t)nw * d.G * (d.D + 1) * sizeof(float);
  return (size_t)2 * ((d.MP + 3) & ~3) * sizeof(uint32_t) + dec;
}

// Workgroups per row: rows that leave most of the 256 CUs idle are spread
// over up to 8 workgroups each (they share the scoring, every one selects the
// whole row, then decodes its share of the kept tokens), as far as k_max
// pages give each split its minimum span; the last split to finish merges.
// Only the first kSyncRows rows have synchronisation counters and key slots.
int step_splits(const Dims& d, int k_max) {
  const long units = (long)d.B * d.Hkv;
  const long minspan = kStepMinSpanSteps * 16 * (step_threads(d) / kWave);
  const long by_tokens = (long)k_max * d.P / minspan;
  if (units > kSyncRows || (size_t)units * d.MP > kXchgWords) return 1;
  return (int)std::max(1L, std::min({(long)kStepMaxSplits, 256 / units, by_tokens}));
}

}  // namespace

int decode_tile_tokens(const Dims& d) {
  if (use_mfma_decode(d)) return 64;
  // the VALU decode's tile (ValuDecode::TILE for kDecodeThreads threads)
  const int C = kv_vec(d.dt), L = d.D / C, SPW = kWave / L;
  return 4 * (16 / (C * kv_bytes(d.dt))) * (kDecodeThreads / kWave) * SPW;
}

int decode_splits(const Dims& d, int k_max) {
  const long span = (long)decode_tile_tokens(d) * decode_tiles_per_split(d, k_max);
  return (int)(((long)k_max * d.P + span - 1) / span);
}

DecodePlan plan_decode(const Dims& d, int k_max) {
  return DecodePlan{decode_splits(d, k_max), decode_tiles_per_split(d, k_max),
                    decode_tile_tokens(d)};
}

size_t workspace_layout(const Dims& d, int k_max, void* base, Workspace* ws) {
  const size_t units = (size_t)d.B * d.Hkv;
  const size_t o_sync = 0;
  const size_t o_xkeys = o_sync + kSyncBytes;
  const size_t o_keys = o_sync + kZeroBytes;
  const size_t o_phys = o_keys + round_up(units * d.MP * sizeof(uint32_t));
  const size_t o_part = o_phys + round_up(units * k_max * sizeof(int32_t));
  const size_t splits = std::max(decode_splits(d, k_max), step_splits(d, k_max));
  const size_t total =
      o_part + round_up((size_t)d.B * d.Hq * splits * partial_stride(d) * sizeof(float));
  if (base && ws) {
    char* c = static_cast<char*>(base);
    ws->sync = reinterpret_cast<uint32_t*>(c + o_sync);
    ws->xkeys = reinterpret_cast<uint32_t*>(c + o_xkeys);
    ws->keys = reinterpret_cast<uint32_t*>(c + o_keys);
    ws->sel_phys = reinterpret_cast<int32_t*>(c + o_phys);
    ws->partials = reinterpret_cast<float*>(c + o_part);
  }
  return total;
}

bool step_fits(const Dims& d) { return step_lds_bytes(d) <= kStepMaxLds; }

StepPlan plan_step(const Dims& d, int k_max, int polls) {
  return StepPlan{step_threads(d), step_splits(d, k_max), polls, step_lds_bytes(d)};
}

hipError_t launch_meta_build(const Dims& d, const void* k_pool, void* meta,
                             const int32_t* bt, const int32_t* seq_lens, hipStream_t s) {
  clear_stale_error();
  return by_dtype(d.dt, [&](auto DT) {
    return meta_build_t<decltype(DT)::value>(d, k_pool, meta, bt, seq_lens, s);
  });
}

hipError_t launch_meta_append(const Dims& d, const void* k_new, const void* v_new,
                              void* k_pool, void* v_pool, void* meta, const int32_t* bt,
                              const int32_t* seq_lens, hipStream_t s) {
  clear_stale_error();
  return by_dtype(d.dt, [&](auto DT) {
    return meta_append_t<decltype(DT)::value>(d, k_new, v_new, k_pool, v_pool, meta, bt,
                                              seq_lens, s);
  });
}

hipError_t launch_score_select(const Dims& d, const float* q, const void* meta,
                               const int32_t* bt, const int32_t* seq_lens, int k_max,
                               const int32_t* k_per_seq, const SelectPolicy& pol,
                               int32_t* sel, int32_t* sel_count, float* scores_out,
                               const Workspace& ws, hipStream_t s) {
  clear_stale_error();
  return by_dtype(d.dt, [&](auto DT) {
    return score_select_t<decltype(DT)::value>(d, q, meta, bt, seq_lens, k_max, k_per_seq, pol,
                                               sel, sel_count, scores_out, ws, s);
  });
}

hipError_t launch_decode(const Dims& d, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* bt, const int32_t* seq_lens,
                         const int32_t* sel, const int32_t* sel_phys,
                         const int32_t* sel_count, int k_max, float scale,
                         const Workspace& ws, float* out, hipStream_t s) {
  const DecodePlan plan = plan_decode(d, k_max);
  clear_stale_error();
  return by_dtype(d.dt, [&](auto DT) {
    return decode_t<decltype(DT)::value>(d, plan, q, k_pool, v_pool, bt, seq_lens, sel,
                                         sel_phys, sel_count, k_max, scale, ws, out, s);
  });
}

hipError_t launch_step(const Dims& d, int polls, const float* q, const void* k_new,
                       const void* v_new, void* k_pool, void* v_pool, void* meta,
                       const int32_t* bt, const int32_t* seq_lens, int k_max,
                       const int32_t* k_per_seq, const SelectPolicy& pol, float scale,
                       const int32_t* order, int order_len, int32_t* sel,
                       int32_t* sel_count, float* scores_out, const Workspace& ws,
                       float* out, hipStream_t s) {
  const StepPlan plan = plan_step(d, k_max, polls);
  if (plan.lds > kStepMaxLds) return hipErrorInvalidValue;
  clear_stale_error();
  return by_dtype(d.dt, [&](auto DT) {
    return step_t<decltype(DT)::value>(d, plan, q, k_new, v_new, k_pool, v_pool, meta, bt,
                                       seq_lens, k_max, k_per_seq, pol, scale, order,
                                       order_len, sel, sel_count, scores_out, ws, out, s);
  });
}

int step_splits_for(const Dims& d, int k_max) { return step_splits(d, k_max); }

hipError_t step_per_cu(const Dims& d, int k_max, int* per_cu) {
  const StepPlan plan = plan_step(d, k_max, kDefaultExchangePolls);
  return by_dtype(d.dt, [&](auto DT) {
    return step_per_cu_t<decltype(DT)::value>(d, plan, per_cu);
  });
}

// Longest-processing-time-first list scheduling with the workgroup
// dispatcher as the queue.  The dispatcher starts workgroups in index order:
// the first num_cus*per_cu of them are resident at once, workgroup
// j*num_cus + c of that first wave on the same CU as workgroup c (measured on
// MI355X), and every later one starts when a resident one ends.  So the
// heaviest rows make the first wave: each, heaviest first, goes to the CU
// with the least weight so far among those holding fewer than per_cu rows
// (the second row of a CU pairs heavy rows with light ones; with room for
// three, a heavy row may keep its CU to itself while light rows share
// one), and a CU's k-th row is its workgroup of round k.  Slots a CU does not
// use are idle workgroups (-1), so that every workgroup of the wave still
// lands on its CU.  Rows after the first wave follow in descending weight:
// each takes the next slot to free up.
bool schedule_rows(const double* w, int B, int Hkv, int num_cus, int per_cu, int32_t* order,
                   long cap, long* len) {
  const int units = B * Hkv;
  const long C = std::max(1, num_cus), m = std::max(1, per_cu);
  const long first = std::min<long>(units, C * m);
  // rows heaviest first, equal weights in row order: the sequences sorted,
  // each followed by its KV heads (all of a sequence's rows weigh the same)
  std::vector<int> seq(B);
  std::iota(seq.begin(), seq.end(), 0);
  std::sort(seq.begin(), seq.end(),
            [&](int a, int b) { return w[a] > w[b] || (w[a] == w[b] && a < b); });
  std::vector<int> rank(units);
  for (int i = 0; i < B; ++i)
    for (int h = 0; h < Hkv; ++h) rank[(size_t)i * Hkv + h] = seq[i] * Hkv + h;
  auto wrow = [&](int u) { return w[u / Hkv]; };
  // the first wave: the CU with the least weight among those with a free
  // slot (equal weights: lower CU first) takes the next row
  using Slot = std::pair<double, long>;  // (weight so far, CU)
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> free_cus;
  for (long c = 0; c < std::min(C, first); ++c) free_cus.push({0.0, c});
  std::vector<int> count(std::min(C, first), 0);
  std::vector<long> where(first);  // first-wave slot of rank r: round * C + CU
  long wave = 0;  // workgroups of the first wave (idle ones at its end left out
                 // when no rows follow)
  for (long r = 0; r < first; ++r) {
    const Slot s = free_cus.top();
    free_cus.pop();
    where[r] = count[s.second] * C + s.second;
    wave = std::max(wave, where[r] + 1);
    if (++count[s.second] < m) free_cus.push({s.first + wrow(rank[r]), s.second});
  }
  if (units > first) wave = (wave + C - 1) / C * C;
  *len = wave + (units - first);
  if (order == nullptr) return true;
  if (*len > cap) return false;
  std::fill(order, order + wave, -1);
  for (long r = 0; r < first; ++r) order[where[r]] = rank[r];
  for (long r = first; r < units; ++r) order[wave + (r - first)] = rank[r];
  return true;
}

}  // namespace tsv
