// gfx950 (CDNA4) device code for query-aware page selection with sparse
// paged decode.  Method: TinyServe, "Query-Aware Cache Selection for Efficient
// LLM Serving" (abstract; method details, key design): per-page bounding boxes
// of the keys, a query-to-box score, the highest-scoring pages kept, masked
// attention over those pages only.
//
// The fused step is one kernel, k_step: every (sequence, KV head) row is
// handled by workgroups of its own that append, score, select and attend
// (rows too few to fill the chip are spread over several workgroups, which
// share the scoring and merge their shares without another launch).
//
// Phased kernels (separate select / decode calls, and rows too wide for the
// one-launch step's local memory), in the order a decode step runs them:
//   k_meta_append    write the new token, widen its page's box
//   k_score_select   one workgroup per (sequence, KV head): stream the page
//                    boxes (coalesced 16-byte rows), score them on the VALU
//                    with DPP butterflies, radix top-K in LDS
//   k_decode_split   one workgroup per (sequence, KV head, token tile): gather
//                    the selected pages' K/V straight from the pool, masked
//                    softmax partial state of the tile
//   k_merge          combine the tiles' partial states into the output
// plus k_meta_build, the full rebuild of every box.
//
// Wave64 throughout; all reductions stay inside a wavefront (DPP / ds_swizzle
// / bpermute) except one LDS step across the workgroup's waves.
//
// Everything here has internal linkage; tsv_kernels.hip includes it once per
// translation unit (one per KV type and kernel family).
#pragma once
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "tsv_launch.h"

namespace tsv {

#ifdef TSV_PHASE_STAMPS
// Phase stamps of the testing build: thread 0 of every workgroup of the
// one-launch step records the GPU's 100 MHz real-time counter at the step's
// phase boundaries (slot 0 start, 1 block-table row staged, 2 scored (with
// the split rows' key exchange), 3 selected, 4 decoded, 5 end), and its
// (row, split) in slot 6.  The last launch's stamps are read back through
// tsv_debug_phase_stamps.
constexpr int kStampWorkgroups = 8192, kStampSlots = 8;
__device__ unsigned long long g_phase_stamps[kStampWorkgroups][kStampSlots];
#define TSV_STAMP(i)                                                      \
  do {                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < kStampWorkgroups)                \
      g_phase_stamps[blockIdx.x][i] = __builtin_amdgcn_s_memrealtime();   \
  } while (0)
#define TSV_STAMP_VALUE(i, v)                                             \
  do {                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < kStampWorkgroups)                \
      g_phase_stamps[blockIdx.x][i] = (v);                                \
  } while (0)
#else
#define TSV_STAMP(i) \
  do {               \
  } while (0)
#define TSV_STAMP_VALUE(i, v) \
  do {                        \
  } while (0)
#endif

namespace {

constexpr int kWave = 64;

template <int DT>
struct KV {
  static constexpr int bytes = kv_bytes(DT);
  static constexpr int vec = kv_vec(DT);  // elements of one lane load
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// One lane load of LB = 8 or 16 bytes (8 bytes land in .x/.y).
template <int LB>
__device__ __forceinline__ uint4 ldb(const void* p) {
  static_assert(LB == 8 || LB == 16, "lane loads are 8 or 16 bytes");
  if constexpr (LB == 8) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    return make_uint4(x.x, x.y, 0u, 0u);
  } else {
    return ld16(p);
  }
}

// The same lane load marked non-temporal (`nt`): for data that one step reads
// once.  On the page boxes it measured 4-11% faster steps than plain loads
// (except fp8 boxes read four rows per lane, 7% slower); on K/V it did not
// pay in the one-launch step.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int LB>
__device__ __forceinline__ uint4 ldb_nt(const void* p) {
  static_assert(LB == 8 || LB == 16, "lane loads are 8 or 16 bytes");
  if constexpr (LB == 8) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint4(x.x, x.y, 0u, 0u);
  } else {
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
  }
}

// A K/V load of type T (4, 8 or 16 bytes), non-temporal when NTKV: the
// phased decode kernels, which stream K/V with no other phase beside them,
// measured 9% faster with it; the one-launch step measured slower.
template <bool NTKV, class T>
__device__ __forceinline__ T ld_kv(const void* p) {
  if constexpr (!NTKV) {
    return *reinterpret_cast<const T*>(p);
  } else if constexpr (sizeof(T) == 16) {
    const uint4 r = ldb_nt<16>(p);
    T t;
    __builtin_memcpy(&t, &r, 16);
    return t;
  } else if constexpr (sizeof(T) == 8) {
    const uint4 r = ldb_nt<8>(p);
    T t;
    __builtin_memcpy(&t, &r, 8);
    return t;
  } else {
    static_assert(sizeof(T) == 4, "K/V loads are 4, 8 or 16 bytes");
    const uint32_t x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    T t;
    __builtin_memcpy(&t, &x, 4);
    return t;
  }
}

// Four OCP fp8 values (bytes 0..3 of w; E4M3 for DT_F8, E5M2 for DT_F8E5)
// widened to fp32, exactly.
template <int DT>
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  f32x2 a, b;
  if constexpr (DT == DT_F8) {
    a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  } else {
    a = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    b = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  }
  f[0] = a.x;
  f[1] = a.y;
  f[2] = b.x;
  f[3] = b.y;
}

// Widen one lane load of C elements to fp32 (exact).
template <int DT, int C = KV<DT>::vec>
__device__ __forceinline__ void unpack(const uint4 r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else if constexpr (is_fp8(DT)) {
#pragma unroll
    for (int i = 0; i < C / 4; ++i) fp8x4_to_f32<DT>(w[i], f + 4 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
      f[2 * i] = (float)h.x;
      f[2 * i + 1] = (float)h.y;
    }
  }
}

template <int DT>
__device__ __forceinline__ float elem_to_f32(uint32_t bits) {
  if constexpr (DT == DT_F32) return __uint_as_float(bits);
  else if constexpr (DT == DT_BF16) return __uint_as_float(bits << 16);
  else if constexpr (DT == DT_F8) return __builtin_amdgcn_cvt_f32_fp8((int)bits, 0);
  else if constexpr (DT == DT_F8E5) return __builtin_amdgcn_cvt_f32_bf8((int)bits, 0);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

template <int DT>
__device__ __forceinline__ uint32_t load_elem(const void* base, size_t i) {
  if constexpr (DT == DT_F32) return reinterpret_cast<const uint32_t*>(base)[i];
  else if constexpr (is_fp8(DT)) return reinterpret_cast<const uint8_t*>(base)[i];
  else return reinterpret_cast<const uint16_t*>(base)[i];
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, size_t i, uint32_t bits) {
  if constexpr (DT == DT_F32) reinterpret_cast<uint32_t*>(base)[i] = bits;
  else if constexpr (is_fp8(DT)) reinterpret_cast<uint8_t*>(base)[i] = (uint8_t)bits;
  else reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)bits;
}

// ---------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowRor8 = 0x128;

// The value of lane ^ 32 / lane ^ 16, by the gfx950 lane-swap instructions
// (v_permlane32_swap / v_permlane16_swap: plain VALU, where a shuffle would
// take the LDS crossbar).  With x in both operands, the swap leaves lane l's
// partner value in the first result when bit 5 (bit 4) of l is set, else in
// the second.  All 64 lanes must be active.
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

// Sum over aligned groups of L lanes.  Lane k of a group holds the partial
// sum of its own contiguous channel run; every step adds the sibling subtree
// (after a step all lanes of a subtree hold the same value, so the mirror
// permutations pick a lane of the sibling subtree), which reproduces a
// balanced pairwise tree over the group's channels exactly.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (L >= 2) x = x + dpp<kQuadXor1>(x);
  if constexpr (L >= 4) x = x + dpp<kQuadXor2>(x);
  if constexpr (L >= 8) x = x + dpp<kRowHalfMirror>(x);
  if constexpr (L >= 16) x = x + dpp<kRowMirror>(x);
  if constexpr (L >= 32) x = x + xor16(x);
  if constexpr (L >= 64) x = x + xor32(x);
  return x;
}

// Combine lanes that differ only in the bits >= log2(L) (the other slots of
// the wave).  Requires L >= 8.
template <int L, class Op>
__device__ __forceinline__ float across_slots(float x, Op op) {
  static_assert(L >= 8, "slot reduction assumes at least 8 lanes per slot");
  if constexpr (L <= 8) x = op(x, dpp<kRowRor8>(x));
  if constexpr (L <= 16) x = op(x, xor16(x));
  if constexpr (L <= 32) x = op(x, xor32(x));
  return x;
}

// The value of lane ^ MASK (MASK = 8, 16, 32).
template <int MASK>
__device__ __forceinline__ float xor_lane(float x) {
  if constexpr (MASK == 8) return dpp<kRowRor8>(x);
  else if constexpr (MASK == 16) return xor16(x);
  else return xor32(x);
}

// Balanced pairwise fp32 sum of t[0..N): T(lo,hi) = T(lo,mid) + T(mid,hi).
template <int N>
__device__ __forceinline__ float tree_sum(const float* t) {
  if constexpr (N == 1) return t[0];
  else return tree_sum<N / 2>(t) + tree_sum<N / 2>(t + N / 2);
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane
// row (row_shr 1, 2, 4, 8), then row totals carried with row_bcast 15 / 31.
__device__ __forceinline__ int wave_incl_scan(int x, int /*lane*/) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int t = tmp[i];
    off += i < w ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

// Order-preserving map of fp32 (no NaN) to uint32: a > b <=> key(a) > key(b).
// The least key of a non-NaN score is 0x007fffff (-inf); only one NaN
// pattern maps to 0.
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Device-scope (agent) atomic stores and loads: coherent across every CU and
// XCD of the GPU without cache-wide maintenance; used for the few words that
// workgroups of one launch exchange.
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Returns once this thread's earlier stores have completed at their scope
// (s_waitcnt vmcnt(0); the fence keeps the compiler from moving them past).
__device__ __forceinline__ void stores_done() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited on
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return min(max(x, lo), hi);
}

// Copy n 32-bit words from global memory to LDS, threads nt apart, issuing
// R loads per thread before the first store so that one memory latency
// covers R*nt words (indices are clamped, so the loads need no branches).
template <int R, class T, class F>
__device__ __forceinline__ void stage_row(const int32_t* __restrict__ src, int n, int nt,
                                          T* dst, F&& fn) {
  for (int base = 0; base < n; base += R * nt) {
    int32_t v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = src[min(base + r * nt + (int)threadIdx.x, n - 1)];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int p = base + r * nt + (int)threadIdx.x;
      if (p < n) dst[p] = fn(v[r]);
    }
  }
}

// ---------------------------------------------------------------------------
// K0: metadata
// ---------------------------------------------------------------------------

// grid (ceil(Hkv*D/256), MP, B): one thread per (sequence, page, head, channel)
template <int DT>
__global__ __launch_bounds__(256) void k_meta_build(
    const void* __restrict__ k_pool, void* __restrict__ meta,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    int Hkv, int D, int P, int MP, int NP) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int p = blockIdx.y, b = blockIdx.z;
  if (i >= Hkv * D) return;
  const int len = clampi(seq_lens[b], 0, MP * P);
  if (p * P >= len) return;
  const int h = i / D, d = i - h * D;
  const int v = min(P, len - p * P);
  const size_t phys = (size_t)clampi(bt[(size_t)b * MP + p], 0, NP - 1);
  const size_t base = ((phys * Hkv + h) * P) * D + d;
  uint32_t bmin = load_elem<DT>(k_pool, base), bmax = bmin;
  float vmin = elem_to_f32<DT>(bmin), vmax = vmin;
  for (int s = 1; s < v; ++s) {
    const uint32_t e = load_elem<DT>(k_pool, base + (size_t)s * D);
    const float x = elem_to_f32<DT>(e);
    if (x < vmin) { vmin = x; bmin = e; }
    if (x > vmax) { vmax = x; bmax = e; }
  }
  const size_t m = ((phys * Hkv + h) * 2) * D + d;
  store_elem<DT>(meta, m, bmin);
  store_elem<DT>(meta, m + D, bmax);
}

// one thread per (sequence, head, channel)
template <int DT>
__global__ __launch_bounds__(256) void k_meta_append(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    void* __restrict__ k_pool, void* __restrict__ v_pool, void* __restrict__ meta,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens, int B,
    int Hkv, int D, int P, int MP, int NP) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * Hkv * D) return;
  const int b = i / (Hkv * D), r = i - b * Hkv * D, h = r / D, d = r - h * D;
  const int len = min(seq_lens[b], MP * P);
  if (len < 1) return;
  const int pos = len - 1, p = pos / P, slot = pos - p * P;
  const size_t phys = (size_t)clampi(bt[(size_t)b * MP + p], 0, NP - 1);
  const uint32_t kb = load_elem<DT>(k_new, i), vb = load_elem<DT>(v_new, i);
  const size_t dst = ((phys * Hkv + h) * P + slot) * D + d;
  store_elem<DT>(k_pool, dst, kb);
  store_elem<DT>(v_pool, dst, vb);
  const size_t m = ((phys * Hkv + h) * 2) * D + d;
  if (slot == 0) {
    store_elem<DT>(meta, m, kb);
    store_elem<DT>(meta, m + D, kb);
  } else {
    const float k = elem_to_f32<DT>(kb);
    if (k < elem_to_f32<DT>(load_elem<DT>(meta, m))) store_elem<DT>(meta, m, kb);
    if (k > elem_to_f32<DT>(load_elem<DT>(meta, m + D))) store_elem<DT>(meta, m + D, kb);
  }
}

// ---------------------------------------------------------------------------
// K1: page scoring, streamed per (sequence, KV head), and top-K selection
// ---------------------------------------------------------------------------
//
// Lane layout of the scoring loop: a page's box row is 2*D*bytes; each lane
// loads 16 bytes of the min row and 16 bytes of the max row, i.e. C
// contiguous channels, so L = D/C lanes cover a page and one wave scores
// 64/L pages per load.  Consecutive lanes read consecutive 16-byte pieces of
// the same row, so every wave load is a run of whole 64/128-byte segments.
// A batch is PB = waves * (64/L) * U pages; a workgroup walks its batches
// with the next batch's rows already in flight while it scores the current
// one (two register buffers).
//
// Term per channel: fma(qneg, mn, qpos*mx) with qpos = max(q,0),
// qneg = min(q,0).  One of qpos/qneg is zero, so the result is the single
// rounding of q*mx (q >= 0) or q*mn (q < 0), which is max(fl(q*mn), fl(q*mx))
// because mn <= mx and rounding is monotone; zero signs can differ, which
// only shows in an all-zero sum and -0 is stored as +0.
// 16 waves per scoring workgroup where the registers allow it (128 per
// lane), else 8; 4 waves when one batch of that size covers a whole row
template <int G>
constexpr int score_threads() { return G <= 1 ? 1024 : 512; }

template <int DT, int D, int G, int NTH>
struct ScoreCfg {
  static constexpr int EB = KV<DT>::bytes, C = KV<DT>::vec, L = D / C;
  // a lane holds the queries of at most 8 heads; a group of 16 splits its
  // heads over HS = 2 slices of L lanes that load the same box channels
  static constexpr int HS = G > 8 ? 2 : 1, GH = G / HS;
  static constexpr int PPW = kWave / (L * HS);  // pages per wave per load
  static constexpr int U = G >= 4 ? 1 : 4;  // rows per lane per batch
  static constexpr int NT = NTH, NW = NT / kWave;
  static constexpr int PB = NW * PPW * U;  // pages per batch
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Reduction of x over the 64 lanes with an associative, commutative,
// idempotent op: DPP inside each 16-lane row, then the four row results
// read as scalars.  Wave-uniform result.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
  x = op(x, dpp_u<kQuadXor1>(x));
  x = op(x, dpp_u<kQuadXor2>(x));
  x = op(x, dpp_u<kRowHalfMirror>(x));
  x = op(x, dpp_u<kRowMirror>(x));
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return op(op(r0, r1), op(r2, r3));
}

// LDS scratch of select_block (s_red[0] / s_red[1] must hold all-ones / zero,
// written before a barrier that precedes the call).
template <int NT>
struct SelectLds {
  alignas(16) int hist[2][256];  // passes alternate, so a pass's scan overlaps the next clear
  int red[8];
  int scan[NT / 64];
};

// Top-K of one row by a whole workgroup.  Pages [0, f) and [n - r, n) are
// always kept; the other R = keff - f - r slots take the largest order keys
// among pages [f, n - r), equal keys lowest page first.
//
// Thread t owns the m = ceil(n/NT) consecutive pages [t*m, t*m + m) and keeps
// their keys in registers (M >= m slots: every loop over them has a
// compile-time trip count, so the arrays stay in registers without indexed
// access).  The threshold is found most-significant digit first: the bits
// every candidate shares are fixed at once (block AND / OR), then 8-bit
// digits are counted in an LDS histogram (double-buffered: the waves that do
// not scan it clear the next pass's) until the boundary bucket is taken
// whole or no bits are left.  One block-wide scan of packed (kept-above,
// equal-to-threshold) counts then gives every thread its output slots, so
// the pages come out in ascending order without sorting.
//
// Leaves the kept pages, ascending, in LDS: s_key[0..cnt) logical pages,
// s_phys[0..cnt) physical pages, and returns cnt.  With srow non-null also
// writes the logical pages to srow (-1 padded to k_max), the physical pages
// to prow (if non-null) and the count to *count.  Ends with a barrier.
template <int NT, int M>
__device__ __forceinline__ int select_block_m(uint32_t* s_key, uint32_t* s_phys, int n,
                                              int keff, int f, int r, int k_max,
                                              int32_t* __restrict__ srow,
                                              int32_t* __restrict__ prow,
                                              int32_t* __restrict__ count, SelectLds<NT>& sl) {
  constexpr int NW = NT / kWave;
  static_assert(NT >= 256, "one histogram bin per thread is cleared");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int m = (n + NT - 1) / NT;  // <= M
  const int p0 = tid * m, nl = max(n - 1, 0);
  const int R = keff - f - r, ncand = n - f - r, pr = n - r;  // candidates [f, pr)
  const bool take_all = R >= ncand, radix = R > 0 && R < ncand;
  uint32_t kk[M], ph[M];
  bool cand[M], valid[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int p = p0 + i, pc = min(p, nl);
    kk[i] = s_key[pc];
    ph[i] = s_phys[pc];
    valid[i] = i < m && p < n;
    cand[i] = valid[i] && p >= f && p < pr;
  }
  uint32_t tmask = 0, tau = 0;  // (key & tmask) > tau: kept; == tau: the first `need`
  int need = 0;
  if (radix) {
    uint32_t a = ~0u, o = 0u;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      a &= cand[i] ? kk[i] : ~0u;
      o |= cand[i] ? kk[i] : 0u;
    }
    a = wave_reduce(a, [](uint32_t u, uint32_t v) { return u & v; });
    o = wave_reduce(o, [](uint32_t u, uint32_t v) { return u | v; });
    if (lane == 0) {
      atomicAnd(reinterpret_cast<unsigned*>(&sl.red[0]), a);
      atomicOr(reinterpret_cast<unsigned*>(&sl.red[1]), o);
    }
    if (tid < 256) sl.hist[0][tid] = 0;
    __syncthreads();
    a = (uint32_t)sl.red[0];
    o = (uint32_t)sl.red[1];
    int remaining = R;
    if (a == o) {  // every candidate has the same key: lowest pages win
      tmask = ~0u;
      tau = a;
    } else {
      int top = 31 - __clz(a ^ o);
      tmask = top == 31 ? 0u : ~((2u << top) - 1u);
      tau = a & tmask;
      for (int pass = 0;; ++pass) {
        const int width = min(8, top + 1), shift = top + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        const int nb = 1 << width;
        int* hist = sl.hist[pass & 1];
#pragma unroll
        for (int i = 0; i < M; ++i)
          if (cand[i] && (kk[i] & tmask) == tau) atomicAdd(&hist[(kk[i] >> shift) & dmask], 1);
        __syncthreads();
        if (wave == 0) {
          int c[4], sum = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int bin = nb - 1 - 4 * lane - j;
            c[j] = bin >= 0 ? hist[bin] : 0;
            sum += c[j];
          }
          int before = wave_incl_scan(sum, lane) - sum;  // keys in higher digits
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (before < remaining && before + c[j] >= remaining) {
              sl.red[2] = nb - 1 - 4 * lane - j;
              sl.red[3] = remaining - before;
              sl.red[4] = c[j];
            }
            before += c[j];
          }
        } else {
          // the other waves clear the next pass's histogram meanwhile
          for (int i = tid - kWave; i < 256; i += NT - kWave) sl.hist[(pass + 1) & 1][i] = 0;
        }
        __syncthreads();
        const int dg = sl.red[2], cb = sl.red[4];
        remaining = sl.red[3];
        tau |= (uint32_t)dg << shift;
        tmask |= dmask << shift;
        if (remaining == cb || shift == 0) break;
        top = shift - 1;
      }
    }
    need = remaining;
  }
  int nkeep = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const uint32_t km = kk[i] & tmask;
    nkeep += (valid[i] && !cand[i]) || (cand[i] && (take_all || (radix && km > tau)));
    neq += radix && cand[i] && km == tau;
  }
  int tot;
  const int ex = block_excl_scan<NW>((neq << 16) | nkeep, sl.scan, &tot);
  int eqi = ex >> 16;
  int pos = (ex & 0xffff) + min(eqi, need);
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const uint32_t km = kk[i] & tmask;
    bool keep = (valid[i] && !cand[i]) || (cand[i] && (take_all || (radix && km > tau)));
    if (radix && cand[i] && km == tau) keep = eqi++ < need;
    if (keep) {
      if (pos < k_max) {  // never false: the count is at most min(K_b, n_b)
        if (srow) srow[pos] = p0 + i;
        if (prow) prow[pos] = (int32_t)ph[i];
        s_key[pos] = (uint32_t)(p0 + i);
        s_phys[pos] = ph[i];
      }
      ++pos;
    }
  }
  const int total = min((tot & 0xffff) + min(tot >> 16, need), k_max);
  if (srow) {
    for (int i = total + tid; i < k_max; i += NT) {
      srow[i] = -1;
      if (prow) prow[i] = 0;
    }
    if (tid == 0) *count = total;
  }
  __syncthreads();
  return total;
}

// select_block_m for the row's m = ceil(n / NT) pages per thread, rounded up
// to a power of two (a uniform branch).  s_red[0] / s_red[1] must hold
// all-ones / zero, written before a barrier that precedes the call.
template <int NT>
__device__ __forceinline__ int select_block(uint32_t* s_key, uint32_t* s_phys, int n, int keff,
                                            int f, int r, int k_max, int32_t* __restrict__ srow,
                                            int32_t* __restrict__ prow,
                                            int32_t* __restrict__ count, SelectLds<NT>& sl) {
  constexpr int MAXM = kMaxPagesPerSeq / NT;
  const int m = (n + NT - 1) / NT;
  if (m <= 1)
    return select_block_m<NT, 1>(s_key, s_phys, n, keff, f, r, k_max, srow, prow, count, sl);
  if (m <= 2)
    return select_block_m<NT, 2>(s_key, s_phys, n, keff, f, r, k_max, srow, prow, count, sl);
  if constexpr (MAXM > 4) {
    if (m <= 4)
      return select_block_m<NT, 4>(s_key, s_phys, n, keff, f, r, k_max, srow, prow, count, sl);
  }
  if constexpr (MAXM > 8) {
    if (m <= 8)
      return select_block_m<NT, 8>(s_key, s_phys, n, keff, f, r, k_max, srow, prow, count, sl);
  }
  return select_block_m<NT, MAXM>(s_key, s_phys, n, keff, f, r, k_max, srow, prow, count, sl);
}

// Rows of at most this many pages are selected by one wave (select_wave),
// one page per lane: faster than the workgroup's digit search only there.
constexpr int kWaveSelectPages = kWave;

// Top-K of one row of at most 64 pages by wave 0 of the workgroup, with the
// same result as select_block: pages [0, f) and [n - r, n) always kept, the
// other R = keff - f - r slots to the largest order keys among pages
// [f, n - r), equal keys lowest page first; the kept pages left ascending in
// s_key / s_phys [0, cnt).  Lane l holds page l in registers, so no barrier
// is needed until the end: the shared high bits of the candidates are fixed
// by a wave AND / OR, then 8-bit digits are counted in an LDS histogram (LDS
// operations of one wave complete in order) until the boundary bucket is
// taken whole or no bits are left.  The output position of a kept page is
// the number of kept lanes below it (a ballot), so the pages come out
// ascending without a sort.  All threads return the count; ends with a
// barrier.
template <int NT>
__device__ __forceinline__ int select_wave(uint32_t* s_key, uint32_t* s_phys, int n, int keff,
                                           int f, int r, int k_max, SelectLds<NT>& sl) {
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x < kWave) {
    const int R = keff - f - r, pr = n - r, ncand = pr - f;
    const bool take_all = R >= ncand, radix = R > 0 && R < ncand;
    int* hist = sl.hist[0];
    const int p = lane, pc = min(p, max(n - 1, 0));
    const uint32_t kk = s_key[pc], ph = s_phys[pc];
    const bool valid = p < n, cand = valid && p >= f && p < pr;
    uint32_t tmask = 0, tau = 0;  // (key & tmask) > tau: kept; == tau: the first `need`
    int need = 0;
    if (radix) {
      const uint32_t a =
          wave_reduce(cand ? kk : ~0u, [](uint32_t u, uint32_t v) { return u & v; });
      const uint32_t o = wave_reduce(cand ? kk : 0u, [](uint32_t u, uint32_t v) { return u | v; });
      int remaining = R;
      if (a == o) {  // every candidate has the same key: lowest pages win
        tmask = ~0u;
        tau = a;
      } else {
        int top = 31 - __clz(a ^ o);
        tmask = top == 31 ? 0u : ~((2u << top) - 1u);
        tau = a & tmask;
        for (;;) {
          const int width = min(8, top + 1), shift = top + 1 - width;
          const uint32_t dmask = (1u << width) - 1u;
          const int nb = 1 << width;
          reinterpret_cast<int4*>(hist)[lane] = int4{0, 0, 0, 0};  // 256 bins
          if (cand && (kk & tmask) == tau) atomicAdd(&hist[(kk >> shift) & dmask], 1);
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          int c[4], sum = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {  // digits in decreasing order
            const int bin = nb - 1 - 4 * lane - j;
            c[j] = bin >= 0 ? hist[bin] : 0;
            sum += c[j];
          }
          int before = wave_incl_scan(sum, lane) - sum;  // keys in higher digits
          int dg = -1, rem = 0, cb = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (before < remaining && before + c[j] >= remaining) {
              dg = nb - 1 - 4 * lane - j;
              rem = remaining - before;
              cb = c[j];
            }
            before += c[j];
          }
          const int src = __ffsll(__ballot(dg >= 0)) - 1;  // exactly one lane
          dg = __builtin_amdgcn_readlane(dg, src);
          remaining = __builtin_amdgcn_readlane(rem, src);
          cb = __builtin_amdgcn_readlane(cb, src);
          tau |= (uint32_t)dg << shift;
          tmask |= dmask << shift;
          if (remaining == cb || shift == 0) break;
          top = shift - 1;
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        }
      }
      need = remaining;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    const uint32_t km = kk & tmask;
    const bool eq = radix && cand && km == tau;
    bool keep = (valid && !cand) || (cand && (take_all || (radix && km > tau)));
    if (eq) keep = __popcll(__ballot(eq) & below) < need;
    const unsigned long long bk = __ballot(keep);
    const int pos = __popcll(bk & below);
    if (keep && pos < k_max) {  // pos < k_max always: at most min(K_b, n_b) are kept
      s_key[pos] = (uint32_t)p;
      s_phys[pos] = ph;
    }
    if (lane == 0) sl.red[5] = min(__popcll(bk), k_max);
  }
  __syncthreads();
  return sl.red[5];
}

// Scores batches bstart, bstart + bstride, ... of one unit's n pages into
// s_key (order keys).  s_phys holds the unit's block-table row.  GSUM: the
// group's heads are summed (fp32, increasing head order), else maxed.  No
// barrier.
template <int DT, int D, int G, int NT, bool GSUM>
__device__ __forceinline__ void score_pages(const float* __restrict__ q,
                                            const void* __restrict__ meta,
                                            const uint32_t* s_phys, int b, int h, int Hq,
                                            int Hkv, int n, int bstart, int bstride,
                                            uint32_t* s_key) {
  using Cfg = ScoreCfg<DT, D, G, NT>;
  constexpr int EB = Cfg::EB, C = Cfg::C, L = Cfg::L, PPW = Cfg::PPW, U = Cfg::U;
  constexpr int NW = Cfg::NW, PB = Cfg::PB, HS = Cfg::HS, GH = Cfg::GH;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nbatch = (n + PB - 1) / PB;
  // lane: channel run `chunk` of page slot `slot`, heads hs*GH .. hs*GH+GH-1
  const int chunk = lane % L, hs = (lane / L) % HS, slot = lane / (L * HS);
  float qp[GH][C], qn[GH][C];
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    const float* qg = q + ((size_t)b * Hq + h * G + hs * GH + g) * D + chunk * C;
#pragma unroll
    for (int cc = 0; cc < C; cc += 4) {
      const float4 x4 = *reinterpret_cast<const float4*>(qg + cc);
      const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qp[g][cc + k] = xs[k] > 0.f ? xs[k] : 0.f;
        qn[g][cc + k] = xs[k] < 0.f ? xs[k] : 0.f;
      }
    }
  }
  const char* mb = reinterpret_cast<const char*>(meta);
  // masked lanes read a valid row (page n-1) and drop it: no branches around
  // the loads, so the compiler's load counters track both buffers exactly
  auto load_batch = [&](int bi, uint4 (&mn)[U], uint4 (&mx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = min(bi * PB + u * (NW * PPW) + wave * PPW + slot, n - 1);
      const size_t row = ((size_t)s_phys[p] * Hkv + h) * 2 * D + chunk * C;
      if constexpr (U == 1 || C * EB == 16) {
        mn[u] = ldb_nt<C * EB>(mb + row * EB);
        mx[u] = ldb_nt<C * EB>(mb + (row + D) * EB);
      } else {  // 8-byte lanes, four rows each: plain loads measured faster
        mn[u] = ldb<C * EB>(mb + row * EB);
        mx[u] = ldb<C * EB>(mb + (row + D) * EB);
      }
    }
  };
  auto score_batch = [&](int bi, const uint4 (&rmn)[U], const uint4 (&rmx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = bi * PB + u * (NW * PPW) + wave * PPW + slot;
      float mn[C], mx[C];
      unpack<DT, C>(rmn[u], mn);
      unpack<DT, C>(rmx[u], mx);
      float best = 0.f, sc[GH];
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        float t[C];
#pragma unroll
        for (int cc = 0; cc < C; ++cc)
          t[cc] = __builtin_fmaf(qn[g][cc], mn[cc], qp[g][cc] * mx[cc]);
        sc[g] = group_sum<L>(tree_sum<C>(t));
        if constexpr (GSUM) best = g == 0 ? sc[g] : best + sc[g];
        else best = g == 0 ? sc[g] : fmaxf(best, sc[g]);
      }
      if constexpr (HS == 2) {
        // slice 0 combines slice 1's heads: the max is exact in any order,
        // the sum continues head by head (heads 8..15 after 0..7)
        if constexpr (GSUM) {
#pragma unroll
          for (int g = 0; g < GH; ++g) best = best + xor_lane<L>(sc[g]);
        } else {
          best = fmaxf(best, xor_lane<L>(best));
        }
      }
      best = best == 0.f ? 0.f : best;  // -0 -> +0
      if (p < n && chunk == 0 && hs == 0) s_key[p] = order_key(best);
    }
  };
  // a ring of DEPTH batches in flight: batch bi's slot is refilled with
  // batch bi + DEPTH*bstride right after bi is scored.  The loads take no
  // branch (indices past the last batch reload the last one), and the
  // steady-state loop refills every slot, so each wait in it leaves the same
  // DEPTH-1 batches in flight: a load issued under a condition would make
  // the compiler drain the whole ring at the top of every round.  fp8 lanes
  // load 8 bytes, so their ring is twice as deep for the same bytes in
  // flight (single-row batches only: four-row batches would not fit
  // 1024-thread workgroups' registers).
  constexpr int DEPTH = U == 1 ? 4 * (16 / (C * EB)) : 2;
  if (bstart >= nbatch) return;
  uint4 rmn[DEPTH][U], rmx[DEPTH][U];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_batch(min(bstart + i * bstride, nbatch - 1), rmn[i], rmx[i]);
  int base = bstart;
  for (; base + DEPTH * bstride < nbatch; base += DEPTH * bstride) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int bi = base + i * bstride;
      score_batch(bi, rmn[i], rmx[i]);
      load_batch(min(bi + DEPTH * bstride, nbatch - 1), rmn[i], rmx[i]);
    }
  }
  // the last round: the batches still in the ring
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    const int bi = base + i * bstride;
    if (bi < nbatch) score_batch(bi, rmn[i], rmx[i]);
  }
}

// One workgroup per (unit, split): scores batches split, split + NS, ...
// of the unit's pages.  With NS == 1 the keys stay in LDS and the workgroup
// selects at the end; otherwise the keys go to the workspace for k_select.
template <int G>
constexpr int score_min_waves() { return 1; }

template <int DT, int D, int G, int NTH>
__global__ __launch_bounds__(NTH, score_min_waves<G>()) void k_score_select(
    const float* __restrict__ q, const void* __restrict__ meta,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    int Hq, int Hkv, int P, int MP, int NP, int NS, int k_max,
    const int32_t* __restrict__ k_per_seq, SelectPolicy pol,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
    float* __restrict__ scores_out, uint32_t* __restrict__ keys,
    int32_t* __restrict__ sel_phys) {
  using Cfg = ScoreCfg<DT, D, G, NTH>;
  constexpr int NT = Cfg::NT, PB = Cfg::PB;
  extern __shared__ uint32_t smem[];
  uint32_t* s_phys = smem;       // [MP] physical page of every logical page
  uint32_t* s_key = smem + MP;   // [MP] order keys (NS == 1)
  __shared__ SelectLds<NT> sl;

  const int unit = blockIdx.x / NS, split = blockIdx.x - unit * NS;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x;
  if (tid == 0) {
    sl.red[0] = -1;
    sl.red[1] = 0;
  }
  // the whole block-table row (MP entries, all allocated) is staged without
  // waiting for the length, so both loads share one memory latency
  const int32_t* bt_row = bt + (size_t)b * MP;
  stage_row<4>(bt_row, MP, NT, s_phys, [NP](int32_t e) { return (uint32_t)clampi(e, 0, NP - 1); });
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int kb = clampi(k_per_seq ? k_per_seq[b] : k_max, 1, k_max);
  const int n = (len + P - 1) / P;
  const int nbatch = (n + PB - 1) / PB;
  if (split > 0 && split >= nbatch) return;  // whole workgroup: no pages
  __syncthreads();
  // one copy of the scoring loop per aggregation; the branch is uniform
  if (pol.group_sum)
    score_pages<DT, D, G, NT, true>(q, meta, s_phys, b, h, Hq, Hkv, n, split, NS, s_key);
  else
    score_pages<DT, D, G, NT, false>(q, meta, s_phys, b, h, Hq, Hkv, n, split, NS, s_key);
  __syncthreads();
  // this workgroup's pages: keys for k_select (split rows), optional scores
  if (NS > 1 || scores_out) {
    uint32_t* krow = keys + (size_t)unit * MP;
    float* srow_out = scores_out ? scores_out + (size_t)unit * MP : nullptr;
    for (int b2 = split; b2 < nbatch; b2 += NS)
      for (int i = tid; i < PB; i += NT) {
        const int p = b2 * PB + i;
        if (p < n) {
          const uint32_t k = s_key[p];
          if (NS > 1) krow[p] = k;
          if (srow_out) srow_out[p] = key_to_score(k);
        }
      }
  }
  if (NS > 1) return;
  const int keff = min(kb, n), f = min(pol.n_sink, keff), r = min(pol.n_recent, keff - f);
  select_block<NT>(s_key, s_phys, n, keff, f, r, k_max, sel + (size_t)unit * k_max,
                   sel_phys + (size_t)unit * k_max, sel_count + unit, sl);
}

// Selection of units scored by several workgroups: one workgroup per
// (sequence, KV head) loads the unit's keys and block-table row into LDS.
constexpr int kSelectThreads = 256;

__global__ __launch_bounds__(kSelectThreads) void k_select(
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens, int Hkv, int P,
    int MP, int NP, int k_max, const int32_t* __restrict__ k_per_seq, SelectPolicy pol,
    const uint32_t* __restrict__ keys, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ sel_phys) {
  constexpr int NT = kSelectThreads;
  extern __shared__ uint32_t smem[];
  uint32_t* s_phys = smem;      // [MP]
  uint32_t* s_key = smem + MP;  // [MP]
  __shared__ SelectLds<NT> sl;
  const int unit = blockIdx.x, b = unit / Hkv;
  if (threadIdx.x == 0) {
    sl.red[0] = -1;
    sl.red[1] = 0;
  }
  stage_row<8>(reinterpret_cast<const int32_t*>(keys + (size_t)unit * MP), MP, NT, s_key,
               [](int32_t k) { return (uint32_t)k; });
  stage_row<8>(bt + (size_t)b * MP, MP, NT, s_phys,
               [NP](int32_t e) { return (uint32_t)clampi(e, 0, NP - 1); });
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int kb = clampi(k_per_seq ? k_per_seq[b] : k_max, 1, k_max);
  const int n = (len + P - 1) / P;
  __syncthreads();
  const int keff = min(kb, n), f = min(pol.n_sink, keff), r = min(pol.n_recent, keff - f);
  select_block<NT>(s_key, s_phys, n, keff, f, r, k_max, sel + (size_t)unit * k_max,
                   sel_phys + (size_t)unit * k_max, sel_count + unit, sl);
}

// ---------------------------------------------------------------------------
// K2: split decode over the selected-token stream, merge by the last tile
// ---------------------------------------------------------------------------
//
// The selected pages of a (sequence, KV head), in sel order, form a stream of
// cnt*P token slots; workgroup `split` covers stream slots
// [split*TILE, (split+1)*TILE).  Each lane owns C channels of one token row
// (L = D/C lanes per row, 64/L rows per wave per load); all J loads of K and V
// are issued before any arithmetic, so a workgroup keeps TILE*2*D*bytes in
// flight.  Masked slots (past the length, or past the last selected page) are
// never loaded: their V stays zero and their logit -inf, so a NaN in an
// unused slot cannot reach the output.
//
// Each tile leaves (max, sum, acc[D]) per query head in `partials`, and
// k_merge, launched after the tiles, combines a unit's tiles into `out`.  A
// unit with one tile writes `out` directly; a unit with nothing selected gets
// zero rows from its first tile slot.

// Token span of one split when a row's t_all selected tokens are spread over
// at most S workgroups of at least `minspan` tokens each (a multiple of 16,
// so every split starts on a 16-token step).  Depends on the row's data only,
// never on the launch width.
__device__ __forceinline__ long step_span(long t_all, int S, int minspan) {
  const long se = min((long)S, max(1L, t_all / minspan));
  const long per = (t_all + se - 1) / se;
  return max(16L, (per + 15) & ~15L);
}

// K3: merge of the tiles' partial states of one (sequence, query head) per
// wave, for units with more than one tile.  Lane s holds tile s's (max,
// denominator); the weighted sums are read with all of a lane's loads in
// flight together.
template <int D>
__global__ __launch_bounds__(256) void k_merge(
    const float* __restrict__ partials, const int32_t* __restrict__ sel_count, int B,
    int Hq, int Hkv, int G, int log2P, int k_max, int S_max, int tile,
    float* __restrict__ out) {
  constexpr int PER = D / kWave, UNR = 8;
  const int gw = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (gw >= B * Hq) return;
  const int b = gw / Hq, hq = gw - b * Hq, h = hq / G;
  const int cnt = clampi(sel_count[(size_t)b * Hkv + h], 0, k_max);
  const int ns = (int)((((long)cnt << log2P) + tile - 1) / tile);
  if (ns <= 1) return;  // finished by the decode tile itself
  const float* base = partials + (size_t)gw * S_max * (D + 2);
  // global max and denominator, 64 tiles per pass
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += kWave) {
    const int s = s0 + lane;
    float m = s < ns ? base[(size_t)s * (D + 2) + D] : -INFINITY;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    M = fmaxf(M, m);
  }
  if (M == -INFINITY) {
#pragma unroll
    for (int i = 0; i < PER; ++i) out[(size_t)gw * D + lane + kWave * i] = 0.f;
    return;
  }
  float l = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kWave) {
    const int s = s0 + lane;
    float t = 0.f;
    if (s < ns) {
      const float* ps = base + (size_t)s * (D + 2);
      t = __builtin_amdgcn_exp2f(ps[D] - M) * ps[D + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
    l += t;
  }
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += UNR) {
    float w[UNR], v[UNR][PER];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int s = s0 + u;
      const float* ps = base + (size_t)min(s, ns - 1) * (D + 2);
      w[u] = s < ns ? ps[D] : -INFINITY;
#pragma unroll
      for (int i = 0; i < PER; ++i) v[u][i] = ps[lane + kWave * i];
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float wt = __builtin_amdgcn_exp2f(w[u] - M);  // -inf state -> 0
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(wt, v[u][i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
    out[(size_t)gw * D + lane + kWave * i] = l > 0.f ? acc[i] / l : 0.f;
}


// End of a split: wave w left its unnormalised sum in s_acc[w][g][0..D),
// its denominator in s_acc[w][g][D] and its running max in s_mw[w][g].  A
// unit covered by one split writes out directly; otherwise the split's
// (max, denominator, sum) goes to `partials` for k_merge (DEV: with
// device-scope stores, for a merge by another workgroup of the same launch).
template <int D, int G, int NT, int NW, bool DEV = false>
__device__ __forceinline__ void finish_split(float (*s_acc)[G][D + 1], float (*s_mw)[G],
                             float* __restrict__ partials, float* __restrict__ out, int b,
                             int h, int Hq, int S_max, int split, int ns) {
  for (int i = threadIdx.x; i < G * (D + 1); i += NT) {
    const int g = i / (D + 1), d = i - g * (D + 1);
    float M = s_mw[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_mw[w][g]);
    const float Ms = M == -INFINITY ? 0.f : M;
    float sum = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = __builtin_amdgcn_exp2f(s_mw[w][g] - Ms);
      sum = __builtin_fmaf(a, s_acc[w][g][d], sum);
      l = __builtin_fmaf(a, s_acc[w][g][D], l);
    }
    if (ns == 1) {
      if (d < D) out[((size_t)b * Hq + h * G + g) * D + d] = l > 0.f ? sum / l : 0.f;
    } else {
      float* dst = partials + (((size_t)b * Hq + h * G + g) * S_max + split) * (D + 2);
      if constexpr (DEV) {
        if (d < D) {
          st_dev(dst + d, sum);
        } else {
          st_dev(dst + D, M);
          st_dev(dst + D + 1, l);
        }
      } else if (d < D) {
        dst[d] = sum;
      } else {
        dst[D] = M;
        dst[D + 1] = l;
      }
    }
  }
}


// Fold the running softmax state of the partner slot (lane ^ MASK) into
// this lane's: both end with the combined state.
template <int MASK, int G, int C>
__device__ __forceinline__ void merge_slot_state(float (&m)[G], float (&l)[G],
                                                 float (&acc)[G][C]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mo = xor_lane<MASK>(m[g]);
    const float lo = xor_lane<MASK>(l[g]);
    const float M = fmaxf(m[g], mo);
    const float Ms = M == -INFINITY ? 0.f : M;
    const float a = __builtin_amdgcn_exp2f(m[g] - Ms), ao = __builtin_amdgcn_exp2f(mo - Ms);
    l[g] = __builtin_fmaf(l[g], a, lo * ao);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float xo = xor_lane<MASK>(acc[g][c]);
      acc[g][c] = __builtin_fmaf(acc[g][c], a, xo * ao);
    }
    m[g] = M;
  }
}

// Selected-token stream of one (sequence, KV head): entry e of the list
// (e0 + e in sel order) is logical page s_lp[e] at physical page s_ph[e];
// token ts of the stream is slot ts mod P of entry ts / P - e0, and exists
// when it lies before the sequence length.  npg entries are listed.
struct TokenList {
  const int* lp;
  const uint32_t* ph;
  int npg, e0, len, log2P, Hkv, h, D;
  // pool element offset of stream token ts, or -1 when it does not exist
  __device__ __forceinline__ long off(long ts) const {
    const int P = 1 << log2P;
    const int e = (int)(ts >> log2P) - e0;
    const int st = (int)(ts & (P - 1));
    const int ec = min(e, npg - 1);
    const int l = lp[ec];
    if (e >= npg || l < 0 || l * P + st >= len) return -1;
    return (long)((((size_t)ph[ec] * Hkv + h) * P + st) * D);
  }
  // slot 0 of the first entry: a token that exists (masked loads read it)
  __device__ __forceinline__ long safe() const {
    return (long)((((size_t)ph[0] * Hkv + h) << log2P) * D);
  }
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ long uniform64(long x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(x & 0xffffffffL));
  const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
  return ((long)hi << 32) | (unsigned)lo;
}

// The 16 stream tokens [tw, tw + 16) of one MFMA wave step (tw a multiple of
// 16, EB-byte KV elements) lie in one list entry when P >= 16 and in two consecutive
// entries when P == 8.  Wave-uniform: token t < split sits at k0/v0 + t*D
// elements and exists if t < lim0; token t >= split at k1/v1 + (t-split)*D,
// existing if t - split < lim1.  Slots that do not exist are still inside
// their page (or in a listed page), so reading them is in bounds.
struct StepMap {
  const char *k0, *k1, *v0, *v1;
  int split, lim0, lim1;
};

template <int EB>
__device__ __forceinline__ StepMap step_map(const TokenList& tl, const char* kb, const char* vb,
                                            long tw) {
  const int P = 1 << tl.log2P;
  const int e = uniform((int)(tw >> tl.log2P) - tl.e0);
  const int st0 = uniform((int)(tw & (P - 1)));
  StepMap m;
  m.split = min(16, P - st0);
  const int ec = clampi(e, 0, tl.npg - 1);
  const int l0 = uniform(tl.lp[ec]);
  const int p0 = uniform((int)tl.ph[ec]);
  m.lim0 = uniform(e < tl.npg && l0 >= 0 ? clampi(tl.len - (l0 * P + st0), 0, m.split) : 0);
  const size_t b0 = ((((size_t)p0 * tl.Hkv + tl.h) << tl.log2P) + st0) * tl.D * EB;
  m.k0 = kb + b0;
  m.v0 = vb + b0;
  m.lim1 = 0;
  m.k1 = m.k0;
  m.v1 = m.v0;
  if (m.split < 16) {
    const int ec1 = clampi(e + 1, 0, tl.npg - 1);
    const int l1 = uniform(tl.lp[ec1]);
    const int p1 = uniform((int)tl.ph[ec1]);
    m.lim1 = uniform(e + 1 < tl.npg && l1 >= 0 ? clampi(tl.len - l1 * P, 0, 16 - m.split) : 0);
    const size_t b1 = (((size_t)p1 * tl.Hkv + tl.h) << tl.log2P) * tl.D * EB;
    m.k1 = kb + b1;
    m.v1 = vb + b1;
  }
  return m;
}

// VALU decode of stream tokens [t0, t_end) by the NT threads of a
// workgroup, in tiles of TILE tokens.  Every lane slot keeps a running (max,
// sum, acc) over its tokens; tile t+1's K/V loads are issued before tile t is
// processed.  Ends with each wave's state in s_acc[wave] / s_mw[wave] (no
// barrier).
template <int DT, int D, int G, int NT>
struct ValuDecode {
  static constexpr int EB = KV<DT>::bytes, C = KV<DT>::vec, L = D / C;
  // loads in flight per lane and buffer: 16-wave workgroups hold half as many;
  // fp8 lanes load 8 bytes, so they hold twice as many tokens for the same
  // bytes in flight
  static constexpr int SPW = kWave / L, NW = NT / kWave, TPI = NW * SPW,
                       J = (NT >= 1024 ? 2 : 4) * (16 / (C * EB));
  static constexpr int TILE = J * TPI;
};

template <int DT, int D, int G, int NT, int GS = G, bool NTKV = false>
__device__ __forceinline__ void valu_decode_range(const float* __restrict__ qg0,
                                                  const char* __restrict__ kb,
                                                  const char* __restrict__ vb,
                                                  const TokenList& tl, long t0, long t_end,
                                                  float qscale, float (*s_acc)[GS][D + 1],
                                                  float (*s_mw)[GS], int g0 = 0) {
  using VD = ValuDecode<DT, D, G, NT>;
  constexpr int EB = VD::EB, C = VD::C, L = VD::L, SPW = VD::SPW, TPI = VD::TPI, J = VD::J;
  constexpr int TILE = VD::TILE;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int chunk = lane % L, slot = lane / L;
  float qs[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qg = qg0 + (size_t)g * D + chunk * C;
#pragma unroll
    for (int c = 0; c < C; c += 4) {
      const float4 x4 = *reinterpret_cast<const float4*>(qg + c);
      qs[g][c] = x4.x * qscale;
      qs[g][c + 1] = x4.y * qscale;
      qs[g][c + 2] = x4.z * qscale;
      qs[g][c + 3] = x4.w * qscale;
    }
  }
  const int ntiles = (int)((t_end - t0 + TILE - 1) / TILE);
  const long safe_off = tl.safe() + chunk * C;
  auto load_tile = [&](int it, uint4 (&kr)[J], uint4 (&vr)[J], bool (&ok)[J]) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const long ts = t0 + (long)it * TILE + j * TPI + wave * SPW + slot;
      const long o = tl.off(ts);
      ok[j] = o >= 0 && ts < t_end;  // the list may go on past this range
      const long off = ok[j] ? o + chunk * C : safe_off;
      if constexpr (C * EB == 16) {
        kr[j] = ld_kv<NTKV, uint4>(kb + off * EB);
        vr[j] = ld_kv<NTKV, uint4>(vb + off * EB);
      } else {
        const uint2 k2 = ld_kv<NTKV, uint2>(kb + off * EB), v2 = ld_kv<NTKV, uint2>(vb + off * EB);
        kr[j] = make_uint4(k2.x, k2.y, 0u, 0u);
        vr[j] = make_uint4(v2.x, v2.y, 0u, 0u);
      }
    }
  };
  float m_run[G], l_run[G], acc[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) acc[g][c] = 0.f;
  }
  auto process = [&](const uint4 (&kr)[J], const uint4 (&vr)[J], const bool (&ok)[J]) {
    float z[G][J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float kf[C];
      unpack<DT, C>(kr[j], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) a = __builtin_fmaf(qs[g][c], kf[c], a);
        a = group_sum<L>(a);
        z[g][j] = ok[j] ? a : -INFINITY;
      }
    }
    float ms[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float tm = z[g][0];
#pragma unroll
      for (int j = 1; j < J; ++j) tm = fmaxf(tm, z[g][j]);
      const float mn = fmaxf(m_run[g], tm);
      const float a = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[g] - mn);
      l_run[g] *= a;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[g][c] *= a;
      m_run[g] = mn;
      ms[g] = mn == -INFINITY ? 0.f : mn;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float vf[C];
      unpack<DT, C>(ok[j] ? vr[j] : make_uint4(0, 0, 0, 0), vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pz = __builtin_amdgcn_exp2f(z[g][j] - ms[g]);
        l_run[g] += pz;
#pragma unroll
        for (int c = 0; c < C; ++c) acc[g][c] = __builtin_fmaf(pz, vf[c], acc[g][c]);
      }
    }
  };
  {
    uint4 ka[J], va[J], kb2[J], vb2[J];
    bool oka[J], okb[J];
    if (ntiles > 0) load_tile(0, ka, va, oka);
    for (int it = 0; it < ntiles; it += 2) {
      if (it + 1 < ntiles) load_tile(it + 1, kb2, vb2, okb);
      process(ka, va, oka);
      if (it + 1 >= ntiles) break;
      if (it + 2 < ntiles) load_tile(it + 2, ka, va, oka);
      process(kb2, vb2, okb);
    }
  }
  // merge the wave's token slots, then hand each wave's state to LDS
  if constexpr (L <= 8) merge_slot_state<8, G, C>(m_run, l_run, acc);
  if constexpr (L <= 16) merge_slot_state<16, G, C>(m_run, l_run, acc);
  if constexpr (L <= 32) merge_slot_state<32, G, C>(m_run, l_run, acc);
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int c = 0; c < C; ++c) s_acc[wave][g0 + g][chunk * C + c] = acc[g][c];
      if (chunk == 0) {
        s_acc[wave][g0 + g][D] = l_run[g];
        s_mw[wave][g0 + g] = m_run[g];
      }
    }
  }
}

template <int DT, int D, int G, int NT, bool MF, int CH, bool NTKV = false>
__device__ __forceinline__ void decode_group(const float* __restrict__ qg0,
                                             const char* __restrict__ kb,
                                             const char* __restrict__ vb, const TokenList& tl,
                                             long t0, long t_end, float qscale,
                                             float (*s_acc)[G][D + 1], float (*s_mw)[G]);

// Stages sel entries [e0, e0 + ecap) of a unit (logical page, physical
// page) into LDS for a split decode workgroup.
__device__ __forceinline__ void stage_split_list(const int32_t* __restrict__ sel,
                                                 const int32_t* __restrict__ sel_phys,
                                                 const int32_t* __restrict__ bt, int unit,
                                                 int b, int MP, int NP, int k_max, int e0,
                                                 int ecap, int nt, int* s_lp, uint32_t* s_ph) {
  for (int i = threadIdx.x; i < ecap; i += nt) {
    const int lp = sel[(size_t)unit * k_max + e0 + i];
    const int ph = sel_phys ? sel_phys[(size_t)unit * k_max + e0 + i]
                            : bt[(size_t)b * MP + clampi(lp, 0, MP - 1)];
    s_lp[i] = lp;
    s_ph[i] = (uint32_t)clampi(ph, 0, NP - 1);
  }
}

// One workgroup per (sequence, KV head, split); a split is TPW consecutive
// tiles of the selected-token stream.  Slots and waves are merged once, at
// the end; a unit covered by one split writes `out`, others leave partial
// states for k_merge.
template <int DT, int D, int G, int NT>
__global__ __launch_bounds__(NT) void k_decode_split(
    const float* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ sel_count,
    int Hq, int Hkv, int log2P, int MP, int NP, int k_max, int S_max, int TPW,
    float qscale, float* __restrict__ partials, float* __restrict__ out) {
  using VD = ValuDecode<DT, D, G, NT>;
  constexpr int NW = VD::NW, TILE = VD::TILE;
  constexpr int MAXE = kMaxTilesPerSplit * TILE / 8;  // sel entries of a split (P >= 8)
  __shared__ int s_lp[MAXE];
  __shared__ uint32_t s_ph[MAXE];
  __shared__ float s_acc[NW][G][D + 1];
  __shared__ float s_mw[NW][G];

  const int unit = blockIdx.x / S_max, split = blockIdx.x - unit * S_max;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const long span = (long)TPW * TILE;
  const long t0 = (long)split * span;
  const int e0 = (int)(t0 >> log2P);                                  // < k_max by the grid
  const int ecap = (int)min(max(1L, span >> log2P), (long)(k_max - e0));  // <= MAXE
  stage_split_list(sel, sel_phys, bt, unit, b, MP, NP, k_max, e0, ecap, NT, s_lp, s_ph);
  const int cnt = clampi(sel_count[unit], 0, k_max);
  const int len = clampi(seq_lens[b], 0, MP << log2P);
  const long t_all = (long)cnt << log2P;
  const long t_end = min(t_all, t0 + span);
  if (t0 >= t_end) {  // whole workgroup: no work
    if (cnt == 0 && split == 0)
      for (int i = threadIdx.x; i < G * D; i += NT) out[((size_t)b * Hq + h * G) * D + i] = 0.f;
    return;
  }
  __syncthreads();
  const TokenList tl{s_lp, s_ph, min(cnt - e0, ecap), e0, len, log2P, Hkv, h, D};
  decode_group<DT, D, G, NT, false, 1, true>(q + ((size_t)b * Hq + h * G) * D,
                                  reinterpret_cast<const char*>(k_pool),
                                  reinterpret_cast<const char*>(v_pool), tl, t0, t_end, qscale,
                                  s_acc, s_mw);
  __syncthreads();
  finish_split<D, G, NT, NW>(s_acc, s_mw, partials, out, b, h, Hq, S_max, split,
                             (int)((t_all + span - 1) / span));
}

// ---------------------------------------------------------------------------
// K2 for grouped-query heads (G = 4, 8) on 16-bit or fp8 KV: both
// contractions on MFMA, 16 tokens per wave step (fp8 widened to bf16)
// ---------------------------------------------------------------------------
//
// Both fp32 operands that meet a 16-bit KV operand (q, and the
// probabilities p) are split into hi + lo 16-bit parts, so the products keep
// ~16 more mantissa bits than one 16-bit operand would.  A group has G <= 8
// heads, so the two parts share one MFMA: hi in fragment rows/columns
// 0 .. G-1, lo in 8 .. 8+G-1.
//   logits^T[token][c] = K[token][:] . Q[c][:]   (v_mfma_f32_16x16x32)
//     A = K rows straight from the pool (lane: token n16, 8 channels at
//     32*ch + 8*c4), B = Q^T with column c = q_hi of head c (c < 8) or q_lo
//     of head c - 8.  Lane (n16, c4) ends with the partial logits of column
//     n16 for tokens 4*c4 + r; one DPP row rotation by 8 adds the partner
//     column, so lanes n16 and n16 ^ 8 both hold the logits of head n16 & 7.
//   out[c][d] += sum_token P[c][token] * V[token][d]   (v_mfma_f32_16x16x16)
//     A = P with row c = p_hi of head c (c < 8) or p_lo of head c - 8: the
//     lane's 4 probabilities, split, are exactly its A fragment.  Rows c and
//     c + 8 are added once, at the end.  B needs 4 consecutive tokens of one
//     channel per lane: lane
//     (n16, c4) loads the W = D/16 channels W*n16 .. W*n16 + W-1 of tokens
//     4*c4 .. 4*c4 + 3 (four 8- or 16-byte loads, whole rows per wave load)
//     and v_perm packs channel W*n16 + e of the four tokens into the B
//     fragment of output tile e, so V never goes through LDS.  Output tile e
//     holds channel W*n16 + e in column n16.
// Rows of the 16-row fragments beyond G carry zero queries and are never
// stored.  Masked tokens read a valid token's row and are then dropped: their
// logits are -inf, so p = 0 multiplies finite values.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
struct Mma;
template <>
struct Mma<DT_BF16> {
  typedef bf16x8_t vec8;
  typedef s16x4_t vec4;  // bf16 bits
  typedef __bf16 elem;
  static constexpr float kPScale = 1.f;
  static __device__ __forceinline__ f32x4_t mma32(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mma16(vec4 a, vec4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ short bits(elem x) { return __builtin_bit_cast(short, x); }
};
template <>
struct Mma<DT_F16> {
  typedef f16x8_t vec8;
  typedef f16x4_t vec4;
  typedef _Float16 elem;
  // probabilities are scaled by 2^12 before the f16 split so that their low
  // parts stay normal numbers; the sum is scaled back exactly afterwards
  static constexpr float kPScale = 4096.f;
  static __device__ __forceinline__ f32x4_t mma32(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mma16(vec4 a, vec4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ short bits(elem x) { return __builtin_bit_cast(short, x); }
};

// Two OCP fp8 values (bytes 0, 1 of w, or 2, 3 with HI; E4M3 for DT_F8,
// E5M2 for DT_F8E5) as a bf16 pair, low half first, in one conversion
// (scale 1).  Exact: every E4M3 and every E5M2 value is a bf16 value.
template <int DT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  if constexpr (DT == DT_F8)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w, 1.0f, HI));
}

template <int DT>
__device__ __forceinline__ void split_hi_lo(float x, typename Mma<DT>::elem& hi,
                                            typename Mma<DT>::elem& lo) {
  using E = typename Mma<DT>::elem;
  hi = (E)x;
  lo = (E)(x - (float)hi);
}

template <int DT, int D>
struct MfmaDecode {
  static constexpr int WS = 16;         // tokens per wave step
  static constexpr int NCH = D / 32;    // 32-channel chunks (logits: K, output: V)
  static constexpr int NDT = D / 16;    // 16-channel tiles of the output
};

// MFMA decode of stream tokens [t0, t_end) by the NW waves of a workgroup.
// 16-token steps are dealt round-robin to the waves; a wave takes its steps
// CH at a time (a chunk): the chunk's K and V loads are all issued together,
// one chunk ahead of the arithmetic, and the running softmax state is
// rescaled once per chunk.  Page lookups are wave-uniform (scalar), each
// lane keeps one K and one V address per step.  Ends with each wave's state
// in s_acc[wave] / s_mw[wave] (no barrier).  fp8 KV is widened to bf16 in
// registers (exactly) and takes the bf16 instructions.
template <int DT, int D, int G, int NW, int CH, int GS = G, bool NTKV = false>
__device__ __forceinline__ void mfma_decode_range(const float* __restrict__ qg0,
                                                  const char* __restrict__ kb,
                                                  const char* __restrict__ vb,
                                                  const TokenList& tl, long t0, long t_end,
                                                  float qscale, float (*s_acc)[GS][D + 1],
                                                  float (*s_mw)[GS], int g0 = 0) {
  constexpr int MDT = is_fp8(DT) ? DT_BF16 : DT;  // MFMA operand type
  constexpr int EB = KV<DT>::bytes;
  using M = Mma<MDT>;
  using MD = MfmaDecode<DT, D>;
  using vec8 = typename M::vec8;
  using vec4 = typename M::vec4;
  using E = typename M::elem;
  constexpr int WS = MD::WS, NCH = MD::NCH, NDT = MD::NDT;
  constexpr int VW = D / 32;  // bf16/f16 dwords of V per token and lane (W = 2*VW channels)
  constexpr int VR = VW * EB / 2;  // dwords of V as loaded
  using KRaw = std::conditional_t<EB == 1, uint2, uint4>;  // 8 channels of K as loaded
  static_assert(G <= 8, "hi and lo parts of the group share one 16-row fragment");
  const int lane = threadIdx.x & (kWave - 1), wave = uniform(threadIdx.x / kWave);
  const int n16 = lane & 15, c4 = lane >> 4;
  const int head = n16 & 7;           // head of fragment row / column n16
  const bool has = head < G, lo_part = n16 >= 8;
  t0 = uniform64(t0);
  t_end = uniform64(t_end);
  // B operand of the logits: column n16, 8 channels per chunk
  vec8 qf[NCH];
  {
    const float* qg = qg0 + (size_t)(has ? head : 0) * D + 8 * c4;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const float4 a = *reinterpret_cast<const float4*>(qg + 32 * ch);
      const float4 c = *reinterpret_cast<const float4*>(qg + 32 * ch + 4);
      const float xs[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        E hi, lo;
        split_hi_lo<MDT>(has ? xs[j] : 0.f, hi, lo);
        qf[ch][j] = lo_part ? lo : hi;
      }
    }
  }
  const int nsteps = uniform((int)((t_end - t0 + WS - 1) / WS));
  const int mine = nsteps > wave ? (nsteps - wave + NW - 1) / NW : 0;
  // per-lane byte offsets: K row n16 (8 channels at 8*c4), V rows 4*c4 .. +3
  // (W channels at W*n16)
  const int k_lane = (n16 * D + 8 * c4) * EB;
  const int v_lane = 2 * VW * n16 * EB;
  struct Chunk {
    KRaw k[CH][NCH];           // token n16, channels 32*ch + 8*c4 .. + 7
    uint32_t v[CH][4][VR];     // token 4*c4 + j, channels W*n16 .. W*n16 + W-1
    int vlim[CH];              // tokens 4*c4 + j with j < vlim exist
  };
  // the chunk of the wave's steps i0 .. i0+CH-1 (clamped to its last step,
  // so the loads need no branch)
  auto load = [&](int i0, Chunk& c) {
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const int i = min(i0 + cc, mine - 1);
      const StepMap sm = step_map<EB>(tl, kb, vb, t0 + (long)(wave + i * NW) * WS);
      const char* kp = n16 < sm.split ? sm.k0 + k_lane : sm.k1 + (k_lane - sm.split * D * EB);
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
        c.k[cc][ch] = ld_kv<NTKV, KRaw>(kp + 32 * EB * ch);
      const bool first = 4 * c4 < sm.split;
      const char* vp = (first ? sm.v0 : sm.v1 - sm.split * D * EB) + 4 * c4 * D * EB + v_lane;
      c.vlim[cc] = i0 + cc < mine ? (first ? sm.lim0 - 4 * c4 : sm.lim1 - (4 * c4 - sm.split))
                                  : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const char* vj = vp + j * D * EB;
        if constexpr (VR == 1) {
          c.v[cc][j][0] = ld_kv<NTKV, uint32_t>(vj);
        } else if constexpr (VR == 2) {
          const uint2 x = ld_kv<NTKV, uint2>(vj);
          c.v[cc][j][0] = x.x;
          c.v[cc][j][1] = x.y;
        } else {
          const uint4 x = ld_kv<NTKV, uint4>(vj);
          c.v[cc][j][0] = x.x;
          c.v[cc][j][1] = x.y;
          c.v[cc][j][2] = x.z;
          c.v[cc][j][3] = x.w;
        }
      }
    }
  };
  float m_run = -INFINITY, l_run = 0.f;  // head n16 & 7
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int i0, const Chunk& c) {
    // logits of head n16 & 7 for tokens 4*c4 + r of each step, log2 units;
    // tokens that do not exist (or steps past the wave's last) get -inf
    float z[CH][4];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
#pragma unroll
      for (int r = 0; r < 4; ++r) z[cc][r] = -INFINITY;
      if (i0 + cc >= mine) continue;  // padding of the wave's last chunk
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        if constexpr (EB == 1) {
          const KRaw r = c.k[cc][ch];
          const uint4 kw = {fp8x2_to_bf16x2<DT, false>(r.x), fp8x2_to_bf16x2<DT, true>(r.x),
                            fp8x2_to_bf16x2<DT, false>(r.y), fp8x2_to_bf16x2<DT, true>(r.y)};
          acc = M::mma32(__builtin_bit_cast(vec8, kw), qf[ch], acc);
        } else {
          acc = M::mma32(__builtin_bit_cast(vec8, c.k[cc][ch]), qf[ch], acc);
        }
      }
      const int lim = has ? c.vlim[cc] : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float zr = acc[r] + dpp<kRowRor8>(acc[r]);  // hi + lo columns
        z[cc][r] = r < lim ? zr * qscale : -INFINITY;
      }
    }
    float tm = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < CH; ++cc)
      tm = fmaxf(tm, fmaxf(fmaxf(z[cc][0], z[cc][1]), fmaxf(z[cc][2], z[cc][3])));
    tm = fmaxf(tm, xor16(tm));
    tm = fmaxf(tm, xor32(tm));
    const float mn = fmaxf(m_run, tm);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
    const float ms = mn == -INFINITY ? 0.f : mn;
    m_run = mn;
    l_run *= alpha;
    // output row 4*c4 + r belongs to head (4*c4 + r) & 7, whose factor sits
    // in lane (4*c4 + r) & 7
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a0 = r < G ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r))
                             : 1.f;
      const float a1 = 4 + r < G
                           ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 + r))
                           : 1.f;
      const float ar = (c4 & 1) ? a1 : a0;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt][r] *= ar;
    }
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      if (i0 + cc >= mine) break;
      vec4 pa;  // row n16: p_hi (n16 < 8) or p_lo (n16 >= 8) of head n16 & 7
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pz = __builtin_amdgcn_exp2f(z[cc][r] - ms);
        l_run += pz;
        E hi, lo;
        split_hi_lo<MDT>(pz * M::kPScale, hi, lo);
        if constexpr (MDT == DT_BF16) pa[r] = M::bits(lo_part ? lo : hi);
        else pa[r] = lo_part ? lo : hi;
      }
      // V of tokens that do not exist is zeroed (their slots may hold
      // anything; p = 0 alone would not silence a NaN)
      uint32_t w[4][VW];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int x = 0; x < VR; ++x) {
          const uint32_t raw = j < c.vlim[cc] ? c.v[cc][j][x] : 0u;
          if constexpr (EB == 1) {
            w[j][2 * x] = fp8x2_to_bf16x2<DT, false>(raw);
            w[j][2 * x + 1] = fp8x2_to_bf16x2<DT, true>(raw);
          } else {
            w[j][x] = raw;
          }
        }
#pragma unroll
      for (int e = 0; e < NDT; ++e) {
        // channel W*n16 + e of tokens 4*c4 + 0..3: the low (e even) or high
        // half of dword e/2 of each token
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint2 frag = {__builtin_amdgcn_perm(w[1][e >> 1], w[0][e >> 1], sel),
                            __builtin_amdgcn_perm(w[3][e >> 1], w[2][e >> 1], sel)};
        o[e] = M::mma16(pa, __builtin_bit_cast(vec4, frag), o[e]);
      }
    }
  };
  if (mine > CH) {
    Chunk ca, cb;
    load(0, ca);
    for (int i = 0; i < mine; i += 2 * CH) {
      load(i + CH, cb);
      compute(i, ca);
      if (i + CH >= mine) break;
      load(i + 2 * CH, ca);
      compute(i + CH, cb);
    }
  } else if (mine > 0) {  // one chunk: nothing to prefetch
    Chunk ca;
    load(0, ca);
    compute(0, ca);
  }
  l_run += xor16(l_run);
  l_run += xor32(l_run);
  // out fragment: row 4*c4 + r, channel W*n16 + e; rows g (c4 < 2) and
  // g + 8 (c4 + 2) hold the hi and lo parts of head g
#pragma unroll
  for (int e = 0; e < NDT; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sum = o[e][r] + xor32(o[e][r]);
      const int g = 4 * c4 + r;
      if (g < G) s_acc[wave][g0 + g][NDT * n16 + e] = sum * (1.f / M::kPScale);
    }
  if (lane < G) {
    s_acc[wave][g0 + lane][D] = l_run;
    s_mw[wave][g0 + lane] = m_run;
  }
}

// Decode of all G heads of a group into the waves' combine areas s_acc /
// s_mw [NW][G]: on MFMA (MF) or the VALU.  A lane holds the queries and sums
// of at most 8 heads (4 with fp32 KV, whose lanes hold 4 channels of twice
// the bytes), so larger groups run as several passes over the same tokens,
// the later ones mostly reading them from L2.
template <int DT, int D, int G, int NT, bool MF, int CH, bool NTKV>
__device__ __forceinline__ void decode_group(const float* __restrict__ qg0,
                                             const char* __restrict__ kb,
                                             const char* __restrict__ vb, const TokenList& tl,
                                             long t0, long t_end, float qscale,
                                             float (*s_acc)[G][D + 1], float (*s_mw)[G]) {
  constexpr int GMAX = DT == DT_F32 ? 4 : 8;
  constexpr int GP = G > GMAX ? GMAX : G;  // heads per pass
#pragma unroll
  for (int g0 = 0; g0 < G; g0 += GP) {
    if constexpr (MF)
      mfma_decode_range<DT, D, GP, NT / kWave, CH, G, NTKV>(qg0 + (size_t)g0 * D, kb, vb, tl,
                                                            t0, t_end, qscale, s_acc, s_mw, g0);
    else
      valu_decode_range<DT, D, GP, NT, G, NTKV>(qg0 + (size_t)g0 * D, kb, vb, tl, t0, t_end,
                                                qscale, s_acc, s_mw, g0);
  }
}

// Split decode workgroup for grouped-query heads on 16-bit or fp8 KV: four
// waves, splits of TPW steps of 64 tokens.
template <int DT, int D, int G>
__global__ __launch_bounds__(256, D == 128 ? 2 : 3) void k_decode_mfma(
    const float* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ sel_count,
    int Hq, int Hkv, int log2P, int MP, int NP, int k_max, int S_max, int TPW,
    float qscale, float* __restrict__ partials, float* __restrict__ out) {
  constexpr int NT = 256, NW = NT / kWave, TILE = NW * MfmaDecode<DT, D>::WS;
  constexpr int MAXE = kMaxTilesPerSplit * TILE / 8;
  __shared__ int s_lp[MAXE];
  __shared__ uint32_t s_ph[MAXE];
  __shared__ float s_acc[NW][G][D + 1];
  __shared__ float s_mw[NW][G];

  const int unit = blockIdx.x / S_max, split = blockIdx.x - unit * S_max;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const long span = (long)TPW * TILE;
  const long t0 = (long)split * span;
  const int e0 = (int)(t0 >> log2P);
  const int ecap = (int)min(max(1L, span >> log2P), (long)(k_max - e0));
  stage_split_list(sel, sel_phys, bt, unit, b, MP, NP, k_max, e0, ecap, NT, s_lp, s_ph);
  const int cnt = clampi(sel_count[unit], 0, k_max);
  const int len = clampi(seq_lens[b], 0, MP << log2P);
  const long t_all = (long)cnt << log2P;
  const long t_end = min(t_all, t0 + span);
  if (t0 >= t_end) {  // whole workgroup: no work
    if (cnt == 0 && split == 0)
      for (int i = threadIdx.x; i < G * D; i += NT) out[((size_t)b * Hq + h * G) * D + i] = 0.f;
    return;
  }
  __syncthreads();
  const TokenList tl{s_lp, s_ph, min(cnt - e0, ecap), e0, len, log2P, Hkv, h, D};
  decode_group<DT, D, G, NT, true, 1, true>(q + ((size_t)b * Hq + h * G) * D,
                                  reinterpret_cast<const char*>(k_pool),
                                  reinterpret_cast<const char*>(v_pool), tl, t0, t_end, qscale,
                                  s_acc, s_mw);
  __syncthreads();
  finish_split<D, G, NT, NW>(s_acc, s_mw, partials, out, b, h, Hq, S_max, split,
                             (int)((t_all + span - 1) / span));
}

// ---------------------------------------------------------------------------
// The whole decode step of one (sequence, KV head) in one workgroup
// ---------------------------------------------------------------------------
//
// [append the new token] -> score every page -> block-wide top-K -> decode
// the kept pages' tokens with all waves -> combine the waves -> out.  The
// selection stays in LDS between the phases (it is also written to sel /
// sel_count for the caller).  A row spread over S workgroups exchanges page
// keys once (each scores 1/S of the pages) and the last of them to finish
// merges the S partial states, so the step stays one launch.

template <int DT, int D, int G>
constexpr bool step_uses_mfma() { return DT != DT_F32 && (G == 4 || G == 8 || G == 16); }

// Dynamic LDS of k_step: block-table row and keys (MP words each, rounded to
// 4), then the decode staging area.
template <int DT, int D, int G, int NT>
constexpr size_t step_decode_lds() {
  constexpr int NW = NT / kWave;
  return (size_t)NW * G * (D + 1) * 4;
}

// 4-wave workgroups are meant to run two to a CU: at most 256 registers each
// (fp32 groups of eight heads excepted: their VALU decode needs more)
template <int DT, int D, int G, int NT>
constexpr int step_min_blocks() { return NT == 256 && (G <= 4 || DT != DT_F32) ? 2 : 1; }

// Split rows: the S workgroups of a row exchange page keys through the row's
// slots in the workspace, then meet once more through a counter of finished
// decodes (word 0 of the row's line of counters).  Slots and counter are zero
// between calls.  Everything they exchange (page keys, partial states, the
// counter) is written and read with device-scope atomic stores and loads,
// which are coherent across the chip on their own: no cache-wide writeback or
// invalidation is needed.
constexpr int kSyncDone = 0;

// Reads the keys of the pages that the row's other splits score (batch b of
// PB pages belongs to split b mod S) from the row's slots into s_key, up to
// `polls` times, until none of them reads 0 (not yet written).  A slot is
// written once per call, with a key that is never 0, so a non-zero read is
// that split's key of this call.  Returns 1 when every key has arrived, 0
// when the reads ran out first (then s_key holds no usable foreign keys).
// Uniform over the workgroup.  A thread reads its slots four at a time, so
// that their round trips overlap.
template <int NT, int PB>
__device__ __forceinline__ int poll_row_keys(const uint32_t* xrow, uint32_t* s_key, int n, int S,
                                             int split, int polls) {
  constexpr int R = 4;
  for (int it = 0; it < polls; ++it) {
    int missing = 0;
    for (int p0 = threadIdx.x; p0 < n; p0 += R * NT) {
      uint32_t v[R];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int p = p0 + j * NT;
        v[j] = p < n && (p / PB) % S != split ? ld_dev(xrow + p) : 1u;
      }
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int p = p0 + j * NT;
        if (p < n && (p / PB) % S != split) {
          s_key[p] = v[j];
          missing |= v[j] == 0u;
        }
      }
    }
    if (!__syncthreads_or(missing)) return 1;
    __builtin_amdgcn_s_sleep(2);
  }
  return 0;
}

// Called by one thread after every thread of the workgroup stored its share
// of the partial state and waited for it (and for its key stores): 1 for the
// last of the row's S splits to finish, else 0.  Never waits.  The last
// split resets the counter; every split has left the key exchange by then,
// so it also clears the row's key slots, and the row's prefix of the
// workspace is all zero again when the kernel ends.
__device__ __forceinline__ int row_finish(uint32_t* c, int S) {
  const uint32_t o =
      __hip_atomic_fetch_add(c + kSyncDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (o != (uint32_t)S - 1) return 0;
  st_dev(c + kSyncDone, 0u);
  return 1;
}

// Merge of a split row's S partial states (one with max -inf when its split
// had no tokens) into out, splits in increasing order whichever workgroup
// runs it, so the result does not depend on which split finished last.
template <int D, int G, int NT>
__device__ __forceinline__ void merge_row(const float* __restrict__ partials, int S,
                                          float* __restrict__ orow, size_t hq0) {
  for (int i = threadIdx.x; i < G * D; i += NT) {
    const int g = i / D, d = i - g * D;
    const float* base = partials + (hq0 + g) * S * (D + 2);
    float m[kStepMaxSplits], l[kStepMaxSplits], a[kStepMaxSplits];
#pragma unroll
    for (int s = 0; s < kStepMaxSplits; ++s) {
      if (s >= S) break;
      const float* ps = base + (size_t)s * (D + 2);
      m[s] = ld_dev(ps + D);
      l[s] = ld_dev(ps + D + 1);
      a[s] = ld_dev(ps + d);
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kStepMaxSplits; ++s) {
      if (s >= S) break;
      M = fmaxf(M, m[s]);
    }
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int s = 0; s < kStepMaxSplits; ++s) {
      if (s >= S) break;
      if (m[s] == -INFINITY) continue;  // an empty slot: its sums were never written
      const float w = __builtin_amdgcn_exp2f(m[s] - M);
      L = __builtin_fmaf(w, l[s], L);
      acc = __builtin_fmaf(w, a[s], acc);
    }
    orow[i] = L > 0.f ? acc / L : 0.f;
  }
}

template <int DT, int D, int G, int NT>
// The arguments a workgroup needs first (its row, the block-table row, the
// length and budget) lead the list: the first 14 dwords of the arguments
// arrive in scalar registers with the wave (kernarg preloading), the rest
// through the usual loads, which complete while the row is staged.
__global__ __launch_bounds__(NT, (step_min_blocks<DT, D, G, NT>())) void k_step(
    const int32_t* __restrict__ order, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq, int S,
    int units, int Hkv, int MP, int log2P, int NP, const float* __restrict__ q,
    const void* __restrict__ k_new, const void* __restrict__ v_new, void* __restrict__ k_pool,
    void* __restrict__ v_pool, void* __restrict__ meta, int Hq, int k_max, SelectPolicy pol,
    float qscale, int polls, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
    float* __restrict__ scores_out, uint32_t* __restrict__ sync, uint32_t* __restrict__ xkeys,
    float* __restrict__ partials, float* __restrict__ out) {
  constexpr int NW = NT / kWave;
  constexpr bool MF = step_uses_mfma<DT, D, G>();
  constexpr int PB = ScoreCfg<DT, D, G, NT>::PB;
  extern __shared__ __align__(16) uint32_t smem[];
  const int MPa = (MP + 3) & ~3;
  uint32_t* s_phys = smem;
  uint32_t* s_key = smem + MPa;
  char* dec = reinterpret_cast<char*>(smem + 2 * MPa);
  __shared__ SelectLds<NT> sl;
  __shared__ float s_mw[NW][G];
  __shared__ int s_flag;

  // workgroup -> (row, split): the S splits of a row share blockIdx mod 8,
  // i.e. one XCD and its L2, which then serves the keys they exchange.  A
  // scheduled launch (S = 1) takes its row from the caller's order instead;
  // entries outside [0, units) leave their workgroup idle.
  TSV_STAMP(0);
  int unit, split;
  if (order != nullptr) {
    unit = order[blockIdx.x];
    split = 0;
    if ((unsigned)unit >= (unsigned)units) return;
  } else {
    const int grp = blockIdx.x / (8 * S), within = blockIdx.x - grp * 8 * S;
    split = within >> 3;
    unit = grp * 8 + (within & 7);
    if (unit >= units) return;
  }
  TSV_STAMP_VALUE(6, ((unsigned long long)unit << 32) | (unsigned)split);
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x;
  const int P = 1 << log2P;
  uint32_t* rsync = sync + (size_t)unit * kSyncWordsPerRow;  // used only when S > 1
  if (tid == 0) {
    sl.red[0] = -1;
    sl.red[1] = 0;
  }
  const int32_t* bt_row = bt + (size_t)b * MP;
  stage_row<4>(bt_row, MP, NT, s_phys, [NP](int32_t e) { return (uint32_t)clampi(e, 0, NP - 1); });
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int kb = clampi(k_per_seq ? k_per_seq[b] : k_max, 1, k_max);
  const int n = (len + P - 1) >> log2P;
  if (k_new != nullptr && len >= 1 && tid < D) {
    // the new token is slot (len-1) mod P of page (len-1)/P; its box widens
    // (or opens, on slot 0) before any box of the row is read.  Every split
    // of a row writes the same values, so each sees the appended token
    // whatever the order in which the splits run.
    const int pos = len - 1, p = pos >> log2P, slot = pos & (P - 1);
    const size_t phys = (size_t)clampi(bt_row[p], 0, NP - 1);
    const size_t i = ((size_t)b * Hkv + h) * D + tid;
    const uint32_t kb = load_elem<DT>(k_new, i), vb = load_elem<DT>(v_new, i);
    const size_t dst = ((phys * Hkv + h) * P + slot) * D + tid;
    store_elem<DT>(k_pool, dst, kb);
    store_elem<DT>(v_pool, dst, vb);
    const size_t m = ((phys * Hkv + h) * 2) * D + tid;
    if (slot == 0) {
      store_elem<DT>(meta, m, kb);
      store_elem<DT>(meta, m + D, kb);
    } else {
      const float k = elem_to_f32<DT>(kb);
      if (k < elem_to_f32<DT>(load_elem<DT>(meta, m))) store_elem<DT>(meta, m, kb);
      if (k > elem_to_f32<DT>(load_elem<DT>(meta, m + D))) store_elem<DT>(meta, m + D, kb);
    }
  }
  __syncthreads();  // block-table row staged; the appended token visible to the workgroup
  TSV_STAMP(1);
  // Scoring.  A split row's S workgroups score every S-th batch of pages
  // each and exchange the keys through the row's slots; a split whose wait
  // times out scores the remaining batches itself (bit-identical keys).
  const int nbatch = (n + PB - 1) / PB;
  const bool xchg = S > 1 && nbatch > 1;  // the same for every split of the row
  bool share = xchg;
  uint32_t* xrow = xkeys + (size_t)unit * MP;
  for (int bstart = share ? split : 0, bstride = share ? S : 1;;) {
    if (pol.group_sum)  // uniform branch: one copy of the scoring loop per aggregation
      score_pages<DT, D, G, NT, true>(q, meta, s_phys, b, h, Hq, Hkv, n, bstart, bstride, s_key);
    else
      score_pages<DT, D, G, NT, false>(q, meta, s_phys, b, h, Hq, Hkv, n, bstart, bstride, s_key);
    if (!share) break;
    __syncthreads();
    // publish this split's keys; each slot tells its readers by itself
    // whether it has been written (a published key is never 0: the one NaN
    // key that is becomes 1, here and in this split's own copy, so that every
    // split of the row ranks the same keys), so nothing waits for these
    // stores here
    for (int bi = split; bi < nbatch; bi += S)
      for (int i = tid; i < PB; i += NT) {
        const int p = bi * PB + i;
        if (p < n) {
          const uint32_t k = max(s_key[p], 1u);
          s_key[p] = k;
          st_dev(xrow + p, k);
        }
      }
    if (poll_row_keys<NT, PB>(xrow, s_key, n, S, split, polls)) break;
    __syncthreads();  // no thread still reads s_key for the stores above
    share = false;    // timed out: score every batch here
    bstart = 0;
    bstride = 1;
  }
  __syncthreads();
  TSV_STAMP(2);
  // The rest of the row (select, decode, finish) is its critical path, while
  // a workgroup beside it on the CU may still be scoring, bound by vector ALU
  // throughput: this row's waves take instruction-issue priority from here.
  __builtin_amdgcn_s_setprio(2);
  if (scores_out && split == 0) {  // uniform over the workgroup
    float* srow_out = scores_out + (size_t)unit * MP;
    for (int p = tid; p < n; p += NT) srow_out[p] = key_to_score(s_key[p]);
    // the selection below overwrites s_key with page indices
    __syncthreads();
  }
  const int keff = min(kb, n), f = min(pol.n_sink, keff), r = min(pol.n_recent, keff - f);
  // the selection stays in LDS; it is written out at the end, so that no
  // barrier before the decode waits for those stores
  const int cnt =
      n <= kWaveSelectPages
          ? select_wave<NT>(s_key, s_phys, n, keff, f, r, k_max, sl)
          : select_block<NT>(s_key, s_phys, n, keff, f, r, k_max, nullptr, nullptr, nullptr, sl);
  TSV_STAMP(3);
  int32_t* srow = sel + (size_t)unit * k_max;
  const size_t hq0 = (size_t)b * Hq + h * G;
  float* orow = out + hq0 * D;
  // this split's share of the selected-token stream (none when cnt == 0)
  const long t_all = (long)cnt << log2P;
  const long span = S > 1 ? step_span(t_all, S, kStepMinSpanSteps * 16 * NW) : t_all;
  const long t0 = (long)split * span, t_end = min(t_all, t0 + span);
  if (t0 < t_end) {
    const TokenList tl{reinterpret_cast<const int*>(s_key), s_phys, cnt, 0, len, log2P, Hkv, h, D};
    const float* qg0 = q + hq0 * D;
    const char* kbp = reinterpret_cast<const char*>(k_pool);
    const char* vbp = reinterpret_cast<const char*>(v_pool);
    typedef float AccRow[G][D + 1];
    AccRow* s_acc = reinterpret_cast<AccRow*>(dec);
    // chunks of two 16-token steps: a split's waves often hold only two steps,
    // and longer chunks unroll into more code that every workgroup fetches once
    if constexpr (MF)
      decode_group<DT, D, G, NT, true, 2>(qg0, kbp, vbp, tl, t0, t_end, qscale, s_acc, s_mw);
    else
      decode_group<DT, D, G, NT, false, 2>(qg0, kbp, vbp, tl, t0, t_end, qscale, s_acc, s_mw);
    __syncthreads();
    TSV_STAMP(4);
    finish_split<D, G, NT, NW, true>(s_acc, s_mw, partials, out, b, h, Hq, S, split, S);
  } else if (S == 1) {  // no tokens at all
    for (int i = tid; i < G * D; i += NT) orow[i] = 0.f;
  } else {  // a split without tokens leaves an empty state (max -inf)
    for (int g = tid; g < G; g += NT) {
      float* dst = partials + ((hq0 + g) * S + split) * (D + 2);
      st_dev(dst + D, -INFINITY);
      st_dev(dst + D + 1, 0.f);
    }
  }
  if (split == 0) {
    for (int i = tid; i < k_max; i += NT) srow[i] = i < cnt ? (int32_t)s_key[i] : -1;
    if (tid == 0) sel_count[unit] = cnt;
  }
  if (S == 1) {
    TSV_STAMP(5);
    return;
  }
  // the last split of the row to get here clears the row's key slots (every
  // split has read them and its own key stores have landed) and merges the S
  // partial states
  stores_done();
  __syncthreads();
  if (tid == 0) s_flag = row_finish(rsync, S);
  __syncthreads();
  if (!s_flag) {
    TSV_STAMP(5);
    return;
  }
  if (xchg)
    for (int p = tid; p < n; p += NT) st_dev(xrow + p, 0u);
  merge_row<D, G, NT>(partials, S, orow, hq0);
  TSV_STAMP(5);
}

}  // namespace
}  // namespace tsv
