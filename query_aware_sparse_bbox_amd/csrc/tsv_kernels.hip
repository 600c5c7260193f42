// gfx950 (CDNA4) kernels for query-aware page selection with sparse paged
// decode.  Method: TinyServe, "Query-Aware Cache Selection for Efficient LLM
// Serving" (abstract; method details, key design): per-page bounding boxes of
// the keys, a query-to-box score, the highest-scoring pages kept, masked
// attention over those pages only.
//
// Kernels, in the order a decode step runs them:
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
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "tsv_launch.h"

namespace tsv {
namespace {

constexpr int kWave = 64;
constexpr int kMaxTilesPerSplit = 8;  // decode tiles one workgroup streams

template <int DT>
struct KV {
  static constexpr int bytes = DT == DT_F32 ? 4 : 2;
  static constexpr int per16 = 16 / bytes;  // elements in one 16-byte load
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Widen one 16-byte load of KV-dtype elements to fp32 (exact).
template <int DT>
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
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

template <int DT>
__device__ __forceinline__ uint32_t load_elem(const void* base, size_t i) {
  if constexpr (DT == DT_F32) return reinterpret_cast<const uint32_t*>(base)[i];
  else return reinterpret_cast<const uint16_t*>(base)[i];
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, size_t i, uint32_t bits) {
  if constexpr (DT == DT_F32) reinterpret_cast<uint32_t*>(base)[i] = bits;
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
  if constexpr (L >= 32) x = x + __shfl_xor(x, 16);
  if constexpr (L >= 64) x = x + __shfl_xor(x, 32);
  return x;
}

// Combine lanes that differ only in the bits >= log2(L) (the other slots of
// the wave).  Requires L >= 8.
template <int L, class Op>
__device__ __forceinline__ float across_slots(float x, Op op) {
  static_assert(L >= 8, "slot reduction assumes at least 8 lanes per slot");
  if constexpr (L <= 8) x = op(x, dpp<kRowRor8>(x));
  if constexpr (L <= 16) x = op(x, __shfl_xor(x, 16));
  if constexpr (L <= 32) x = op(x, __shfl_xor(x, 32));
  return x;
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
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
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
  static constexpr int EB = KV<DT>::bytes, C = KV<DT>::per16, L = D / C;
  static constexpr int PPW = kWave / L;  // pages per wave per load
  static constexpr int U = G >= 4 ? 1 : 4;  // rows per lane per batch
  static constexpr int NT = NTH, NW = NT / kWave;
  static constexpr int PB = NW * PPW * U;  // pages per batch
};

// Lanes below this one that have their bit set in `mask`.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Top-K of one unit, run by a single wave: the first f pages always, then
// the R = keff - f largest keys among pages [f, n) (equal keys: lower page
// first), found by an 8-bit-digit radix search over an LDS histogram.  Keys
// are visited as rows of 64 pages (lane l takes page j*64 + l); KC rows at a
// time are read into registers with all reads in flight before the first
// histogram update, so a pass costs one LDS round trip per KC rows.  Output
// slots come from per-row ballots (pages ascend row by row, lane by lane),
// so no scan sits in the loops.  Writes the chosen pages in ascending order,
// -1 padding to k_max, their physical pages and the count.
constexpr int kSelectRows = 8;

__device__ __forceinline__ void select_wave(const uint32_t* s_key, const uint32_t* s_phys, int n, int keff,
                            int f, int k_max, int32_t* __restrict__ srow,
                            int32_t* __restrict__ prow, int32_t* __restrict__ count,
                            int* s_hist) {
  constexpr int KC = kSelectRows;
  const int lane = threadIdx.x & (kWave - 1);
  const int rows = (n + kWave - 1) / kWave;
  const int R = keff - f, ncand = n - f;
  const bool take_all = R >= ncand, radix = R > 0 && R < ncand;
  const int nl = max(n - 1, 0);
  uint32_t tau = 0;
  int need = 0;
  if (radix) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = R;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s_hist[lane + kWave * j] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      for (int c0 = 0; c0 < rows; c0 += KC) {
        uint32_t kk[KC];
#pragma unroll
        for (int r = 0; r < KC; ++r) kk[r] = s_key[min((c0 + r) * kWave + lane, nl)];
#pragma unroll
        for (int r = 0; r < KC; ++r) {
          const int p = (c0 + r) * kWave + lane;
          if (p < n && p >= f && (kk[r] & pmask) == prefix)
            atomicAdd(&s_hist[(kk[r] >> shift) & 255], 1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      __builtin_amdgcn_wave_barrier();
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[255 - 4 * lane - j];
        sum += c[j];
      }
      int before = wave_incl_scan(sum, lane) - sum;  // keys in higher digits
      int found = -1, rem = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < remaining && before + c[j] >= remaining) {
          found = 255 - 4 * lane - j;
          rem = remaining - before;
        }
        before += c[j];
      }
      const int src = __ffsll((unsigned long long)__ballot(found >= 0)) - 1;
      const int dgt = __shfl(found, src);
      remaining = __shfl(rem, src);
      prefix |= (uint32_t)dgt << shift;
      pmask |= 0xFFu << shift;
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      __builtin_amdgcn_wave_barrier();
    }
    tau = prefix;
    need = remaining;  // keys equal to tau to take, lowest pages first
  }
  int eq_seen = 0, base = 0;
  for (int c0 = 0; c0 < rows; c0 += KC) {
    uint32_t kk[KC], ph[KC];
#pragma unroll
    for (int r = 0; r < KC; ++r) {
      const int pc = min((c0 + r) * kWave + lane, nl);
      kk[r] = s_key[pc];
      ph[r] = s_phys[pc];
    }
#pragma unroll
    for (int r = 0; r < KC; ++r) {
      const int p = (c0 + r) * kWave + lane;
      const bool cand = p < n && p >= f;
      const bool eq = radix && cand && kk[r] == tau;
      const unsigned long long eqm = __ballot(eq);
      const bool ch = (p < n && p < f) ||
                      (cand && (radix ? (kk[r] > tau ||
                                         (eq && eq_seen + lanes_below(eqm) < need))
                                      : take_all));
      const unsigned long long chm = __ballot(ch);
      const int pos = base + lanes_below(chm);
      if (ch && pos < k_max) {  // the count never exceeds min(K_b, n_b); kept in bounds
        srow[pos] = p;
        prow[pos] = (int32_t)ph[r];
      }
      eq_seen += __popcll(eqm);
      base += __popcll(chm);
    }
  }
  const int total = min(base, k_max);
  for (int i = total + lane; i < k_max; i += kWave) {
    srow[i] = -1;
    prow[i] = 0;
  }
  if (lane == 0) *count = total;
}

// One workgroup per (unit, split): scores batches split, split + NS, ...
// of the unit's pages.  With NS == 1 the keys stay in LDS and wave 0 selects
// at the end; otherwise the keys go to the workspace for k_select.
template <int G>
constexpr int score_min_waves() { return G == 4 ? 4 : 1; }

template <int DT, int D, int G, int NTH>
__global__ __launch_bounds__(NTH, score_min_waves<G>()) void k_score_select(
    const float* __restrict__ q, const void* __restrict__ meta,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    int Hq, int Hkv, int P, int MP, int NP, int NS, int k_max,
    const int32_t* __restrict__ k_per_seq, int n_sink,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
    float* __restrict__ scores_out, uint32_t* __restrict__ keys,
    int32_t* __restrict__ sel_phys) {
  using Cfg = ScoreCfg<DT, D, G, NTH>;
  constexpr int EB = Cfg::EB, C = Cfg::C, L = Cfg::L, PPW = Cfg::PPW, U = Cfg::U;
  constexpr int NT = Cfg::NT, NW = Cfg::NW, PB = Cfg::PB;
  extern __shared__ uint32_t smem[];
  uint32_t* s_phys = smem;       // [MP] physical page of every logical page
  uint32_t* s_key = smem + MP;   // [MP] order keys (NS == 1)
  __shared__ int s_hist[256];

  const int unit = blockIdx.x / NS, split = blockIdx.x - unit * NS;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // the whole block-table row (MP entries, all allocated) is staged without
  // waiting for the length, so both loads share one memory latency
  const int32_t* bt_row = bt + (size_t)b * MP;
  stage_row<4>(bt_row, MP, NT, s_phys, [NP](int32_t e) { return (uint32_t)clampi(e, 0, NP - 1); });
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int n = (len + P - 1) / P;
  const int nbatch = (n + PB - 1) / PB;
  if (split > 0 && split >= nbatch) return;  // whole workgroup: no pages

  const int chunk = lane % L, slot = lane / L;
  float qp[G][C], qn[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qg = q + ((size_t)b * Hq + h * G + g) * D + chunk * C;
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
  __syncthreads();

  const char* mb = reinterpret_cast<const char*>(meta);
  // masked lanes read a valid row (page n-1) and drop it: no branches around
  // the loads, so the compiler's load counters track both buffers exactly
  auto load_batch = [&](int bi, uint4 (&mn)[U], uint4 (&mx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = min(bi * PB + u * (NW * PPW) + wave * PPW + slot, n - 1);
      const size_t row = ((size_t)s_phys[p] * Hkv + h) * 2 * D + chunk * C;
      mn[u] = ld16(mb + row * EB);
      mx[u] = ld16(mb + (row + D) * EB);
    }
  };
  auto score_batch = [&](int bi, const uint4 (&rmn)[U], const uint4 (&rmx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = bi * PB + u * (NW * PPW) + wave * PPW + slot;
      float mn[C], mx[C];
      unpack<DT>(rmn[u], mn);
      unpack<DT>(rmx[u], mx);
      float best = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float t[C];
#pragma unroll
        for (int cc = 0; cc < C; ++cc)
          t[cc] = __builtin_fmaf(qn[g][cc], mn[cc], qp[g][cc] * mx[cc]);
        const float sc = group_sum<L>(tree_sum<C>(t));
        best = g == 0 ? sc : fmaxf(best, sc);
      }
      best = best == 0.f ? 0.f : best;  // -0 -> +0
      if (p < n && chunk == 0) s_key[p] = order_key(best);
    }
  };
  uint4 amn[U], amx[U], bmn[U], bmx[U];
  int bi = split;
  if (bi < nbatch) load_batch(bi, amn, amx);
  while (bi < nbatch) {
    const int nx = bi + NS;
    if (nx < nbatch) load_batch(nx, bmn, bmx);
    score_batch(bi, amn, amx);
    if (nx >= nbatch) break;
    const int nx2 = nx + NS;
    if (nx2 < nbatch) load_batch(nx2, amn, amx);
    score_batch(nx, bmn, bmx);
    bi = nx2;
  }
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
  if (NS > 1 || wave != 0) return;
  int kb = k_per_seq ? k_per_seq[b] : k_max;
  kb = clampi(kb, 1, k_max);
  const int keff = min(kb, n), f = min(n_sink, keff);
  select_wave(s_key, s_phys, n, keff, f, k_max, sel + (size_t)unit * k_max,
              sel_phys + (size_t)unit * k_max, sel_count + unit, s_hist);
}

// Selection of units scored by several workgroups: one wave per (sequence,
// KV head) loads the unit's keys and block-table row into LDS.
__global__ __launch_bounds__(64) void k_select(
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens, int Hkv, int P,
    int MP, int NP, int k_max, const int32_t* __restrict__ k_per_seq, int n_sink,
    const uint32_t* __restrict__ keys, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ sel_phys) {
  extern __shared__ uint32_t smem[];
  uint32_t* s_phys = smem;      // [MP]
  uint32_t* s_key = smem + MP;  // [MP]
  __shared__ int s_hist[256];
  const int unit = blockIdx.x, b = unit / Hkv;
  stage_row<16>(reinterpret_cast<const int32_t*>(keys + (size_t)unit * MP), MP, kWave, s_key,
                [](int32_t k) { return (uint32_t)k; });
  stage_row<16>(bt + (size_t)b * MP, MP, kWave, s_phys,
                [NP](int32_t e) { return (uint32_t)clampi(e, 0, NP - 1); });
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int n = (len + P - 1) / P;
  __syncthreads();
  int kb = k_per_seq ? k_per_seq[b] : k_max;
  kb = clampi(kb, 1, k_max);
  const int keff = min(kb, n), f = min(n_sink, keff);
  select_wave(s_key, s_phys, n, keff, f, k_max, sel + (size_t)unit * k_max,
              sel_phys + (size_t)unit * k_max, sel_count + unit, s_hist);
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
// Each tile leaves (max, sum, acc[D]) per query head in `partials`; the last
// tile of a unit to finish (arrival counter) merges them into `out`.  A unit
// with one tile writes `out` directly; a unit with nothing selected gets zero
// rows from its first tile slot.

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
// (max, denominator, sum) goes to `partials` for k_merge.
template <int D, int G, int NT, int NW>
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
      if (d < D) {
        dst[d] = sum;
      } else {
        dst[D] = M;
        dst[D + 1] = l;
      }
    }
  }
}

// Lanes `lane` and `lane ^ MASK` (MASK = 8, 16, 32: other token slots).
template <int MASK>
__device__ __forceinline__ float xor_lane(float x) {
  if constexpr (MASK == 8) return dpp<kRowRor8>(x);
  else return __shfl_xor(x, MASK);
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

// One workgroup per (sequence, KV head, split); a split is TPW consecutive
// tiles of TILE stream tokens.  Every lane slot keeps a running (max, sum,
// acc) over its tokens; tile t+1's K/V loads are issued before tile t is
// processed.  Slots and waves are merged once, at the end.
template <int DT, int D, int G, int NT>
__global__ __launch_bounds__(NT) void k_decode_split(
    const float* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ sel_count,
    int Hq, int Hkv, int log2P, int MP, int NP, int k_max, int S_max, int TPW,
    float qscale, float* __restrict__ partials, float* __restrict__ out) {
  constexpr int EB = KV<DT>::bytes, C = KV<DT>::per16, L = D / C;
  constexpr int SPW = kWave / L, NW = NT / kWave, TPI = NW * SPW, J = 4;
  constexpr int TILE = J * TPI;
  constexpr int MAXE = kMaxTilesPerSplit * TILE / 8;  // sel entries of a split (P >= 8)
  __shared__ int s_lp[MAXE];
  __shared__ uint32_t s_ph[MAXE];
  __shared__ float s_acc[NW][G][D + 1];
  __shared__ float s_mw[NW][G];

  const int P = 1 << log2P;
  const int unit = blockIdx.x / S_max, split = blockIdx.x - unit * S_max;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const long span = (long)TPW * TILE;
  const long t0 = (long)split * span;
  const int e0 = (int)(t0 >> log2P);                                  // < k_max by the grid
  const int ecap = (int)min(max(1L, span >> log2P), (long)(k_max - e0));  // <= MAXE
  for (int i = tid; i < ecap; i += NT) {
    const int lp = sel[(size_t)unit * k_max + e0 + i];
    const int ph = sel_phys ? sel_phys[(size_t)unit * k_max + e0 + i]
                            : bt[(size_t)b * MP + clampi(lp, 0, MP - 1)];
    s_lp[i] = lp;
    s_ph[i] = (uint32_t)clampi(ph, 0, NP - 1);
  }
  const int cnt = clampi(sel_count[unit], 0, k_max);
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int chunk = lane % L, slot = lane / L;
  float qs[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qg = q + ((size_t)b * Hq + h * G + g) * D + chunk * C;
#pragma unroll
    for (int c = 0; c < C; c += 4) {
      const float4 x4 = *reinterpret_cast<const float4*>(qg + c);
      qs[g][c] = x4.x * qscale;
      qs[g][c + 1] = x4.y * qscale;
      qs[g][c + 2] = x4.z * qscale;
      qs[g][c + 3] = x4.w * qscale;
    }
  }
  const long t_all = (long)cnt << log2P;
  const long t_end = min(t_all, t0 + span);
  if (t0 >= t_end) {  // whole workgroup: no work
    if (cnt == 0 && split == 0)
      for (int i = tid; i < G * D; i += NT) out[((size_t)b * Hq + h * G) * D + i] = 0.f;
    return;
  }
  __syncthreads();
  const int npg = min(cnt - e0, ecap);
  const int ntiles = (int)((t_end - t0 + TILE - 1) / TILE);

  const char* kb = reinterpret_cast<const char*>(k_pool);
  const char* vb = reinterpret_cast<const char*>(v_pool);
  // masked slots read slot 0 of the first selected page (always a valid
  // token) and are dropped by `ok`: the loads need no branches
  const size_t safe_off = (((size_t)s_ph[0] * Hkv + h) * P) * D + chunk * C;
  auto load_tile = [&](int it, uint4 (&kr)[J], uint4 (&vr)[J], bool (&ok)[J]) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const long ts = t0 + (long)it * TILE + j * TPI + wave * SPW + slot;
      const int e = (int)(ts >> log2P) - e0;
      const int st = (int)(ts & (P - 1));
      const int ec = min(e, npg - 1);
      const int lp = s_lp[ec];
      ok[j] = e < npg && lp >= 0 && lp * P + st < len;
      const size_t off =
          ok[j] ? (((size_t)s_ph[ec] * Hkv + h) * P + st) * D + chunk * C : safe_off;
      kr[j] = ld16(kb + off * EB);
      vr[j] = ld16(vb + off * EB);
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
      unpack<DT>(kr[j], kf);
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
      unpack<DT>(ok[j] ? vr[j] : make_uint4(0, 0, 0, 0), vf);
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
    load_tile(0, ka, va, oka);
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
      for (int c = 0; c < C; ++c) s_acc[wave][g][chunk * C + c] = acc[g][c];
      if (chunk == 0) {
        s_acc[wave][g][D] = l_run[g];
        s_mw[wave][g] = m_run[g];
      }
    }
  }
  __syncthreads();
  finish_split<D, G, NT, NW>(s_acc, s_mw, partials, out, b, h, Hq, S_max, split,
                             (int)((t_all + span - 1) / span));
}

// ---------------------------------------------------------------------------
// K2 for grouped-query heads (G = 4, 8) on 16-bit KV: both contractions on
// MFMA, streamed 16 tokens per wave step
// ---------------------------------------------------------------------------
//
// A workgroup's four waves walk its split in steps of 64 tokens, 16 per wave,
// keeping a running (max, sum, out) per query head across steps.
//   logits^T[token][g] = K[token][:] . q[g][:]   (v_mfma_f32_16x16x32)
//     A = K rows straight from the pool (lane: token n16, 8 channels at
//     32*ch + 8*c4), B = q^T; q is split into hi + lo 16-bit parts so the
//     product keeps ~16 more mantissa bits than one 16-bit operand would.
//     Lane (n16, c4) ends with the logits of head g = n16 for tokens
//     4*c4 + r.
//   out[g][d] += sum_token p[g][token] * V[token][d]   (v_mfma_f32_16x16x16)
//     A = p (hi + lo parts): the lane's 4 probabilities are exactly its A
//     fragment; B = V read column-wise from the wave's 16 V rows staged in
//     LDS (rows padded by 16 bytes so the four lane groups hit disjoint
//     banks).
// Rows of the 16-row fragments beyond G carry zero queries and are never
// stored.  Masked tokens read a valid token's row and are then dropped: their
// V rows are zero in LDS and their logits -inf, so p = 0 multiplies a finite
// zero.
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

template <int DT>
__device__ __forceinline__ void split_hi_lo(float x, typename Mma<DT>::elem& hi,
                                            typename Mma<DT>::elem& lo) {
  using E = typename Mma<DT>::elem;
  hi = (E)x;
  lo = (E)(x - (float)hi);
}

template <int DT, int D, int G>
__global__ __launch_bounds__(256, 3) void k_decode_mfma(
    const float* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ sel_count,
    int Hq, int Hkv, int log2P, int MP, int NP, int k_max, int S_max, int TPW,
    float qscale, float* __restrict__ partials, float* __restrict__ out) {
  using M = Mma<DT>;
  using vec8 = typename M::vec8;
  using vec4 = typename M::vec4;
  using E = typename M::elem;
  constexpr int NT = 256, NW = NT / kWave, WS = 16, TILE = NW * WS;
  constexpr int NCH = D / 32;   // 32-channel chunks of the logit contraction
  constexpr int NDT = D / 16;   // 16-channel tiles of the output
  constexpr int ROW = D + 8;    // LDS row stride in 16-bit elements
  constexpr int LR = D / 8;     // lanes per V row (16 bytes each)
  constexpr int RPI = kWave / LR, NVL = WS / RPI;
  constexpr int MAXE = kMaxTilesPerSplit * TILE / 8;
  static_assert(G <= 16, "one 16-row fragment holds the query group");
  __shared__ int s_lp[MAXE];
  __shared__ uint32_t s_ph[MAXE];
  __shared__ __align__(16) uint16_t s_v[NW][WS][ROW];
  __shared__ float s_acc[NW][G][D + 1];
  __shared__ float s_mw[NW][G];

  const int P = 1 << log2P;
  const int unit = blockIdx.x / S_max, split = blockIdx.x - unit * S_max;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int n16 = lane & 15, c4 = lane >> 4;
  const long span = (long)TPW * TILE;
  const long t0 = (long)split * span;
  const int e0 = (int)(t0 >> log2P);
  const int ecap = (int)min(max(1L, span >> log2P), (long)(k_max - e0));
  for (int i = tid; i < ecap; i += NT) {
    const int lp = sel[(size_t)unit * k_max + e0 + i];
    const int ph = sel_phys ? sel_phys[(size_t)unit * k_max + e0 + i]
                            : bt[(size_t)b * MP + clampi(lp, 0, MP - 1)];
    s_lp[i] = lp;
    s_ph[i] = (uint32_t)clampi(ph, 0, NP - 1);
  }
  const int cnt = clampi(sel_count[unit], 0, k_max);
  const int len = clampi(seq_lens[b], 0, MP * P);
  // B operand of the logits: column g = n16, 8 channels per chunk
  vec8 qhi[NCH], qlo[NCH];
  {
    const bool has = n16 < G;
    const float* qg = q + ((size_t)b * Hq + h * G + (has ? n16 : 0)) * D + 8 * c4;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const float4 a = *reinterpret_cast<const float4*>(qg + 32 * ch);
      const float4 c = *reinterpret_cast<const float4*>(qg + 32 * ch + 4);
      const float xs[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        E hi, lo;
        split_hi_lo<DT>(has ? xs[j] : 0.f, hi, lo);
        qhi[ch][j] = hi;
        qlo[ch][j] = lo;
      }
    }
  }
  const long t_all = (long)cnt << log2P;
  const long t_end = min(t_all, t0 + span);
  if (t0 >= t_end) {  // whole workgroup: no work
    if (cnt == 0 && split == 0)
      for (int i = tid; i < G * D; i += NT) out[((size_t)b * Hq + h * G) * D + i] = 0.f;
    return;
  }
  __syncthreads();
  const int npg = min(cnt - e0, ecap);
  const int nsteps = (int)((t_end - t0 + TILE - 1) / TILE);
  // pool element offset of split-local token `t`, or -1 when masked
  auto token_off = [&](long t) -> long {
    const long ts = t0 + t;
    const int e = (int)(ts >> log2P) - e0;
    const int st = (int)(ts & (P - 1));
    const int ec = min(e, npg - 1);
    const int lp = s_lp[ec];
    if (e >= npg || lp < 0 || lp * P + st >= len) return -1;
    return (long)((((size_t)s_ph[ec] * Hkv + h) * P + st) * D);
  };
  // masked tokens read slot 0 of the first selected page (a valid token)
  const long safe_off = (long)((((size_t)s_ph[0] * Hkv + h) * P) * D);
  const char* kb = reinterpret_cast<const char*>(k_pool);
  const char* vb = reinterpret_cast<const char*>(v_pool);

  float m_run = -INFINITY, l_run = 0.f;  // head g = n16
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < nsteps; ++it) {
    const long tw = (long)it * TILE + wave * WS;  // the wave's first token
    const long koff = token_off(tw + n16);
    uint4 kr[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
      kr[ch] = ld16(kb + ((koff >= 0 ? koff : safe_off) + 32 * ch + 8 * c4) * 2);
    uint4 vr[NVL];
    bool vok[NVL];
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const long off = token_off(tw + u * RPI + lane / LR);
      vok[u] = off >= 0;
      vr[u] = ld16(vb + ((vok[u] ? off : safe_off) + (lane % LR) * 8) * 2);
    }
    // the previous step's reads of s_v are issued before these writes
    // (LDS requests of one wave complete in order)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < NVL; ++u)
      *reinterpret_cast<uint4*>(&s_v[wave][u * RPI + lane / LR][(lane % LR) * 8]) =
          vok[u] ? vr[u] : make_uint4(0, 0, 0, 0);
    // logits of head n16 for tokens 4*c4 + r, log2 units
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const vec8 a = __builtin_bit_cast(vec8, koff >= 0 ? kr[ch] : make_uint4(0, 0, 0, 0));
      acc = M::mma32(a, qhi[ch], acc);
      acc = M::mma32(a, qlo[ch], acc);
    }
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = token_off(tw + 4 * c4 + r) >= 0 ? acc[r] * qscale : -INFINITY;
    float tm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float mn = fmaxf(m_run, tm);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
    const float ms = mn == -INFINITY ? 0.f : mn;
    m_run = mn;
    l_run *= alpha;
    // output rows are heads 4*c4 + r: their factors come from lanes 4*c4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * c4 + r);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt][r] *= ar;
    }
    vec4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pz = __builtin_amdgcn_exp2f(z[r] - ms);
      l_run += pz;
      E hi, lo;
      split_hi_lo<DT>(pz * M::kPScale, hi, lo);
      if constexpr (DT == DT_BF16) {
        phi[r] = M::bits(hi);
        plo[r] = M::bits(lo);
      } else {
        phi[r] = hi;
        plo[r] = lo;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      s16x4_t vv;
#pragma unroll
      for (int j = 0; j < 4; ++j) vv[j] = (short)s_v[wave][4 * c4 + j][16 * dt + n16];
      const vec4 bv = __builtin_bit_cast(vec4, vv);
      o[dt] = M::mma16(phi, bv, o[dt]);
      o[dt] = M::mma16(plo, bv, o[dt]);
    }
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // out fragment: head 4*c4 + r, channel 16*dt + n16
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * c4 + r;
      if (g < G) s_acc[wave][g][16 * dt + n16] = o[dt][r] * (1.f / M::kPScale);
    }
  if (lane < G) {
    s_acc[wave][lane][D] = l_run;
    s_mw[wave][lane] = m_run;
  }
  __syncthreads();
  finish_split<D, G, NT, NW>(s_acc, s_mw, partials, out, b, h, Hq, S_max, split,
                             (int)((t_all + span - 1) / span));
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <int V>
using IC = std::integral_constant<int, V>;

template <class Fn>
hipError_t by_dtype(int dt, Fn&& fn) {
  switch (dt) {
    case DT_F32: return fn(IC<DT_F32>{});
    case DT_F16: return fn(IC<DT_F16>{});
    case DT_BF16: return fn(IC<DT_BF16>{});
  }
  return hipErrorInvalidValue;
}

template <class Fn>
hipError_t by_dt_d_g(const Dims& d, Fn&& fn) {
  return by_dtype(d.dt, [&](auto DT) -> hipError_t {
    auto byG = [&](auto HD) -> hipError_t {
      switch (d.G) {
        case 1: return fn(DT, HD, IC<1>{});
        case 2: return fn(DT, HD, IC<2>{});
        case 4: return fn(DT, HD, IC<4>{});
        case 8: return fn(DT, HD, IC<8>{});
      }
      return hipErrorInvalidValue;
    };
    switch (d.D) {
      case 64: return byG(IC<64>{});
      case 128: return byG(IC<128>{});
    }
    return hipErrorInvalidValue;
  });
}

constexpr int kDecodeThreads = 256;

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

size_t round_up(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Grouped-query heads on 16-bit KV take the MFMA decode (64-token steps);
// everything else the VALU decode.  Both stream TPW steps per workgroup.
bool use_mfma_decode(const Dims& d) {
  return d.dt != DT_F32 && (d.G == 4 || d.G == 8);
}

int decode_tile_tokens(const Dims& d) {
  if (use_mfma_decode(d)) return 64;
  const int bytes = d.dt == DT_F32 ? 4 : 2;
  const int C = 16 / bytes, L = d.D / C, SPW = kWave / L;
  return 4 * (kDecodeThreads / kWave) * SPW;
}

// Tiles per workgroup: enough workgroups to fill the chip several times
// over, each streaming as many tiles as that allows.
int decode_tiles_per_split(const Dims& d, int k_max) {
  const long tile = decode_tile_tokens(d);
  const long tiles_per_row = ((long)k_max * d.P + tile - 1) / tile;
  const long total = tiles_per_row * d.B * d.Hkv;
  return (int)std::max(1L, std::min((long)kMaxTilesPerSplit, total / 1024));
}

int decode_splits(const Dims& d, int k_max) {
  const long span = (long)decode_tile_tokens(d) * decode_tiles_per_split(d, k_max);
  return (int)(((long)k_max * d.P + span - 1) / span);
}

size_t workspace_layout(const Dims& d, int k_max, void* base, Workspace* ws) {
  const size_t units = (size_t)d.B * d.Hkv;
  const size_t o_keys = 0;
  const size_t o_phys = o_keys + round_up(units * d.MP * sizeof(uint32_t));
  const size_t o_part = o_phys + round_up(units * k_max * sizeof(int32_t));
  const size_t total = o_part + round_up((size_t)d.B * d.Hq * decode_splits(d, k_max) *
                                         partial_stride(d) * sizeof(float));
  if (base && ws) {
    char* c = static_cast<char*>(base);
    ws->keys = reinterpret_cast<uint32_t*>(c + o_keys);
    ws->sel_phys = reinterpret_cast<int32_t*>(c + o_phys);
    ws->partials = reinterpret_cast<float*>(c + o_part);
  }
  return total;
}

hipError_t launch_meta_build(const Dims& d, const void* k_pool, void* meta,
                             const int32_t* bt, const int32_t* seq_lens,
                             hipStream_t s) {
  return by_dtype(d.dt, [&](auto DT) -> hipError_t {
    constexpr int dt = decltype(DT)::value;
    dim3 grid((d.Hkv * d.D + 255) / 256, d.MP, d.B);
    hipLaunchKernelGGL(k_meta_build<dt>, grid, dim3(256), 0, s, k_pool, meta, bt,
                       seq_lens, d.Hkv, d.D, d.P, d.MP, d.NP);
    return hipGetLastError();
  });
}

hipError_t launch_meta_append(const Dims& d, const void* k_new,
                              const void* v_new, void* k_pool, void* v_pool,
                              void* meta, const int32_t* bt,
                              const int32_t* seq_lens, hipStream_t s) {
  return by_dtype(d.dt, [&](auto DT) -> hipError_t {
    constexpr int dt = decltype(DT)::value;
    const int total = d.B * d.Hkv * d.D;
    hipLaunchKernelGGL(k_meta_append<dt>, dim3((total + 255) / 256), dim3(256), 0, s,
                       k_new, v_new, k_pool, v_pool, meta, bt, seq_lens, d.B, d.Hkv,
                       d.D, d.P, d.MP, d.NP);
    return hipGetLastError();
  });
}

hipError_t launch_score_select(const Dims& d, const float* q, const void* meta,
                               const int32_t* bt, const int32_t* seq_lens,
                               int k_max, const int32_t* k_per_seq, int n_sink,
                               int32_t* sel, int32_t* sel_count, float* scores_out,
                               const Workspace& ws, hipStream_t s) {
  return by_dt_d_g(d, [&](auto DT, auto HD, auto GG) -> hipError_t {
    constexpr int dt = decltype(DT)::value, hd = decltype(HD)::value,
                  g = decltype(GG)::value;
    using Big = ScoreCfg<dt, hd, g, score_threads<g>()>;
    using Small = ScoreCfg<dt, hd, g, 256>;
    const bool small = d.MP <= Small::PB;
    const int PB = small ? Small::PB : Big::PB;
    const int units = d.B * d.Hkv;
    // enough rows to fill the chip: one streaming workgroup per row, top-K in
    // place; otherwise split every row over several workgroups
    const int batches = (d.MP + PB - 1) / PB;
#ifndef TSV_SCORE_ROWS_ONE_WG
#define TSV_SCORE_ROWS_ONE_WG 256
#endif
    const int NS = units >= TSV_SCORE_ROWS_ONE_WG
                       ? 1
                       : std::max(1, std::min(batches, (512 + units - 1) / units));
    const size_t shmem = 2 * sizeof(uint32_t) * (size_t)d.MP;
    if (small)
      hipLaunchKernelGGL((k_score_select<dt, hd, g, 256>), dim3(units * NS), dim3(256), shmem,
                         s, q, meta, bt, seq_lens, d.Hq, d.Hkv, d.P, d.MP, d.NP, NS, k_max,
                         k_per_seq, n_sink, sel, sel_count, scores_out, ws.keys, ws.sel_phys);
    else
      hipLaunchKernelGGL((k_score_select<dt, hd, g, Big::NT>), dim3(units * NS), dim3(Big::NT),
                         shmem, s, q, meta, bt, seq_lens, d.Hq, d.Hkv, d.P, d.MP, d.NP, NS,
                         k_max, k_per_seq, n_sink, sel, sel_count, scores_out, ws.keys,
                         ws.sel_phys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || NS == 1) return e;
    hipLaunchKernelGGL(k_select, dim3(units), dim3(kWave), 2 * sizeof(uint32_t) * (size_t)d.MP,
                       s, bt, seq_lens, d.Hkv, d.P, d.MP, d.NP, k_max, k_per_seq, n_sink,
                       ws.keys, sel, sel_count, ws.sel_phys);
    return hipGetLastError();
  });
}

hipError_t launch_decode(const Dims& d, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* bt,
                         const int32_t* seq_lens, const int32_t* sel,
                         const int32_t* sel_phys, const int32_t* sel_count,
                         int k_max, float scale, const Workspace& ws, float* out,
                         hipStream_t s) {
  const int S_max = decode_splits(d, k_max);
  const int TPW = decode_tiles_per_split(d, k_max);
  const int log2P = ilog2(d.P);
  const float qscale = scale * 1.44269504088896340736f;  // fold log2(e)
  const bool mfma = use_mfma_decode(d);
  hipError_t e = by_dt_d_g(d, [&](auto DT, auto HD, auto GG) -> hipError_t {
    constexpr int dt = decltype(DT)::value, hd = decltype(HD)::value,
                  g = decltype(GG)::value;
    if constexpr (dt != DT_F32 && (g == 4 || g == 8)) {
      if (mfma) {
        hipLaunchKernelGGL((k_decode_mfma<dt, hd, g>), dim3(d.B * d.Hkv * S_max), dim3(256),
                           0, s, q, k_pool, v_pool, bt, seq_lens, sel, sel_phys, sel_count,
                           d.Hq, d.Hkv, log2P, d.MP, d.NP, k_max, S_max, TPW, qscale,
                           ws.partials, out);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((k_decode_split<dt, hd, g, kDecodeThreads>),
                       dim3(d.B * d.Hkv * S_max), dim3(kDecodeThreads), 0, s, q,
                       k_pool, v_pool, bt, seq_lens, sel, sel_phys, sel_count, d.Hq,
                       d.Hkv, log2P, d.MP, d.NP, k_max, S_max, TPW, qscale, ws.partials,
                       out);
    return hipGetLastError();
  });
  if (e != hipSuccess || S_max == 1) return e;
  const int waves = d.B * d.Hq;
  const int tile = decode_tile_tokens(d) * TPW;
  if (d.D == 64)
    hipLaunchKernelGGL(k_merge<64>, dim3((waves + 3) / 4), dim3(256), 0, s, ws.partials,
                       sel_count, d.B, d.Hq, d.Hkv, d.G, log2P, k_max, S_max, tile, out);
  else
    hipLaunchKernelGGL(k_merge<128>, dim3((waves + 3) / 4), dim3(256), 0, s, ws.partials,
                       sel_count, d.B, d.Hq, d.Hkv, d.G, log2P, k_max, S_max, tile, out);
  return hipGetLastError();
}

}  // namespace tsv
