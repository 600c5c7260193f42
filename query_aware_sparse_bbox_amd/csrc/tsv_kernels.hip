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

#include <type_traits>

#include "tsv_launch.h"

namespace tsv {
namespace {

constexpr int kWave = 64;

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

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(x, o);
    if (lane >= o) x += t;
  }
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

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return min(max(x, lo), hi);
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
// K1: page scoring over (unit, page chunk) workgroups; the last chunk of a
// unit to finish selects that unit's top-K
// ---------------------------------------------------------------------------
//
// Lane layout of the scoring loop: a page's box row is 2*D*bytes; each lane
// loads 16 bytes of the min row and 16 bytes of the max row, i.e. C
// contiguous channels, so L = D/C lanes cover a page and one wave scores
// 64/L pages per load.  Consecutive lanes read consecutive 16-byte pieces of
// the same row, so every wave load is a run of whole 64/128-byte segments.
// A workgroup scores CH = waves * (64/L) * U pages with all U rows of every
// lane in flight at once.
//
// Term per channel: fma(qneg, mn, qpos*mx) with qpos = max(q,0),
// qneg = min(q,0).  One of qpos/qneg is zero, so the result is the single
// rounding of q*mx (q >= 0) or q*mn (q < 0), which is max(fl(q*mn), fl(q*mx))
// because mn <= mx and rounding is monotone; zero signs can differ, which
// only shows in an all-zero sum and -0 is stored as +0.
template <int DT, int D, int G>
struct ScoreCfg {
  static constexpr int EB = KV<DT>::bytes, C = KV<DT>::per16, L = D / C;
  static constexpr int PPW = kWave / L;  // pages per wave per load
  static constexpr int U = G >= 8 ? 1 : (G >= 4 ? 2 : 4);  // rows in flight per lane
  static constexpr int NT = 256, NW = NT / kWave;
  static constexpr int CH = NW * PPW * U;  // pages per workgroup
};

// Top-K of one unit from its n order keys in LDS: the first f pages always,
// then the R = keff - f largest keys among pages [f, n), equal keys to the
// lower page; writes the chosen pages ascending, -1 padding and the count.
template <int NT>
__device__ void select_from_keys(const uint32_t* s_key, int n, int keff, int f,
                                 int k_max, const int32_t* __restrict__ bt_row,
                                 int NP, int32_t* __restrict__ srow,
                                 int32_t* __restrict__ prow,
                                 int32_t* __restrict__ count, int* s_hist,
                                 int* s_tmp, int* s_bc) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int R = keff - f, ncand = n - f;
  const bool take_all = R >= ncand, radix = R > 0 && R < ncand;
  uint32_t tau = 0;
  int need = 0;
  if (radix) {
    // R-th largest key among the candidates, 8 bits at a time
    uint32_t prefix = 0, pmask = 0;
    int remaining = R;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += NT) s_hist[i] = 0;
      __syncthreads();
      for (int p = f + tid; p < n; p += NT) {
        const uint32_t k = s_key[p];
        if ((k & pmask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (wave == 0) {
        int c[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = s_hist[255 - 4 * lane - j];
          sum += c[j];
        }
        int before = wave_incl_scan(sum, lane) - sum;  // keys in higher digits
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (before < remaining && before + c[j] >= remaining) {
            s_bc[0] = 255 - 4 * lane - j;
            s_bc[1] = remaining - before;
          }
          before += c[j];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_bc[0] << shift;
      pmask |= 0xFFu << shift;
      remaining = s_bc[1];
    }
    tau = prefix;
    need = remaining;  // keys equal to tau to take, lowest pages first
  }

  // contiguous page range per thread keeps the output in ascending order
  const int m = (n + NT - 1) / NT;
  const int p0 = min(tid * m, n), p1 = min(p0 + m, n);
  int eq_local = 0;
  if (radix)
    for (int p = max(p0, f); p < p1; ++p) eq_local += s_key[p] == tau;
  int total;
  const int eq_rank0 = block_excl_scan<NW>(eq_local, s_tmp, &total);
  auto chosen = [&](int p, int& eq_rank) -> bool {
    if (p < f) return true;
    if (!radix) return take_all;
    const uint32_t k = s_key[p];
    if (k > tau) return true;
    if (k == tau) return eq_rank++ < need;
    return false;
  };
  int cnt_local = 0;
  {
    int r = eq_rank0;
    for (int p = p0; p < p1; ++p) cnt_local += chosen(p, r);
  }
  int pos = block_excl_scan<NW>(cnt_local, s_tmp, &total);
  {
    int r = eq_rank0;
    for (int p = p0; p < p1; ++p)
      if (chosen(p, r)) {
        if (pos < k_max) {  // total never exceeds min(K_b, n_b); kept in bounds regardless
          srow[pos] = p;
          prow[pos] = clampi(bt_row[p], 0, NP - 1);
        }
        ++pos;
      }
  }
  for (int i = total + tid; i < k_max; i += NT) {
    srow[i] = -1;
    prow[i] = 0;
  }
  if (tid == 0) *count = min(total, k_max);
}

template <int DT, int D, int G>
__global__ __launch_bounds__(256) void k_score_select(
    const float* __restrict__ q, const void* __restrict__ meta,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    int Hq, int Hkv, int P, int MP, int NP, int NC, int k_max,
    const int32_t* __restrict__ k_per_seq, int n_sink,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
    float* __restrict__ scores_out, uint32_t* __restrict__ keys,
    int32_t* __restrict__ sel_phys) {
  using Cfg = ScoreCfg<DT, D, G>;
  constexpr int EB = Cfg::EB, C = Cfg::C, L = Cfg::L, PPW = Cfg::PPW, U = Cfg::U;
  constexpr int NT = Cfg::NT, NW = Cfg::NW, CH = Cfg::CH, PPB = NW * PPW;
  __shared__ uint32_t s_key[CH];
  __shared__ uint32_t s_phys[CH];
  __shared__ int s_hist[256];
  __shared__ int s_tmp[NW];
  __shared__ int s_bc[2];

  const int unit = blockIdx.x / NC, c = blockIdx.x - unit * NC;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int n = (len + P - 1) / P;
  const int nchunks = (n + CH - 1) / CH;
  if (c >= max(nchunks, 1)) return;  // whole workgroup: no pages
  const int p_base = c * CH;
  const int npc = min(CH, n - p_base);  // <= 0 only for an empty sequence
  const int32_t* bt_row = bt + (size_t)b * MP;
  for (int i = tid; i < npc; i += NT) s_phys[i] = (uint32_t)clampi(bt_row[p_base + i], 0, NP - 1);

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
  uint4 rmn[U], rmx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int pl = u * PPB + wave * PPW + slot;
    rmn[u] = make_uint4(0, 0, 0, 0);
    rmx[u] = rmn[u];
    if (pl < npc) {
      const size_t row = ((size_t)s_phys[pl] * Hkv + h) * 2 * D + chunk * C;
      rmn[u] = ld16(mb + row * EB);
      rmx[u] = ld16(mb + (row + D) * EB);
    }
  }
  uint32_t* krow = keys + (size_t)unit * MP;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int pl = u * PPB + wave * PPW + slot;
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
    if (pl < npc && chunk == 0) {
      const uint32_t key = order_key(best);
      s_key[pl] = key;
      if (nchunks > 1) krow[p_base + pl] = key;
      if (scores_out) scores_out[(size_t)unit * MP + p_base + pl] = best;
    }
  }

  // a unit that fits one chunk selects right here; longer units are selected
  // by k_select once every chunk's keys are in memory
  if (nchunks > 1) return;
  __syncthreads();
  int kb = k_per_seq ? k_per_seq[b] : k_max;
  kb = clampi(kb, 1, k_max);
  const int keff = min(kb, n), f = min(n_sink, keff);
  select_from_keys<NT>(s_key, n, keff, f, k_max, bt_row, NP, sel + (size_t)unit * k_max,
                       sel_phys + (size_t)unit * k_max, sel_count + unit, s_hist, s_tmp,
                       s_bc);
}

// Selection of the units that span several score chunks: one workgroup per
// (sequence, KV head) loads the unit's keys into LDS and runs the same top-K.
template <int CH>
__global__ __launch_bounds__(256) void k_select(
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens, int Hkv,
    int P, int MP, int NP, int k_max, const int32_t* __restrict__ k_per_seq, int n_sink,
    const uint32_t* __restrict__ keys, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ sel_phys) {
  constexpr int NT = 256, NW = NT / kWave;
  extern __shared__ uint32_t s_key[];  // [MP]
  __shared__ int s_hist[256];
  __shared__ int s_tmp[NW];
  __shared__ int s_bc[2];
  const int unit = blockIdx.x, b = unit / Hkv;
  const int len = clampi(seq_lens[b], 0, MP * P);
  const int n = (len + P - 1) / P;
  if (n <= CH) return;  // selected by the score kernel
  const uint32_t* krow = keys + (size_t)unit * MP;
  for (int p = threadIdx.x; p < n; p += NT) s_key[p] = krow[p];
  __syncthreads();
  int kb = k_per_seq ? k_per_seq[b] : k_max;
  kb = clampi(kb, 1, k_max);
  const int keff = min(kb, n), f = min(n_sink, keff);
  select_from_keys<NT>(s_key, n, keff, f, k_max, bt + (size_t)b * MP, NP,
                       sel + (size_t)unit * k_max, sel_phys + (size_t)unit * k_max,
                       sel_count + unit, s_hist, s_tmp, s_bc);
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

// End of a decode tile: s_acc[w][g][0..D) holds each wave's unnormalised
// sum, s_acc[w][g][D] its softmax denominator, all relative to the tile max
// s_mt[g].  A unit with one tile writes out directly; otherwise the tile's
// (max, denominator, sum) goes to `partials` for k_merge.
template <int D, int G, int NT, int NW>
__device__ void finish_tile(float (*s_acc)[G][D + 1], const float* s_mt,
                            float* __restrict__ partials, float* __restrict__ out, int b,
                            int h, int Hq, int S_max, int split, int ns) {
  const int tid = threadIdx.x;
  if (ns == 1) {  // the only tile of the unit: finish here
    for (int i = tid; i < G * D; i += NT) {
      const int g = i / D, d = i - g * D;
      float sum = 0.f, l = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sum += s_acc[w][g][d];
        l += s_acc[w][g][D];
      }
      out[((size_t)b * Hq + h * G + g) * D + d] = l > 0.f ? sum / l : 0.f;
    }
    return;
  }
  for (int i = tid; i < G * (D + 1); i += NT) {
    const int g = i / (D + 1), d = i - g * (D + 1);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += s_acc[w][g][d];
    float* dst = partials + (((size_t)b * Hq + h * G + g) * S_max + split) * (D + 2);
    if (d < D) {
      dst[d] = sum;
    } else {
      dst[D] = s_mt[g];
      dst[D + 1] = sum;
    }
  }
}

template <int DT, int D, int G, int NT>
__global__ __launch_bounds__(NT) void k_decode_split(
    const float* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ sel_count,
    int Hq, int Hkv, int log2P, int MP, int NP, int k_max, int S_max,
    float qscale, float* __restrict__ partials, float* __restrict__ out) {
  constexpr int EB = KV<DT>::bytes, C = KV<DT>::per16, L = D / C;
  constexpr int SPW = kWave / L, NW = NT / kWave, TPI = NW * SPW, J = 4;
  constexpr int TILE = J * TPI;
  constexpr int MAXPG = TILE / 8;  // pages a tile can touch (P >= 8)
  __shared__ int s_lp[MAXPG];
  __shared__ uint32_t s_ph[MAXPG];
  __shared__ float s_red[NW][G];
  __shared__ float s_acc[NW][G][D + 1];
  __shared__ float s_mt[G];

  const int P = 1 << log2P;
  const int unit = blockIdx.x / S_max, split = blockIdx.x - unit * S_max;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const long t0 = (long)split * TILE;
  const int e0 = (int)(t0 >> log2P);                        // < k_max by the grid
  const int ecap = min(max(1, TILE >> log2P), k_max - e0);  // sel entries in reach
  // selection entries, count and query are independent loads: issue together
  if (tid < ecap) {
    const int lp = sel[(size_t)unit * k_max + e0 + tid];
    const int ph = sel_phys ? sel_phys[(size_t)unit * k_max + e0 + tid]
                            : bt[(size_t)b * MP + clampi(lp, 0, MP - 1)];
    s_lp[tid] = lp;
    s_ph[tid] = (uint32_t)clampi(ph, 0, NP - 1);
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
  if (t0 >= ((long)cnt << log2P)) {  // whole workgroup: no work
    if (cnt == 0 && split == 0)
      for (int i = tid; i < G * D; i += NT) out[((size_t)b * Hq + h * G) * D + i] = 0.f;
    return;
  }
  __syncthreads();
  const int npg = min(cnt - e0, ecap);

  const char* kb = reinterpret_cast<const char*>(k_pool);
  const char* vb = reinterpret_cast<const char*>(v_pool);
  uint4 kr[J], vr[J];
  bool ok[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const long ts = t0 + j * TPI + wave * SPW + slot;
    const int e = (int)(ts >> log2P) - e0;
    const int st = (int)(ts & (P - 1));
    kr[j] = make_uint4(0, 0, 0, 0);
    vr[j] = kr[j];
    ok[j] = false;
    if (e < npg) {
      const int lp = s_lp[e];
      if (lp >= 0 && lp * P + st < len) {
        ok[j] = true;
        const size_t off = (((size_t)s_ph[e] * Hkv + h) * P + st) * D + chunk * C;
        kr[j] = ld16(kb + off * EB);
        vr[j] = ld16(vb + off * EB);
      }
    }
  }

  // logits (log2 domain), tile max
  float z[G][J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float kf[C];
    unpack<DT>(kr[j], kf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) acc = __builtin_fmaf(qs[g][c], kf[c], acc);
      acc = group_sum<L>(acc);
      z[g][j] = ok[j] ? acc : -INFINITY;
    }
  }
  auto fmax_op = [](float a, float c) { return fmaxf(a, c); };
  auto add_op = [](float a, float c) { return a + c; };
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = z[g][0];
#pragma unroll
    for (int j = 1; j < J; ++j) m = fmaxf(m, z[g][j]);
    m = across_slots<L>(m, fmax_op);
    if (lane == 0) s_red[wave][g] = m;
  }
  __syncthreads();
  float mt[G], ms[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = s_red[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, s_red[w][g]);
    mt[g] = m;
    ms[g] = m == -INFINITY ? 0.f : m;
  }

  float acc[G][C], ls[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    ls[g] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) acc[g][c] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float vf[C];
    unpack<DT>(vr[j], vf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pz = __builtin_amdgcn_exp2f(z[g][j] - ms[g]);
      ls[g] += pz;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[g][c] = __builtin_fmaf(pz, vf[c], acc[g][c]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    ls[g] = across_slots<L>(ls[g], add_op);
#pragma unroll
    for (int c = 0; c < C; ++c) acc[g][c] = across_slots<L>(acc[g][c], add_op);
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int c = 0; c < C; ++c) s_acc[wave][g][chunk * C + c] = acc[g][c];
      if (chunk == 0) s_acc[wave][g][D] = ls[g];
    }
  }
  if (tid == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) s_mt[g] = mt[g];
  }
  __syncthreads();
  finish_tile<D, G, NT, NW>(s_acc, s_mt, partials, out, b, h, Hq, S_max, split,
                            (int)((((long)cnt << log2P) + TILE - 1) / TILE));
}

// ---------------------------------------------------------------------------
// K2 for grouped-query heads (G = 4, 8) on 16-bit KV: both contractions on
// MFMA (v_mfma_f32_16x16x32_{bf16,f16})
// ---------------------------------------------------------------------------
//
// Per wave, 32 stream tokens as two 16-row tiles.
//   logits^T[token][g] = K[token][:] . q[g][:]
//     A = K rows straight from the pool (lane: token n16, 8 channels at
//     32*ch + 8*c4), B = q^T; q is split into hi + lo 16-bit parts so the
//     product keeps ~16 more mantissa bits than one 16-bit operand would.
//     Lane (n16, c4) ends with the logits of head g = n16 for tokens
//     4*c4 + r of each tile.
//   out[g][d] += sum_token p[g][token] * V[token][d]
//     A = p (hi + lo parts): the lane's own 8 probabilities are exactly the
//     A fragment when the 32 contraction slots are ordered
//     (tile0 rows 4c4..4c4+3, tile1 rows 4c4..4c4+3); B = V in the same slot
//     order, read column-wise from the wave's V rows staged in LDS (rows
//     padded by 16 bytes so the four lane groups hit disjoint banks).
// Rows of the 16-row fragments beyond G carry zero queries and are never
// stored.  Masked tokens are never loaded: their V rows are zero in LDS and
// their logits -inf, so p = 0 multiplies a finite zero.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
struct Mma;
template <>
struct Mma<DT_BF16> {
  typedef bf16x8_t vec;
  typedef __bf16 elem;
  static constexpr float kPScale = 1.f;
  static __device__ __forceinline__ f32x4_t mma(vec a, vec b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mma<DT_F16> {
  typedef f16x8_t vec;
  typedef _Float16 elem;
  // probabilities are scaled by 2^12 before the f16 split so that their low
  // parts stay normal numbers; the sum is scaled back exactly afterwards
  static constexpr float kPScale = 4096.f;
  static __device__ __forceinline__ f32x4_t mma(vec a, vec b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <int DT>
__device__ __forceinline__ void split_hi_lo(float x, typename Mma<DT>::elem& hi,
                                            typename Mma<DT>::elem& lo) {
  using E = typename Mma<DT>::elem;
  hi = (E)x;
  lo = (E)(x - (float)hi);
}

template <int DT, int D, int G>
__global__ __launch_bounds__(256) void k_decode_mfma(
    const float* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ sel_count,
    int Hq, int Hkv, int log2P, int MP, int NP, int k_max, int S_max,
    float qscale, float* __restrict__ partials, float* __restrict__ out) {
  using M = Mma<DT>;
  using vec = typename M::vec;
  constexpr int NT = 256, NW = NT / kWave, WT = 32, TILE = NW * WT;
  constexpr int NCH = D / 32;   // 32-channel chunks of the logit contraction
  constexpr int NDT = D / 16;   // 16-channel tiles of the output
  constexpr int ROW = D + 8;    // LDS row stride in 16-bit elements
  constexpr int LR = D / 8;     // lanes per V row (16 bytes each)
  constexpr int RPI = kWave / LR, NVL = WT / RPI;
  constexpr int MAXPG = TILE / 8;
  static_assert(G <= 16, "one 16-row fragment holds the query group");
  __shared__ int s_lp[MAXPG];
  __shared__ uint32_t s_ph[MAXPG];
  __shared__ __align__(16) uint16_t s_v[NW][WT][ROW];
  __shared__ float s_red[NW][16];
  __shared__ float s_acc[NW][G][D + 1];
  __shared__ float s_mt[G];

  const int P = 1 << log2P;
  const int unit = blockIdx.x / S_max, split = blockIdx.x - unit * S_max;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int n16 = lane & 15, c4 = lane >> 4;
  const long t0 = (long)split * TILE;
  const int e0 = (int)(t0 >> log2P);
  const int ecap = min(max(1, TILE >> log2P), k_max - e0);
  if (tid < ecap) {
    const int lp = sel[(size_t)unit * k_max + e0 + tid];
    const int ph = sel_phys ? sel_phys[(size_t)unit * k_max + e0 + tid]
                            : bt[(size_t)b * MP + clampi(lp, 0, MP - 1)];
    s_lp[tid] = lp;
    s_ph[tid] = (uint32_t)clampi(ph, 0, NP - 1);
  }
  const int cnt = clampi(sel_count[unit], 0, k_max);
  const int len = clampi(seq_lens[b], 0, MP * P);
  // B operand of the logits: column g = n16, 8 channels per chunk
  vec qhi[NCH], qlo[NCH];
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
        typename M::elem hi, lo;
        split_hi_lo<DT>(has ? xs[j] : 0.f, hi, lo);
        qhi[ch][j] = hi;
        qlo[ch][j] = lo;
      }
    }
  }
  if (t0 >= ((long)cnt << log2P)) {  // whole workgroup: no work
    if (cnt == 0 && split == 0)
      for (int i = tid; i < G * D; i += NT) out[((size_t)b * Hq + h * G) * D + i] = 0.f;
    return;
  }
  __syncthreads();
  const int npg = min(cnt - e0, ecap);
  // pool element offset of wave-local token `tw`, or -1 when masked
  auto token_off = [&](int tw) -> long {
    const long ts = t0 + wave * WT + tw;
    const int e = (int)(ts >> log2P) - e0;
    const int st = (int)(ts & (P - 1));
    if (e >= npg) return -1;
    const int lp = s_lp[e];
    if (lp < 0 || lp * P + st >= len) return -1;
    return (long)((((size_t)s_ph[e] * Hkv + h) * P + st) * D);
  };

  const char* kb = reinterpret_cast<const char*>(k_pool);
  const char* vb = reinterpret_cast<const char*>(v_pool);
  uint4 kr[2][NCH];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const long off = token_off(16 * i + n16);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
      kr[i][ch] = off >= 0 ? ld16(kb + (off + 32 * ch + 8 * c4) * 2) : make_uint4(0, 0, 0, 0);
  }
  uint4 vr[NVL];
#pragma unroll
  for (int u = 0; u < NVL; ++u) {
    const long off = token_off(u * RPI + lane / LR);
    vr[u] = off >= 0 ? ld16(vb + (off + (lane % LR) * 8) * 2) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < NVL; ++u)
    *reinterpret_cast<uint4*>(&s_v[wave][u * RPI + lane / LR][(lane % LR) * 8]) = vr[u];

  // logits of head n16 for tokens 4*c4 + r of tile i, log2 units
  float z[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const vec a = __builtin_bit_cast(vec, kr[i][ch]);
      acc = M::mma(a, qhi[ch], acc);
      acc = M::mma(a, qlo[ch], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) z[i][r] = token_off(16 * i + 4 * c4 + r) >= 0 ? acc[r] * qscale : -INFINITY;
  }
  float m = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                  fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (lane < 16) s_red[wave][lane] = m;
  __syncthreads();  // also publishes the V rows in LDS
  float mt = s_red[0][n16];
#pragma unroll
  for (int w = 1; w < NW; ++w) mt = fmaxf(mt, s_red[w][n16]);
  const float ms = mt == -INFINITY ? 0.f : mt;
  if (wave == 0 && lane < G) s_mt[lane] = mt;

  // probabilities: the A fragment of the second contraction
  vec phi, plo;
  float lsum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(z[j >> 2][j & 3] - ms);
    lsum += p;
    typename M::elem hi, lo;
    split_hi_lo<DT>(p * M::kPScale, hi, lo);
    phi[j] = hi;
    plo[j] = lo;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    s16x8_t vv;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = (j < 4) ? (4 * c4 + j) : (16 + 4 * c4 + (j - 4));
      vv[j] = (short)s_v[wave][row][16 * dt + n16];
    }
    const vec bv = __builtin_bit_cast(vec, vv);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = M::mma(phi, bv, acc);
    acc = M::mma(plo, bv, acc);
    o[dt] = acc;
  }
  // out fragment: head 4*c4 + r, channel 16*dt + n16
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * c4 + r;
      if (g < G) s_acc[wave][g][16 * dt + n16] = o[dt][r] * (1.f / M::kPScale);
    }
  if (lane < G) s_acc[wave][lane][D] = lsum;
  __syncthreads();
  finish_tile<D, G, NT, NW>(s_acc, s_mt, partials, out, b, h, Hq, S_max, split,
                            (int)((((long)cnt << log2P) + TILE - 1) / TILE));
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

// Grouped-query heads on 16-bit KV take the MFMA decode (128-token tiles).
bool use_mfma_decode(const Dims& d) {
  return d.dt != DT_F32 && (d.G == 4 || d.G == 8);
}

int decode_tile_tokens(const Dims& d) {
  if (use_mfma_decode(d)) return 128;
  const int bytes = d.dt == DT_F32 ? 4 : 2;
  const int C = 16 / bytes, L = d.D / C, SPW = kWave / L;
  return 4 * (kDecodeThreads / kWave) * SPW;
}

int decode_splits(const Dims& d, int k_max) {
  const long stream = (long)k_max * d.P;
  const int tile = decode_tile_tokens(d);
  return (int)((stream + tile - 1) / tile);
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
    using Cfg = ScoreCfg<dt, hd, g>;
    const int NC = (d.MP + Cfg::CH - 1) / Cfg::CH;
    hipLaunchKernelGGL((k_score_select<dt, hd, g>), dim3(d.B * d.Hkv * NC), dim3(Cfg::NT), 0,
                       s, q, meta, bt, seq_lens, d.Hq, d.Hkv, d.P, d.MP, d.NP, NC, k_max,
                       k_per_seq, n_sink, sel, sel_count, scores_out, ws.keys, ws.sel_phys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || NC == 1) return e;
    // units longer than one chunk are selected once all their keys exist
    hipLaunchKernelGGL((k_select<Cfg::CH>), dim3(d.B * d.Hkv), dim3(256),
                       sizeof(uint32_t) * (size_t)d.MP, s, bt, seq_lens, d.Hkv, d.P, d.MP,
                       d.NP, k_max, k_per_seq, n_sink, ws.keys, sel, sel_count, ws.sel_phys);
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
                           d.Hq, d.Hkv, log2P, d.MP, d.NP, k_max, S_max, qscale,
                           ws.partials, out);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((k_decode_split<dt, hd, g, kDecodeThreads>),
                       dim3(d.B * d.Hkv * S_max), dim3(kDecodeThreads), 0, s, q,
                       k_pool, v_pool, bt, seq_lens, sel, sel_phys, sel_count, d.Hq,
                       d.Hkv, log2P, d.MP, d.NP, k_max, S_max, qscale, ws.partials, out);
    return hipGetLastError();
  });
  if (e != hipSuccess || S_max == 1) return e;
  const int waves = d.B * d.Hq;
  const int tile = decode_tile_tokens(d);
  if (d.D == 64)
    hipLaunchKernelGGL(k_merge<64>, dim3((waves + 3) / 4), dim3(256), 0, s, ws.partials,
                       sel_count, d.B, d.Hq, d.Hkv, d.G, log2P, k_max, S_max, tile, out);
  else
    hipLaunchKernelGGL(k_merge<128>, dim3((waves + 3) / 4), dim3(256), 0, s, ws.partials,
                       sel_count, d.B, d.Hq, d.Hkv, d.G, log2P, k_max, S_max, tile, out);
  return hipGetLastError();
}

}  // namespace tsv
