// Launchers of the gfx950 kernels for one KV type.  The build compiles this
// file once per KV type (TSV_DT) and kernel family (TSV_PART: phased kernels
// or the one-launch step), so the instantiations of the device templates
// spread over several objects that compile in parallel.
#include <algorithm>
#include <type_traits>

#include "tsv_device.h"

#ifndef TSV_DT
#error "define TSV_DT (the KV type) and TSV_PART (kernel family) when compiling"
#endif

#define TSV_PART_PHASED 0
#define TSV_PART_STEP 1

namespace tsv {
namespace {

template <int V>
using IC = std::integral_constant<int, V>;

// fn(IC<D>, IC<G>) for the call's head_dim and group size
template <class Fn>
hipError_t by_d_g(const Dims& d, Fn&& fn) {
  auto byG = [&](auto HD) -> hipError_t {
    switch (d.G) {
      case 1: return fn(HD, IC<1>{});
      case 2: return fn(HD, IC<2>{});
      case 4: return fn(HD, IC<4>{});
      case 8: return fn(HD, IC<8>{});
      case 16: return fn(HD, IC<16>{});
    }
    return hipErrorInvalidValue;
  };
  switch (d.D) {
    case 64: return byG(IC<64>{});
    case 128: return byG(IC<128>{});
  }
  return hipErrorInvalidValue;
}

// Rows at least this many: every row of the phased score is one workgroup.
constexpr int kScoreRowsOneWorkgroup = 256;

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

constexpr float kLog2e = 1.44269504088896340736f;

}  // namespace

template <int dt>
hipError_t meta_build_t(const Dims& d, const void* k_pool, void* meta, const int32_t* bt,
                        const int32_t* seq_lens, hipStream_t s) {
  dim3 grid((d.Hkv * d.D + 255) / 256, d.MP, d.B);
  hipLaunchKernelGGL(k_meta_build<dt>, grid, dim3(256), 0, s, k_pool, meta, bt, seq_lens, d.Hkv,
                     d.D, d.P, d.MP, d.NP);
  return hipGetLastError();
}

template <int dt>
hipError_t meta_append_t(const Dims& d, const void* k_new, const void* v_new, void* k_pool,
                         void* v_pool, void* meta, const int32_t* bt, const int32_t* seq_lens,
                         hipStream_t s) {
  const int total = d.B * d.Hkv * d.D;
  hipLaunchKernelGGL(k_meta_append<dt>, dim3((total + 255) / 256), dim3(256), 0, s, k_new, v_new,
                     k_pool, v_pool, meta, bt, seq_lens, d.B, d.Hkv, d.D, d.P, d.MP, d.NP);
  return hipGetLastError();
}

template <int dt>
hipError_t score_select_t(const Dims& d, const float* q, const void* meta, const int32_t* bt,
                          const int32_t* seq_lens, int k_max, const int32_t* k_per_seq,
                          const SelectPolicy& pol, int32_t* sel, int32_t* sel_count,
                          float* scores_out, const Workspace& ws, hipStream_t s) {
  return by_d_g(d, [&](auto HD, auto GG) -> hipError_t {
    constexpr int hd = decltype(HD)::value, g = decltype(GG)::value;
    using Big = ScoreCfg<dt, hd, g, score_threads<g>()>;
    using Small = ScoreCfg<dt, hd, g, 256>;
    const bool small = d.MP <= Small::PB;
    const int PB = small ? Small::PB : Big::PB;
    const int units = d.B * d.Hkv;
    // enough rows to fill the chip: one streaming workgroup per row, top-K in
    // place; otherwise split every row over several workgroups
    const int batches = (d.MP + PB - 1) / PB;
    const int NS = units >= kScoreRowsOneWorkgroup
                       ? 1
                       : std::max(1, std::min(batches, (512 + units - 1) / units));
    const size_t shmem = 2 * sizeof(uint32_t) * (size_t)d.MP;
    if (small)
      hipLaunchKernelGGL((k_score_select<dt, hd, g, 256>), dim3(units * NS), dim3(256), shmem, s,
                         q, meta, bt, seq_lens, d.Hq, d.Hkv, d.P, d.MP, d.NP, NS, k_max,
                         k_per_seq, pol, sel, sel_count, scores_out, ws.keys, ws.sel_phys);
    else
      hipLaunchKernelGGL((k_score_select<dt, hd, g, Big::NT>), dim3(units * NS), dim3(Big::NT),
                         shmem, s, q, meta, bt, seq_lens, d.Hq, d.Hkv, d.P, d.MP, d.NP, NS,
                         k_max, k_per_seq, pol, sel, sel_count, scores_out, ws.keys,
                         ws.sel_phys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || NS == 1) return e;
    hipLaunchKernelGGL(k_select, dim3(units), dim3(kSelectThreads),
                       2 * sizeof(uint32_t) * (size_t)d.MP, s, bt, seq_lens, d.Hkv, d.P, d.MP,
                       d.NP, k_max, k_per_seq, pol, ws.keys, sel, sel_count, ws.sel_phys);
    return hipGetLastError();
  });
}

template <int dt>
hipError_t decode_t(const Dims& d, const DecodePlan& plan, const float* q, const void* k_pool,
                    const void* v_pool, const int32_t* bt, const int32_t* seq_lens,
                    const int32_t* sel, const int32_t* sel_phys, const int32_t* sel_count,
                    int k_max, float scale, const Workspace& ws, float* out, hipStream_t s) {
  const int S_max = plan.S_max, TPW = plan.TPW;
  const int log2P = ilog2(d.P);
  const float qscale = scale * kLog2e;  // exp2 in the softmax
  hipError_t e = by_d_g(d, [&](auto HD, auto GG) -> hipError_t {
    constexpr int hd = decltype(HD)::value, g = decltype(GG)::value;
    if constexpr (dt != DT_F32 && (g == 4 || g == 8 || g == 16)) {
      hipLaunchKernelGGL((k_decode_mfma<dt, hd, g>), dim3(d.B * d.Hkv * S_max), dim3(256), 0, s,
                         q, k_pool, v_pool, bt, seq_lens, sel, sel_phys, sel_count, d.Hq, d.Hkv,
                         log2P, d.MP, d.NP, k_max, S_max, TPW, qscale, ws.partials, out);
    } else {
      hipLaunchKernelGGL((k_decode_split<dt, hd, g, kDecodeThreads>), dim3(d.B * d.Hkv * S_max),
                         dim3(kDecodeThreads), 0, s, q, k_pool, v_pool, bt, seq_lens, sel,
                         sel_phys, sel_count, d.Hq, d.Hkv, log2P, d.MP, d.NP, k_max, S_max, TPW,
                         qscale, ws.partials, out);
    }
    return hipGetLastError();
  });
  if (e != hipSuccess || S_max == 1) return e;
  const int waves = d.B * d.Hq;
  const int tile = plan.tile_tokens * TPW;
  if (d.D == 64)
    hipLaunchKernelGGL(k_merge<64>, dim3((waves + 3) / 4), dim3(256), 0, s, ws.partials,
                       sel_count, d.B, d.Hq, d.Hkv, d.G, log2P, k_max, S_max, tile, out);
  else
    hipLaunchKernelGGL(k_merge<128>, dim3((waves + 3) / 4), dim3(256), 0, s, ws.partials,
                       sel_count, d.B, d.Hq, d.Hkv, d.G, log2P, k_max, S_max, tile, out);
  return hipGetLastError();
}

template <int dt>
hipError_t step_t(const Dims& d, const StepPlan& plan, const float* q, const void* k_new,
                  const void* v_new, void* k_pool, void* v_pool, void* meta, const int32_t* bt,
                  const int32_t* seq_lens, int k_max, const int32_t* k_per_seq,
                  const SelectPolicy& pol, float scale, const int32_t* order, int order_len,
                  int32_t* sel, int32_t* sel_count, float* scores_out, const Workspace& ws,
                  float* out, hipStream_t s) {
  const int log2P = ilog2(d.P);
  const float qscale = scale * kLog2e;  // exp2 in the softmax
  const int units = d.B * d.Hkv, S = plan.S;
  // a row order replaces the workgroup -> row mapping of one-workgroup rows
  const int32_t* ord = S == 1 ? order : nullptr;
  const dim3 grid(ord ? order_len : (units + 7) / 8 * 8 * S);
  return by_d_g(d, [&](auto HD, auto GG) -> hipError_t {
    constexpr int hd = decltype(HD)::value, g = decltype(GG)::value;
    auto go = [&](auto NTc) -> hipError_t {
      constexpr int nthr = decltype(NTc)::value;
      hipLaunchKernelGGL((k_step<dt, hd, g, nthr>), grid, dim3(nthr), plan.lds, s, ord, bt,
                         seq_lens, k_per_seq, S, units, d.Hkv, d.MP, log2P, d.NP, q, k_new,
                         v_new, k_pool, v_pool, meta, d.Hq, k_max, pol, qscale, plan.polls, sel,
                         sel_count, scores_out, ws.sync, ws.xkeys, ws.partials, out);
      return hipGetLastError();
    };
    return plan.nt == 256 ? go(IC<256>{}) : go(IC<512>{});
  });
}

template <int dt>
hipError_t step_per_cu_t(const Dims& d, const StepPlan& plan, int* per_cu) {
  return by_d_g(d, [&](auto HD, auto GG) -> hipError_t {
    constexpr int hd = decltype(HD)::value, g = decltype(GG)::value;
    auto go = [&](auto NTc) -> hipError_t {
      constexpr int nthr = decltype(NTc)::value;
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          per_cu, reinterpret_cast<const void*>(&k_step<dt, hd, g, nthr>), nthr, plan.lds);
    };
    return plan.nt == 256 ? go(IC<256>{}) : go(IC<512>{});
  });
}

#if TSV_PART == TSV_PART_PHASED
template hipError_t meta_build_t<TSV_DT>(const Dims&, const void*, void*, const int32_t*,
                                         const int32_t*, hipStream_t);
template hipError_t meta_append_t<TSV_DT>(const Dims&, const void*, const void*, void*, void*,
                                          void*, const int32_t*, const int32_t*, hipStream_t);
template hipError_t score_select_t<TSV_DT>(const Dims&, const float*, const void*,
                                           const int32_t*, const int32_t*, int, const int32_t*,
                                           const SelectPolicy&, int32_t*, int32_t*, float*,
                                           const Workspace&, hipStream_t);
template hipError_t decode_t<TSV_DT>(const Dims&, const DecodePlan&, const float*, const void*,
                                     const void*, const int32_t*, const int32_t*,
                                     const int32_t*, const int32_t*, const int32_t*, int, float,
                                     const Workspace&, float*, hipStream_t);
#elif TSV_PART == TSV_PART_STEP
#ifdef TSV_PHASE_STAMPS
// The last step launch's phase stamps of this KV type (testing build).
template <>
hipError_t read_phase_stamps_t<TSV_DT>(void* host, size_t bytes) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_stamps),
                             std::min(bytes, sizeof(g_phase_stamps)), 0, hipMemcpyDeviceToHost);
}
#endif
template hipError_t step_t<TSV_DT>(const Dims&, const StepPlan&, const float*, const void*,
                                   const void*, void*, void*, void*, const int32_t*,
                                   const int32_t*, int, const int32_t*, const SelectPolicy&,
                                   float, const int32_t*, int, int32_t*, int32_t*, float*,
                                   const Workspace&, float*, hipStream_t);
template hipError_t step_per_cu_t<TSV_DT>(const Dims&, const StepPlan&, int*);
#else
#error "unknown TSV_PART"
#endif

}  // namespace tsv
