// Template dispatch from a runtime (n, shape) to a kernel instantiation.
// Included once per storage format so the two formats compile in parallel.
#pragma once

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "twnorm_launch.hpp"

namespace twl {
namespace detail {

// Keep grid * block below 2^31 work-items; the kernels' grid-stride loops
// cover whatever a smaller grid leaves.
inline int64_t cap_grid(int64_t grid, int block) {
  const int64_t max_grid = (int64_t(1) << 31) / block;
  return std::max<int64_t>(1, std::min(grid, max_grid));
}

template <typename... P, size_t... I>
hipError_t launch_tuple(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t s,
                        std::tuple<P...>& args, std::index_sequence<I...>) {
  void* ptrs[] = {static_cast<void*>(&std::get<I>(args))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, 0, s);
}

// Resident workgroups per CU of (kernel, block size), looked up once.
inline hipError_t resident_per_cu(const void* kern, int block, int* out) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({kern, block});
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, block, 0);
  if (e != hipSuccess) return e;
  occ = std::max(occ, 1);
  cache[{kern, block}] = occ;
  *out = occ;
  return hipSuccess;
}

// Launch `kern` over `work` workgroups.  With persistent_cus > 0 the grid is
// capped at the workgroups that many CUs hold at once (the kernels loop over
// the rest): the CU-limited mode, and the fused kernel's persistent,
// software-pipelined row loop.  With persistent_cus == 0 the grid is `work`.
template <typename... P, typename... A>
hipError_t go_capped(void (*kern)(P...), int block, int64_t work, int persistent_cus,
                     int per_cu_cap, hipStream_t s, A... a) {
  if (work <= 0) return hipSuccess;
  int64_t grid = work;
  if (persistent_cus > 0) {
    int occ = 0;
    hipError_t e = resident_per_cu(reinterpret_cast<const void*>(kern), block, &occ);
    if (e != hipSuccess) return e;
    if (per_cu_cap > 0) occ = std::min(occ, per_cu_cap);
    grid = std::min<int64_t>(grid, int64_t(persistent_cus) * occ);
  }
  grid = cap_grid(grid, block);
  std::tuple<P...> args(a...);
  return launch_tuple(kern, dim3(static_cast<uint32_t>(grid)), dim3(block), s, args,
                      std::index_sequence_for<P...>{});
}

template <typename... P, typename... A>
hipError_t go(void (*kern)(P...), int block, int64_t work, int persistent_cus, hipStream_t s,
              A... a) {
  return go_capped(kern, block, work, persistent_cus, 0, s, a...);
}

template <class D, int N>
hipError_t fused_n(const Launch& L, const FusedArgs& a, hipStream_t s) {
  const int block = 64 * L.waves;
  const int64_t work_rows = a.rows;
  // Wide rows.  Whole chip: one workgroup per row, so the hardware dispatcher
  // hands the remaining rows to workgroups as earlier ones retire, which
  // evens out the end of the call (measured faster than the persistent loop
  // on the whole chip: 29.9 against 30.4 us at N=8, 1024 x 8192).  CU-limited
  // calls, or a forced residency cap: persistent grid on those CUs, each
  // workgroup walking its rows with the next row's loads in flight (faster on
  // 8-32 CUs, where each CU must keep its own pipeline full).
  const int grid_cus = L.cu_limit > 0 ? L.cu_limit : (L.wgs_per_cu > 0 ? L.device_cus : 0);
#define TW_ROWS(KK)                                                                            \
  (L.waves <= 4   ? go_capped(twk::fused_rows_kernel<D, N, KK, 4>, block, work_rows, grid_cus, L.wgs_per_cu, s, a.pp,  \
                       a.residual, a.weight, a.outs, a.residual_out, a.rows, a.chunks, a.hidden_f, \
                       a.eps)                                                                   \
   : L.waves <= 8 ? go_capped(twk::fused_rows_kernel<D, N, KK, 8>, block, work_rows, grid_cus, L.wgs_per_cu, s, a.pp,  \
                       a.residual, a.weight, a.outs, a.residual_out, a.rows, a.chunks, a.hidden_f, \
                       a.eps)                                                                   \
                  : go_capped(twk::fused_rows_kernel<D, N, KK, 16>, block, work_rows, grid_cus, L.wgs_per_cu, s, a.pp, \
                       a.residual, a.weight, a.outs, a.residual_out, a.rows, a.chunks, a.hidden_f, \
                       a.eps))
  switch (L.k) {
    case 0: {
      const int rows_per_block = 256 / L.team;
      return go(twk::fused_team_kernel<D, N>, 256, (a.rows + rows_per_block - 1) / rows_per_block,
                L.cu_limit, s, a.pp, a.residual, a.weight, a.outs, a.residual_out, a.rows, a.chunks,
                L.team, a.hidden_f, a.eps);
    }
    case 1: return TW_ROWS(1);
    case 2: return TW_ROWS(2);
    case 3: return TW_ROWS(3);
    case 4: return TW_ROWS(4);
    case 6: return TW_ROWS(6);
    case 8: return TW_ROWS(8);
  }
#undef TW_ROWS
  return hipErrorInvalidValue;
}

// Dispatch on the partial count; NLO..NHI bounds the instantiations made by
// one translation unit (the ranges compile in parallel).
template <class D, int NLO, int NHI>
hipError_t fused_range(const Launch& L, const FusedArgs& a, hipStream_t s) {
#define TW_N(NN) \
  case NN:       \
    if constexpr (NN >= NLO && NN <= NHI) return fused_n<D, NN>(L, a, s); \
    break;
  switch (L.n) {
    TW_N(1) TW_N(2) TW_N(3) TW_N(4) TW_N(5) TW_N(6) TW_N(7) TW_N(8)
    TW_N(9) TW_N(10) TW_N(11) TW_N(12) TW_N(13) TW_N(14) TW_N(15) TW_N(16)
  }
#undef TW_N
  return hipErrorInvalidValue;
}

template <class D, int N>
hipError_t reduce_n(const twk::PartialPtrs& pp, twk::u32x4* reduced, int64_t total, int cu_limit,
                    hipStream_t s) {
  // cu_limit here is the persistent grid's CU count (the limit, else the device's)
  constexpr int64_t block = 256 * twk::reduce_slots<N>();
  return go_capped(twk::reduce_kernel<D, N>, 256, (total + block - 1) / block, cu_limit, 2, s, pp,
                   reduced, total);
}

template <class D>
hipError_t reduce(int n, const twk::PartialPtrs& pp, twk::u32x4* reduced, int64_t total,
                  int cu_limit, hipStream_t s) {
  switch (n) {
    case 1: return reduce_n<D, 1>(pp, reduced, total, cu_limit, s);
    case 2: return reduce_n<D, 2>(pp, reduced, total, cu_limit, s);
    case 3: return reduce_n<D, 3>(pp, reduced, total, cu_limit, s);
    case 4: return reduce_n<D, 4>(pp, reduced, total, cu_limit, s);
    case 5: return reduce_n<D, 5>(pp, reduced, total, cu_limit, s);
    case 6: return reduce_n<D, 6>(pp, reduced, total, cu_limit, s);
    case 7: return reduce_n<D, 7>(pp, reduced, total, cu_limit, s);
    case 8: return reduce_n<D, 8>(pp, reduced, total, cu_limit, s);
    case 9: return reduce_n<D, 9>(pp, reduced, total, cu_limit, s);
    case 10: return reduce_n<D, 10>(pp, reduced, total, cu_limit, s);
    case 11: return reduce_n<D, 11>(pp, reduced, total, cu_limit, s);
    case 12: return reduce_n<D, 12>(pp, reduced, total, cu_limit, s);
    case 13: return reduce_n<D, 13>(pp, reduced, total, cu_limit, s);
    case 14: return reduce_n<D, 14>(pp, reduced, total, cu_limit, s);
    case 15: return reduce_n<D, 15>(pp, reduced, total, cu_limit, s);
    case 16: return reduce_n<D, 16>(pp, reduced, total, cu_limit, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace detail
}  // namespace twl
