// Internal launch interface between the C ABI (twnorm_api.hip) and the
// per-dtype kernel instantiations (twnorm_fused_{bf16,f32}.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "twnorm_kernels.hpp"

namespace twl {

struct FusedArgs {
  twk::PartialPtrs pp;
  const twk::u32x4* residual;
  const twk::u32x4* weight;
  twk::OutPtrs outs;
  twk::u32x4* residual_out;
  int64_t rows;
  int chunks;      // 16-byte chunks per row
  float hidden_f;  // features per row, as float (divisor of the mean square)
  float eps;
};

struct Launch {
  int n;           // partials
  int waves;       // wide-row kernel: wavefronts per row
  int k;           // wide-row kernel: chunk slots per lane; 0 = narrow-row kernel
  int team;        // narrow-row kernel: lanes per row
  int cu_limit;    // 0: whole chip; > 0: persistent grid for that many CUs
  int device_cus;  // CUs of the device (persistent whole-chip grid under a cap)
  int wgs_per_cu;  // > 0: persistent grid of at most this many workgroups per
                   // CU; 0: no cap (one workgroup per row on the whole chip)
};

// n in [1, 8] and [9, 16] are instantiated in separate translation units.
hipError_t launch_fused_bf16_n1to8(const Launch& L, const FusedArgs& a, hipStream_t s);
hipError_t launch_fused_bf16_n9to16(const Launch& L, const FusedArgs& a, hipStream_t s);
hipError_t launch_fused_f32_n1to8(const Launch& L, const FusedArgs& a, hipStream_t s);
hipError_t launch_fused_f32_n9to16(const Launch& L, const FusedArgs& a, hipStream_t s);

inline hipError_t launch_fused(bool bf16, const Launch& L, const FusedArgs& a, hipStream_t s) {
  if (bf16) return L.n <= 8 ? launch_fused_bf16_n1to8(L, a, s) : launch_fused_bf16_n9to16(L, a, s);
  return L.n <= 8 ? launch_fused_f32_n1to8(L, a, s) : launch_fused_f32_n9to16(L, a, s);
}
// grid_cus: CUs of the persistent grid (the CU limit, else the device's)
hipError_t launch_reduce_bf16(int n, const twk::PartialPtrs& pp, twk::u32x4* reduced,
                              int64_t total_chunks, int grid_cus, hipStream_t s);
hipError_t launch_reduce_f32(int n, const twk::PartialPtrs& pp, twk::u32x4* reduced,
                             int64_t total_chunks, int grid_cus, hipStream_t s);
hipError_t launch_copy(const twk::u32x4* src, twk::u32x4* dst, int64_t chunks, int cu_limit,
                       hipStream_t s);
// persistent_cus: CUs of the persistent grid (the CU limit, else the device's)
hipError_t launch_mix(int n_src, const twk::MixPtrs& m, int64_t bytes, int persistent_cus,
                      hipStream_t s);

}  // namespace twl
