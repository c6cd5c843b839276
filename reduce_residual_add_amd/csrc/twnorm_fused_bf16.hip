// bf16 storage (float32 arithmetic): fused kernels for 1..8 partials and
// the unfused reduce kernel.
#include "twnorm_launch_impl.hpp"

namespace twl {

hipError_t launch_fused_bf16_n1to8(const Launch& L, const FusedArgs& a, hipStream_t s) {
  return detail::fused_range<twk::Bf16, 1, 8>(L, a, s);
}

hipError_t launch_reduce_bf16(int n, const twk::PartialPtrs& pp, twk::u32x4* reduced,
                              int64_t total_chunks, int grid_cus, hipStream_t s) {
  return detail::reduce<twk::Bf16>(n, pp, reduced, total_chunks, grid_cus, s);
}

}  // namespace twl
