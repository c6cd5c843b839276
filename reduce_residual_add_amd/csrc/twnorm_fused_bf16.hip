// Kernel instantiations for bf16 storage (float32 arithmetic).
#include "twnorm_launch_impl.hpp"

namespace twl {

hipError_t launch_fused_bf16(const Launch& L, const FusedArgs& a, hipStream_t s) {
  return detail::fused<twk::Bf16>(L, a, s);
}

hipError_t launch_reduce_bf16(int n, const twk::PartialPtrs& pp, twk::u32x4* reduced,
                              int64_t total_chunks, int cu_limit, hipStream_t s) {
  return detail::reduce<twk::Bf16>(n, pp, reduced, total_chunks, cu_limit, s);
}

}  // namespace twl
