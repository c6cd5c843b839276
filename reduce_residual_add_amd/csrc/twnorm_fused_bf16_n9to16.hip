// bf16 storage (float32 arithmetic): fused kernels for 9..16 partials.
#include "twnorm_launch_impl.hpp"

namespace twl {

hipError_t launch_fused_bf16_n9to16(const Launch& L, const FusedArgs& a, hipStream_t s) {
  return detail::fused_range<twk::Bf16, 9, 16>(L, a, s);
}

}  // namespace twl
