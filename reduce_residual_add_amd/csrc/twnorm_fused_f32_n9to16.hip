// float32 storage: fused kernels for 9..16 partials.
#include "twnorm_launch_impl.hpp"

namespace twl {

hipError_t launch_fused_f32_n9to16(const Launch& L, const FusedArgs& a, hipStream_t s) {
  return detail::fused_range<twk::F32, 9, 16>(L, a, s);
}

}  // namespace twl
