// float32 storage: fused kernels for 1..8 partials and the unfused reduce
// kernel; plus the streaming copy.
#include "twnorm_launch_impl.hpp"

namespace twk {

// ---------------------------------------------------------------------------
// Measurement aid: plain streaming copy, four 16-byte chunks in flight per
// lane.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t chunks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; c + 3 * stride < chunks; c += 4 * stride) {
    u32x4 a = ld_stream(src + c);
    u32x4 b = ld_stream(src + c + stride);
    u32x4 d = ld_stream(src + c + 2 * stride);
    u32x4 e = ld_stream(src + c + 3 * stride);
    st_stream(dst + c, a);
    st_stream(dst + c + stride, b);
    st_stream(dst + c + 2 * stride, d);
    st_stream(dst + c + 3 * stride, e);
  }
  for (; c < chunks; c += stride) st_stream(dst + c, ld_stream(src + c));
}

}  // namespace twk

namespace twl {

hipError_t launch_fused_f32_n1to8(const Launch& L, const FusedArgs& a, hipStream_t s) {
  return detail::fused_range<twk::F32, 1, 8>(L, a, s);
}

hipError_t launch_reduce_f32(int n, const twk::PartialPtrs& pp, twk::u32x4* reduced,
                             int64_t total_chunks, int cu_limit, hipStream_t s) {
  return detail::reduce<twk::F32>(n, pp, reduced, total_chunks, cu_limit, s);
}

hipError_t launch_copy(const twk::u32x4* src, twk::u32x4* dst, int64_t chunks, int cu_limit,
                       hipStream_t s) {
  const int64_t per_block = 256 * 4;
  return detail::go(twk::stream_copy_kernel, 256, (chunks + per_block - 1) / per_block, cu_limit,
                    s, src, dst, chunks);
}

}  // namespace twl
