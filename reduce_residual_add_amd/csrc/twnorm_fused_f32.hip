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

// ---------------------------------------------------------------------------
// Measurement aid: the fused kernel's traffic pattern without its arithmetic.
// NS sources are walked in blocks, one block per workgroup step, with the
// fused kernel's lane layout (slots of 16 bytes per lane, 256 lanes), its
// cache policies and its order of work: the first destination is stored
// (as the fused kernel stores residual_out), then the next block's loads are
// issued, then the other destinations are stored (as the normalised output
// is).  Up to 9 sources a lane holds 4 slots (16 KiB
// blocks, as the fused kernel on 8192 bf16 features); above that 2 slots
// (8 KiB blocks), so that the loads of one block fit in registers at 2 waves
// per SIMD.  Each destination word is the wrap-around sum of the source
// words.  A block's descriptors cover only the bytes left, so the last,
// short block reads zeros past the end and its stores there are dropped.
// ---------------------------------------------------------------------------
constexpr int mix_slots(int ns) { return ns <= 9 ? 4 : 2; }
constexpr int mix_block(int ns) { return 256 * 16 * mix_slots(ns); }

template <int NS>
__device__ __forceinline__ void mix_load(u32x4 (&raw)[mix_slots(NS)][NS], const MixPtrs& m,
                                         int64_t off, int len, unsigned lane_off) {
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const rsrc_t r = make_rsrc(reinterpret_cast<const char*>(m.src[j]) + off, len);
#pragma unroll
    for (int k = 0; k < mix_slots(NS); ++k) raw[k][j] = buf_load(r, lane_off + k * 4096u);
  }
}

template <int NS>
__global__ void __launch_bounds__(256, 2) stream_mix_kernel(MixPtrs m, int64_t bytes) {
  constexpr int K = mix_slots(NS);
  constexpr int B = mix_block(NS);
  const int64_t blocks = (bytes + B - 1) / B;
  const unsigned lane_off = threadIdx.x * 16u;
  auto len_of = [&](int64_t b) {
    const int64_t left = bytes - b * B;
    return int(left < B ? left : B);
  };
  u32x4 raw[K][NS];
  int64_t b = blockIdx.x;
  if (b < blocks) mix_load<NS>(raw, m, b * B, len_of(b), lane_off);
  for (; b < blocks; b += gridDim.x) {
    u32x4 acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      acc[k] = raw[k][0];
#pragma unroll
      for (int j = 1; j < NS; ++j) acc[k] += raw[k][j];
    }
    const int len = len_of(b);
    const rsrc_t r0 = make_rsrc(reinterpret_cast<char*>(m.dst[0]) + b * B, len);
#pragma unroll
    for (int k = 0; k < K; ++k) buf_store(acc[k], r0, lane_off + k * 4096u);
    const int64_t next = b + gridDim.x;
    if (next < blocks) mix_load<NS>(raw, m, next * B, len_of(next), lane_off);
    for (int d = 1; d < m.n_dst; ++d) {
      const rsrc_t r = make_rsrc(reinterpret_cast<char*>(m.dst[d]) + b * B, len);
#pragma unroll
      for (int k = 0; k < K; ++k) buf_store(acc[k], r, lane_off + k * 4096u);
    }
  }
}

}  // namespace twk

namespace twl {

hipError_t launch_fused_f32_n1to8(const Launch& L, const FusedArgs& a, hipStream_t s) {
  return detail::fused_range<twk::F32, 1, 8>(L, a, s);
}

hipError_t launch_reduce_f32(int n, const twk::PartialPtrs& pp, twk::u32x4* reduced,
                             int64_t total_chunks, int grid_cus, hipStream_t s) {
  return detail::reduce<twk::F32>(n, pp, reduced, total_chunks, grid_cus, s);
}

hipError_t launch_mix(int n_src, const twk::MixPtrs& m, int64_t bytes, int persistent_cus,
                      hipStream_t s) {
#define TW_MIX(NS)                                                                         \
  case NS:                                                                                 \
    return detail::go_capped(twk::stream_mix_kernel<NS>, 256,                              \
                             (bytes + twk::mix_block(NS) - 1) / twk::mix_block(NS),        \
                             persistent_cus, 2, s, m, bytes);
  switch (n_src) {
    TW_MIX(1) TW_MIX(2) TW_MIX(3) TW_MIX(4) TW_MIX(5) TW_MIX(6) TW_MIX(7) TW_MIX(8) TW_MIX(9)
    TW_MIX(10) TW_MIX(11) TW_MIX(12) TW_MIX(13) TW_MIX(14) TW_MIX(15) TW_MIX(16) TW_MIX(17)
  }
#undef TW_MIX
  return hipErrorInvalidValue;
}

hipError_t launch_copy(const twk::u32x4* src, twk::u32x4* dst, int64_t chunks, int cu_limit,
                       hipStream_t s) {
  const int64_t per_block = 256 * 4;
  return detail::go(twk::stream_copy_kernel, 256, (chunks + per_block - 1) / per_block, cu_limit,
                    s, src, dst, chunks);
}

}  // namespace twl
