// Host-side argument validation and launch-shape choice for libtwnorm.
// HIP-free: this translation unit makes no HIP call and includes no HIP
// header, so every error path of the C ABI can be exercised without a GPU.
#pragma once

#include <stdint.h>

#include "twnorm.h"

namespace twv {

// Kernel launch shape for one token row.
//   k > 0 : wide-row kernel, `waves` wavefronts per row, k chunk slots/lane
//   k == 0: narrow-row kernel, `team` lanes per row (power of two <= 32)
struct Shape {
  int waves;
  int k;
  int team;
};

int elem_bytes(tw_dtype dtype);  // 0 for an unknown dtype

// Record a failure message for tw_last_error() and return `s`.
tw_status fail(tw_status s, const char* fmt, ...);
void clear_error();
const char* last_error();

tw_status check_fused(const void* const* partials, int n, int64_t rows, int64_t hidden,
                      tw_dtype dtype, const void* residual, const void* weight, float eps,
                      const void* out, const void* residual_out, int n_cu_limit);
tw_status check_fused_allgather(const void* const* partials, int n, int64_t rows, int64_t hidden,
                                tw_dtype dtype, const void* residual, const void* weight,
                                float eps, const void* const* ag_outs, int n_ag,
                                int64_t ag_row_offset, int64_t ag_total_rows,
                                const void* residual_out, int n_cu_limit);
tw_status check_reduce(const void* const* partials, int n, int64_t rows, int64_t hidden,
                       tw_dtype dtype, const void* reduced, int n_cu_limit);
tw_status check_copy(const void* src, const void* dst, int64_t bytes, int n_cu_limit);
tw_status check_mix(const void* const* srcs, int n_src, const void* const* dsts, int n_dst,
                    int64_t bytes, int n_cu_limit);

// Shape for (dtype, hidden, n) when `rows` rows run on `cus` of the device's
// `device_cus` CUs; honours the calling thread's tw_set_fused_shape override.
tw_status choose_shape(tw_dtype dtype, int64_t hidden, int n, int64_t rows, int cus, int device_cus,
                       Shape* shape);

// True if the wide-row kernel for (dtype, n, waves, k) needs scratch memory
// (from the build's register-fit table).
bool shape_spills(tw_dtype dtype, int n, int waves, int k);

// Force (waves, k) for wide rows ((0, 0) restores the automatic choice) and,
// with wgs_per_cu > 0, run the wide-row kernel on a persistent grid of at
// most wgs_per_cu workgroups per CU (0 = the default grid), for the calling
// thread's later calls.
tw_status set_override(int waves, int k, int wgs_per_cu);
int wgs_per_cu_cap();

}  // namespace twv
