// C entry points over the HIP-free validator, built with g++ into a test-only
// shared library so that property tests can drive every alias rule from
// Python without any call reaching the HIP runtime.
#include "twnorm_validate.hpp"

extern "C" {

int shim_check_fused(const void* const* partials, int n, long long rows, long long hidden,
                     int dtype, const void* residual, const void* weight, float eps,
                     const void* out, const void* residual_out, int n_cu_limit) {
  return twv::check_fused(partials, n, rows, hidden, static_cast<tw_dtype>(dtype), residual,
                          weight, eps, out, residual_out, n_cu_limit);
}

int shim_check_fused_allgather(const void* const* partials, int n, long long rows,
                               long long hidden, int dtype, const void* residual,
                               const void* weight, float eps, const void* const* ag_outs, int n_ag,
                               long long ag_row_offset, long long ag_total_rows,
                               const void* residual_out, int n_cu_limit) {
  return twv::check_fused_allgather(partials, n, rows, hidden, static_cast<tw_dtype>(dtype),
                                    residual, weight, eps, ag_outs, n_ag, ag_row_offset,
                                    ag_total_rows, residual_out, n_cu_limit);
}

int shim_check_reduce(const void* const* partials, int n, long long rows, long long hidden,
                      int dtype, const void* reduced, int n_cu_limit) {
  return twv::check_reduce(partials, n, rows, hidden, static_cast<tw_dtype>(dtype), reduced,
                           n_cu_limit);
}

}  // extern "C"
