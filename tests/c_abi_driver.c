/*
 * A caller of libtwnorm written in plain C99: no C++, no Python, no torch in
 * the process.  It exercises the C ABI as a C program sees it: device memory
 * from hipMalloc, a stream from hipStreamCreate, status codes and
 * tw_last_error().
 *
 *   c_abi_driver IN OUT
 *
 * IN holds int32 n, int32 dtype (tw_dtype), int64 rows, int64 hidden,
 * float32 eps, then the n partials, the residual and the weight as raw
 * storage bytes (row-major).  OUT receives out, then residual_out.
 *
 * Besides the fused call it checks, and reports on stderr:
 *   - the ABI version;
 *   - that n = 0 is refused with TW_ERR_INVALID_ARG and a message, and that
 *     the refused call wrote nothing;
 *   - that the in-place update (residual_out == residual) gives the same
 *     bytes as the out-of-place call.
 * Exit status 0 on success, 1 on any failure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "twnorm.h"

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : -1; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  if (tw_abi_version() != TW_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header says %d\n", tw_abi_version(), TW_ABI_VERSION);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t n = 0, dtype = 0;
  int64_t rows = 0, hidden = 0;
  float eps = 0.0f;
  if (read_all(in, &n, 4) || read_all(in, &dtype, 4) || read_all(in, &rows, 8) ||
      read_all(in, &hidden, 8) || read_all(in, &eps, 4)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  if (n < 1 || n > TW_MAX_PARTIALS || rows < 1 || hidden < 1 || (dtype != TW_BF16 && dtype != TW_F32)) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  const size_t elem = dtype == TW_BF16 ? 2 : 4;
  const size_t tensor = (size_t)rows * (size_t)hidden * elem;
  const size_t wbytes = (size_t)hidden * elem;

  unsigned char* host = malloc(tensor * (size_t)(n + 1) + wbytes);
  unsigned char* host_out = malloc(tensor * 3);
  if (host == NULL || host_out == NULL) return 1;
  if (read_all(in, host, tensor * (size_t)(n + 1) + wbytes)) {
    fprintf(stderr, "short body\n");
    return 1;
  }
  fclose(in);

  void* d_parts[TW_MAX_PARTIALS];
  void *d_res, *d_res2, *d_w, *d_out, *d_rout, *d_out2;
  for (int i = 0; i < n; ++i) {
    HIP_OK(hipMalloc(&d_parts[i], tensor));
    HIP_OK(hipMemcpy(d_parts[i], host + (size_t)i * tensor, tensor, hipMemcpyHostToDevice));
  }
  HIP_OK(hipMalloc(&d_res, tensor));
  HIP_OK(hipMalloc(&d_res2, tensor));
  HIP_OK(hipMalloc(&d_w, wbytes));
  HIP_OK(hipMalloc(&d_out, tensor));
  HIP_OK(hipMalloc(&d_rout, tensor));
  HIP_OK(hipMalloc(&d_out2, tensor));
  HIP_OK(hipMemcpy(d_res, host + (size_t)n * tensor, tensor, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_res2, host + (size_t)n * tensor, tensor, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, host + (size_t)(n + 1) * tensor, wbytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(d_out, 0, tensor));

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  const void* const* parts = (const void* const*)d_parts;

  /* refused call: nothing enqueued, nothing written */
  tw_status st = tw_fused_reduce_rmsnorm(parts, 0, rows, hidden, (tw_dtype)dtype, d_res, d_w, eps,
                                         d_out, d_rout, 0, s);
  if (st != TW_ERR_INVALID_ARG || tw_last_error()[0] == '\0') {
    fprintf(stderr, "n = 0 gave %d (%s)\n", (int)st, tw_status_string(st));
    return 1;
  }
  fprintf(stderr, "refused as expected: %s: %s\n", tw_status_string(st), tw_last_error());
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(host_out, d_out, tensor, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < tensor; ++i)
    if (host_out[i] != 0) {
      fprintf(stderr, "the refused call wrote to out\n");
      return 1;
    }

  /* out of place */
  st = tw_fused_reduce_rmsnorm(parts, n, rows, hidden, (tw_dtype)dtype, d_res, d_w, eps, d_out,
                               d_rout, 0, s);
  if (st != TW_OK) {
    fprintf(stderr, "fused call: %s: %s\n", tw_status_string(st), tw_last_error());
    return 1;
  }
  /* in place on a second copy of the residual */
  st = tw_fused_reduce_rmsnorm(parts, n, rows, hidden, (tw_dtype)dtype, d_res2, d_w, eps, d_out2,
                               d_res2, 0, s);
  if (st != TW_OK) {
    fprintf(stderr, "in-place call: %s: %s\n", tw_status_string(st), tw_last_error());
    return 1;
  }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(host_out, d_out, tensor, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host_out + tensor, d_rout, tensor, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host, d_out2, tensor, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host + tensor, d_res2, tensor, hipMemcpyDeviceToHost));
  if (memcmp(host, host_out, 2 * tensor) != 0) {
    fprintf(stderr, "in-place and out-of-place results differ\n");
    return 1;
  }

  FILE* out = fopen(argv[2], "wb");
  if (out == NULL || fwrite(host_out, 1, 2 * tensor, out) != 2 * tensor) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(out);

  HIP_OK(hipStreamDestroy(s));
  for (int i = 0; i < n; ++i) HIP_OK(hipFree(d_parts[i]));
  HIP_OK(hipFree(d_res));
  HIP_OK(hipFree(d_res2));
  HIP_OK(hipFree(d_w));
  HIP_OK(hipFree(d_out));
  HIP_OK(hipFree(d_rout));
  HIP_OK(hipFree(d_out2));
  free(host);
  free(host_out);
  fprintf(stderr, "ok\n");
  return 0;
}
