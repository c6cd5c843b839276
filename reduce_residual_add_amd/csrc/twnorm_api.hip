// C-ABI entry points of libtwnorm (declared in include/twnorm.h, and the
// measurement aids in include/twnorm_bench.h).
//
// Each entry point validates its arguments without touching HIP
// (twnorm_validate.cpp), picks the launch shape from (dtype, hidden, n) and
// the call's rows and CUs (every shape gives the same bits), and enqueues one kernel on the caller's stream -- or, for a CU limit, on a
// cached CU-masked stream that is ordered after the caller's stream and
// before its later work by a pair of events (no join when the caller already
// is that masked stream).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <map>
#include <mutex>
#include <vector>

#include "twnorm.h"
#include "twnorm_bench.h"
#include "twnorm_launch.hpp"
#include "twnorm_validate.hpp"

namespace {

struct DeviceState {
  int cus = 0;
  // CU-masked streams: key k > 0 = first k mask bits, k < 0 = complement of
  // the first -k bits
  std::map<int, hipStream_t> masked;
  hipEvent_t ev_in = nullptr;
  hipEvent_t ev_out = nullptr;
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;
// Set by tw_shutdown(): the masked streams and events are gone and are not
// created again.  Guarded by g_mu.
bool g_shut_down = false;

// Report a failed HIP call.  HIP also keeps the error as the thread's sticky
// "last error"; it is read back and cleared here so that it cannot surface
// later in an unrelated caller's launch check.
tw_status hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();
  return twv::fail(TW_ERR_HIP, "%s: %s (hipError %d)", what, hipGetErrorString(e),
                   static_cast<int>(e));
}

// Per-device cache entry for the current device.  Caller holds g_mu.
tw_status device_state(DeviceState** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  DeviceState& d = g_dev[dev];
  if (d.cus == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
    if (cus < 1) return twv::fail(TW_ERR_HIP, "device reports %d CUs", cus);
    d.cus = cus;
  }
  if (d.ev_in == nullptr) {
    e = hipEventCreateWithFlags(&d.ev_in, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    e = hipEventCreateWithFlags(&d.ev_out, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  }
  *out = &d;
  return TW_OK;
}

// CU count of the current device, cached per device without a lock.
tw_status current_device_cus(int* cus_out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus_out = c;
      return TW_OK;
    }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
  if (cus < 1) return twv::fail(TW_ERR_HIP, "device reports %d CUs", cus);
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  *cus_out = cus;
  return TW_OK;
}

void shutdown_at_exit() { (void)tw_shutdown(); }

// CU-masked streams keep the default priority.  Each owns a hardware queue of
// its own, and a process gets few of them (4 by default, shared with the
// ordinary streams), so at most kMaxMaskedStreams distinct masks are cached
// per device, for the life of the process; creating and destroying queues on
// every call is avoided on purpose.
constexpr size_t kMaxMaskedStreams = 3;

// The stream for `key`: > 0, the CUs of the first `key` mask bits (the
// hardware spreads consecutive bits round-robin over the 8 XCDs, then over
// their shader engines); < 0, the CUs the first -key bits leave out (for work
// beside a CU-limited call).  Caller holds g_mu.
tw_status masked_stream(DeviceState& d, int key, hipStream_t* out) {
  auto it = d.masked.find(key);
  if (it != d.masked.end()) {
    *out = it->second;
    return TW_OK;
  }
  if (g_shut_down)
    return twv::fail(TW_ERR_UNSUPPORTED,
                     "tw_shutdown() has released the CU-masked streams; CU-limited calls are "
                     "no longer available in this process");
  if (d.masked.size() >= kMaxMaskedStreams)
    return twv::fail(TW_ERR_UNSUPPORTED,
                     "CU mask %s%d: this process already uses %zu distinct CU masks (the "
                     "maximum; each needs its own hardware queue)",
                     key < 0 ? "complement of " : "", key < 0 ? -key : key, d.masked.size());
  std::vector<uint32_t> mask((d.cus + 31) / 32, 0u);
  const int lo = key > 0 ? 0 : -key, hi = key > 0 ? key : d.cus;
  for (int i = lo; i < hi; ++i) mask[i / 32] |= 1u << (i % 32);
  hipStream_t s = nullptr;
  // The queues must be destroyed while the HIP runtime is still alive: an
  // atexit handler registered now runs before the runtime's own teardown,
  // which was registered when the runtime was loaded.
  static bool registered = false;
  if (!registered) {
    registered = true;
    std::atexit(shutdown_at_exit);
  }
  hipError_t e = hipExtStreamCreateWithCUMask(&s, static_cast<uint32_t>(mask.size()), mask.data());
  if (e != hipSuccess) return hip_fail(e, "hipExtStreamCreateWithCUMask");
  d.masked[key] = s;
  *out = s;
  return TW_OK;
}

// Run `launch(cu_limit, stream)` on the whole chip or on a CU-limited stream.
template <typename F>
tw_status run(int n_cu_limit, hipStream_t caller, const char* what, F&& launch) {
  if (n_cu_limit > 0) {
    int cus = 0;
    tw_status st = current_device_cus(&cus);
    if (st != TW_OK) return st;
    if (n_cu_limit >= cus) n_cu_limit = 0;   // the whole chip
  }
  if (n_cu_limit == 0) {
    hipError_t e = launch(0, caller);
    return e == hipSuccess ? TW_OK : hip_fail(e, what);
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_shut_down)
    return twv::fail(TW_ERR_UNSUPPORTED,
                     "tw_shutdown() has released the CU-masked streams; CU-limited calls are "
                     "no longer available in this process");
  DeviceState* d = nullptr;
  tw_status st = device_state(&d);
  if (st != TW_OK) return st;
  hipStream_t ms = nullptr;
  st = masked_stream(*d, n_cu_limit, &ms);
  if (st != TW_OK) return st;
  if (caller == ms) {
    // already on the masked stream (tw_cu_masked_stream): no join needed
    const hipError_t le = launch(n_cu_limit, ms);
    return le == hipSuccess ? TW_OK : hip_fail(le, what);
  }
  hipError_t e = hipEventRecord(d->ev_in, caller);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = hipStreamWaitEvent(ms, d->ev_in, 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  const hipError_t le = launch(n_cu_limit, ms);
  e = hipEventRecord(d->ev_out, ms);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = hipStreamWaitEvent(caller, d->ev_out, 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  return le == hipSuccess ? TW_OK : hip_fail(le, what);
}

// Everything after validation: shape, device, launch.  `outs` holds the
// destinations of the normalised rows (one buffer for the plain call).
tw_status fused_launch(const void* const* partials, int n, int64_t rows, int64_t hidden,
                       tw_dtype dtype, const void* residual, const void* weight, float eps,
                       const twk::OutPtrs& outs, void* residual_out, int n_cu_limit,
                       void* stream) {
  if (rows == 0) return TW_OK;
  int cus = 0;
  tw_status st = current_device_cus(&cus);
  if (st != TW_OK) return st;
  const int call_cus = (n_cu_limit > 0 && n_cu_limit < cus) ? n_cu_limit : cus;
  twv::Shape sh{};
  st = twv::choose_shape(dtype, hidden, n, rows, call_cus, cus, &sh);
  if (st != TW_OK) return st;

  twl::FusedArgs a{};
  for (int i = 0; i < n; ++i) a.pp.p[i] = static_cast<const twk::u32x4*>(partials[i]);
  a.residual = static_cast<const twk::u32x4*>(residual);
  a.weight = static_cast<const twk::u32x4*>(weight);
  a.outs = outs;
  a.residual_out = static_cast<twk::u32x4*>(residual_out);
  a.rows = rows;
  a.chunks = static_cast<int>(hidden * twv::elem_bytes(dtype) / 16);
  a.hidden_f = static_cast<float>(hidden);
  a.eps = eps;
  twl::Launch L{n, sh.waves, sh.k, sh.team, 0, cus, twv::wgs_per_cu_cap()};
  return run(n_cu_limit, static_cast<hipStream_t>(stream), "fused kernel launch",
             [&](int cu, hipStream_t s) {
               L.cu_limit = cu;
               return twl::launch_fused(dtype == TW_BF16, L, a, s);
             });
}

tw_status fused_impl(const void* const* partials, int n, int64_t rows, int64_t hidden,
                     tw_dtype dtype, const void* residual, const void* weight, float eps,
                     void* out, void* residual_out, int n_cu_limit, void* stream) {
  tw_status st = twv::check_fused(partials, n, rows, hidden, dtype, residual, weight, eps, out,
                                  residual_out, n_cu_limit);
  if (st != TW_OK) return st;
  twk::OutPtrs outs{};
  outs.p[0] = static_cast<twk::u32x4*>(out);
  outs.n = 1;
  outs.row0 = 0;
  return fused_launch(partials, n, rows, hidden, dtype, residual, weight, eps, outs, residual_out,
                      n_cu_limit, stream);
}

}  // namespace

extern "C" {

tw_status tw_fused_reduce_rmsnorm(const void* const* partials, int n, int64_t rows,
                                  int64_t hidden, tw_dtype dtype, const void* residual,
                                  const void* weight, float eps, void* out, void* residual_out,
                                  int n_cu_limit, void* stream) {
  twv::clear_error();
  return fused_impl(partials, n, rows, hidden, dtype, residual, weight, eps, out, residual_out,
                    n_cu_limit, stream);
}

tw_status tw_fused_reduce_rmsnorm_allgather(const void* const* partials, int n, int64_t rows,
                                            int64_t hidden, tw_dtype dtype, const void* residual,
                                            const void* weight, float eps, void* const* ag_outs,
                                            int n_ag, int64_t ag_row_offset,
                                            int64_t ag_total_rows, void* residual_out,
                                            int n_cu_limit, void* stream) {
  twv::clear_error();
  tw_status st = twv::check_fused_allgather(partials, n, rows, hidden, dtype, residual, weight,
                                            eps, ag_outs, n_ag, ag_row_offset, ag_total_rows,
                                            residual_out, n_cu_limit);
  if (st != TW_OK) return st;
  twk::OutPtrs outs{};
  for (int j = 0; j < n_ag; ++j) outs.p[j] = static_cast<twk::u32x4*>(ag_outs[j]);
  outs.n = n_ag;
  outs.row0 = ag_row_offset;
  return fused_launch(partials, n, rows, hidden, dtype, residual, weight, eps, outs, residual_out,
                      n_cu_limit, stream);
}

tw_status tw_rmsnorm(const void* reduced, int64_t rows, int64_t hidden, tw_dtype dtype,
                     const void* residual, const void* weight, float eps, void* out,
                     void* residual_out, int n_cu_limit, void* stream) {
  twv::clear_error();
  const void* parts[1] = {reduced};
  return fused_impl(parts, 1, rows, hidden, dtype, residual, weight, eps, out, residual_out,
                    n_cu_limit, stream);
}

tw_status tw_reduce(const void* const* partials, int n, int64_t rows, int64_t hidden,
                    tw_dtype dtype, void* reduced, int n_cu_limit, void* stream) {
  twv::clear_error();
  tw_status st = twv::check_reduce(partials, n, rows, hidden, dtype, reduced, n_cu_limit);
  if (st != TW_OK) return st;
  if (rows == 0) return TW_OK;
  twk::PartialPtrs pp{};
  for (int i = 0; i < n; ++i) pp.p[i] = static_cast<const twk::u32x4*>(partials[i]);
  const int64_t total = rows * (hidden * twv::elem_bytes(dtype) / 16);
  auto* red = static_cast<twk::u32x4*>(reduced);
  int cus = 0;
  st = current_device_cus(&cus);
  if (st != TW_OK) return st;
  return run(n_cu_limit, static_cast<hipStream_t>(stream), "reduce kernel launch",
             [&](int cu, hipStream_t s) {
               const int grid_cus = cu > 0 ? cu : cus;
               return dtype == TW_BF16 ? twl::launch_reduce_bf16(n, pp, red, total, grid_cus, s)
                                       : twl::launch_reduce_f32(n, pp, red, total, grid_cus, s);
             });
}

static tw_status masked_stream_entry(int n_cu_limit, bool complement, void** stream) {
  twv::clear_error();
  if (stream == nullptr) return twv::fail(TW_ERR_INVALID_ARG, "stream is NULL");
  if (n_cu_limit < 1) return twv::fail(TW_ERR_INVALID_ARG, "n_cu_limit must be >= 1");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_shut_down)
    return twv::fail(TW_ERR_UNSUPPORTED,
                     "tw_shutdown() has released the CU-masked streams");
  DeviceState* d = nullptr;
  tw_status st = device_state(&d);
  if (st != TW_OK) return st;
  if (n_cu_limit >= d->cus)
    return twv::fail(TW_ERR_INVALID_ARG, "n_cu_limit %d is not below the device's %d CUs",
                     n_cu_limit, d->cus);
  hipStream_t ms = nullptr;
  st = masked_stream(*d, complement ? -n_cu_limit : n_cu_limit, &ms);
  if (st != TW_OK) return st;
  *stream = static_cast<void*>(ms);
  return TW_OK;
}

tw_status tw_cu_masked_stream(int n_cu_limit, void** stream) {
  return masked_stream_entry(n_cu_limit, false, stream);
}

tw_status tw_cu_complement_stream(int n_cu_limit, void** stream) {
  return masked_stream_entry(n_cu_limit, true, stream);
}

tw_status tw_shutdown(void) {
  twv::clear_error();
  std::lock_guard<std::mutex> lock(g_mu);
  g_shut_down = true;
  tw_status result = TW_OK;
  for (auto& dev : g_dev) {
    DeviceState& d = dev.second;
    for (auto& m : d.masked) {
      // wait for the stream's work, then release it and its hardware queue
      hipError_t e = hipStreamSynchronize(m.second);
      if (e == hipSuccess) e = hipStreamDestroy(m.second);
      if (e != hipSuccess) result = hip_fail(e, "releasing a CU-masked stream");
    }
    d.masked.clear();
    for (hipEvent_t* ev : {&d.ev_in, &d.ev_out}) {
      if (*ev == nullptr) continue;
      const hipError_t e = hipEventDestroy(*ev);
      if (e != hipSuccess) result = hip_fail(e, "hipEventDestroy");
      *ev = nullptr;
    }
  }
  return result;
}

tw_status tw_stream_copy(const void* src, void* dst, int64_t bytes, int n_cu_limit, void* stream) {
  twv::clear_error();
  tw_status st = twv::check_copy(src, dst, bytes, n_cu_limit);
  if (st != TW_OK) return st;
  if (bytes == 0) return TW_OK;
  return run(n_cu_limit, static_cast<hipStream_t>(stream), "copy kernel launch",
             [&](int cu, hipStream_t s) {
               return twl::launch_copy(static_cast<const twk::u32x4*>(src),
                                       static_cast<twk::u32x4*>(dst), bytes / 16, cu, s);
             });
}

tw_status tw_stream_mix(const void* const* srcs, int n_src, void* const* dsts, int n_dst,
                        int64_t bytes, int n_cu_limit, void* stream) {
  twv::clear_error();
  tw_status st = twv::check_mix(srcs, n_src, dsts, n_dst, bytes, n_cu_limit);
  if (st != TW_OK) return st;
  if (bytes == 0) return TW_OK;
  int cus = 0;
  st = current_device_cus(&cus);
  if (st != TW_OK) return st;
  twk::MixPtrs m{};
  for (int i = 0; i < n_src; ++i) m.src[i] = static_cast<const twk::u32x4*>(srcs[i]);
  for (int j = 0; j < n_dst; ++j) m.dst[j] = static_cast<twk::u32x4*>(dsts[j]);
  m.n_dst = n_dst;
  return run(n_cu_limit, static_cast<hipStream_t>(stream), "mix kernel launch",
             [&](int cu, hipStream_t s) {
               return twl::launch_mix(n_src, m, bytes, cu > 0 ? cu : cus, s);
             });
}

}  // extern "C"
