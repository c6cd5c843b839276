// Host-side argument validation and launch-shape choice (no HIP calls).
#include "twnorm_validate.hpp"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace twv {

namespace {

thread_local char g_err[512] = {0};

// Launch-shape override of tw_set_fused_shape: per host thread, so one
// thread's tuning never changes another thread's calls.
thread_local int g_override_waves = 0;
thread_local int g_override_k = 0;
thread_local int g_wgs_per_cu = 0;

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, int64_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Checks shared by every entry point that takes [rows, hidden] tensors.
tw_status check_shape(int64_t rows, int64_t hidden, tw_dtype dtype, int n_cu_limit,
                      int64_t* tensor_bytes) {
  const int b = elem_bytes(dtype);
  if (b == 0) return fail(TW_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
  if (rows < 0) return fail(TW_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (hidden < 1) return fail(TW_ERR_INVALID_ARG, "hidden must be >= 1 (got %lld)", (long long)hidden);
  if (n_cu_limit < 0) return fail(TW_ERR_INVALID_ARG, "n_cu_limit must be >= 0 (got %d)", n_cu_limit);
  if (hidden > INT64_MAX / 16 / b)
    return fail(TW_ERR_INVALID_ARG, "hidden %lld too large", (long long)hidden);
  const int64_t row_bytes = hidden * b;
  if (rows > 0 && rows > INT64_MAX / row_bytes)
    return fail(TW_ERR_INVALID_ARG, "rows * hidden overflows 64-bit byte counts");
  if (row_bytes % 16 != 0)
    return fail(TW_ERR_UNSUPPORTED, "hidden * sizeof(dtype) = %lld is not a multiple of 16",
                (long long)row_bytes);
  if (row_bytes > TW_MAX_HIDDEN_BYTES)
    return fail(TW_ERR_UNSUPPORTED, "row of %lld bytes exceeds the %d-byte maximum",
                (long long)row_bytes, TW_MAX_HIDDEN_BYTES);
  *tensor_bytes = rows * row_bytes;
  return TW_OK;
}

tw_status check_partials(const void* const* partials, int n) {
  if (partials == nullptr) return fail(TW_ERR_INVALID_ARG, "partials array is NULL");
  if (n < 1 || n > TW_MAX_PARTIALS)
    return fail(TW_ERR_INVALID_ARG, "n must be in [1, %d] (got %d)", TW_MAX_PARTIALS, n);
  for (int i = 0; i < n; ++i)
    if (partials[i] == nullptr) return fail(TW_ERR_INVALID_ARG, "partials[%d] is NULL", i);
  return TW_OK;
}

}  // namespace

int elem_bytes(tw_dtype dtype) {
  switch (dtype) {
    case TW_BF16: return 2;
    case TW_F32: return 4;
  }
  return 0;
}

tw_status fail(tw_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = '\0'; }

const char* last_error() { return g_err; }

// Inputs and residual_out of the fused paths; sets the bytes of one
// [rows, hidden] tensor.
static tw_status check_fused_inputs(const void* const* partials, int n, int64_t rows,
                                    int64_t hidden, tw_dtype dtype, const void* residual,
                                    const void* weight, float eps, const void* residual_out,
                                    int n_cu_limit, int64_t* tensor_bytes) {
  tw_status st = check_partials(partials, n);
  if (st != TW_OK) return st;
  if (residual == nullptr) return fail(TW_ERR_INVALID_ARG, "residual is NULL");
  if (weight == nullptr) return fail(TW_ERR_INVALID_ARG, "weight is NULL");
  if (residual_out == nullptr) return fail(TW_ERR_INVALID_ARG, "residual_out is NULL");
  if (!(eps >= 0.0f) || std::isinf(eps))
    return fail(TW_ERR_INVALID_ARG, "eps must be finite and >= 0 (got %g)", (double)eps);
  st = check_shape(rows, hidden, dtype, n_cu_limit, tensor_bytes);
  if (st != TW_OK) return st;
  for (int i = 0; i < n; ++i)
    if (misaligned(partials[i]))
      return fail(TW_ERR_UNSUPPORTED, "partials[%d] is not 16-byte aligned", i);
  if (misaligned(residual) || misaligned(weight) || misaligned(residual_out))
    return fail(TW_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  const int64_t tb = *tensor_bytes;
  const Span s_res = span(residual, tb), s_rout = span(residual_out, tb),
             s_w = span(weight, hidden * elem_bytes(dtype));
  for (int i = 0; i < n; ++i)
    if (overlap(s_rout, span(partials[i], tb)))
      return fail(TW_ERR_ALIAS, "residual_out overlaps partials[%d]", i);
  if (overlap(s_rout, s_w)) return fail(TW_ERR_ALIAS, "residual_out overlaps weight");
  if (residual_out != residual && overlap(s_rout, s_res))
    return fail(TW_ERR_ALIAS, "residual_out partially overlaps residual");
  return TW_OK;
}

// An output span may overlap no input, residual_out or other output.
static tw_status check_output_span(const char* name, Span s_o, const void* const* partials, int n,
                                   int64_t tb, const void* residual, const void* weight,
                                   int64_t wb, const void* residual_out) {
  for (int i = 0; i < n; ++i)
    if (overlap(s_o, span(partials[i], tb)))
      return fail(TW_ERR_ALIAS, "%s overlaps partials[%d]", name, i);
  if (overlap(s_o, span(residual, tb))) return fail(TW_ERR_ALIAS, "%s overlaps residual", name);
  if (overlap(s_o, span(weight, wb))) return fail(TW_ERR_ALIAS, "%s overlaps weight", name);
  if (overlap(s_o, span(residual_out, tb)))
    return fail(TW_ERR_ALIAS, "%s overlaps residual_out", name);
  return TW_OK;
}

tw_status check_fused(const void* const* partials, int n, int64_t rows, int64_t hidden,
                      tw_dtype dtype, const void* residual, const void* weight, float eps,
                      const void* out, const void* residual_out, int n_cu_limit) {
  if (out == nullptr) return fail(TW_ERR_INVALID_ARG, "out is NULL");
  int64_t tb = 0;
  tw_status st = check_fused_inputs(partials, n, rows, hidden, dtype, residual, weight, eps,
                                    residual_out, n_cu_limit, &tb);
  if (st != TW_OK) return st;
  if (misaligned(out)) return fail(TW_ERR_UNSUPPORTED, "out is not 16-byte aligned");
  return check_output_span("out", span(out, tb), partials, n, tb, residual, weight,
                           hidden * elem_bytes(dtype), residual_out);
}

tw_status check_fused_allgather(const void* const* partials, int n, int64_t rows, int64_t hidden,
                                tw_dtype dtype, const void* residual, const void* weight,
                                float eps, const void* const* ag_outs, int n_ag,
                                int64_t ag_row_offset, int64_t ag_total_rows,
                                const void* residual_out, int n_cu_limit) {
  if (ag_outs == nullptr) return fail(TW_ERR_INVALID_ARG, "ag_outs array is NULL");
  if (n_ag < 1 || n_ag > TW_MAX_PARTIALS)
    return fail(TW_ERR_INVALID_ARG, "n_ag must be in [1, %d] (got %d)", TW_MAX_PARTIALS, n_ag);
  for (int j = 0; j < n_ag; ++j)
    if (ag_outs[j] == nullptr) return fail(TW_ERR_INVALID_ARG, "ag_outs[%d] is NULL", j);
  if (ag_row_offset < 0) return fail(TW_ERR_INVALID_ARG, "ag_row_offset must be >= 0");
  int64_t tb = 0;
  tw_status st = check_fused_inputs(partials, n, rows, hidden, dtype, residual, weight, eps,
                                    residual_out, n_cu_limit, &tb);
  if (st != TW_OK) return st;
  if (ag_total_rows < 0 || ag_row_offset > ag_total_rows - rows)
    return fail(TW_ERR_INVALID_ARG, "rows [%lld, %lld) do not fit the %lld-row gather buffers",
                (long long)ag_row_offset, (long long)(ag_row_offset + rows),
                (long long)ag_total_rows);
  const int64_t row_bytes = hidden * elem_bytes(dtype);
  if (ag_total_rows > INT64_MAX / row_bytes)
    return fail(TW_ERR_INVALID_ARG, "gather buffer size overflows 64-bit byte counts");
  const int64_t gb = ag_total_rows * row_bytes;
  char name[32];
  for (int j = 0; j < n_ag; ++j) {
    if (misaligned(ag_outs[j]))
      return fail(TW_ERR_UNSUPPORTED, "ag_outs[%d] is not 16-byte aligned", j);
    snprintf(name, sizeof(name), "ag_outs[%d]", j);
    st = check_output_span(name, span(ag_outs[j], gb), partials, n, tb, residual, weight,
                           row_bytes, residual_out);
    if (st != TW_OK) return st;
    for (int i = 0; i < j; ++i)
      if (overlap(span(ag_outs[j], gb), span(ag_outs[i], gb)))
        return fail(TW_ERR_ALIAS, "ag_outs[%d] overlaps ag_outs[%d]", j, i);
  }
  return TW_OK;
}

tw_status check_reduce(const void* const* partials, int n, int64_t rows, int64_t hidden,
                       tw_dtype dtype, const void* reduced, int n_cu_limit) {
  tw_status st = check_partials(partials, n);
  if (st != TW_OK) return st;
  if (reduced == nullptr) return fail(TW_ERR_INVALID_ARG, "reduced is NULL");
  int64_t tb = 0;
  st = check_shape(rows, hidden, dtype, n_cu_limit, &tb);
  if (st != TW_OK) return st;
  for (int i = 0; i < n; ++i)
    if (misaligned(partials[i]))
      return fail(TW_ERR_UNSUPPORTED, "partials[%d] is not 16-byte aligned", i);
  if (misaligned(reduced)) return fail(TW_ERR_UNSUPPORTED, "reduced is not 16-byte aligned");
  const Span s_red = span(reduced, tb);
  for (int i = 0; i < n; ++i)
    if (partials[i] != reduced && overlap(s_red, span(partials[i], tb)))
      return fail(TW_ERR_ALIAS, "reduced partially overlaps partials[%d]", i);
  return TW_OK;
}

tw_status check_copy(const void* src, const void* dst, int64_t bytes, int n_cu_limit) {
  if (src == nullptr || dst == nullptr) return fail(TW_ERR_INVALID_ARG, "src or dst is NULL");
  if (bytes < 0) return fail(TW_ERR_INVALID_ARG, "bytes must be >= 0");
  if (n_cu_limit < 0) return fail(TW_ERR_INVALID_ARG, "n_cu_limit must be >= 0");
  if (bytes % 16 != 0) return fail(TW_ERR_UNSUPPORTED, "bytes must be a multiple of 16");
  if (misaligned(src) || misaligned(dst))
    return fail(TW_ERR_UNSUPPORTED, "src and dst must be 16-byte aligned");
  if (overlap(span(src, bytes), span(dst, bytes))) return fail(TW_ERR_ALIAS, "src and dst overlap");
  return TW_OK;
}

tw_status check_mix(const void* const* srcs, int n_src, const void* const* dsts, int n_dst,
                    int64_t bytes, int n_cu_limit) {
  if (srcs == nullptr || dsts == nullptr) return fail(TW_ERR_INVALID_ARG, "srcs or dsts is NULL");
  if (n_src < 1 || n_src > TW_MAX_PARTIALS + 1)
    return fail(TW_ERR_INVALID_ARG, "n_src must be in [1, %d]", TW_MAX_PARTIALS + 1);
  if (n_dst < 1 || n_dst > TW_MAX_PARTIALS)
    return fail(TW_ERR_INVALID_ARG, "n_dst must be in [1, %d]", TW_MAX_PARTIALS);
  if (bytes < 0) return fail(TW_ERR_INVALID_ARG, "bytes must be >= 0");
  if (n_cu_limit < 0) return fail(TW_ERR_INVALID_ARG, "n_cu_limit must be >= 0");
  for (int i = 0; i < n_src; ++i)
    if (srcs[i] == nullptr) return fail(TW_ERR_INVALID_ARG, "srcs[%d] is NULL", i);
  for (int j = 0; j < n_dst; ++j)
    if (dsts[j] == nullptr) return fail(TW_ERR_INVALID_ARG, "dsts[%d] is NULL", j);
  if (bytes % 16 != 0) return fail(TW_ERR_UNSUPPORTED, "bytes must be a multiple of 16");
  for (int i = 0; i < n_src; ++i)
    if (misaligned(srcs[i])) return fail(TW_ERR_UNSUPPORTED, "srcs[%d] is not 16-byte aligned", i);
  for (int j = 0; j < n_dst; ++j) {
    if (misaligned(dsts[j])) return fail(TW_ERR_UNSUPPORTED, "dsts[%d] is not 16-byte aligned", j);
    const Span d = span(dsts[j], bytes);
    for (int i = 0; i < n_src; ++i)
      if (overlap(d, span(srcs[i], bytes)))
        return fail(TW_ERR_ALIAS, "dsts[%d] overlaps srcs[%d]", j, i);
    for (int k = 0; k < j; ++k)
      if (overlap(d, span(dsts[k], bytes)))
        return fail(TW_ERR_ALIAS, "dsts[%d] overlaps dsts[%d]", j, k);
  }
  return TW_OK;
}

// Register-fit table of the wide-row kernels, generated at build time from the
// compiler's resource remarks (reduce_residual_add_amd/build.py): which chunk
// counts K run without scratch for each (dtype, n, launch bound).
#include "twnorm_fit_table.inc"

static const int kAllowedK[] = {1, 2, 3, 4, 6, 8};

static int k_index(int k) {
  for (int i = 0; i < 6; ++i)
    if (kKValues[i] == k) return i;
  return -1;
}

static int bucket_of(int waves) { return waves <= 4 ? 0 : (waves <= 8 ? 1 : 2); }

bool shape_spills(tw_dtype dtype, int n, int waves, int k) {
  const int ki = k_index(k);
  if (ki < 0 || n < 1 || n > 16) return true;
  const int dt = dtype == TW_BF16 ? 0 : 1;
  return ((kFitMask[dt][n][bucket_of(waves)] >> ki) & 1) == 0;
}

// Shapes measured fastest on MI355X (HBM-resident inputs, every K with its
// fewest covering waves timed at 1024 and 4096 rows, one workgroup per row,
// partials loaded in groups where a whole row exceeds the register target)
// for row widths used in practice.  Widths and partial counts not listed take
// the default rule below, which won the rest of the sweep (for example 4 x 6
// on 12288-wide rows with 4-16 partials and 4 x 8 on 16384-wide rows with
// 4-16 partials).
struct TunedShape {
  int elem_bytes;
  int64_t chunks;
  int n_lo, n_hi;
  int waves, k;
};
static const TunedShape kTuned[] = {
    {2, 1024, 5, 16, 4, 4},  // 8192 bf16 features, many partials
    {2, 1024, 1, 3, 8, 2},   // 8192 bf16 features, few partials
    {2, 512, 1, 2, 1, 8},    // 4096 bf16, 1-2 partials: one wave per row, no barrier (+3%)
    {2, 512, 3, 5, 8, 1},    // 4096 bf16, 3-5 partials (+1-6% over 4 x 2 and 1 x 8)
    {2, 512, 6, 16, 1, 8},   // 4096 bf16, 6-16 partials (+8-11% over 4 x 2)
    {2, 640, 1, 2, 5, 2},    // 5120 bf16 features, 1-2 partials: every lane busy (+4% over 4 x 3)
    {2, 896, 1, 3, 7, 2},    // 7168 bf16 features, few partials (+4% over 4 x 4 at 1024 rows)
    {2, 1536, 1, 3, 12, 2},  // 12288 bf16 features, few partials
    {2, 2048, 1, 1, 16, 2},  // 16384 bf16 features, one partial (+10% over 4 x 8)
    {2, 2048, 2, 2, 8, 4},   // 16384 bf16 features, two partials (+4% over 4 x 8)
    // 2560-3584 bf16 features: each entry gained over the 4 x 2 default at
    // both 1024 and 4096 rows; partial counts where no shape did keep it
    {2, 320, 2, 5, 5, 1},    // 2560 bf16, 2-5 partials: every lane busy (+0.2-3.5%)
    {2, 320, 8, 8, 5, 1},    // 2560 bf16, 8 partials (+0.3-1.6%)
    {2, 384, 2, 2, 3, 2},    // 3072 bf16, 2 partials (+0.3-1.3%)
    {2, 384, 3, 4, 6, 1},    // 3072 bf16, 3-4 partials (+0.2-2.9%)
    {2, 384, 8, 16, 1, 6},   // 3072 bf16, 8-16 partials: one wave per row (+2.7-5.8%)
    {2, 448, 3, 4, 7, 1},    // 3584 bf16, 3-4 partials (+0.3-2.9%)
    {2, 448, 8, 16, 1, 8},   // 3584 bf16, 8-16 partials: one wave per row (+1.3-8.4%)
};

// Shapes measured fastest when a call runs on at most half of the CUs: on 8,
// 16, 32 and 64 CUs, 8 x 2 beats the whole-chip 4 x 4 by 4-6% on 8192-wide
// rows with 8 partials; on 8 and 32 CUs, 10 x 1 beats 8 x 2 by 15-20% on
// 5120-wide rows with 4 partials (every lane busy, three rows in flight per
// CU) and the whole-chip 4 x 3 by 1-14% with 8-16 partials; 7 x 2 beats the
// whole-chip 4 x 4 by 1-10% on 7168-wide rows with 4-12 partials (not 16);
// 8 x 3 beats the whole-chip default 4 x 6 by 1-7% on 12288-wide rows with
// 1-4 partials (not 8; the whole-chip 12 x 2 exceeds the limited calls'
// workgroups); 2 x 4 beats 8 x 1 by 3-5% on 4096-wide rows with 2 partials
// and by 1-2% with 4.
static const TunedShape kTunedLimited[] = {
    {2, 1024, 5, 16, 8, 2},
    {2, 640, 3, 16, 10, 1},
    {2, 896, 4, 12, 7, 2},
    {2, 1536, 1, 4, 8, 3},
    {2, 512, 1, 4, 2, 4},
};

// The whole-chip shape of a wide row:
//  * a measured shape for this (width, n) if it spills nothing;
//  * else, for rows of at most 256 chunks, one wavefront with the fewest
//    chunk slots per lane that cover the row, if that spills nothing: no
//    idle wavefront and no barrier.  Measured on MI355X at about 256 MB per
//    call with 2 and 8 partials: on 64-chunk rows (512 bf16 or 256 fp32
//    features) 1 x 1 takes 41-42 us against 49-57 us with 4 x 1, within
//    1.07 of the arithmetic-free traffic pattern; on 96-256 chunks it is the
//    fastest shape or within 1.1% of it (3-9% faster than 4 x 1 at 256).
//    On 8 and 32 CUs it is faster still against 4 x 1: 2.0-2.3x on 64
//    chunks, 1.16-1.30x on 128, 1.02-1.05x on 256;
//  * else 4 wavefronts with the fewest chunk slots per lane that cover the
//    row, if that spills nothing;
//  * else, for each K the fewest wavefronts W <= 16 that cover the row, and
//    among the spill-free (W, K) the fewest idle chunk slots (ties: smaller
//    K); if every candidate spills, the fewest idle slots regardless.
static tw_status throughput_shape(tw_dtype dtype, int b, int64_t chunks, int64_t hidden, int n,
                                  int max_waves, Shape* shape) {
  for (const TunedShape& t : kTuned) {
    if (t.elem_bytes == b && t.chunks == chunks && n >= t.n_lo && n <= t.n_hi &&
        t.waves <= max_waves && !shape_spills(dtype, n, t.waves, t.k)) {
      *shape = Shape{t.waves, t.k, 0};
      return TW_OK;
    }
  }
  if (chunks <= 256) {
    for (int k : kAllowedK) {
      if (64 * k >= chunks) {
        if (!shape_spills(dtype, n, 1, k)) {
          *shape = Shape{1, k, 0};
          return TW_OK;
        }
        break;
      }
    }
  }
  for (int k : kAllowedK) {
    if (4 * 64 * k >= chunks) {
      if (!shape_spills(dtype, n, 4, k)) {
        *shape = Shape{4, k, 0};
        return TW_OK;
      }
      break;
    }
  }
  int best_w = 0, best_k = 0, any_w = 0, any_k = 0;
  int64_t best_waste = -1, any_waste = -1;
  for (int k : kAllowedK) {
    const int64_t w = (chunks + 64 * k - 1) / (64 * k);
    if (w > max_waves) continue;
    const int64_t waste = w * 64 * k - chunks;
    if (any_waste < 0 || waste < any_waste) {
      any_waste = waste;
      any_w = (int)w;
      any_k = k;
    }
    if (!shape_spills(dtype, n, (int)w, k) && (best_waste < 0 || waste < best_waste)) {
      best_waste = waste;
      best_w = (int)w;
      best_k = k;
    }
  }
  if (any_waste < 0)
    return fail(TW_ERR_UNSUPPORTED, "hidden %lld too wide for workgroups of at most %d wavefronts",
                (long long)hidden, max_waves);
  *shape = best_waste >= 0 ? Shape{best_w, best_k, 0} : Shape{any_w, any_k, 0};
  return TW_OK;
}

// Widest workgroup, in wavefronts, that a CU-limited call launches: 640
// threads, the widest shape the GPU tests run on CU-masked queues.  An
// exploratory probe that ran 1024-thread workgroups (with register loads and
// with direct-to-LDS loads) on an 8-CU mask stalled, cause not established;
// 1024-thread workgroups had run on a 32-CU mask before.  Until the cause is
// known, CU-limited calls stay on the tested sizes.
constexpr int kMaxLimitedWaves = 10;

// Automatic shape.  The results do not depend on it (the order of every
// addition is fixed by the row width), so it may follow the call:
//  * rows of at most 32 chunks: narrow-row kernel, smallest power-of-two team;
//  * fewer rows than CUs (decode-sized calls, one workgroup per row, most CUs
//    idle): as many wavefronts as the row fills (at most 16, or
//    kMaxLimitedWaves on a CU-limited call) with the fewest chunk slots per
//    lane, so each lane issues the fewest loads in a row, if that spills
//    nothing;
//  * else the whole-chip shape above, or, when the call runs on at most half
//    of the device's CUs, a shape measured for that regime if there is one.
// A CU-limited call never uses more than kMaxLimitedWaves wavefronts per
// workgroup, so rows wider than kMaxLimitedWaves x 64 x 8 chunks (40960 bf16)
// return TW_ERR_UNSUPPORTED there.
tw_status choose_shape(tw_dtype dtype, int64_t hidden, int n, int64_t rows, int cus, int device_cus,
                       Shape* shape) {
  const int b = elem_bytes(dtype);
  if (b == 0) return fail(TW_ERR_INVALID_ARG, "unknown dtype");
  if (n < 1 || n > TW_MAX_PARTIALS) return fail(TW_ERR_INVALID_ARG, "n out of range");
  const int64_t chunks = hidden * b / 16;
  const bool limited = cus < device_cus;
  const int max_waves = limited ? kMaxLimitedWaves : 16;
  const int ow = g_override_waves, ok = g_override_k;
  if (ow > 0 && ok > 0) {
    if ((int64_t)ow * 64 * ok < chunks)
      return fail(TW_ERR_UNSUPPORTED, "forced shape %d waves x %d chunks cannot cover %lld chunks",
                  ow, ok, (long long)chunks);
    if (ow > max_waves)
      return fail(TW_ERR_UNSUPPORTED,
                  "forced shape of %d waves exceeds the %d-wavefront workgroups of CU-limited calls",
                  ow, max_waves);
    *shape = Shape{ow, ok, 0};
    return TW_OK;
  }
  if (chunks <= 32) {
    int team = 1;
    while (team < chunks) team <<= 1;
    *shape = Shape{0, 0, team};
    return TW_OK;
  }
  if (rows < cus) {
    const int64_t w = std::min<int64_t>(max_waves, (chunks + 63) / 64);
    for (int k : kAllowedK) {
      if (w * 64 * k >= chunks) {
        if (!shape_spills(dtype, n, (int)w, k)) {
          *shape = Shape{(int)w, k, 0};
          return TW_OK;
        }
        break;
      }
    }
  }
  Shape t{};
  tw_status st = throughput_shape(dtype, b, chunks, hidden, n, max_waves, &t);
  if (st != TW_OK) return st;
  // On at most half of the device's CUs a call is bound by what each CU
  // issues and keeps in flight, not by HBM, and other shapes win there.
  if (2 * (int64_t)cus <= device_cus) {
    for (const TunedShape& u : kTunedLimited) {
      if (u.elem_bytes == b && u.chunks == chunks && n >= u.n_lo && n <= u.n_hi &&
          u.waves <= max_waves && !shape_spills(dtype, n, u.waves, u.k)) {
        t = Shape{u.waves, u.k, 0};
        break;
      }
    }
  }
  *shape = t;
  return TW_OK;
}

tw_status set_override(int waves, int k, int wgs_per_cu) {
  bool k_ok = (k == 0);
  for (int a : kAllowedK) k_ok = k_ok || (a == k);
  if (waves < 0 || waves > 16 || !k_ok || ((waves == 0) != (k == 0)) || wgs_per_cu < 0)
    return fail(TW_ERR_INVALID_ARG, "invalid forced shape (%d waves, %d chunks per lane, %d per CU)",
                waves, k, wgs_per_cu);
  g_override_waves = waves;
  g_override_k = k;
  g_wgs_per_cu = wgs_per_cu;
  return TW_OK;
}

int wgs_per_cu_cap() { return g_wgs_per_cu; }

}  // namespace twv

// ---------------------------------------------------------------------------
// HIP-free exported entry points
// ---------------------------------------------------------------------------
#include "twnorm_bench.h"

extern "C" {

const char* tw_status_string(tw_status s) {
  switch (s) {
    case TW_OK: return "TW_OK";
    case TW_ERR_INVALID_ARG: return "TW_ERR_INVALID_ARG";
    case TW_ERR_UNSUPPORTED: return "TW_ERR_UNSUPPORTED";
    case TW_ERR_ALIAS: return "TW_ERR_ALIAS";
    case TW_ERR_HIP: return "TW_ERR_HIP";
  }
  return "TW_UNKNOWN_STATUS";
}

const char* tw_last_error(void) { return twv::last_error(); }

int tw_abi_version(void) { return TW_ABI_VERSION; }

tw_status tw_set_fused_shape(int waves, int chunks_per_lane, int wgs_per_cu) {
  twv::clear_error();
  return twv::set_override(waves, chunks_per_lane, wgs_per_cu);
}

tw_status tw_query_fused_shape(tw_dtype dtype, int64_t hidden, int n, int64_t rows, int cus,
                               int device_cus, int* waves, int* chunks_per_lane,
                               int* team_lanes) {
  twv::clear_error();
  if (waves == nullptr || chunks_per_lane == nullptr || team_lanes == nullptr)
    return twv::fail(TW_ERR_INVALID_ARG, "output pointer is NULL");
  const int b = twv::elem_bytes(dtype);
  if (b == 0) return twv::fail(TW_ERR_INVALID_ARG, "unknown dtype");
  if (hidden < 1) return twv::fail(TW_ERR_INVALID_ARG, "hidden must be >= 1");
  if ((hidden * b) % 16 != 0) return twv::fail(TW_ERR_UNSUPPORTED, "row bytes not a multiple of 16");
  if (hidden * b > TW_MAX_HIDDEN_BYTES) return twv::fail(TW_ERR_UNSUPPORTED, "row too wide");
  if (rows < 0) return twv::fail(TW_ERR_INVALID_ARG, "rows must be >= 0");
  if (cus < 1 || device_cus < cus)
    return twv::fail(TW_ERR_INVALID_ARG, "need 1 <= cus <= device_cus (got %d, %d)", cus, device_cus);
  twv::Shape s{};
  tw_status st = twv::choose_shape(dtype, hidden, n, rows, cus, device_cus, &s);
  if (st != TW_OK) return st;
  *waves = s.waves;
  *chunks_per_lane = s.k;
  *team_lanes = s.team;
  return TW_OK;
}

}  // extern "C"
