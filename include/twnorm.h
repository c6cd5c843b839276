/*
 * twnorm.h -- C ABI of libtwnorm: fused "reduce N tensor-parallel partial
 * outputs + residual add + RMSNorm * weight" for one GPU's token-sharded rows,
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [TW] "TokenWeave 策略详解：以大模型推理为例" (nanhubrain.csdn.net)
 *   [TP] "张量并行Tensor Parallelism" (scmmm.top)
 *   [TWS] "TokenWeave: Efficient Compute-Communication Overlap for
 *         Distributed LLM Inference" (gist.science lay summary)
 *
 * What is computed, per token row t and feature j (float32 arithmetic):
 *   s[t,j]            = p_0[t,j] + p_1[t,j] + ... + p_{n-1}[t,j]   (index order)
 *   x[t,j]            = residual[t,j] + s[t,j]
 *   residual_out[t,j] = round(x[t,j])
 *   out[t,j]          = round(x[t,j] * rsqrt(mean_j' x[t,j']^2 + eps) * weight[j])
 * where the mean runs over all `hidden` features of the token and round() is
 * round-to-nearest-even into the storage type.  The sum of partials is the
 * per-shard half of a token-boundary ReduceScatter ([TW] §2, §3.2; the
 * appendix's zero-padded column partials, and [TP] MLP: Y = sum_i Y_i); the
 * add + norm is [TW] §1's  output = RMSNorm(residual + allreduce_output) *
 * weight, run on this shard's rows only ([TW] §3.3); the new residual is the
 * X = X + Y update of [TP] Self-Attention, fused in registers as in [TW] §5.
 *
 * Common conventions (every entry point):
 *   Layout     Each of partials[i], residual, out, residual_out, reduced is a
 *              row-major contiguous [rows, hidden] array of `dtype`; weight is
 *              [hidden] of `dtype`.  A token shard is a row range, so callers
 *              pass pointers already offset to the shard's first row.
 *   Memory     All data pointers are device pointers owned by the caller.  The
 *              library never allocates, frees or keeps them after returning.
 *              The host array `partials` is read during the call only.
 *   Device     The pointers and `stream` belong to the current HIP device
 *              (hipGetDevice), whose CU count and CU-masked streams the call
 *              uses.  This is not checked (it would cost a runtime query per
 *              pointer): memory of another device is then accessed from this
 *              one.  The Python binding checks it.
 *   Execution  Asynchronous: work is enqueued on `stream` (a hipStream_t
 *              passed as an opaque pointer; NULL = the null stream) and the
 *              call returns.  No device synchronisation, no allocation.
 *   Errors     Arguments are validated first, without any HIP call; on an
 *              error nothing is enqueued and nothing is written.
 *                TW_ERR_INVALID_ARG  null pointer, n outside [1, 16], rows < 0,
 *                                    hidden < 1, eps negative / NaN / Inf,
 *                                    n_cu_limit < 0, unknown dtype, or
 *                                    rows * hidden too large for 64-bit bytes.
 *                TW_ERR_UNSUPPORTED  hidden * sizeof(dtype) not a multiple of
 *                                    16, a pointer not 16-byte aligned,
 *                                    hidden beyond TW_MAX_HIDDEN_BYTES bytes,
 *                                    a fourth distinct n_cu_limit, or a
 *                                    CU limit after tw_shutdown().
 *                TW_ERR_ALIAS        an output overlaps an input it may not
 *                                    (rules per entry point below).
 *                TW_ERR_HIP          a HIP runtime call or the launch failed;
 *                                    tw_last_error() has the HIP message.
 *              rows == 0 is a no-op returning TW_OK (after validation).
 *              Faults inside a kernel surface at the caller's next
 *              synchronisation, as for any HIP launch.
 *   n_cu_limit 0, or any value >= the device's CU count, uses the whole chip.
 *              k in [1, CUs) runs the kernel on at most k CUs (persistent grid
 *              on a cached CU-masked stream, ordered after and before `stream`
 *              by events).  Results are bit-identical for every n_cu_limit.
 *              Such calls launch workgroups of at most 10 wavefronts, so rows
 *              wider than 40960 bf16 (20480 fp32) features return
 *              TW_ERR_UNSUPPORTED with a CU limit.  Under HIP-graph capture
 *              a CU-limited call is captured with its event join and replays
 *              with the same results, but a graph node carries no CU mask:
 *              replayed on another stream, its grid (sized for k CUs) is not
 *              confined to them; replayed on tw_cu_masked_stream(k), it is.
 *              Each distinct CU mask needs a hardware queue of its own until
 *              tw_shutdown(): at most 3 distinct masks (limits k, and
 *              complements from tw_cu_complement_stream) per device and
 *              process; a fourth returns TW_ERR_UNSUPPORTED.
 *   Determinism The order of every addition depends only on (dtype, hidden,
 *              n): partials in index order per element, squares summed per
 *              16-byte chunk, then per group of 64 consecutive chunks by a
 *              fixed pairwise tree, then group by group in row order.  The
 *              same row gives the same bits whatever rows, shard offset,
 *              n_cu_limit or launch shape are.
 *   Threads    Entry points may be called from several host threads; the
 *              per-device cache (CU count, masked streams) is mutex-guarded.
 */
#ifndef TWNORM_H
#define TWNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TW_OK = 0,
  TW_ERR_INVALID_ARG = -1,
  TW_ERR_UNSUPPORTED = -2,
  TW_ERR_ALIAS = -3,
  TW_ERR_HIP = -4
} tw_status;

typedef enum { TW_BF16 = 0, TW_F32 = 1 } tw_dtype;

#define TW_ABI_VERSION 4
#define TW_MAX_PARTIALS 16
/* Largest supported row: 16 waves x 64 lanes x 8 chunks of 16 bytes. */
#define TW_MAX_HIDDEN_BYTES (16 * 64 * 8 * 16)

/*
 * Fused path: out = RMSNorm(residual + sum_i partials[i]) * weight and
 * residual_out = residual + sum_i partials[i], in one pass over HBM.
 *   partials      host array of n device pointers, each [rows, hidden]
 *   n             number of partials, 1..TW_MAX_PARTIALS
 *   rows, hidden  shard size in token rows and features per token
 *   dtype         storage type of every tensor (arithmetic is float32)
 *   residual      [rows, hidden] input
 *   weight        [hidden]
 *   eps           added to the mean square inside the square root, >= 0
 *   out           [rows, hidden] normalised output
 *   residual_out  [rows, hidden] updated residual; may be exactly `residual`
 *                 (in-place update) but may not overlap it partially
 *   n_cu_limit, stream   see above
 * Alias rules: out may not overlap any input or residual_out; residual_out
 * may not overlap a partial or weight, nor residual except by equality.
 */
tw_status tw_fused_reduce_rmsnorm(const void* const* partials, int n, int64_t rows,
                                  int64_t hidden, tw_dtype dtype, const void* residual,
                                  const void* weight, float eps, void* out,
                                  void* residual_out, int n_cu_limit, void* stream);

/*
 * Fused path with the AllGather store: the same computation as
 * tw_fused_reduce_rmsnorm, with the normalised rows written into each of n_ag
 * gather buffers at rows [ag_row_offset, ag_row_offset + rows) instead of one
 * `out` ([TW] §3.4: every rank ends with the full normalised sequence; §5: the
 * fused kernel stores its result straight into the AllGather targets).  On one
 * GPU the n_ag local buffers stand for the ranks' gather buffers; running the
 * N token shards (offsets r * rows) fills every buffer with all T rows.
 *   ag_outs        host array of n_ag device pointers, each a row-major
 *                  [ag_total_rows, hidden] buffer of `dtype`
 *   n_ag           1..TW_MAX_PARTIALS
 *   ag_row_offset  first gather-buffer row this shard writes
 *   ag_total_rows  rows of each gather buffer; ag_row_offset + rows must fit
 * Rows outside [ag_row_offset, ag_row_offset + rows) are not touched.
 * Alias rules: the gather buffers (whole) are pairwise disjoint and overlap no
 * input and not residual_out; residual_out as in tw_fused_reduce_rmsnorm.
 */
tw_status tw_fused_reduce_rmsnorm_allgather(const void* const* partials, int n, int64_t rows,
                                            int64_t hidden, tw_dtype dtype, const void* residual,
                                            const void* weight, float eps, void* const* ag_outs,
                                            int n_ag, int64_t ag_row_offset,
                                            int64_t ag_total_rows, void* residual_out,
                                            int n_cu_limit, void* stream);

/*
 * Unfused comparison path, first half: reduced = round(sum_i partials[i]),
 * the reduce of a ReduceScatter written to HBM ([TW] §4: the intermediate
 * makes a round trip through HBM).  `reduced` may be exactly one of the
 * partials (in place) but may not overlap any partially.
 */
tw_status tw_reduce(const void* const* partials, int n, int64_t rows, int64_t hidden,
                    tw_dtype dtype, void* reduced, int n_cu_limit, void* stream);

/*
 * Unfused comparison path, second half: residual_out = residual + reduced and
 * out = RMSNorm(residual_out) * weight ([TW] §1 formula, §3.3), reading the
 * reduced tensor back from HBM.  Same alias rules as the fused path with
 * `reduced` in the place of the partials.  Identical in results to
 * tw_fused_reduce_rmsnorm with n = 1 and partials = {reduced}.
 */
tw_status tw_rmsnorm(const void* reduced, int64_t rows, int64_t hidden, tw_dtype dtype,
                     const void* residual, const void* weight, float eps, void* out,
                     void* residual_out, int n_cu_limit, void* stream);

/*
 * The library's CU-masked stream for `n_cu_limit` on the current device
 * (created on first use and owned by the library until tw_shutdown(); never
 * destroy it yourself).  Its kernels run only on the CUs of the first
 * n_cu_limit mask bits, which the hardware spreads round-robin over the 8
 * XCDs and then their shader engines.  Calls made on this stream with the
 * same n_cu_limit launch directly, without the per-call event join to the
 * caller's stream: a caller can queue a batch of calls there and order the
 * batch against its other streams itself.  n_cu_limit must be in [1, CUs).
 * Counts toward the 3 distinct limits a process may use.
 */
tw_status tw_cu_masked_stream(int n_cu_limit, void** stream);

/*
 * The library's stream restricted to the CUs that the first n_cu_limit mask
 * bits leave out: other work, such as the GEMM of the other token split, can
 * run there beside CU-limited fused calls without sharing CUs with them (the
 * two-split overlap of [TWS]).  Same ownership and limits as
 * tw_cu_masked_stream; it counts toward the 3 distinct masks of a process.
 */
tw_status tw_cu_complement_stream(int n_cu_limit, void** stream);

/*
 * Ordered teardown of the library's per-device resources: for every device
 * the library used, waits for the work queued on its CU-masked streams, then
 * destroys those streams (and their hardware queues) and the two events that
 * join them to callers' streams.  The HIP runtime must still be alive, so the
 * library registers this function with atexit() when it creates its first
 * CU-masked stream (such a handler runs before the runtime's own teardown),
 * and a caller may call it earlier, e.g. from a language runtime's exit hook.
 * Idempotent.  Afterwards whole-chip calls keep working, while CU-limited
 * calls and the two stream queries return TW_ERR_UNSUPPORTED: the queues are
 * not created a second time.  Streams obtained from tw_cu_masked_stream or
 * tw_cu_complement_stream are invalid after it.  Returns TW_ERR_HIP if a
 * synchronisation or destroy call failed (the rest are still released).
 */
tw_status tw_shutdown(void);

const char* tw_status_string(tw_status s);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* tw_last_error(void);
int tw_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TWNORM_H */
