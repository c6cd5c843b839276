/*
 * twnorm_bench.h -- measurement and tuning entry points of libtwnorm.  They
 * are not part of the method: a caller of the fused reduce + RMSNorm path
 * needs only twnorm.h.  These exist to measure the HBM ceilings the fused
 * kernel is compared with, to scale hardware traffic counters, and to sweep
 * or inspect the fused kernel's launch shape.  Same conventions (layout,
 * ownership, asynchronous execution, errors, n_cu_limit) as twnorm.h.
 */
#ifndef TWNORM_BENCH_H
#define TWNORM_BENCH_H

#include "twnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Measurement aid (not part of the method): dst = src, `bytes` bytes, a
 * plain 16-byte-vector streaming copy used as the practical HBM ceiling and
 * to scale hardware traffic counters.  bytes must be a multiple of 16 and both
 * pointers 16-byte aligned; the ranges may not overlap.
 */
tw_status tw_stream_copy(const void* src, void* dst, int64_t bytes, int n_cu_limit,
                         void* stream);

/*
 * Measurement aid (not part of the method): the fused kernel's HBM traffic
 * without its arithmetic, the practical ceiling of that traffic pattern.
 * Reads n_src tensors of `bytes` bytes and writes n_dst tensors of the same
 * size: every 32-bit word of every dst becomes the wrap-around uint32 sum of
 * that word over the srcs.  The access pattern follows the fused kernel's
 * row walk: 16 KiB blocks, each walked by one 256-lane workgroup (4 slots of
 * 16 bytes per lane), the next block's loads issued before this block's
 * stores, and a persistent grid of at most 2 workgroups per CU, with the
 * fused kernel's cache policies (non-temporal loads, device-scope stores).
 * So a fused call over N partials corresponds to n_src = N + 1, n_dst = 2
 * and bytes = rows * hidden * element size.
 * n_src in [1, TW_MAX_PARTIALS + 1], n_dst in [1, TW_MAX_PARTIALS]; bytes a
 * multiple of 16; every pointer 16-byte aligned; no dst may overlap a src or
 * another dst (srcs may overlap each other).  n_cu_limit as for the fused
 * call.  bytes == 0 is a no-op.
 */
tw_status tw_stream_mix(const void* const* srcs, int n_src, void* const* dsts, int n_dst,
                        int64_t bytes, int n_cu_limit, void* stream);

/*
 * Tuning hook: force the fused kernel's launch shape to `waves` wavefronts
 * per token row with `chunks_per_lane` 16-byte chunks per lane (both 0 =
 * automatic choice), and with `wgs_per_cu` > 0 run rows wider than 32
 * chunks on a persistent grid of at most `wgs_per_cu` workgroups per CU of
 * the call (0 = the default grid: one workgroup per row on the whole chip, a
 * persistent grid of as many workgroups as each CU holds on a CU-limited
 * call).  Applies to the later calls made from the calling thread only (the
 * setting is per host thread, so one thread's tuning never changes or fails
 * another thread's calls); a shape that cannot cover a row returns
 * TW_ERR_UNSUPPORTED at that thread's call, and so does a shape of more than
 * 10 wavefronts at a CU-limited call.  A forced shape also applies to rows of
 * at most 32 chunks, which otherwise take the narrow-row kernel.  Neither the
 * shape nor the grid changes any result bit: every shape adds in the same
 * order.  Returns
 * TW_ERR_INVALID_ARG for
 * waves outside [0,16], chunks_per_lane not in {0,1,2,3,4,6,8}, only one of
 * the two being 0, or wgs_per_cu < 0.
 */
tw_status tw_set_fused_shape(int waves, int chunks_per_lane, int wgs_per_cu);

/* Launch shape the fused kernel would use for (dtype, hidden, n partials)
 * when `rows` rows run on `cus` CUs (the CU limit of the call, else the
 * device's count) of a device with `device_cus` CUs; writes the wavefronts
 * per row and chunks per lane (team_lanes for rows narrower than one
 * wavefront, else 0).  Calls of fewer rows than CUs get as many wavefronts
 * per row as the row fills; calls on at most half of the device's CUs may
 * get a shape measured for that regime instead of the whole-chip one.
 * The results are the same bits for every shape.  Needs
 * 1 <= cus <= device_cus and rows >= 0.  HIP-free. */
tw_status tw_query_fused_shape(tw_dtype dtype, int64_t hidden, int n, int64_t rows, int cus,
                               int device_cus, int* waves, int* chunks_per_lane,
                               int* team_lanes);

#ifdef __cplusplus
}
#endif

#endif /* TWNORM_BENCH_H */
