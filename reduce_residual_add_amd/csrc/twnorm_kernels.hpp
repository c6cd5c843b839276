// Device code of libtwnorm for gfx950 (CDNA4, wave64).
//
// One token row is one independent unit of work: its statistic needs all of
// its `hidden` features and nothing from other rows ("TokenWeave 策略详解：以
// 大模型推理为例", §1: the per-token RMS uses all of a token's features; §2:
// the ReduceScatter must cut along token boundaries for that reason).  So a
// row is owned by one team of lanes and never leaves registers between its
// loads and its stores:
//
//   loads   N partial chunks + 1 residual chunk per 16-byte chunk slot,
//           all issued before the first add (memory-level parallelism);
//           on a persistent grid the next row's loads are in flight while
//           this row finishes
//   sum     s = p_0 + ... + p_{N-1} in index order, x = r + s   (float32)
//   store   residual_out = round(x)            (the X = X + Y update)
//   reduce  sum of x^2: per 16-byte chunk -> one DPP / ds_swizzle butterfly
//           per group of 64 consecutive chunks -> the group sums in row
//           order through LDS (an order fixed by the row width alone)
//   store   out = round(x * rsqrt(ss / H + eps) * w)
//
// The pages' kernel sums the N peers inside the switch fabric with 16-byte
// multimem loads ("融合内核中的体现": multimem_ld_reduce_add<16>); here the N
// partials are local HBM buffers, read with N plain 16-byte loads and summed
// in VGPRs, which is what a 16-byte-per-lane vector load does best on CDNA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxPartials = 16;

struct PartialPtrs {
  const u32x4* p[kMaxPartials];
};

// Destinations of the normalised output: `n` buffers, each written at row
// `row0 + row` (one buffer at row 0 for the plain fused call; one per rank's
// AllGather buffer for the all-gather store).
constexpr int kMaxOutputs = 16;
struct OutPtrs {
  u32x4* p[kMaxOutputs];
  int n;
  int64_t row0;
};

// Sources and destinations of the traffic-pattern measurement aid.
struct MixPtrs {
  const u32x4* src[kMaxPartials + 1];
  u32x4* dst[kMaxOutputs];
  int n_dst;
};

// Storage formats.  A 16-byte chunk holds kElems values.
struct Bf16 {
  static constexpr int kElems = 8;
};
struct F32 {
  static constexpr int kElems = 4;
};

// ---------------------------------------------------------------------------
// Streaming memory access through plain pointers (the narrow-row and copy
// kernels).  Partials, residual and outputs are touched once per call, so
// they carry the non-temporal hint (measured on MI355X: +15-20% HBM
// throughput over default caching).  TW_NT_LOADS / TW_NT_STORES = 0 select
// the default cache policy instead.
// ---------------------------------------------------------------------------
#ifndef TW_NT_LOADS
#define TW_NT_LOADS 1
#endif
#ifndef TW_NT_STORES
#define TW_NT_STORES 1
#endif

__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) {
#if TW_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

__device__ __forceinline__ void st_stream(u32x4* p, u32x4 v) {
#if TW_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Buffer-resource access (the wide-row kernel).  A descriptor in four scalar
// registers holds a row's base address and byte size; lanes pass a 32-bit
// byte offset.  Per row only the scalar base changes, so no lane does 64-bit
// address arithmetic, and the buffer unit's range check turns lanes past the
// row's end into zero loads and dropped stores.
//
// Cache policy (gfx940-family bits: 1 = SC0, 2 = NT, 16 = SC1).  Measured on
// MI355X for this kernel's 9-read : 2-write stream: NT loads beat default
// loads by ~12%; device-scope (SC1) stores beat NT stores by 3-8% on rows of
// 5120-8192 features, and both beat default stores.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer access
#ifndef TW_LOAD_CPOL
#define TW_LOAD_CPOL 2    // NT
#endif

#ifndef TW_STORE_CPOL
#define TW_STORE_CPOL 16  // SC1: device scope
#endif
constexpr int kLoadCpol = TW_LOAD_CPOL;
constexpr int kStoreCpol = TW_STORE_CPOL;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load(rsrc_t r, unsigned byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kLoadCpol);
}

// Default-policy load for data every workgroup re-reads (the weight).
__device__ __forceinline__ u32x4 buf_load_cached(rsrc_t r, unsigned byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ __forceinline__ void buf_store(u32x4 v, rsrc_t r, unsigned byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kStoreCpol);
}

// ---------------------------------------------------------------------------
// Format conversion.  bf16 -> f32 is exact (the bf16 bits are the high half
// of a float32).  f32 -> bf16 uses v_cvt_pk_bf16_f32: round to nearest even,
// NaN stays NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void widen(Bf16, const u32x4& v, float* f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(v[q] << 16);
    f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
  }
}

__device__ __forceinline__ void widen(F32, const u32x4& v, float* f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(v[q]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x4 narrow(Bf16, const float* f) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
  return r;
}

__device__ __forceinline__ u32x4 narrow(F32, const float* f) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = __float_as_uint(f[q]);
  return r;
}

// ---------------------------------------------------------------------------
// Cross-lane sums.  Butterfly over aligned lane groups: quad_perm swaps for
// distance 1 and 2, row_half_mirror / row_mirror for 4 and 8 (earlier steps
// made each 4- / 8-lane block uniform, so a mirror acts as a swap),
// ds_swizzle xor 16 inside each 32-lane half, and the two halves' readlane
// values for 32.  Every lane of a group ends with the same bits, and the
// order of additions depends only on the group size.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swizzle_xor16(float v) {
  // bit-mode swizzle: and_mask 0x1f, or_mask 0, xor_mask 0x10
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of `team` lanes (a power of two, 1..64).  `team`
// must be uniform across the wavefront and every lane must be active.
__device__ __forceinline__ float team_sum(float v, int team) {
  if (team >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if (team >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if (team >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if (team >= 16) v += dpp<0x140>(v);  // row_mirror
  if (team >= 32) v += swizzle_xor16(v);
  if (team >= 64) v = readlane(v, 0) + readlane(v, 32);
  return v;
}

// ---------------------------------------------------------------------------
// Per-chunk arithmetic shared by both kernel shapes.
// raw[0] is the residual chunk, raw[1..N] the partial chunks.
// ---------------------------------------------------------------------------
template <class D, int N>
__device__ __forceinline__ void add_chunk(const u32x4 (&raw)[N + 1], float* x, float& ss) {
  constexpr int E = D::kElems;
  float acc[E], t[E];
  widen(D{}, raw[1], acc);
#pragma unroll
  for (int i = 1; i < N; ++i) {
    widen(D{}, raw[i + 1], t);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += t[e];
  }
  widen(D{}, raw[0], t);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = t[e] + acc[e];
    ss = __builtin_fmaf(x[e], x[e], ss);
  }
}

template <class D>
__device__ __forceinline__ u32x4 scale_chunk(const float* x, float inv, const u32x4& wraw) {
  constexpr int E = D::kElems;
  float w[E], o[E];
  widen(D{}, wraw, w);
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = (x[e] * inv) * w[e];
  return narrow(D{}, o);
}

// ---------------------------------------------------------------------------
// Wide rows: one workgroup of W wavefronts (blockDim.x = 64 W <= 64 MAXW) per
// row, each lane owning K chunk slots c = tid + k * blockDim.x.  Each
// workgroup walks rows blockIdx.x, blockIdx.x + gridDim.x, ...  On the whole
// chip the grid has one workgroup per row, so each walks a single row; on a
// CU-limited call the grid is persistent (at most the workgroups those CUs
// hold at once) and the loop is software-pipelined: as soon as a row's sums
// are in registers, the loads of the workgroup's next row are issued, so HBM
// keeps streaming while the row's sum of squares is reduced, scaled and
// stored.  Raw chunks of one row sit in K * (N + 1) * 4 VGPRs, the float32
// row in K * E.
// MAXW sets the launch bound: 4 (256 threads) leaves the compiler up to 512
// VGPRs per lane, 8 (512 threads) up to 256, 16 (1024 threads) caps it at 128.
// ---------------------------------------------------------------------------
template <int N, int K>
__device__ __forceinline__ void load_row(u32x4 (&raw)[K][N + 1], const PartialPtrs& pp,
                                         const u32x4* residual, int64_t base, int row_bytes,
                                         unsigned lane_off, unsigned slot_stride) {
  const rsrc_t r_row = make_rsrc(residual + base, row_bytes);
#pragma unroll
  for (int k = 0; k < K; ++k) raw[k][0] = buf_load(r_row, lane_off + k * slot_stride);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const rsrc_t p_row = make_rsrc(pp.p[i] + base, row_bytes);
#pragma unroll
    for (int k = 0; k < K; ++k) raw[k][i + 1] = buf_load(p_row, lane_off + k * slot_stride);
  }
}

// How many partials the wide-row kernel loads before it adds: all N, in one
// batch with the residual (the most loads in flight), when a whole row's raw
// chunks, its float32 values, the weight and the addressing fit the VGPR
// target of the launch bound; otherwise as many as fit, group after group,
// with the residual last.  The target keeps two waves per SIMD for 256- and
// 512-thread workgroups (256 VGPRs) and is the 1024-thread bound itself
// (128).  Measured on MI355X against loading whole rows: the same time where
// a row fits (the N=8, 8192-wide kernel is unchanged), 8-13% faster for
// 12-16 partials or 16384-wide rows, and up to 44% where a whole row would
// spill.  The additions keep their order, so the bits do not change.
template <class D, int N, int K, int MAXW>
struct RowPlan {
  static constexpr int kTarget = MAXW <= 8 ? 256 : 128;
  static constexpr int kFixed = K * D::kElems + K * 4 + 48;
  static constexpr bool kWholeRow = (N + 1) * K * 4 + kFixed <= kTarget;
  static constexpr int kFit = (kTarget - kFixed) / (K * 4);
  // partials per group when the whole row does not fit (may be all N: the
  // residual then still waits until they are summed)
  static constexpr int kGroup = kWholeRow ? N : (kFit < 1 ? 1 : (kFit < N ? kFit : N));
};

// `residual` carries no __restrict__: the in-place update passes the same
// buffer as `residual_out`, and each lane stores a chunk only after loading
// it.
template <class D, int N, int K, int MAXW>
__global__ void __launch_bounds__(64 * MAXW)
fused_rows_kernel(PartialPtrs pp, const u32x4* residual, const u32x4* __restrict__ weight,
                  OutPtrs outs, u32x4* residual_out,
                  int64_t rows, int chunks, float hidden_f, float eps) {
  constexpr int E = D::kElems;
  constexpr int G = RowPlan<D, N, K, MAXW>::kGroup;
  constexpr bool kWholeRow = RowPlan<D, N, K, MAXW>::kWholeRow;
  __shared__ float red[2][MAXW * K];
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int row_bytes = chunks * 16;
  const int groups = (chunks + 63) >> 6;  // 64-chunk groups of the row
  const unsigned lane_off = unsigned(tid) * 16u;      // this lane's first chunk
  const unsigned slot_stride = unsigned(nthr) * 16u;  // between a lane's chunk slots

  u32x4 wv[K];
  const rsrc_t w_rsrc = make_rsrc(weight, row_bytes);
#pragma unroll
  for (int k = 0; k < K; ++k) wv[k] = buf_load_cached(w_rsrc, lane_off + k * slot_stride);

  int parity = 0;
  // A row once its float32 values x and each slot's sum of squares q are in
  // registers: the row's sum of squares, the scale and the normalised store.
  // Slot k of wave w holds chunks [64 g, 64 g + 64) with g = k W + w: one
  // butterfly per slot gives each 64-chunk group's sum, and the groups are
  // added in the order of g.  The order of every addition is thus fixed by
  // the row width alone, whatever W and K are, and so are the bits.
  auto finish_row = [&](float (&x)[K][E], float (&q)[K], int64_t row) {
#pragma unroll
    for (int k = 0; k < K; ++k) q[k] = team_sum(q[k], 64);
    float ss = 0.0f;
    if (MAXW > 1 && nwaves > 1) {
      if ((tid & 63) == 0) {
#pragma unroll
        for (int k = 0; k < K; ++k) red[parity][k * nwaves + wave] = q[k];
      }
      __syncthreads();
      for (int g = 0; g < groups; ++g) ss += red[parity][g];
      // Double-buffered: the next row writes the other half, and the row
      // after that is only reached once every wave passed the next barrier,
      // i.e. finished reading this half.
      parity ^= 1;
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (k < groups) ss += q[k];
    }
    const float inv = 1.0f / __builtin_sqrtf(ss / hidden_f + eps);
    u32x4 o[K];
#pragma unroll
    for (int k = 0; k < K; ++k) o[k] = scale_chunk<D>(x[k], inv, wv[k]);
    const int64_t obase = (outs.row0 + row) * chunks;
    for (int j = 0; j < outs.n; ++j) {
      const rsrc_t o_rsrc = make_rsrc(outs.p[j] + obase, row_bytes);
#pragma unroll
      for (int k = 0; k < K; ++k) buf_store(o[k], o_rsrc, lane_off + k * slot_stride);
    }
  };

  // Row walk of this workgroup: first, first + stride, ... below `end`.
  // Slots past the row's end load zeros, so they add nothing to the sums,
  // and their stores fall outside the descriptor's range and are dropped.
  const int64_t first = blockIdx.x, stride = gridDim.x, end = rows;
  if constexpr (kWholeRow) {
    // Whole rows: the residual and all N partials of the row in flight at
    // once, and the next row's loads issued as soon as this row's sums are
    // in registers.
    u32x4 raw[K][N + 1];
    int64_t row = first;
    if (row < end) load_row<N, K>(raw, pp, residual, row * chunks, row_bytes, lane_off, slot_stride);
    for (; row < end; row += stride) {
      const rsrc_t ro_rsrc = make_rsrc(residual_out + row * chunks, row_bytes);
      float x[K][E];
      float q[K];  // sum of squares of each slot's chunk
#pragma unroll
      for (int k = 0; k < K; ++k) {
        q[k] = 0.0f;
        add_chunk<D, N>(raw[k], x[k], q[k]);
        buf_store(narrow(D{}, x[k]), ro_rsrc, lane_off + k * slot_stride);
      }
      // The raw registers are free again: start the next row's loads now.
      const int64_t next = row + stride;
      if (next < end)
        load_row<N, K>(raw, pp, residual, next * chunks, row_bytes, lane_off, slot_stride);
      finish_row(x, q, row);
    }
  } else {
    // Groups of G partials: x accumulates p_0 + p_1 + ... in index order,
    // then x = r + x, the same additions as add_chunk.
    for (int64_t row = first; row < end; row += stride) {
      const int64_t base = row * chunks;
      float x[K][E];
#pragma unroll
      for (int g0 = 0; g0 < N; g0 += G) {
        u32x4 raw[K][G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
          if (g0 + i < N) {
            const rsrc_t p_row = make_rsrc(pp.p[g0 + i] + base, row_bytes);
#pragma unroll
            for (int k = 0; k < K; ++k) raw[k][i] = buf_load(p_row, lane_off + k * slot_stride);
          }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
          for (int i = 0; i < G; ++i) {
            if (g0 + i < N) {
              float t[E];
              widen(D{}, raw[k][i], t);
              if (g0 + i == 0) {
#pragma unroll
                for (int e = 0; e < E; ++e) x[k][e] = t[e];
              } else {
#pragma unroll
                for (int e = 0; e < E; ++e) x[k][e] += t[e];
              }
            }
          }
        }
      }
      const rsrc_t r_row = make_rsrc(residual + base, row_bytes);
      u32x4 rr[K];
#pragma unroll
      for (int k = 0; k < K; ++k) rr[k] = buf_load(r_row, lane_off + k * slot_stride);
      const rsrc_t ro_rsrc = make_rsrc(residual_out + base, row_bytes);
      float q[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float t[E];
        widen(D{}, rr[k], t);
        q[k] = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          x[k][e] = t[e] + x[k][e];
          q[k] = __builtin_fmaf(x[k][e], x[k][e], q[k]);
        }
        buf_store(narrow(D{}, x[k]), ro_rsrc, lane_off + k * slot_stride);
      }
      finish_row(x, q, row);
    }
  }
}

// ---------------------------------------------------------------------------
// Narrow rows (at most 32 chunks): a team of `team` lanes (power of two) per
// row, 256 / team rows per 256-thread workgroup, one chunk per lane.  The
// loop bound depends on blockIdx only, so whole wavefronts iterate together
// and the butterfly always sees every lane active.  The row is one 64-chunk
// group whose lanes past `chunks` hold zeros, and the team butterfly is the
// first levels of the wide kernel's 64-lane one (the levels above add exact
// zeros), so both kernels give the same bits for the same row.
// ---------------------------------------------------------------------------
template <class D, int N>
__global__ void __launch_bounds__(256)
fused_team_kernel(PartialPtrs pp, const u32x4* residual, const u32x4* __restrict__ weight,
                  OutPtrs outs, u32x4* residual_out,
                  int64_t rows, int chunks, int team, float hidden_f, float eps) {
  constexpr int E = D::kElems;
  const int tid = threadIdx.x;
  const int rows_per_block = blockDim.x / team;
  const int my = tid / team;
  const int c = tid - my * team;
  const bool lane_has_chunk = c < chunks;
  u32x4 wv = {0u, 0u, 0u, 0u};
  if (lane_has_chunk) wv = weight[c];

  for (int64_t row0 = (int64_t)blockIdx.x * rows_per_block; row0 < rows;
       row0 += (int64_t)gridDim.x * rows_per_block) {
    const int64_t row = row0 + my;
    const bool act = lane_has_chunk && row < rows;
    const int64_t off = row * chunks + c;
    float x[E];
    float ss = 0.0f;
    if (act) {
      u32x4 raw[N + 1];
      raw[0] = ld_stream(residual + off);
#pragma unroll
      for (int i = 0; i < N; ++i) raw[i + 1] = ld_stream(pp.p[i] + off);
      add_chunk<D, N>(raw, x, ss);
      st_stream(residual_out + off, narrow(D{}, x));
    }
    ss = team_sum(ss, team);
    const float inv = 1.0f / __builtin_sqrtf(ss / hidden_f + eps);
    if (act) {
      const u32x4 o = scale_chunk<D>(x, inv, wv);
      const int64_t ooff = (outs.row0 + row) * chunks + c;
      for (int j = 0; j < outs.n; ++j) st_stream(outs.p[j] + ooff, o);
    }
  }
}

// ---------------------------------------------------------------------------
// Unfused comparison path, first kernel: reduced = round(sum_i p_i), the
// reduce half of a ReduceScatter written to HBM.  It walks the tensors in
// blocks of 256 lanes x K chunk slots with the fused kernel's access order,
// cache policy and pipelining (this block's result stored, then the next
// block's loads issued) on a persistent grid of 2 workgroups per CU, so the
// comparison measures the HBM round trip of the intermediate and nothing
// else.  A block's descriptors cover only the chunks left: lanes past the end
// load zeros and have their stores dropped.
// ---------------------------------------------------------------------------
template <int N>
constexpr int reduce_slots() { return N <= 8 ? 4 : 2; }

template <int N>
__device__ __forceinline__ void reduce_load(u32x4 (&raw)[reduce_slots<N>()][N],
                                            const PartialPtrs& pp, int64_t first_chunk,
                                            int bytes, unsigned lane_off) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const rsrc_t r = make_rsrc(pp.p[i] + first_chunk, bytes);
#pragma unroll
    for (int k = 0; k < reduce_slots<N>(); ++k) raw[k][i] = buf_load(r, lane_off + k * 4096u);
  }
}

template <class D, int N>
__global__ void __launch_bounds__(256, 2)
reduce_kernel(PartialPtrs pp, u32x4* reduced, int64_t total_chunks) {
  constexpr int E = D::kElems;
  constexpr int K = reduce_slots<N>();
  constexpr int64_t kBlock = 256 * K;  // chunks per block
  const unsigned lane_off = threadIdx.x * 16u;
  const int64_t blocks = (total_chunks + kBlock - 1) / kBlock;
  auto bytes_of = [&](int64_t b) {
    const int64_t left = total_chunks - b * kBlock;
    return int(left < kBlock ? left : kBlock) * 16;
  };
  u32x4 raw[K][N];
  int64_t b = blockIdx.x;
  if (b < blocks) reduce_load<N>(raw, pp, b * kBlock, bytes_of(b), lane_off);
  for (; b < blocks; b += gridDim.x) {
    u32x4 o[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float acc[E], t[E];
      widen(D{}, raw[k][0], acc);
#pragma unroll
      for (int i = 1; i < N; ++i) {
        widen(D{}, raw[k][i], t);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += t[e];
      }
      o[k] = narrow(D{}, acc);
    }
    const rsrc_t r = make_rsrc(reduced + b * kBlock, bytes_of(b));
#pragma unroll
    for (int k = 0; k < K; ++k) buf_store(o[k], r, lane_off + k * 4096u);
    const int64_t next = b + gridDim.x;
    if (next < blocks) reduce_load<N>(raw, pp, next * kBlock, bytes_of(next), lane_off);
  }
}

}  // namespace twk
