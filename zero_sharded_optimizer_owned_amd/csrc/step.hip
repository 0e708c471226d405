// The hot path of libzero_shard: rank reduce, overflow/norm check and the
// fused Adam/AdamW step -- HIP kernels for gfx950 and the C entry points that
// validate, plan and launch them.
//
// All kernels stream HBM: the step moves ~34-162 bytes per owned parameter for
// a few dozen fp32 operations, so the design aims at bytes in flight, not at
// arithmetic.  No MFMA: nothing here is a contraction.
//   * every stream is read and written as 128-bit vectors of 8 elements
//     (one vector = 16 B of 16-bit data or 2 x 16 B of fp32); all base
//     indices are multiples of 8, so the vectors of all streams start at the
//     same flat indices and only the ends of a range need scalar peels;
//   * one block per short contiguous piece: the fused step takes one chunk
//     of the owner's chunk table per block (or one group of short chunks),
//     the flat-range kernels one piece of 256 vectors, one vector
//     per thread; blocks are dispatched in order, so the pieces in flight
//     form a narrow window that advances through every stream (no
//     cross-block synchronisation at all);
//   * reductions of the squared norm use fp64 per-thread sums, a wavefront
//     butterfly (DPP/permute shuffles), an LDS stage per block and fixed
//     contiguous folds of the per-block partials -- a fixed tree, so the
//     result is identical run to run;
//   * the rank sum is one fp32 add per rank in rank order and one IEEE
//     division (a multiply by 1/divisor when divisor is a power of two,
//     which gives the same bits), the same instruction sequence on the vector
//     and peel paths, so every path produces identical bits.
// Built with -ffp-contract=off: every fused multiply-add below is written
// explicitly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "internal.h"
#include "launch.h"
#include "scan.h"

namespace zs {
namespace {

// The check's per-block partials are folded by one block when there are at
// most kFoldDirect of them, else first by kFinalBlocks blocks.
constexpr uint64_t kFoldDirect = 4096;
constexpr uint64_t kFinalBlocks = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Element access.  A vector is 8 elements at an index e that is a multiple of
// 8; `Raw` is its storage as loaded (4 VGPRs for 16-bit data, 8 for fp32), so
// a batch of loads can be in flight before any of them is widened.
// `load_stream` marks a load as nontemporal (data read exactly once); the
// fused step uses it for 16-bit rank gradients, the flat reduce for 16-bit
// rank data below 32 ranks, and the 16-bit write-back is a nontemporal store.
// Measured: +1-6% for those kernels; the same hint on fp32 rank data, on
// 64-rank reduces or on fp32 stores made them slower or changed nothing.
// ---------------------------------------------------------------------------
template <int DT>
struct Elem;

template <>
struct Elem<ZERO_F16> {
  typedef half8 Raw;
  static __device__ __forceinline__ Raw load_raw(const void* base, uint64_t e) {
    return *reinterpret_cast<const half8*>(static_cast<const _Float16*>(base) + e);
  }
  static __device__ __forceinline__ Raw load_stream(const void* base, uint64_t e) {
    return __builtin_nontemporal_load(reinterpret_cast<const half8*>(static_cast<const _Float16*>(base) + e));
  }
  static __device__ __forceinline__ float widen(const Raw& h, int k) { return (float)h[k]; }
  static __device__ __forceinline__ float load1(const void* base, uint64_t e) {
    return (float)static_cast<const _Float16*>(base)[e];
  }
  static __device__ __forceinline__ void store8(void* base, uint64_t e, const float (&x)[8]) {
    half8 h;
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = (_Float16)x[k];
    __builtin_nontemporal_store(h, reinterpret_cast<half8*>(static_cast<_Float16*>(base) + e));
  }
  static __device__ __forceinline__ void store1(void* base, uint64_t e, float x) {
    static_cast<_Float16*>(base)[e] = (_Float16)x;
  }
};

// bfloat16: widening is a 16-bit shift; narrowing rounds to nearest, ties to
// even, keeps infinities and turns NaN into a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <>
struct Elem<ZERO_BF16> {
  typedef uint4 Raw;
  static __device__ __forceinline__ Raw load_raw(const void* base, uint64_t e) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
  }
  static __device__ __forceinline__ Raw load_stream(const void* base, uint64_t e) {
    const u32x4 r = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + e));
    return uint4{r[0], r[1], r[2], r[3]};
  }
  static __device__ __forceinline__ float widen(const Raw& w, int k) {
    const uint32_t word = (k >> 1) == 0 ? w.x : (k >> 1) == 1 ? w.y : (k >> 1) == 2 ? w.z : w.w;
    return __uint_as_float((k & 1) ? (word & 0xFFFF0000u) : (word << 16));
  }
  static __device__ __forceinline__ float load1(const void* base, uint64_t e) {
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[e] << 16);
  }
  static __device__ __forceinline__ void store8(void* base, uint64_t e, const float (&x)[8]) {
    uint4 w;
    w.x = bf16_bits(x[0]) | (bf16_bits(x[1]) << 16);
    w.y = bf16_bits(x[2]) | (bf16_bits(x[3]) << 16);
    w.z = bf16_bits(x[4]) | (bf16_bits(x[5]) << 16);
    w.w = bf16_bits(x[6]) | (bf16_bits(x[7]) << 16);
    __builtin_nontemporal_store(u32x4{w.x, w.y, w.z, w.w},
                                reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + e));
  }
  static __device__ __forceinline__ void store1(void* base, uint64_t e, float x) {
    static_cast<uint16_t*>(base)[e] = (uint16_t)bf16_bits(x);
  }
};

struct F32x8 {
  float4v lo, hi;
};

template <>
struct Elem<ZERO_F32> {
  typedef F32x8 Raw;
  static __device__ __forceinline__ Raw load_raw(const void* base, uint64_t e) {
    const float4v* p = reinterpret_cast<const float4v*>(static_cast<const float*>(base) + e);
    return F32x8{p[0], p[1]};
  }
  static __device__ __forceinline__ Raw load_stream(const void* base, uint64_t e) { return load_raw(base, e); }
  static __device__ __forceinline__ float widen(const Raw& r, int k) {
    return k < 4 ? r.lo[k] : r.hi[k - 4];
  }
  static __device__ __forceinline__ float load1(const void* base, uint64_t e) {
    return static_cast<const float*>(base)[e];
  }
  static __device__ __forceinline__ void store8(void* base, uint64_t e, const float (&x)[8]) {
    float4v* p = reinterpret_cast<float4v*>(static_cast<float*>(base) + e);
    p[0] = float4v{x[0], x[1], x[2], x[3]};
    p[1] = float4v{x[4], x[5], x[6], x[7]};
  }
  static __device__ __forceinline__ void store1(void* base, uint64_t e, float x) {
    static_cast<float*>(base)[e] = x;
  }
};

// fp32 vector load into registers.
__device__ __forceinline__ void load8f(const float* base, uint64_t e, float (&x)[8]) {
  const F32x8 r = Elem<ZERO_F32>::load_raw(base, e);
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = Elem<ZERO_F32>::widen(r, k);
}

// ---------------------------------------------------------------------------
// The rank reduce: s = start; s += g_r in rank order (fp32); s / divisor.
// ---------------------------------------------------------------------------
struct RankSet {
  const void* ptr[ZERO_MAX_RANKS];
  uint32_t R;
  uint64_t base;       // flat index of element 0 of every rank buffer
  float divisor;
  float inv_divisor;   // exact reciprocal when divisor is a power of two
  int32_t div_pow2;
};

__device__ __forceinline__ float divide(float s, const RankSet& rs) {
  // x * 2^-k and x / 2^k are the same real number, so both round identically.
  return rs.div_pow2 ? s * rs.inv_divisor : s / rs.divisor;
}

// The same division for whole vectors, with the (uniform) test taken once.
template <int U>
__device__ __forceinline__ void divide_vec(float (&s)[U][8], const RankSet& rs) {
  if (rs.div_pow2) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) s[u][k] = s[u][k] * rs.inv_divisor;
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) s[u][k] = s[u][k] / rs.divisor;
  }
}

// Batch of ranks whose loads are issued together before their adds.
template <int DT>
struct RankBatch {
  static constexpr int value = DT == ZERO_F32 ? 4 : 8;  // 32 VGPRs of raw data per vector
};

template <int DT, int U, int B, bool STREAM = false>
__device__ __forceinline__ void load_batch(const RankSet& rs, uint32_t r0, const uint64_t (&f)[U],
                                           typename Elem<DT>::Raw (&x)[B][U]) {
#pragma unroll
  for (int j = 0; j < B; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[j][u] = STREAM ? Elem<DT>::load_stream(rs.ptr[r0 + j], f[u] - rs.base)
                       : Elem<DT>::load_raw(rs.ptr[r0 + j], f[u] - rs.base);
}

template <int DT, int U, int B>
__device__ __forceinline__ void add_batch(const typename Elem<DT>::Raw (&x)[B][U], float (&s)[U][8]) {
#pragma unroll
  for (int j = 0; j < B; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) s[u][k] = s[u][k] + Elem<DT>::widen(x[j][u], k);
}

// s += g_0 + ... + g_{R-1} (in rank order) for a runtime R, then divide.
// Whole batches are double-buffered: batch b+1 is in flight while batch b is
// added; the loads of the last R mod B ranks are issued together before their
// adds.  STREAM loads the rank data with the nontemporal hint.
template <int DT, int U, bool STREAM = false>
__device__ __forceinline__ void reduce_vec(const RankSet& rs, const uint64_t (&f)[U],
                                           float (&s)[U][8]) {
  constexpr int B = RankBatch<DT>::value;
  typedef typename Elem<DT>::Raw Raw;
  const uint32_t full = rs.R / B * B;
  uint32_t r0 = 0;
  if (full > 0) {
    Raw xa[B][U], xb[B][U];
    load_batch<DT, U, B, STREAM>(rs, 0, f, xa);
    for (; r0 + 2 * B <= full; r0 += 2 * B) {
      load_batch<DT, U, B, STREAM>(rs, r0 + B, f, xb);
      add_batch<DT, U, B>(xa, s);
      if (r0 + 2 * B < full) load_batch<DT, U, B, STREAM>(rs, r0 + 2 * B, f, xa);
      add_batch<DT, U, B>(xb, s);
    }
    if (r0 < full) {  // an odd number of whole batches: the last one is in xa
      add_batch<DT, U, B>(xa, s);
      r0 += B;
    }
  }
  const uint32_t rem = rs.R - r0;  // < B, the same for every thread
  if (rem > 0) {
    Raw x[B - 1][U];
#pragma unroll
    for (int j = 0; j < B - 1; ++j) {
      if ((uint32_t)j < rem) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          x[j][u] = STREAM ? Elem<DT>::load_stream(rs.ptr[r0 + j], f[u] - rs.base)
                           : Elem<DT>::load_raw(rs.ptr[r0 + j], f[u] - rs.base);
      }
    }
#pragma unroll
    for (int j = 0; j < B - 1; ++j) {
      if ((uint32_t)j < rem) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < 8; ++k) s[u][k] = s[u][k] + Elem<DT>::widen(x[j][u], k);
      }
    }
  }
  divide_vec<U>(s, rs);
}

template <int DT>
__device__ __forceinline__ float reduce_one(const RankSet& rs, uint64_t f, float start) {
  float s = start;
  for (uint32_t r = 0; r < rs.R; ++r) s = s + Elem<DT>::load1(rs.ptr[r], f - rs.base);
  return divide(s, rs);
}

// ---------------------------------------------------------------------------
// Squared-norm / overflow reduction: wave butterfly, LDS across waves.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = x + __shfl_xor(x, off, 64);
  return x;
}

// Block-wide (sum, any) with a fixed order; the result is valid in thread 0.
__device__ __forceinline__ void block_reduce(double& sq, int& bad) {
  __shared__ double s_sum[kWavesPerBlock];
  __shared__ int s_bad[kWavesPerBlock];
  sq = wave_sum(sq);
  const int any = __any(bad);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_sum[w] = sq;
    s_bad[w] = any;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = s_sum[0];
    int b = s_bad[0];
    for (int i = 1; i < kWavesPerBlock; ++i) {
      t = t + s_sum[i];
      b |= s_bad[i];
    }
    sq = t;
    bad = b;
  }
}

__device__ __forceinline__ void check_accum(float g, double& sq, int& bad) {
  const double d = (double)g;
  sq = fma(d, d, sq);  // d*d is exact in fp64, so the fma rounds only the sum
  bad |= !__builtin_isfinite(g);
}

struct CheckOut {
  double* partial;   // [parts] one per block of the first stage
  int32_t* flags;    // [parts]
  double* partial2;  // [kFinalBlocks] second stage (large part counts)
  int32_t* flags2;   // [kFinalBlocks]
};

// ---------------------------------------------------------------------------
// K1: owner reduce over a contiguous flat range, optional fused check.
// ---------------------------------------------------------------------------
struct ReduceArgs {
  RankSet rs;
  uint64_t begin, end;
  uint64_t piece;  // vectors per block piece, a multiple of kBlock
  int xcd_order;   // pieces in XCD-contiguous runs (xcd_contiguous) rather than dealt round-robin
  float* out;
  uint64_t out_base;
  CheckOut chk;
};

// What the reduce does with the existing output (the `accumulate` argument).
enum AccumMode : int {
  kOverwrite = 0,      // out = sum / D
  kStartFromOut = 1,   // out = (out + sum) / D
  kAddMean = 2         // out = out + sum / D   (per-backward reduce, then accumulate)
};

// Flat-range kernels split the range into pieces of `piece` vectors: block b
// takes piece b, its threads on consecutive 128-bit vectors of every stream,
// so a block streams one short contiguous piece of each stream and exits, and
// blocks are dispatched in order.  A grid smaller than the piece count (only
// for ranges beyond kMaxChunkGrid pieces) takes the rest with a grid stride.
template <int DT, int MODE, bool CHECK, bool STREAM>
__global__ void __launch_bounds__(kBlock) reduce_kernel(const ReduceArgs a) {
  const uint64_t f0 = a.begin, f1 = a.end;
  const uint64_t a0 = min(f1, (f0 + 7) & ~7ull);
  const uint64_t a1 = max(a0, f1 & ~7ull);
  double sq = 0.0;
  int bad = 0;
  if (blockIdx.x == 0) {
    const uint64_t t = threadIdx.x;
    uint64_t f = ~0ull;
    if (t < a0 - f0) f = f0 + t;
    else if (t >= 8 && t - 8 < f1 - a1) f = a1 + (t - 8);
    if (f != ~0ull) {
      const float old = MODE != kOverwrite ? a.out[f - a.out_base] : 0.0f;
      float g = reduce_one<DT>(a.rs, f, MODE == kStartFromOut ? old : 0.0f);
      if (MODE == kAddMean) g = old + g;
      a.out[f - a.out_base] = g;
      if (CHECK) check_accum(g, sq, bad);
    }
  }
  const uint64_t v0 = a0 / 8, n_vec = a1 / 8 - v0;
  const uint64_t blk = a.xcd_order ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * a.piece;
  for (uint64_t p0 = blk * a.piece; p0 < n_vec; p0 += stride) {
    const uint64_t p1 = min(n_vec, p0 + a.piece);
    for (uint64_t v = p0 + threadIdx.x; v < p1; v += kBlock) {
      const uint64_t f[1] = {(v0 + v) * 8};
      float s[1][8], old[8];
      if (MODE == kStartFromOut) {
        load8f(a.out, f[0] - a.out_base, s[0]);
      } else {
        if (MODE == kAddMean) load8f(a.out, f[0] - a.out_base, old);
#pragma unroll
        for (int k = 0; k < 8; ++k) s[0][k] = 0.0f;
      }
      reduce_vec<DT, 1, STREAM>(a.rs, f, s);
      if (MODE == kAddMean) {
#pragma unroll
        for (int k = 0; k < 8; ++k) s[0][k] = old[k] + s[0][k];
      }
      Elem<ZERO_F32>::store8(a.out, f[0] - a.out_base, s[0]);
      if (CHECK) {
#pragma unroll
        for (int k = 0; k < 8; ++k) check_accum(s[0][k], sq, bad);
      }
    }
  }
  if (CHECK) {
    block_reduce(sq, bad);
    if (threadIdx.x == 0) {  // indexed by piece, so the fold's tree is the same in either order
      a.chk.partial[blk] = sq;
      a.chk.flags[blk] = bad;
    }
  }
}

// ---------------------------------------------------------------------------
// K2: check of a stored fp32 gradient (first stage), and the final stages.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) check_kernel(const float* g, uint64_t n, CheckOut chk) {
  const uint64_t a1 = n & ~7ull;
  double sq = 0.0;
  int bad = 0;
  if (blockIdx.x == 0 && threadIdx.x < n - a1) check_accum(g[a1 + threadIdx.x], sq, bad);
  const uint64_t n_vec = a1 / 8;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  // one read stream: XCD-contiguous runs of pieces (measured +4.6%)
  const uint64_t blk = xcd_contiguous(blockIdx.x, gridDim.x);
  for (uint64_t v = blk * kBlock + threadIdx.x; v < n_vec; v += stride) {
    float x[8];
    load8f(g, v * 8, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) check_accum(x[k], sq, bad);
  }
  block_reduce(sq, bad);
  if (threadIdx.x == 0) {  // indexed by piece: the fold's tree does not depend on the order
    chk.partial[blk] = sq;
    chk.flags[blk] = bad;
  }
}

// Folds parts (sum, any) pairs: block b takes the contiguous slice
// [b * per, min(parts, (b + 1) * per)) in a fixed order and writes its result
// to (out_sum[b], out_flag[b]).  The same part count always gives the same
// tree, so the result is identical run to run.
__global__ void __launch_bounds__(kBlock) check_fold_kernel(const double* sum, const int32_t* flag,
                                                            uint64_t parts, uint64_t per,
                                                            double* out_sum, int32_t* out_flag) {
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = min(parts, lo + per);
  double sq = 0.0;
  int bad = 0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += kBlock) {
    sq = sq + sum[i];
    bad |= flag[i];
  }
  block_reduce(sq, bad);
  if (threadIdx.x == 0) {
    out_sum[blockIdx.x] = sq;
    out_flag[blockIdx.x] = bad ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// K3/K4: fused owner step over the chunk table.
// ---------------------------------------------------------------------------
struct AdamConst {
  float beta1, one_minus_beta1, beta2, one_minus_beta2;
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
  float decay;  // 1 - lr * wd for AdamW, else 1
  float l2;     // wd for classic Adam, else 0
  float clip;
};

__device__ __forceinline__ void adam_update(float g, float& w, float& m, float& v,
                                            const AdamConst& c) {
  float gc = g * c.clip;
  if (c.l2 != 0.0f) gc = fmaf(c.l2, w, gc);
  m = fmaf(c.beta1, m, c.one_minus_beta1 * gc);
  v = fmaf(c.beta2, v, (c.one_minus_beta2 * gc) * gc);
  const float denom = fmaf(__builtin_sqrtf(v), c.inv_sqrt_bc2, c.eps);
  const float upd = m / denom;
  w = fmaf(-c.step_size, upd, w * c.decay);
}

struct AdamArgs {
  RankSet rs;
  const zero_chunk* chunks;
  uint64_t n_chunks;
  const uint64_t* groups;  // [n_groups + 1] first chunk of each block's work, or NULL
  uint64_t n_groups;
  uint64_t begin, end;
  const float* reduced_g;
  float *w, *m, *v;
  uint64_t local_base;
  void* p16;
  uint64_t param_base;
  AdamConst c;
};

// Gradient source of the fused step, fixed at compile time:
//   RC > 0  : exactly RC rank buffers (all loads unrolled, none guarded);
//   RC == 0 : any number of rank buffers, loaded in double-buffered batches;
//   RC == kReduced : a stored owner-local fp32 reduced gradient.
constexpr int kReduced = -1;

// NT: load 16-bit rank gradients with the nontemporal hint (the per-chunk
// path; the packed path reads them without it, see there).
template <int GDT, int PDT, int RC, int U, bool NT = (GDT != ZERO_F32)>
__device__ __forceinline__ void adam_vec(const AdamArgs& a, const uint64_t (&f)[U]) {
  float g[U][8], w[U][8], m[U][8], v[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int k = 0; k < 8; ++k) g[u][k] = 0.0f;
  // Every load of the iteration is issued before the first add: one memory
  // round trip per iteration.
  if constexpr (RC > 0) {
    typename Elem<GDT>::Raw x[RC][U];
    load_batch<GDT, U, RC, /*STREAM=*/NT>(a.rs, 0, f, x);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load8f(a.w, f[u] - a.local_base, w[u]);
      load8f(a.m, f[u] - a.local_base, m[u]);
      load8f(a.v, f[u] - a.local_base, v[u]);
    }
    // Keep the scheduler from sinking the state loads below the adds.
    __builtin_amdgcn_sched_barrier(0);
    add_batch<GDT, U, RC>(x, g);
    divide_vec<U>(g, a.rs);
  } else if constexpr (RC == kReduced) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load8f(a.reduced_g, f[u] - a.local_base, g[u]);
      load8f(a.w, f[u] - a.local_base, w[u]);
      load8f(a.m, f[u] - a.local_base, m[u]);
      load8f(a.v, f[u] - a.local_base, v[u]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load8f(a.w, f[u] - a.local_base, w[u]);
      load8f(a.m, f[u] - a.local_base, m[u]);
      load8f(a.v, f[u] - a.local_base, v[u]);
    }
    reduce_vec<GDT, U>(a.rs, f, g);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int k = 0; k < 8; ++k) adam_update(g[u][k], w[u][k], m[u][k], v[u][k], a.c);
    Elem<ZERO_F32>::store8(a.w, f[u] - a.local_base, w[u]);
    Elem<ZERO_F32>::store8(a.m, f[u] - a.local_base, m[u]);
    Elem<ZERO_F32>::store8(a.v, f[u] - a.local_base, v[u]);
    if constexpr (PDT != ZERO_NONE) Elem<PDT>::store8(a.p16, f[u] - a.param_base, w[u]);
  }
}

template <int GDT, int PDT, int RC>
__device__ __forceinline__ void adam_one(const AdamArgs& a, uint64_t f) {
  const float g =
      RC == kReduced ? a.reduced_g[f - a.local_base] : reduce_one<GDT>(a.rs, f, 0.0f);
  const uint64_t l = f - a.local_base;
  float w = a.w[l], m = a.m[l], v = a.v[l];
  adam_update(g, w, m, v, a.c);
  a.w[l] = w;
  a.m[l] = m;
  a.v[l] = v;
  if constexpr (PDT != ZERO_NONE) Elem<PDT>::store1(a.p16, f - a.param_base, w);
}

// One chunk by one block: the block's threads take the chunk's 128-bit
// vectors in order (thread t on vectors t, t + kBlock, ...); threads 0-6 take
// the scalar head before the first vector boundary, threads 8-14 the tail
// after the last one.
template <int GDT, int PDT, int RC>
__device__ __forceinline__ void adam_chunk(const AdamArgs& a, const zero_chunk ch, uint32_t t) {
  const uint64_t f0 = max(ch.flat, a.begin);
  const uint64_t f1 = min(ch.flat + ch.len, a.end);
  if (f0 >= f1) return;
  const uint64_t a0 = min(f1, (f0 + 7) & ~7ull);
  const uint64_t a1 = max(a0, f1 & ~7ull);
  if (t < a0 - f0) adam_one<GDT, PDT, RC>(a, f0 + t);
  else if (t >= 8 && t - 8 < f1 - a1) adam_one<GDT, PDT, RC>(a, a1 + t - 8);
  const uint64_t vend = a1 / 8;
  for (uint64_t vi = a0 / 8 + t; vi < vend; vi += kBlock) {
    const uint64_t f[1] = {vi * 8};
    adam_vec<GDT, PDT, RC, 1>(a, f);
  }
}

// Several short chunks by one block.  Each chunk is cut into work units --
// its 128-bit vectors, and its scalar head and tail elements -- and the
// block's threads take the units of all its chunks together: first every
// chunk's vectors, then every chunk's scalar elements, so that a wavefront
// mostly runs one of the two routines rather than both one after the other
// (thread t on units t, t + kBlock, ...).  A unit's chunk is found by binary
// search over the prefix sums of the per-chunk vector (or scalar) counts.
// The units run the same element and vector routines as one block per chunk,
// so the results are identical.  Chunks are taken kBlock at a time.
// Rank gradients are loaded here without the nontemporal hint: a chunk's
// scalar tail runs after the vector phase and reads a cache line that the
// chunk's last vector already brought in; with the hint that line tends to
// have left the cache by then and is read twice (measured on 100-element
// tensors: 5% more bytes fetched and 13% lower throughput with the hint).
// The packed path's LDS: per-chunk first element, vector count and head
// length; prefix sums of the vector and scalar counts; the scans' wave totals.
struct PackedLds {
  uint64_t f0[kBlock];
  uint64_t nvec[kBlock];
  uint64_t pv[kBlock + 1], ps[kBlock + 1];
  uint64_t wave_v[kWavesPerBlock], wave_s[kWavesPerBlock];
  uint32_t head[kBlock];
};

template <int GDT, int PDT, int RC>
__device__ void adam_packed(const AdamArgs& a, uint64_t c0, uint64_t c1, uint32_t t) {
  __shared__ PackedLds lds;
  uint64_t* const s_f0 = lds.f0;
  uint32_t* const s_head = lds.head;
  uint64_t* const s_nvec = lds.nvec;
  uint64_t* const s_pv = lds.pv;
  uint64_t* const s_ps = lds.ps;
  for (uint64_t s0 = c0; s0 < c1; s0 += kBlock) {
    const uint32_t m = (uint32_t)min((uint64_t)kBlock, c1 - s0);
    uint64_t nv = 0, ns = 0;
    if (t < m) {
      const zero_chunk ch = a.chunks[s0 + t];
      const uint64_t f0 = max(ch.flat, a.begin);
      const uint64_t f1 = max(f0, min(ch.flat + ch.len, a.end));
      const uint64_t a0 = min(f1, (f0 + 7) & ~7ull);
      const uint64_t a1 = max(a0, f1 & ~7ull);
      s_f0[t] = f0;
      s_head[t] = (uint32_t)(a0 - f0);
      s_nvec[t] = (a1 - a0) / 8;
      nv = (a1 - a0) / 8;
      ns = (a0 - f0) + (f1 - a1);
    }
    // prefix sums of the vector and scalar counts over the block
    s_pv[t + 1] = block_inclusive_scan(nv, lds.wave_v);
    s_ps[t + 1] = block_inclusive_scan(ns, lds.wave_s);
    if (t == 0) s_pv[0] = s_ps[0] = 0;
    __syncthreads();
    const uint64_t n_vec = s_pv[m], n_all = n_vec + s_ps[m];
    for (uint64_t u = t; u < n_all; u += kBlock) {
      const bool vec = u < n_vec;
      const uint64_t k = vec ? u : u - n_vec;
      const uint64_t* pre = vec ? s_pv : s_ps;
      uint32_t lo = 0, hi = m;  // the chunk j with pre[j] <= k < pre[j + 1]
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (pre[mid] <= k) lo = mid;
        else hi = mid;
      }
      const uint64_t r = k - pre[lo];
      const uint64_t f0 = s_f0[lo];
      const uint64_t head = s_head[lo], nvec = s_nvec[lo];
      if (vec) {
        const uint64_t f[1] = {f0 + head + 8 * r};
        adam_vec<GDT, PDT, RC, 1, /*NT=*/false>(a, f);
      } else {
        adam_one<GDT, PDT, RC>(a, r < head ? f0 + r : f0 + head + 8 * nvec + (r - head));
      }
    }
    __syncthreads();  // the next slice reuses the arrays
  }
}

// Multi-tensor kernel, one block per chunk.  A block streams one short
// contiguous piece of every stream and exits; blocks are dispatched in chunk
// order, which keeps the pieces in flight across the chip inside a narrow
// window of each stream.  A grid smaller than the chunk count takes the
// remaining chunks with a grid stride.  With rank gradients the XCDs take
// runs of two consecutive chunks (xcd_runs): measured +7% for 8 bf16 ranks on
// two boxes, within 0.6% for 4 fp16 or 16 fp32 ranks; from a stored gradient
// the plain order is 2% faster, so it keeps that.
template <int GDT, int PDT, int RC>
__global__ void __launch_bounds__(kBlock) adam_kernel(const AdamArgs a) {
  constexpr uint64_t kRun = RC == kReduced ? 1 : 2;
  for (uint64_t c = xcd_runs(blockIdx.x, gridDim.x, kRun); c < a.n_chunks; c += gridDim.x)
    adam_chunk<GDT, PDT, RC>(a, a.chunks[c], threadIdx.x);
}

// The same step over a group table: one block per group, i.e. one long chunk
// or several short ones packed together.  A kernel of its own, so that the
// per-chunk kernel carries neither the packing code nor its LDS arrays (with
// them it ran 2-6% slower).
template <int GDT, int PDT, int RC>
__global__ void __launch_bounds__(kBlock) adam_group_kernel(const AdamArgs a) {
  const uint32_t t = threadIdx.x;
  for (uint64_t w = blockIdx.x; w < a.n_groups; w += gridDim.x) {
    const uint64_t c0 = a.groups[w];
    const uint64_t c1 = min(a.groups[w + 1], a.n_chunks);
    if (c1 <= c0) continue;
    if (c1 - c0 == 1) adam_chunk<GDT, PDT, RC>(a, a.chunks[c0], t);
    else adam_packed<GDT, PDT, RC>(a, c0, c1, t);
  }
}

// ---------------------------------------------------------------------------
// Host-side planning and validation.
// ---------------------------------------------------------------------------
bool is_pow2_float(float d, float* inv) {
  int e = 0;
  const float mant = std::frexp(d, &e);
  if (mant != 0.5f) return false;
  const float r = std::ldexp(1.0f, 1 - e);  // 1/d exactly
  if (!std::isfinite(r) || r == 0.0f || std::fpclassify(r) == FP_SUBNORMAL) return false;
  *inv = r;
  return true;
}

int fill_ranks(RankSet* rs, const void* const* rank_grads, uint32_t R, int dtype, uint64_t base,
               uint64_t begin, float divisor, const char* who) {
  if (R == 0 || R > ZERO_MAX_RANKS)
    return fail(ZERO_EINVAL, "%s: R = %u outside [1, %d]", who, R, ZERO_MAX_RANKS);
  if (!rank_grads) return fail(ZERO_EINVAL, "%s: rank_grads is NULL", who);
  if (dtype != ZERO_F16 && dtype != ZERO_BF16 && dtype != ZERO_F32)
    return fail(ZERO_EINVAL, "%s: unknown gradient dtype %d", who, dtype);
  if (base % 8 != 0) return fail(ZERO_EINVAL, "%s: grad_base must be a multiple of 8", who);
  if (begin < base) return fail(ZERO_EINVAL, "%s: begin lies below grad_base", who);
  if (!(divisor > 0.0f) || !std::isfinite(divisor))
    return fail(ZERO_EINVAL, "%s: divisor must be finite and > 0", who);
  for (uint32_t r = 0; r < R; ++r) {
    if (!rank_grads[r]) return fail(ZERO_EINVAL, "%s: rank buffer %u is NULL", who, r);
    if (!aligned16(rank_grads[r]))
      return fail(ZERO_EINVAL, "%s: rank buffer %u is not 16-byte aligned", who, r);
    rs->ptr[r] = rank_grads[r];
  }
  for (uint32_t r = R; r < ZERO_MAX_RANKS; ++r) rs->ptr[r] = nullptr;
  rs->R = R;
  rs->base = base;
  rs->divisor = divisor;
  float inv = 0.0f;
  rs->div_pow2 = is_pow2_float(divisor, &inv) ? 1 : 0;
  rs->inv_divisor = inv;
  return ZERO_OK;
}

// Blocks of a flat-range kernel over n_vec vectors: one per piece.
uint32_t flat_grid(uint64_t n_vec, uint64_t piece = kBlock) {
  return chunk_grid((n_vec + piece - 1) / piece, 0);
}

// Vectors per block piece of the rank reduce: one per thread.  (Two per
// thread were 2% faster for 64 fp16 ranks dealt round-robin to the XCDs; in
// the XCD-contiguous order with two blocks per CU that many ranks now take,
// one per thread is 1.5-2% faster than two and 2-3% faster than four.)
uint64_t reduce_piece(uint32_t) { return kBlock; }

// The XCD-contiguous piece order (each XCD streams one contiguous run of the
// range) for one source (measured +7.7% for a bf16 source added into fp32)
// and from 32 sources on (+3 to +3.5% for 64 fp16 ranks with the fused check,
// together with the two-block cap below, on two boxes); 16 sources stay
// round-robin (the contiguous order measured -3.8% there).
int reduce_xcd_order(uint32_t R) { return R == 1 || R >= 32 ? 1 : 0; }

// Workspace of a check whose first stage has `parts` blocks: the per-block
// (sum, flag) pairs, then the second-stage pairs.
uint64_t check_ws_bytes(uint64_t parts) {
  const uint64_t first = (parts * (sizeof(double) + sizeof(int32_t)) + 255) / 256 * 256;
  return first + kFinalBlocks * (sizeof(double) + sizeof(int32_t));
}

// Most first-stage blocks a check over n elements can use (any begin).
uint64_t check_parts(uint64_t n) { return flat_grid(n / 8 + 1); }

int check_workspace(void* ws, size_t ws_bytes, uint64_t n, const char* who) {
  if (!ws) return fail(ZERO_EINVAL, "%s: workspace is NULL", who);
  const uint64_t need = check_ws_bytes(check_parts(n));
  if (ws_bytes < need)
    return fail(ZERO_EINVAL, "%s: workspace needs %llu bytes for %llu elements, got %zu", who,
                (unsigned long long)need, (unsigned long long)n, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(ZERO_EINVAL, "%s: workspace must be 256-byte aligned", who);
  return ZERO_OK;
}

CheckOut check_layout(void* ws, uint64_t parts) {
  char* b = static_cast<char*>(ws);
  const uint64_t first = (parts * (sizeof(double) + sizeof(int32_t)) + 255) / 256 * 256;
  CheckOut c;
  c.partial = reinterpret_cast<double*>(b);
  c.flags = reinterpret_cast<int32_t*>(b + parts * sizeof(double));
  c.partial2 = reinterpret_cast<double*>(b + first);
  c.flags2 = reinterpret_cast<int32_t*>(b + first + kFinalBlocks * sizeof(double));
  return c;
}

// Folds the first stage's `parts` pairs into the two outputs in a fixed tree.
void finish_check(const CheckOut& c, uint64_t parts, int32_t* d_overflow, double* d_sumsq,
                  hipStream_t s) {
  if (parts <= kFoldDirect) {
    hipLaunchKernelGGL(check_fold_kernel, 1, kBlock, 0, s, c.partial, c.flags, parts, parts, d_sumsq,
                       d_overflow);
    return;
  }
  const uint64_t per = (parts + kFinalBlocks - 1) / kFinalBlocks;
  const uint64_t blocks = (parts + per - 1) / per;
  hipLaunchKernelGGL(check_fold_kernel, (uint32_t)blocks, kBlock, 0, s, c.partial, c.flags, parts, per,
                     c.partial2, c.flags2);
  hipLaunchKernelGGL(check_fold_kernel, 1, kBlock, 0, s, c.partial2, c.flags2, blocks, blocks,
                     d_sumsq, d_overflow);
}

// Blocks of the flat reduce resident on one CU: uncapped (registers decide),
// except two for 16 to 31 ranks of 16-bit data without the fused check
// (measured on 16 bf16 ranks: +2.4% and +2.2% on two boxes; the same cap
// costs one source 10%, and three or four blocks change nothing) and two
// from 32 ranks on in the XCD-contiguous order (measured on 64 fp16 ranks
// with the check: uncapped -2%, three per CU -1.3%; in the round-robin order
// the cap had cost 1%).
uint32_t reduce_lds(int dt, uint32_t R, bool check) {
  const bool cap = R >= 32 || (dt != ZERO_F32 && R >= 16 && !check);
  return cap ? lds_for_blocks_per_cu(2, 0) : 0;
}

template <int DT, int MODE, bool STREAM>
void launch_reduce_s(const ReduceArgs& a, bool check, uint32_t grid, hipStream_t s) {
  const uint32_t lds = reduce_lds(DT, a.rs.R, check);
  if (check) hipLaunchKernelGGL((reduce_kernel<DT, MODE, true, STREAM>), grid, kBlock, lds, s, a);
  else hipLaunchKernelGGL((reduce_kernel<DT, MODE, false, STREAM>), grid, kBlock, lds, s, a);
}

// 16-bit rank data is loaded with the nontemporal hint below 32 ranks
// (measured: +3% for one source, +6% for 16; -3% for 64 ranks).
template <int DT, int MODE>
void launch_reduce_m(const ReduceArgs& a, bool check, uint32_t grid, hipStream_t s) {
  if constexpr (DT != ZERO_F32) {
    if (a.rs.R < 32) {
      launch_reduce_s<DT, MODE, true>(a, check, grid, s);
      return;
    }
  }
  launch_reduce_s<DT, MODE, false>(a, check, grid, s);
}

template <int DT>
void launch_reduce(const ReduceArgs& a, int mode, bool check, uint32_t grid, hipStream_t s) {
  if (mode == kStartFromOut) launch_reduce_m<DT, kStartFromOut>(a, check, grid, s);
  else if (mode == kAddMean) launch_reduce_m<DT, kAddMean>(a, check, grid, s);
  else launch_reduce_m<DT, kOverwrite>(a, check, grid, s);
}

// Blocks of the fused step resident on one CU.  Fewer blocks in flight keep
// the window of pieces that HBM serves narrow; each block already has every
// load of its vector in flight at once.  Measured on the 3.75e8-element owner
// (one vector per thread, 2048-element chunks): two blocks per CU beat three,
// four or an uncapped launch by 3-10% for 16-bit ranks, a stored gradient and
// up to four fp32 ranks; from eight fp32 ranks on, one block per CU is 4-5%
// faster than two.
template <int GDT, int RC>
uint32_t adam_blocks_per_cu(uint32_t R) {
  return (GDT == ZERO_F32 && RC != kReduced && R >= 8) ? 1 : 2;
}

template <int GDT, int PDT, int RC>
void launch_adam_k(const AdamArgs& a, uint32_t grid, hipStream_t s) {
  const uint32_t lds = lds_for_blocks_per_cu(adam_blocks_per_cu<GDT, RC>(a.rs.R),
                                             a.groups ? (uint32_t)sizeof(PackedLds) : 0u);
  if (a.groups)
    hipLaunchKernelGGL((adam_group_kernel<GDT, PDT, RC>), chunk_grid(a.n_groups, grid), kBlock, lds, s, a);
  else
    hipLaunchKernelGGL((adam_kernel<GDT, PDT, RC>), chunk_grid(a.n_chunks, grid), kBlock, lds, s, a);
}

template <int GDT, int RC>
void launch_adam_p(const AdamArgs& a, int pdt, uint32_t grid, hipStream_t s) {
  if (pdt == ZERO_F16) launch_adam_k<GDT, ZERO_F16, RC>(a, grid, s);
  else if (pdt == ZERO_BF16) launch_adam_k<GDT, ZERO_BF16, RC>(a, grid, s);
  else launch_adam_k<GDT, ZERO_NONE, RC>(a, grid, s);
}

// Rank counts with a fully unrolled kernel; any other count takes the batched one.
template <int GDT>
void launch_adam_r(const AdamArgs& a, int pdt, uint32_t grid, hipStream_t s) {
  switch (a.rs.R) {
    case 1: launch_adam_p<GDT, 1>(a, pdt, grid, s); break;
    case 2: launch_adam_p<GDT, 2>(a, pdt, grid, s); break;
    case 4: launch_adam_p<GDT, 4>(a, pdt, grid, s); break;
    case 8: launch_adam_p<GDT, 8>(a, pdt, grid, s); break;
    case 16: launch_adam_p<GDT, 16>(a, pdt, grid, s); break;
    default: launch_adam_p<GDT, 0>(a, pdt, grid, s); break;
  }
}

}  // namespace
}  // namespace zs

using namespace zs;

extern "C" int zero_reduce_owned(const void* const* rank_grads, uint32_t R, int grad_dtype,
                                 uint64_t grad_base, uint64_t begin, uint64_t n, float divisor,
                                 int accumulate, float* out, uint64_t out_base,
                                 int32_t* d_overflow, double* d_sumsq, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  static const char* who = "zero_reduce_owned";
  clear_error();
  ReduceArgs a;
  std::memset(&a, 0, sizeof a);
  int rc = fill_ranks(&a.rs, rank_grads, R, grad_dtype, grad_base, begin, divisor, who);
  if (rc) return rc;
  if (!out) return fail(ZERO_EINVAL, "%s: out is NULL", who);
  if (!aligned16(out)) return fail(ZERO_EINVAL, "%s: out is not 16-byte aligned", who);
  if (out_base % 8 != 0) return fail(ZERO_EINVAL, "%s: out_base must be a multiple of 8", who);
  if (begin < out_base) return fail(ZERO_EINVAL, "%s: begin lies below out_base", who);
  if (n > UINT64_MAX - begin) return fail(ZERO_EINVAL, "%s: begin + n overflows", who);
  if (accumulate < kOverwrite || accumulate > kAddMean)
    return fail(ZERO_EINVAL, "%s: accumulate must be 0, 1 or 2", who);
  const bool check = d_overflow != nullptr || d_sumsq != nullptr;
  if (check) {
    if (!d_overflow || !d_sumsq)
      return fail(ZERO_EINVAL, "%s: give both d_overflow and d_sumsq, or neither", who);
    if ((rc = check_workspace(workspace, ws_bytes, n, who))) return rc;
  }
  if (n == 0) return ZERO_OK;
  if ((rc = begin_launch())) return rc;
  a.begin = begin;
  a.end = begin + n;
  a.out = out;
  a.out_base = out_base;
  const uint64_t a0 = std::min<uint64_t>(a.end, (begin + 7) & ~7ull);
  const uint64_t a1 = std::max<uint64_t>(a0, a.end & ~7ull);
  a.piece = reduce_piece(R);
  a.xcd_order = reduce_xcd_order(R);
  const uint32_t grid = flat_grid(a1 / 8 - a0 / 8, a.piece);
  if (check) a.chk = check_layout(workspace, grid);
  switch (grad_dtype) {
    case ZERO_F16: launch_reduce<ZERO_F16>(a, accumulate, check, grid, stream); break;
    case ZERO_BF16: launch_reduce<ZERO_BF16>(a, accumulate, check, grid, stream); break;
    default: launch_reduce<ZERO_F32>(a, accumulate, check, grid, stream); break;
  }
  if ((rc = launch_status(who))) return rc;
  if (check) {
    finish_check(a.chk, grid, d_overflow, d_sumsq, stream);
    if ((rc = launch_status(who))) return rc;
  }
  return ZERO_OK;
}

// ---------------------------------------------------------------------------
// The checked reduce without a caller workspace, for callers that cannot
// allocate device memory.  Its per-block partials live in `scratch`, a
// file-scope device array of kScratchBytes that every GPU the library runs on
// holds until the process ends.  Host code never passes the array's name to a
// kernel: the first call on a device looks up that device's address of the
// array once, and the kernels take that address, as they take a workspace.
// Every block of the check writes the partial it later reads, so the array
// needs no clearing; calls that overlap on one GPU share it and race.
// ---------------------------------------------------------------------------
namespace zs {
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;  // a check over up to ~2.8e9 elements
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // device address of `scratch`, per device
}  // namespace
}  // namespace zs

static __device__ __align__(256) unsigned char scratch[zs::kScratchBytes];

namespace zs {
namespace {
int scratch_address(void** out, const char* who) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ZERO_EHIP, "%s: no current HIP device", who);
  if (dev < 0 || dev >= kScratchDevices)
    return fail(ZERO_EINVAL, "%s: device %d beyond the %d this library serves", who, dev, kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ZERO_EHIP, "%s: looking up the scratch array on device %d failed: %s", who, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ZERO_OK;
}
}  // namespace
}  // namespace zs

extern "C" int zero_reduce_owned_noalloc(const void* const* rank_grads, uint32_t R, int grad_dtype,
                                         uint64_t grad_base, uint64_t begin, uint64_t n, float divisor,
                                         int accumulate, float* out, uint64_t out_base, int32_t* d_overflow,
                                         double* d_sumsq, hipStream_t stream) {
  static const char* who = "zero_reduce_owned_noalloc";
  clear_error();
  if (d_overflow == nullptr && d_sumsq == nullptr)  // no check: nothing needs scratch
    return zero_reduce_owned(rank_grads, R, grad_dtype, grad_base, begin, n, divisor, accumulate, out,
                             out_base, nullptr, nullptr, nullptr, 0, stream);
  const uint64_t need = check_ws_bytes(check_parts(n));
  if (need > kScratchBytes)
    return fail(ZERO_ERANGE,
                "%s: a check over %llu elements needs %llu bytes of partials, more than the %zu-byte "
                "scratch array holds (use zero_reduce_owned with a workspace)",
                who, (unsigned long long)n, (unsigned long long)need, kScratchBytes);
  void* ws = nullptr;
  const int rc = scratch_address(&ws, who);
  if (rc) return rc;
  return zero_reduce_owned(rank_grads, R, grad_dtype, grad_base, begin, n, divisor, accumulate, out, out_base,
                           d_overflow, d_sumsq, ws, kScratchBytes, stream);
}

extern "C" int zero_check_workspace_bytes(uint64_t n, uint64_t* bytes) {
  clear_error();
  if (!bytes) return fail(ZERO_EINVAL, "zero_check_workspace_bytes: bytes is NULL");
  *bytes = check_ws_bytes(check_parts(n));
  return ZERO_OK;
}

extern "C" int zero_grad_check(const float* g, uint64_t n, int32_t* d_overflow, double* d_sumsq,
                               void* workspace, size_t ws_bytes, hipStream_t stream) {
  static const char* who = "zero_grad_check";
  clear_error();
  if (!d_overflow || !d_sumsq) return fail(ZERO_EINVAL, "%s: NULL output", who);
  int rc = check_workspace(workspace, ws_bytes, n, who);
  if (rc) return rc;
  if (n > 0 && !g) return fail(ZERO_EINVAL, "%s: g is NULL", who);
  if (n > 0 && !aligned16(g)) return fail(ZERO_EINVAL, "%s: g is not 16-byte aligned", who);
  if ((rc = begin_launch())) return rc;
  const uint32_t grid = flat_grid(n / 8);
  const CheckOut chk = check_layout(workspace, grid);
  hipLaunchKernelGGL(check_kernel, grid, kBlock, 0, stream, g, n, chk);
  if ((rc = launch_status(who))) return rc;
  finish_check(chk, grid, d_overflow, d_sumsq, stream);
  return launch_status(who);
}

extern "C" int zero_adam_step(const zero_adam_args* p, hipStream_t stream) {
  static const char* who = "zero_adam_step";
  clear_error();
  if (!p) return fail(ZERO_EINVAL, "%s: args is NULL", who);
  AdamArgs a;
  std::memset(&a, 0, sizeof a);
  int rc;
  if (p->step == 0) return fail(ZERO_EINVAL, "%s: step counts from 1", who);
  if (p->begin > p->end) return fail(ZERO_EINVAL, "%s: begin > end", who);
  if (p->n_chunks > 0 && !p->chunks) return fail(ZERO_EINVAL, "%s: chunks is NULL", who);
  if (!p->groups && p->n_groups != 0)
    return fail(ZERO_EINVAL, "%s: n_groups given without a group table", who);
  const bool reduced = p->reduced_g != nullptr;
  if (reduced) {
    if (!aligned16(p->reduced_g))
      return fail(ZERO_EINVAL, "%s: reduced_g is not 16-byte aligned", who);
  } else if ((rc = fill_ranks(&a.rs, p->rank_grads, p->R, p->grad_dtype, p->grad_base, p->begin,
                              p->divisor, who))) {
    return rc;
  }
  if (!p->master || !p->exp_avg || !p->exp_avg_sq)
    return fail(ZERO_EINVAL, "%s: master/exp_avg/exp_avg_sq must be given", who);
  if (!aligned16(p->master) || !aligned16(p->exp_avg) || !aligned16(p->exp_avg_sq))
    return fail(ZERO_EINVAL, "%s: state arrays must be 16-byte aligned", who);
  if (p->local_base % 8 != 0 || p->local_base > p->begin)
    return fail(ZERO_EINVAL, "%s: local_base must be a multiple of 8 and <= begin", who);
  const int pdt = p->param_dtype;
  if (pdt != ZERO_NONE && pdt != ZERO_F16 && pdt != ZERO_BF16)
    return fail(ZERO_EINVAL, "%s: param_dtype must be NONE, F16 or BF16", who);
  if (pdt != ZERO_NONE) {
    if (!p->param16) return fail(ZERO_EINVAL, "%s: param16 is NULL", who);
    if (!aligned16(p->param16)) return fail(ZERO_EINVAL, "%s: param16 is not 16-byte aligned", who);
    if (p->param_base % 8 != 0 || p->param_base > p->begin)
      return fail(ZERO_EINVAL, "%s: param_base must be a multiple of 8 and <= begin", who);
  }
  const double hp[] = {p->lr, p->beta1, p->beta2, p->eps, p->weight_decay, p->clip_coef};
  for (double x : hp)
    if (!std::isfinite(x)) return fail(ZERO_EINVAL, "%s: non-finite hyperparameter", who);
  if (p->lr < 0 || p->eps < 0 || p->weight_decay < 0 || p->clip_coef < 0)
    return fail(ZERO_EINVAL, "%s: lr, eps, weight_decay and clip_coef must be >= 0", who);
  if (p->beta1 < 0 || p->beta1 >= 1 || p->beta2 < 0 || p->beta2 >= 1)
    return fail(ZERO_EINVAL, "%s: betas must lie in [0, 1)", who);
  if (p->n_chunks == 0 || p->begin == p->end || (p->groups && p->n_groups == 0)) return ZERO_OK;
  if ((rc = begin_launch())) return rc;

  // Constants in fp64, each rounded once to fp32.
  const double t = (double)p->step;
  const double bc1 = 1.0 - std::pow(p->beta1, t);
  const double bc2 = 1.0 - std::pow(p->beta2, t);
  a.c.beta1 = (float)p->beta1;
  a.c.one_minus_beta1 = (float)(1.0 - p->beta1);
  a.c.beta2 = (float)p->beta2;
  a.c.one_minus_beta2 = (float)(1.0 - p->beta2);
  a.c.step_size = (float)(p->lr / bc1);
  a.c.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  a.c.eps = (float)p->eps;
  a.c.decay = p->adamw ? (float)(1.0 - p->lr * p->weight_decay) : 1.0f;
  a.c.l2 = p->adamw ? 0.0f : (float)p->weight_decay;
  a.c.clip = (float)p->clip_coef;
  a.chunks = p->chunks;
  a.n_chunks = p->n_chunks;
  a.groups = p->groups;
  a.n_groups = p->groups ? p->n_groups : 0;
  a.begin = p->begin;
  a.end = p->end;
  a.reduced_g = p->reduced_g;
  a.w = p->master;
  a.m = p->exp_avg;
  a.v = p->exp_avg_sq;
  a.local_base = p->local_base;
  a.p16 = pdt != ZERO_NONE ? p->param16 : nullptr;
  a.param_base = p->param_base;

  const uint32_t grid = p->grid_blocks;
  if (reduced) {
    launch_adam_p<ZERO_F32, kReduced>(a, pdt, grid, stream);
  } else {
    switch (p->grad_dtype) {
      case ZERO_F16: launch_adam_r<ZERO_F16>(a, pdt, grid, stream); break;
      case ZERO_BF16: launch_adam_r<ZERO_BF16>(a, pdt, grid, stream); break;
      default: launch_adam_r<ZERO_F32>(a, pdt, grid, stream); break;
    }
  }
  return launch_status(who);
}

