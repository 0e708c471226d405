// The bandwidth probe of libzero_shard: a plain 128-bit streaming kernel whose
// read:write mix is chosen by the caller.  It measures the HBM rate this
// device reaches for a given mix of streams, the ceiling that the optimizer
// kernels are compared with; it is not part of the optimizer step.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "launch.h"

namespace zs {
namespace {

struct ProbeArgs {
  const uint4* src[ZERO_MAX_PROBE_STREAMS];
  uint4* dst[ZERO_MAX_PROBE_STREAMS];
  uint32_t n_src, n_dst;
  uint64_t n_vec;  // 16-byte vectors per stream
  int xcd_order;   // pieces in XCD-contiguous runs (xcd_contiguous)
};

constexpr int kProbeBatch = 4;  // sources whose loads are issued together

// One 16-byte vector per thread and stream: block b covers the vectors
// [p * kBlock, (p + 1) * kBlock) of every stream, where p = b or, in XCD
// order, p = xcd_contiguous(b); blocks are dispatched in order (a grid
// smaller than the piece count takes the rest with a grid stride).
// Loads of kProbeBatch sources are issued before they are combined; the XOR
// is then stored to every destination.  Without destinations the XOR is only
// kept live (an empty asm statement takes it as an operand), so the loads
// stay and nothing is written.
__global__ void __launch_bounds__(kBlock) probe_kernel(const ProbeArgs a) {
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  const uint64_t blk = a.xcd_order ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
  for (uint64_t i = blk * kBlock + threadIdx.x; i < a.n_vec; i += stride) {
    uint4 x = make_uint4(0, 0, 0, 0);
    for (uint32_t s0 = 0; s0 < a.n_src; s0 += kProbeBatch) {
      const uint32_t nb = min((uint32_t)kProbeBatch, a.n_src - s0);
      uint4 y[kProbeBatch];
#pragma unroll
      for (int j = 0; j < kProbeBatch; ++j)
        y[j] = j < (int)nb ? a.src[s0 + j][i] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kProbeBatch; ++j) {
        x.x ^= y[j].x;
        x.y ^= y[j].y;
        x.z ^= y[j].z;
        x.w ^= y[j].w;
      }
    }
    asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
    for (uint32_t d = 0; d < a.n_dst; ++d) a.dst[d][i] = x;
  }
}

}  // namespace
}  // namespace zs

using namespace zs;

extern "C" int zero_stream_probe(const void* const* srcs, uint32_t n_src, void* const* dsts,
                                 uint32_t n_dst, uint64_t bytes, int order, hipStream_t stream) {
  static const char* who = "zero_stream_probe";
  clear_error();
  if (n_src > ZERO_MAX_PROBE_STREAMS || n_dst > ZERO_MAX_PROBE_STREAMS || n_src + n_dst == 0)
    return fail(ZERO_EINVAL, "%s: stream counts %u, %u: each at most %d, not both 0", who, n_src,
                n_dst, ZERO_MAX_PROBE_STREAMS);
  if (order != 0 && order != 1) return fail(ZERO_EINVAL, "%s: order must be 0 or 1, got %d", who, order);
  if (bytes % 16) return fail(ZERO_EINVAL, "%s: %llu bytes is not a multiple of 16", who,
                              (unsigned long long)bytes);
  if (bytes == 0) return ZERO_OK;
  if ((n_src && !srcs) || (n_dst && !dsts)) return fail(ZERO_EINVAL, "%s: NULL pointer array", who);
  ProbeArgs a{};
  for (uint32_t s = 0; s < n_src; ++s) {
    if (!srcs[s] || !aligned16(srcs[s]))
      return fail(ZERO_EINVAL, "%s: source %u is NULL or not 16-byte aligned", who, s);
    a.src[s] = static_cast<const uint4*>(srcs[s]);
  }
  for (uint32_t d = 0; d < n_dst; ++d) {
    if (!dsts[d] || !aligned16(dsts[d]))
      return fail(ZERO_EINVAL, "%s: destination %u is NULL or not 16-byte aligned", who, d);
    a.dst[d] = static_cast<uint4*>(dsts[d]);
  }
  a.n_src = n_src;
  a.n_dst = n_dst;
  a.n_vec = bytes / 16;
  a.xcd_order = order;
  int rc = begin_launch();
  if (rc) return rc;
  hipLaunchKernelGGL(probe_kernel, chunk_grid((a.n_vec + kBlock - 1) / kBlock, 0), kBlock, 0, stream,
                     a);
  return launch_status(who);
}
