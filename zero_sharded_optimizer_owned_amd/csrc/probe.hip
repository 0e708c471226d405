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
  uint64_t src_wide, dst_wide;  // bit s set: stream s takes 2 vectors per thread, else 1
  uint32_t n_src, n_dst;
  uint64_t n_vec;  // threads' worth of work: a stream of width w holds w * n_vec vectors
  int xcd_order;   // pieces in XCD-contiguous runs (xcd_contiguous)
};

constexpr int kProbeBatch = 4;  // sources whose loads are issued together

// One unit of work per thread and stream: thread i of the grid touches the
// vectors [w * i, w * i + w) of a stream of width w (16 or 32 contiguous
// bytes, like one 8-element vector of 16-bit or fp32 data).  Block b covers
// the units [p * kBlock, (p + 1) * kBlock), where p = b or, in XCD order,
// p = xcd_contiguous(b); blocks are dispatched in order (a grid smaller than
// the piece count takes the rest with a grid stride).  Loads of kProbeBatch
// sources are issued before they are combined; the XOR is then stored to
// every destination.  Without destinations the XOR is only kept live (an
// empty asm statement takes it as an operand), so the loads stay and nothing
// is written.
__global__ void __launch_bounds__(kBlock) probe_kernel(const ProbeArgs a) {
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  const uint64_t blk = a.xcd_order ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (uint64_t i = blk * kBlock + threadIdx.x; i < a.n_vec; i += stride) {
    uint4 x = zero;
    for (uint32_t s0 = 0; s0 < a.n_src; s0 += kProbeBatch) {
      const uint32_t nb = min((uint32_t)kProbeBatch, a.n_src - s0);
      uint4 y[kProbeBatch], z[kProbeBatch];
#pragma unroll
      for (int j = 0; j < kProbeBatch; ++j) {
        y[j] = zero;
        z[j] = zero;
        if (j < (int)nb) {
          const uint4* p = a.src[s0 + j];
          if ((a.src_wide >> (s0 + j)) & 1) {
            y[j] = p[2 * i];
            z[j] = p[2 * i + 1];
          } else {
            y[j] = p[i];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kProbeBatch; ++j) {
        x.x ^= y[j].x ^ z[j].x;
        x.y ^= y[j].y ^ z[j].y;
        x.z ^= y[j].z ^ z[j].z;
        x.w ^= y[j].w ^ z[j].w;
      }
    }
    asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
    for (uint32_t d = 0; d < a.n_dst; ++d) {
      if ((a.dst_wide >> d) & 1) {
        a.dst[d][2 * i] = x;
        a.dst[d][2 * i + 1] = x;
      } else {
        a.dst[d][i] = x;
      }
    }
  }
}

}  // namespace
}  // namespace zs

using namespace zs;

extern "C" int zero_stream_probe(const void* const* srcs, const uint8_t* src_widths, uint32_t n_src,
                                 void* const* dsts, const uint8_t* dst_widths, uint32_t n_dst,
                                 uint64_t bytes, int order, hipStream_t stream) {
  static const char* who = "zero_stream_probe";
  clear_error();
  if (n_src > ZERO_MAX_PROBE_STREAMS || n_dst > ZERO_MAX_PROBE_STREAMS || n_src + n_dst == 0)
    return fail(ZERO_EINVAL, "%s: stream counts %u, %u: each at most %d, not both 0", who, n_src,
                n_dst, ZERO_MAX_PROBE_STREAMS);
  if (order != 0 && order != 1) return fail(ZERO_EINVAL, "%s: order must be 0 or 1, got %d", who, order);
  if (bytes % 16) return fail(ZERO_EINVAL, "%s: %llu bytes is not a multiple of 16", who,
                              (unsigned long long)bytes);
  if ((n_src && !srcs) || (n_dst && !dsts)) return fail(ZERO_EINVAL, "%s: NULL pointer array", who);
  ProbeArgs a{};
  for (uint32_t s = 0; s < n_src; ++s) {
    if (!srcs[s] || !aligned16(srcs[s]))
      return fail(ZERO_EINVAL, "%s: source %u is NULL or not 16-byte aligned", who, s);
    a.src[s] = static_cast<const uint4*>(srcs[s]);
    const unsigned w = src_widths ? src_widths[s] : 1;
    if (w != 1 && w != 2) return fail(ZERO_EINVAL, "%s: source %u has width %u", who, s, w);
    if (w == 2) a.src_wide |= 1ull << s;
  }
  for (uint32_t d = 0; d < n_dst; ++d) {
    if (!dsts[d] || !aligned16(dsts[d]))
      return fail(ZERO_EINVAL, "%s: destination %u is NULL or not 16-byte aligned", who, d);
    a.dst[d] = static_cast<uint4*>(dsts[d]);
    const unsigned w = dst_widths ? dst_widths[d] : 1;
    if (w != 1 && w != 2) return fail(ZERO_EINVAL, "%s: destination %u has width %u", who, d, w);
    if (w == 2) a.dst_wide |= 1ull << d;
  }
  if (bytes == 0) return ZERO_OK;
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
