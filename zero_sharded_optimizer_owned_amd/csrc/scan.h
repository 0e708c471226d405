// Block-wide prefix sums for the packed (several pieces per block) kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace zs {

// Inclusive prefix sum of one 64-bit value per thread over a kBlock-thread
// block: a shuffle scan inside each wavefront, then the wavefront totals
// through LDS (`s_wave`, kWavesPerBlock entries).  Every thread of the block
// must call it; it synchronises the block once.  The caller synchronises
// again before reusing `s_wave`.
__device__ __forceinline__ uint64_t block_inclusive_scan(uint64_t x, uint64_t* s_wave) {
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (uint32_t d = 1; d < 64; d <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)x, d, 64);
    const uint32_t hi = __shfl_up((uint32_t)(x >> 32), d, 64);
    if (lane >= d) x += (uint64_t)hi << 32 | lo;
  }
  if (lane == 63) s_wave[w] = x;
  __syncthreads();
  uint64_t before = 0;
  for (uint32_t i = 0; i < w; ++i) before += s_wave[i];
  return x + before;
}

}  // namespace zs
