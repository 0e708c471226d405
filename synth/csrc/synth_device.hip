// Seeded synthetic inputs on the device (test and benchmark infrastructure).
//
// Device twin of synth/__init__.py: element i of a stream is output i of a
// SplitMix64 sequence started at the stream key, turned into an fp32 value by
// one IEEE rounding (normal / uniform / square recipes), then stored as fp32,
// or rounded to fp16 / bf16 (nearest, ties to even).  Same bits as the host
// generator at every index.  Holds no part of the optimizer arithmetic.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float value_f32(uint64_t key, uint64_t idx, int dist, float c) {
  const uint64_t h = mix64(key + (idx + 1) * kGolden);
  if (dist == 1) {
    const int32_t centred = (int32_t)(h >> 40) - 8388608;
    return (float)centred * c;
  }
  const uint64_t s = (h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48);
  const float x = (float)((int32_t)s - 131070) * c;
  return dist == 2 ? x * x : x;
}

__device__ __forceinline__ uint16_t to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void __launch_bounds__(256) fill_kernel(void* dst, int dtype, uint64_t n, uint64_t key,
                                                   uint64_t index0, int dist, float c) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float x = value_f32(key, index0 + i, dist, c);
    if (dtype == 3) {
      static_cast<float*>(dst)[i] = x;
    } else if (dtype == 1) {
      static_cast<__half*>(dst)[i] = __float2half_rn(x);
    } else {
      static_cast<uint16_t*>(dst)[i] = to_bf16_rne(x);
    }
  }
}

}  // namespace

extern "C" {

// Fill dst[0..n) with elements index0..index0+n of stream `key`.
// dtype: 1 fp16, 2 bf16, 3 fp32.  dist: 0 normal, 1 uniform, 2 square.
// c: the fp32 scale of the recipe (normal: sigma*sqrt(3)/65536, uniform: a/2^23).
// Returns 0, or -1 for bad arguments, -3 for a launch error.
int synth_fill(void* dst, int dtype, uint64_t n, uint64_t key, uint64_t index0, int dist, float c,
               hipStream_t stream) {
  if (n == 0) return 0;
  if (dst == nullptr || dtype < 1 || dtype > 3 || dist < 0 || dist > 2) return -1;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, dtype, n, key,
                     index0, dist, c);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
