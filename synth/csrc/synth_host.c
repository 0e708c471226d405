/*
 * Seeded synthetic inputs on the host, multi-threaded (test and benchmark
 * infrastructure, input generation only).
 *
 * Host twin of synth/__init__.py (numpy) and synth/csrc/synth_device.hip:
 * element i of a stream is output i of a SplitMix64 sequence started at the
 * stream key, turned into an fp32 value by one IEEE rounding (normal, uniform
 * or square recipe), then stored as fp32 or rounded to fp16 / bf16 (nearest,
 * ties to even).  Same bits as the other two at every index; the numpy
 * version is the reference the CPU tests hold this one to.  It exists because
 * full-size inputs (tens of billions of values) are too slow to produce in
 * numpy.  Holds no part of the optimizer arithmetic.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const uint64_t kGolden = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline float value_f32(uint64_t key, uint64_t idx, int dist, float c) {
  const uint64_t h = mix64(key + (idx + 1) * kGolden);
  if (dist == 1) {
    const int32_t centred = (int32_t)(h >> 40) - 8388608;
    return (float)centred * c;
  }
  const uint64_t s = (h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48);
  const float x = (float)((int32_t)s - 131070) * c;
  return dist == 2 ? x * x : x;
}

static inline uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}

/* bfloat16: the upper half of the fp32 pattern, rounded to nearest even. */
static inline uint16_t to_bf16(float x) {
  const uint32_t u = f32_bits(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* binary16, nearest even: normal results by rounding the fp32 significand at
 * bit 13 and rebasing the exponent (127 - 15 = 112); results below 2^-14 by
 * scaling to units of the smallest subnormal (2^-24, exact) and rounding to
 * an integer in the default (nearest-even) mode; 65520 and above overflow. */
static inline uint16_t to_f16(float x) {
  const uint32_t u = f32_bits(x);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);
  if (a < 0x38800000u) return (uint16_t)(sign | (uint16_t)nearbyintf(fabsf(x) * 16777216.0f));
  return (uint16_t)(sign | (uint16_t)(((a + 0x0FFFu + ((a >> 13) & 1u)) >> 13) - (112u << 10)));
}

/* dst[0..n) = elements index0 .. index0+n-1 of the stream `key`, stored as
 * dtype (1 fp16, 2 bf16: uint16 patterns; 3 fp32).  dist: 0 normal,
 * 1 uniform, 2 square; c is the recipe's fp32 scale.  Returns 0 or -1. */
int synth_host_fill(void *dst, int dtype, uint64_t n, uint64_t key, uint64_t index0, int dist, float c) {
  if (n == 0) return 0;
  if (!dst || dtype < 1 || dtype > 3 || dist < 0 || dist > 2) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    const float x = value_f32(key, index0 + (uint64_t)i, dist, c);
    if (dtype == 3) ((float *)dst)[i] = x;
    else if (dtype == 1) ((uint16_t *)dst)[i] = to_f16(x);
    else ((uint16_t *)dst)[i] = to_bf16(x);
  }
  return 0;
}
