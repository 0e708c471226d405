// Launch planning shared by the device sources of libzero_shard.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace zs {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;

// Compute units of the current device (queried once per device).
int cu_count(int* out);
// Before an entry point's launches: clears a pending error left by earlier,
// unrelated HIP calls (so launch_status reports only this call's launches)
// and returns the compute-unit count.
int begin_launch(int* cus);
bool aligned16(const void* p);
// ZERO_OK, or ZERO_EHIP with a message if the last launch failed.
int launch_status(const char* who);
// Blocks that fit on all CUs at once, capped by the chunks' wavefronts
// (`requested` != 0 overrides).
uint32_t persistent_grid(uint32_t per_cu, uint64_t n_chunks, int cus, uint32_t requested);

// Blocks of `kernel` that fit on one CU at once.
template <typename K>
uint32_t blocks_per_cu(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kBlock, 0) != hipSuccess || n < 1) n = 1;
  return (uint32_t)n;
}

}  // namespace zs
