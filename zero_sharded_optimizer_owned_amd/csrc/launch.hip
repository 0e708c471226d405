// Launch planning shared by the device sources of libzero_shard.
#include "launch.h"

namespace zs {

int begin_launch() {
  (void)hipGetLastError();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ZERO_EHIP, "no current HIP device");
  return ZERO_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ZERO_OK;
}

uint32_t chunk_grid(uint64_t n_pieces, uint32_t requested) {
  if (requested) return requested;
  if (n_pieces == 0) return 1;
  return n_pieces < kMaxChunkGrid ? (uint32_t)n_pieces : kMaxChunkGrid;
}

}  // namespace zs
