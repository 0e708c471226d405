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

namespace {
constexpr int kMaxDevices = 64;
int g_lds_cu[kMaxDevices];   // LDS bytes per CU, 0 = not yet queried
int g_lds_blk[kMaxDevices];  // largest LDS allocation of one block
}  // namespace

uint32_t lds_for_blocks_per_cu(uint32_t per_cu, uint32_t static_bytes) {
  int dev = 0;
  if (per_cu == 0 || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cu = __atomic_load_n(&g_lds_cu[dev], __ATOMIC_ACQUIRE);
  int blk = __atomic_load_n(&g_lds_blk[dev], __ATOMIC_RELAXED);
  if (cu == 0) {
    if (hipDeviceGetAttribute(&blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        cu <= 0 || blk <= 0)
      return 0;
    __atomic_store_n(&g_lds_blk[dev], blk, __ATOMIC_RELAXED);
    __atomic_store_n(&g_lds_cu[dev], cu, __ATOMIC_RELEASE);
  }
  // A block's whole LDS (its static arrays plus the reservation) must exceed
  // a (per_cu + 1)-th of the CU's LDS, with a granule of margin: per_cu
  // blocks fit, one more does not.
  const uint64_t target = (uint64_t)cu / (per_cu + 1) + 1024;
  const uint64_t dyn = target > static_bytes ? (target - static_bytes + 1023) / 1024 * 1024 : 0;
  const uint64_t total = dyn + static_bytes;
  if (total * per_cu > (uint64_t)cu || total > (uint64_t)blk) return 0;
  return (uint32_t)dyn;
}

uint32_t chunk_grid(uint64_t n_pieces, uint32_t requested) {
  if (requested) return requested;
  if (n_pieces == 0) return 1;
  return n_pieces < kMaxChunkGrid ? (uint32_t)n_pieces : kMaxChunkGrid;
}

}  // namespace zs
