// Launch planning shared by the device sources of libzero_shard.
#include "launch.h"

namespace zs {

namespace {
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];  // 0 = not yet queried
}  // namespace

int cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ZERO_EHIP, "hipGetDevice failed");
  if (dev >= 0 && dev < kMaxDevices && __atomic_load_n(&g_cu_count[dev], __ATOMIC_RELAXED) > 0) {
    *out = __atomic_load_n(&g_cu_count[dev], __ATOMIC_RELAXED);
    return ZERO_OK;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return fail(ZERO_EHIP, "querying the compute-unit count failed");
  if (dev >= 0 && dev < kMaxDevices) __atomic_store_n(&g_cu_count[dev], cus, __ATOMIC_RELAXED);
  *out = cus;
  return ZERO_OK;
}

int begin_launch(int* cus) {
  (void)hipGetLastError();
  return cu_count(cus);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ZERO_OK;
}

// A persistent grid: every block resident at once, but no more blocks than
// there are chunks for their wavefronts.
uint32_t persistent_grid(uint32_t per_cu, uint64_t n_chunks, int cus, uint32_t requested) {
  if (requested) return requested;
  const uint64_t resident = (uint64_t)per_cu * (uint64_t)cus;
  const uint64_t by_chunks = (n_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  return (uint32_t)(by_chunks < resident ? by_chunks : resident);
}

}  // namespace zs
