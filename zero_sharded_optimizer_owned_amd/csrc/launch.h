// Launch planning shared by the device sources of libzero_shard.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace zs {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;

// Before an entry point's launches: clears a pending error left by earlier,
// unrelated HIP calls (so launch_status reports only this call's launches)
// and checks that a device is current.
int begin_launch();
bool aligned16(const void* p);
// ZERO_OK, or ZERO_EHIP with a message if the last launch failed.
int launch_status(const char* who);

// Every kernel of the library gives one block one short contiguous piece of
// work (a chunk, a span, or 256 consecutive vectors of a flat range) and
// launches one block per piece: the hardware dispatches blocks in index
// order, so the pieces in flight stay inside a narrow, advancing window of
// each stream, which is what HBM streams fastest.  The grid is capped so that
// its thread count stays within the launch limit (`requested` != 0
// overrides); kernels take any pieces past the grid with a grid stride.
constexpr uint32_t kMaxChunkGrid = 1u << 23;
uint32_t chunk_grid(uint64_t n_pieces, uint32_t requested);

// The dispatcher deals a launch's blocks to the chip's 8 XCDs in turn (block b
// to XCD b mod 8), so neighbouring pieces run on different XCDs at the same
// time.  xcd_contiguous maps block b of a G-block grid to a piece index such
// that each XCD takes one contiguous run of about G/8 pieces instead (a
// bijection of [0, G)).  Measured with the streaming probe: contiguous runs
// stream one source 6% faster and a 1:1 copy 2.4% faster, but lose 1-2% from
// about ten streams on; kernels opt in where their own A/B says so.
constexpr uint64_t kXcds = 8;
__host__ __device__ __forceinline__ uint64_t xcd_contiguous(uint64_t b, uint64_t G) {
  const uint64_t x = b % kXcds, k = b / kXcds, q = G / kXcds, r = G % kXcds;
  return x * q + (x < r ? x : r) + k;
}

// Between the two: the XCDs take runs of K consecutive pieces in turn (XCD x
// gets pieces xK .. xK+K-1, then 8K + xK .. , and so on); a last partial
// round keeps the plain order.  A bijection of [0, G); K = 1 is the identity.
__host__ __device__ __forceinline__ uint64_t xcd_runs(uint64_t b, uint64_t G, uint64_t K) {
  const uint64_t span = kXcds * K, full = G / span * span;
  if (b >= full) return b;
  return b / span * span + (b % kXcds) * K + (b / kXcds) % K;
}

// Dynamic LDS bytes that let at most `per_cu` blocks of a kernel reside on one
// CU at a time, for a kernel whose own arrays take `static_bytes` of LDS (the
// reservation only caps residency; nothing reads it).  0 -- no cap -- when
// the device cannot give one block that much, or when the query fails.  The
// device's LDS sizes are queried once per device.
uint32_t lds_for_blocks_per_cu(uint32_t per_cu, uint32_t static_bytes);

}  // namespace zs
