// Host check of the piece orders in launch.h (built with hipcc --cuda-host-only
// by tests/test_abi_host.py): each remapping is a bijection of [0, G) for any
// grid size, xcd_runs with K = 1 is the identity, xcd_contiguous gives every
// XCD (block b runs on XCD b mod 8) one contiguous run of pieces, and
// xcd_runs gives it runs of K consecutive pieces in every full round.
#include <cstdio>
#include <vector>

#include "launch.h"

static int fails = 0;
#define CHECK(c, ...)                   \
  do {                                  \
    if (!(c)) {                         \
      ++fails;                          \
      if (fails < 10) printf(__VA_ARGS__); \
    }                                   \
  } while (0)

int main() {
  const uint64_t grids[] = {1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 128, 1000, 4096, 4097, 65537, 183106};
  const uint64_t runs[] = {1, 2, 3, 4, 16, 64};
  for (uint64_t G : grids) {
    std::vector<int> seen(G, 0);
    std::vector<uint64_t> lo(zs::kXcds, ~0ull), hi(zs::kXcds, 0), cnt(zs::kXcds, 0);
    for (uint64_t b = 0; b < G; ++b) {
      const uint64_t p = zs::xcd_contiguous(b, G);
      CHECK(p < G, "contiguous: %llu -> %llu outside %llu\n", (unsigned long long)b, (unsigned long long)p,
            (unsigned long long)G);
      if (p < G) seen[p]++;
      const uint64_t x = b % zs::kXcds;
      lo[x] = p < lo[x] ? p : lo[x];
      hi[x] = p > hi[x] ? p : hi[x];
      cnt[x]++;
    }
    for (uint64_t p = 0; p < G; ++p) CHECK(seen[p] == 1, "contiguous: piece %llu taken %d times (G %llu)\n",
                                           (unsigned long long)p, seen[p], (unsigned long long)G);
    for (uint64_t x = 0; x < zs::kXcds; ++x)
      if (cnt[x]) CHECK(hi[x] - lo[x] + 1 == cnt[x], "contiguous: XCD %llu not one run (G %llu)\n",
                        (unsigned long long)x, (unsigned long long)G);
    for (uint64_t K : runs) {
      std::vector<int> seen2(G, 0);
      const uint64_t span = zs::kXcds * K, full = G / span * span;
      for (uint64_t b = 0; b < G; ++b) {
        const uint64_t p = zs::xcd_runs(b, G, K);
        CHECK(p < G, "runs %llu: out of range\n", (unsigned long long)K);
        if (p < G) seen2[p]++;
        if (K == 1) CHECK(p == b, "runs 1 is not the identity\n");
        // within a full round, the next block of the same XCD takes the next piece
        if (b + zs::kXcds < full && (b / zs::kXcds) % K != K - 1)
          CHECK(zs::xcd_runs(b + zs::kXcds, G, K) == p + 1, "runs %llu: not consecutive at block %llu\n",
                (unsigned long long)K, (unsigned long long)b);
      }
      for (uint64_t p = 0; p < G; ++p) CHECK(seen2[p] == 1, "runs %llu: piece %llu taken %d times (G %llu)\n",
                                             (unsigned long long)K, (unsigned long long)p, seen2[p],
                                             (unsigned long long)G);
    }
  }
  if (fails) {
    printf("%d failures\n", fails);
    return 1;
  }
  printf("clean\n");
  return 0;
}
