// Sanitizer driver for the host half of libzero_shard (test infrastructure):
// layouts, chunk tables (counted, then filled, then with too small a
// capacity), dense offsets, state accounting, the clip scalar, the step
// decision over all owners and the stage-3 span builders
// over random tensor lists, plus the argument errors, in an
// AddressSanitizer / UndefinedBehaviorSanitizer build.  It also checks the
// chunk table's coverage: every real element of an owner exactly once, no
// padding (chunks may run across tensors that no padding separates).  Exit
// status 0 = clean run.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "zero_shard.h"

namespace {
uint64_t g_state = 0x243F6A8885A308D3ull;
uint64_t next() {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return g_state;
}
uint64_t below(uint64_t n) { return n ? next() % n : 0; }

int fails = 0;
void expect(bool ok, const char* what, int trial) {
  if (!ok) {
    std::fprintf(stderr, "trial %d: %s (%s)\n", trial, what, zero_last_error());
    ++fails;
  }
}
}  // namespace

int main() {
  static const uint32_t kAligns[] = {1, 2, 8, 64, 128};
  for (int trial = 0; trial < 400; ++trial) {
    const uint32_t T = 1 + (uint32_t)below(12);
    std::vector<uint64_t> numel(T);
    for (auto& x : numel) x = 1 + below(below(2) ? 50 : 5000);
    const uint32_t R = 1 + (uint32_t)below(70);
    const uint32_t A = kAligns[below(5)];
    std::vector<uint64_t> off(T), b(R), e(R);
    uint64_t total = 0;
    expect(zero_shard_layout(numel.data(), T, R, A, off.data(), &total, b.data(), e.data()) == ZERO_OK,
           "layout", trial);
    const uint32_t C = 8 * (1 + (uint32_t)below(300));
    for (uint32_t r = 0; r < R; ++r) {
      uint64_t count = 0;
      expect(zero_chunk_table(numel.data(), off.data(), T, b[r], e[r], C, nullptr, 0, &count) == ZERO_OK,
             "chunk count", trial);
      std::vector<zero_chunk> ch(count + 1);
      uint64_t got = 0;
      expect(zero_chunk_table(numel.data(), off.data(), T, b[r], e[r], C, ch.data(), count, &got) ==
                     ZERO_OK && got == count,
             "chunk fill", trial);
      if (count > 0) {
        uint64_t again = 0;
        expect(zero_chunk_table(numel.data(), off.data(), T, b[r], e[r], C, ch.data(), count - 1,
                                &again) == ZERO_ERANGE && again == count,
               "chunk capacity", trial);
      }
      // coverage: the chunks tile the real elements of [b, e) in order
      std::vector<unsigned char> hit(e[r] - b[r], 0);
      for (uint64_t i = 0; i < count; ++i) {
        const zero_chunk& c = ch[i];
        expect(c.tensor < T && c.len > 0 && c.len <= C, "chunk fields", trial);
        if (c.tensor >= T) continue;
        const uint64_t t0 = off[c.tensor], t1 = t0 + numel[c.tensor];
        expect(c.flat >= b[r] && c.flat + c.len <= e[r] && c.flat >= t0 && c.flat < t1,
               "chunk bounds", trial);
        for (uint64_t f = c.flat; f < c.flat + c.len && f >= b[r] && f < e[r]; ++f) ++hit[f - b[r]];
      }
      for (uint64_t f = b[r]; f < e[r]; ++f) {
        bool real = false;
        for (uint32_t k = 0; k < T; ++k) real = real || (f >= off[k] && f < off[k] + numel[k]);
        if (hit[f - b[r]] != (real ? 1 : 0)) {
          expect(false, "coverage", trial);
          break;
        }
      }
    }
    zero_ratio q[4];
    expect(zero_state_bytes(1 + below(1ull << 40), R, 2, 2, 12, q) == ZERO_OK, "state bytes", trial);
    float coef = 0.0f;
    expect(zero_clip_coef((double)below(1000), 1.0, 1e-6, &coef) == ZERO_OK, "clip", trial);
    std::vector<int32_t> flags(R);
    std::vector<double> partial(R);
    for (uint32_t r = 0; r < R; ++r) {
      flags[r] = below(50) == 0;
      partial[r] = (double)below(1000);
    }
    int32_t update = -1;
    expect(zero_step_decision(flags.data(), partial.data(), R, 1.0, 1e-6, &update, &coef) == ZERO_OK,
           "step decision", trial);
    std::vector<uint64_t> doff(T);
    uint64_t dtotal = 0;
    expect(zero_dense_offsets(numel.data(), T, doff.data(), &dtotal) == ZERO_OK && dtotal >= T,
           "dense offsets", trial);

    std::vector<uint32_t> live;
    for (uint32_t k = 0; k < T; ++k)
      if (below(2)) live.push_back(k);
    std::vector<uint64_t> shard(T);
    uint64_t resident = 0, gathered = 0;
    expect(zero3_storage(numel.data(), T, R, live.data(), (uint32_t)live.size(), shard.data(), &resident,
                         &gathered) == ZERO_OK,
           "zero3 storage", trial);
    const uint32_t span = 1 + (uint32_t)below(3000);
    uint64_t ns = 0;
    expect(zero3_gather_spans(numel.data(), T, R, live.data(), (uint32_t)live.size(), span, nullptr, 0,
                              &ns) == ZERO_OK,
           "gather count", trial);
    std::vector<zero_copy_span> sp(ns + 1);
    uint64_t ns2 = 0;
    expect(zero3_gather_spans(numel.data(), T, R, live.data(), (uint32_t)live.size(), span, sp.data(), ns,
                              &ns2) == ZERO_OK && ns2 == ns,
           "gather fill", trial);
    const uint32_t rank = (uint32_t)below(R);
    expect(zero3_partition_spans(numel.data(), T, R, rank, span, nullptr, 0, &ns) == ZERO_OK,
           "partition count", trial);
    sp.assign(ns + 1, zero_copy_span{});
    expect(zero3_partition_spans(numel.data(), T, R, rank, span, sp.data(), ns, &ns2) == ZERO_OK && ns2 == ns,
           "partition fill", trial);
    if (ns > 0)
      expect(zero3_partition_spans(numel.data(), T, R, rank, span, sp.data(), ns - 1, &ns2) == ZERO_ERANGE,
             "partition capacity", trial);
  }
  // argument errors
  uint64_t one = 1, o = 0, tot = 0, bb = 0, ee = 0, cnt = 0;
  expect(zero_shard_layout(&one, 1, 0, 1, &o, &tot, &bb, &ee) == ZERO_EINVAL, "R = 0", -1);
  expect(zero_shard_layout(nullptr, 1, 1, 1, &o, &tot, &bb, &ee) == ZERO_EINVAL, "NULL numel", -1);
  expect(zero_chunk_table(&one, &o, 1, 0, 1, 7, nullptr, 0, &cnt) == ZERO_EINVAL, "chunk not x8", -1);
  uint64_t huge[2] = {~0ull - 5, 10};
  uint64_t off2[2], b2[2], e2[2];
  expect(zero_shard_layout(huge, 2, 2, 64, off2, &tot, b2, e2) == ZERO_ERANGE, "64-bit overflow", -1);
  if (fails) return 1;
  std::puts("host driver: clean");
  return 0;
}
