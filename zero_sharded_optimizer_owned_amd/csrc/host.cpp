// Host half of libzero_shard: layout, chunk table, state accounting, clip
// scalar and the thread-local error message.  No device code here.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace zs {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

}  // namespace zs

using zs::fail;
using u128 = unsigned __int128;

extern "C" const char* zero_last_error(void) { return zs::g_last_error.c_str(); }

// Owner ranges over the padded total P: [floor(P r / R), floor(P (r+1) / R)).
// ([Deep dive] "Reduce first, then update the owned slice", contiguous
// ownership; the products are taken in 128 bits.)
extern "C" int zero_shard_layout(const uint64_t* numel, uint32_t n_tensors, uint32_t ranks,
                                 uint32_t align_elems, uint64_t* tensor_offset,
                                 uint64_t* padded_total, uint64_t* owner_begin,
                                 uint64_t* owner_end) {
  zs::clear_error();
  if (!numel || !tensor_offset || !padded_total || !owner_begin || !owner_end)
    return fail(ZERO_EINVAL, "zero_shard_layout: NULL pointer argument");
  if (n_tensors == 0) return fail(ZERO_EINVAL, "zero_shard_layout: no tensors");
  if (ranks == 0) return fail(ZERO_EINVAL, "zero_shard_layout: ranks must be >= 1");
  if (align_elems == 0) return fail(ZERO_EINVAL, "zero_shard_layout: alignment must be >= 1");
  u128 total = 0;
  for (uint32_t k = 0; k < n_tensors; ++k) {
    if (numel[k] == 0) return fail(ZERO_EINVAL, "zero_shard_layout: tensor %u has 0 elements", k);
    const u128 padded = ((u128)numel[k] + align_elems - 1) / align_elems * align_elems;
    if (total + padded > (u128)UINT64_MAX)
      return fail(ZERO_ERANGE, "zero_shard_layout: padded total exceeds 64 bits");
    total += padded;
  }
  // All checks passed: write outputs.
  u128 off = 0;
  for (uint32_t k = 0; k < n_tensors; ++k) {
    tensor_offset[k] = (uint64_t)off;
    off += ((u128)numel[k] + align_elems - 1) / align_elems * align_elems;
  }
  *padded_total = (uint64_t)total;
  for (uint32_t r = 0; r < ranks; ++r) {
    owner_begin[r] = (uint64_t)(total * r / ranks);
    owner_end[r] = (uint64_t)(total * (r + 1) / ranks);
  }
  return ZERO_OK;
}

// Dense (unpadded) start of every tensor: the running sum of the sizes before
// it ([Deep dive] "Resume training and export weights separately": an export
// consolidates the weights without the layout's padding).
extern "C" int zero_dense_offsets(const uint64_t* numel, uint32_t n_tensors, uint64_t* dense_offset,
                                  uint64_t* dense_total) {
  zs::clear_error();
  if (n_tensors > 0 && (!numel || !dense_offset))
    return fail(ZERO_EINVAL, "zero_dense_offsets: NULL tensor arrays");
  if (!dense_total) return fail(ZERO_EINVAL, "zero_dense_offsets: dense_total is NULL");
  u128 total = 0;
  for (uint32_t k = 0; k < n_tensors; ++k) {
    if (numel[k] == 0) return fail(ZERO_EINVAL, "zero_dense_offsets: tensor %u has 0 elements", k);
    total += numel[k];
    if (total > (u128)UINT64_MAX)
      return fail(ZERO_ERANGE, "zero_dense_offsets: dense total exceeds 64 bits");
  }
  uint64_t pos = 0;
  for (uint32_t k = 0; k < n_tensors; ++k) {
    dense_offset[k] = pos;
    pos += numel[k];
  }
  *dense_total = pos;
  return ZERO_OK;
}

extern "C" int zero_chunk_table(const uint64_t* numel, const uint64_t* tensor_offset,
                                uint32_t n_tensors, uint64_t begin, uint64_t end,
                                uint32_t max_chunk_elems, zero_chunk* out, uint64_t capacity,
                                uint64_t* n_chunks) {
  zs::clear_error();
  if (!n_chunks) return fail(ZERO_EINVAL, "zero_chunk_table: n_chunks is NULL");
  if (n_tensors > 0 && (!numel || !tensor_offset))
    return fail(ZERO_EINVAL, "zero_chunk_table: NULL tensor arrays");
  if (begin > end) return fail(ZERO_EINVAL, "zero_chunk_table: begin > end");
  if (max_chunk_elems < 8 || max_chunk_elems % 8 != 0)
    return fail(ZERO_EINVAL, "zero_chunk_table: max_chunk_elems must be a positive multiple of 8");
  if (capacity > 0 && !out) return fail(ZERO_EINVAL, "zero_chunk_table: out is NULL");
  for (uint32_t k = 0; k < n_tensors; ++k) {
    if (numel[k] == 0) return fail(ZERO_EINVAL, "zero_chunk_table: tensor %u has 0 elements", k);
    if ((u128)tensor_offset[k] + numel[k] > (u128)UINT64_MAX)
      return fail(ZERO_EINVAL, "zero_chunk_table: tensor %u extends past 2^64", k);
    if (k > 0 && tensor_offset[k] < tensor_offset[k - 1] + numel[k - 1])
      return fail(ZERO_EINVAL, "zero_chunk_table: tensor %u overlaps or precedes tensor %u", k,
                  k - 1);
  }
  const uint64_t C = max_chunk_elems;
  uint64_t count = 0;
  for (uint32_t k = 0; k < n_tensors;) {
    // a run of tensors k .. j-1 with no padding between them
    uint32_t j = k + 1;
    while (j < n_tensors && tensor_offset[j] == tensor_offset[j - 1] + numel[j - 1]) ++j;
    const uint64_t r0 = tensor_offset[k], r1 = tensor_offset[j - 1] + numel[j - 1];
    uint64_t b = r0 > begin ? r0 : begin;
    const uint64_t e = r1 < end ? r1 : end;
    uint32_t t = k;  // the tensor that holds flat index b
    while (b < e) {
      while (tensor_offset[t] + numel[t] <= b) ++t;
      const uint64_t cut = (b / C + 1) * C;  // next multiple of C after b
      const uint64_t stop = cut < e ? cut : e;
      if (out && count < capacity) {
        out[count].flat = b;
        out[count].len = (uint32_t)(stop - b);
        out[count].tensor = t;
      }
      ++count;
      b = stop;
    }
    k = j;
  }
  *n_chunks = count;
  if (out == nullptr && capacity == 0) return ZERO_OK;
  if (count > capacity)
    return fail(ZERO_ERANGE, "zero_chunk_table: %llu chunks needed, capacity %llu",
                (unsigned long long)count, (unsigned long long)capacity);
  return ZERO_OK;
}

namespace {
// Greedy grouping shared by the chunk and span group builders: consecutive
// items go into one group while their work units total at most max_units and
// their elements at most max_elems; an item of more than max_units units is a
// group of its own.  `units(i)` and `elems(i)` describe item i.  Writes group
// starts and the sentinel n, returns the group count.
template <typename U, typename E>
uint64_t greedy_groups(uint64_t n, uint64_t max_units, uint64_t max_elems, U units, E elems,
                       uint64_t* out, uint64_t capacity) {
  const uint64_t kUnits = max_units;
  uint64_t g = 0;
  for (uint64_t i = 0; i < n;) {
    if (out && g < capacity) out[g] = i;
    ++g;
    uint64_t u = units(i), e = elems(i), j = i + 1;
    if (u <= kUnits) {
      while (j < n) {
        const uint64_t uj = units(j);
        if (u + uj > kUnits || e + elems(j) > max_elems) break;
        u += uj;
        e += elems(j);
        ++j;
      }
    }
    i = j;
  }
  if (out && g < capacity) out[g] = n;  // sentinel
  return g;
}
}  // namespace

extern "C" int zero_chunk_groups(const zero_chunk* chunks, uint64_t n_chunks, uint32_t max_group_elems,
                                 uint64_t* out, uint64_t capacity, uint64_t* n_groups) {
  zs::clear_error();
  if (!n_groups) return fail(ZERO_EINVAL, "zero_chunk_groups: n_groups is NULL");
  if (n_chunks > 0 && !chunks) return fail(ZERO_EINVAL, "zero_chunk_groups: chunks is NULL");
  if (max_group_elems == 0) return fail(ZERO_EINVAL, "zero_chunk_groups: max_group_elems must be > 0");
  if (capacity > 0 && !out) return fail(ZERO_EINVAL, "zero_chunk_groups: out is NULL");
  // work units of a chunk: scalar head, 128-bit vectors, scalar tail
  auto units = [](const zero_chunk& c) -> uint64_t {
    const uint64_t f0 = c.flat, f1 = c.flat + c.len;
    uint64_t a0 = (f0 + 7) & ~7ull;
    if (a0 > f1) a0 = f1;
    uint64_t a1 = f1 & ~7ull;
    if (a1 < a0) a1 = a0;
    return (a0 - f0) + (a1 - a0) / 8 + (f1 - a1);
  };
  auto cunits = [&](uint64_t i) { return units(chunks[i]); };
  auto celems = [&](uint64_t i) -> uint64_t { return chunks[i].len; };
  // one unit per thread of a 256-thread block: a unit of the step is heavy
  // (every rank's data, then master and moments), and more units per thread
  // measured slower (2.7 against 3.0 TB/s for 100-element tensors)
  const uint64_t g = greedy_groups(n_chunks, 256, max_group_elems, cunits, celems, out, capacity);
  *n_groups = g;
  if (out == nullptr && capacity == 0) return ZERO_OK;
  if (g + 1 > capacity)
    return fail(ZERO_ERANGE, "zero_chunk_groups: %llu entries needed, capacity %llu",
                (unsigned long long)(g + 1), (unsigned long long)capacity);
  return ZERO_OK;
}


extern "C" int zero_span_groups(const zero_copy_span* spans, uint64_t n_spans, uint32_t elem_bytes,
                                uint32_t max_group_elems, uint64_t* out, uint64_t capacity,
                                uint64_t* n_groups) {
  zs::clear_error();
  if (!n_groups) return fail(ZERO_EINVAL, "zero_span_groups: n_groups is NULL");
  if (n_spans > 0 && !spans) return fail(ZERO_EINVAL, "zero_span_groups: spans is NULL");
  if (elem_bytes != 2 && elem_bytes != 4)
    return fail(ZERO_EINVAL, "zero_span_groups: elem_bytes must be 2 or 4");
  if (max_group_elems == 0) return fail(ZERO_EINVAL, "zero_span_groups: max_group_elems must be > 0");
  if (capacity > 0 && !out) return fail(ZERO_EINVAL, "zero_span_groups: out is NULL");
  const uint64_t V = 16 / elem_bytes;
  // units: scalar head, vectors, scalar tail when source and destination share
  // their 16-byte phase, else one unit per element
  auto units = [&](uint64_t i) -> uint64_t {
    const zero_copy_span& sp = spans[i];
    const uint64_t len = sp.len;
    if ((sp.src - sp.dst) % V != 0) return len;
    uint64_t head = (V - sp.dst % V) % V;
    if (head > len) head = len;
    const uint64_t nvec = (len - head) / V;
    return len - nvec * (V - 1);
  };
  auto elems = [&](uint64_t i) -> uint64_t { return spans[i].len; };
  // up to eight units per thread: a unit of a copy is light, and spans whose
  // phases differ are one unit per element (69-element spans: 1.40 TB/s with
  // 2048 units per group, 0.53 with 256)
  const uint64_t g = greedy_groups(n_spans, 2048, max_group_elems, units, elems, out, capacity);
  *n_groups = g;
  if (out == nullptr && capacity == 0) return ZERO_OK;
  if (g + 1 > capacity)
    return fail(ZERO_ERANGE, "zero_span_groups: %llu entries needed, capacity %llu",
                (unsigned long long)(g + 1), (unsigned long long)capacity);
  return ZERO_OK;
}

namespace {
// whole + shared / R as a reduced fraction; whole and shared are exact
// products of 64-bit by 32-bit values (at most 2^98), R < 2^64.
int make_ratio(u128 whole, u128 shared, uint64_t R, zero_ratio* out) {
  // Reduce shared / R first so that whole * den stays within 128 bits.
  u128 a = shared, b = R;
  while (b) {
    const u128 t = a % b;
    a = b;
    b = t;
  }
  const u128 g = shared == 0 ? (u128)R : a;
  const u128 sn = shared / g, den = (u128)R / g;
  if (whole > (u128)UINT64_MAX || den > (u128)UINT64_MAX) return ZERO_ERANGE;
  const u128 num = whole * den + sn;  // < 2^64 * 2^64: fits
  if (num > (u128)UINT64_MAX) return ZERO_ERANGE;
  out->num = (uint64_t)num;
  out->den = (uint64_t)den;
  return ZERO_OK;
}
}  // namespace

// [Deep dive] "Count state before choosing a stage"; [ZeRO Q&A] "Memory
// Footprint Reduction Matrix".
extern "C" int zero_state_bytes(uint64_t params, uint64_t ranks, uint32_t param_bytes,
                                uint32_t grad_bytes, uint32_t optim_bytes, zero_ratio out[4]) {
  zs::clear_error();
  if (!out) return fail(ZERO_EINVAL, "zero_state_bytes: out is NULL");
  if (params == 0 || ranks == 0 || param_bytes == 0 || grad_bytes == 0 || optim_bytes == 0)
    return fail(ZERO_EINVAL, "zero_state_bytes: counts and byte widths must be positive");
  const u128 P = params, p = param_bytes, g = grad_bytes, o = optim_bytes;
  zero_ratio tmp[4];
  const u128 parts[4][2] = {
      {P * (p + g + o), 0},  // DP
      {P * (p + g), P * o},  // ZeRO-1
      {P * p, P * (g + o)},  // ZeRO-2
      {0, P * (p + g + o)},  // ZeRO-3
  };
  for (int s = 0; s < 4; ++s) {
    if (make_ratio(parts[s][0], parts[s][1], ranks, &tmp[s]) != ZERO_OK)
      return fail(ZERO_ERANGE, "zero_state_bytes: result exceeds 64 bits");
  }
  std::memcpy(out, tmp, sizeof tmp);
  return ZERO_OK;
}

extern "C" int zero_clip_coef(double sumsq, double max_norm, double eps, float* coef) {
  zs::clear_error();
  if (!coef) return fail(ZERO_EINVAL, "zero_clip_coef: coef is NULL");
  if (!std::isfinite(sumsq) || sumsq < 0.0)
    return fail(ZERO_EINVAL, "zero_clip_coef: sumsq must be finite and >= 0");
  if (!std::isfinite(max_norm) || max_norm <= 0.0)
    return fail(ZERO_EINVAL, "zero_clip_coef: max_norm must be finite and > 0");
  if (!std::isfinite(eps) || eps < 0.0)
    return fail(ZERO_EINVAL, "zero_clip_coef: eps must be finite and >= 0");
  const double c = max_norm / (std::sqrt(sumsq) + eps);
  *coef = (float)(c < 1.0 ? c : 1.0);
  return ZERO_OK;
}

// The step decision from every owner's check: skip when any owner saw a
// non-finite gradient value, else clip with the norm of the whole gradient,
// whose square is the sum of the owners' partials taken in owner order.
extern "C" int zero_step_decision(const int32_t* overflow, const double* sumsq, uint32_t n_owners,
                                  double max_norm, double eps, int32_t* update, float* coef) {
  zs::clear_error();
  if (!overflow || !sumsq || !update || !coef) return fail(ZERO_EINVAL, "zero_step_decision: NULL pointer");
  if (n_owners == 0) return fail(ZERO_EINVAL, "zero_step_decision: no owners");
  int32_t any = 0;
  for (uint32_t r = 0; r < n_owners; ++r) any |= overflow[r] != 0;
  if (any) {
    *update = 0;
    *coef = 0.0f;
    return ZERO_OK;
  }
  double total = 0.0;
  for (uint32_t r = 0; r < n_owners; ++r) {
    if (!std::isfinite(sumsq[r]) || sumsq[r] < 0.0)
      return fail(ZERO_EINVAL, "zero_step_decision: owner %u's squared norm is negative or not finite", r);
    total += sumsq[r];
  }
  const int rc = zero_clip_coef(total, max_norm, eps, coef);
  if (rc) return rc;
  *update = 1;
  return ZERO_OK;
}

// ---------------------------------------------------------------------------
// ZeRO-3 per-tensor partitioning ([Deep dive] "Stage 3 needs a live working
// set"): tensor k is cut into R shards of s_k = ceil(n_k / R) elements; rank
// r's shard buffer holds its shard of every tensor in tensor order (tensor k
// at so_k = sum of s_j, j < k); a live tensor is gathered into a separate
// full buffer of R * s_k elements, shards in rank order.
// ---------------------------------------------------------------------------
namespace {
int check_stage3(const uint64_t* numel, uint32_t n_tensors, uint32_t ranks, const uint32_t* live,
                 uint32_t n_live, const char* who) {
  if (ranks == 0) return fail(ZERO_EINVAL, "%s: ranks must be >= 1", who);
  if (n_tensors == 0 || !numel) return fail(ZERO_EINVAL, "%s: no tensors", who);
  for (uint32_t k = 0; k < n_tensors; ++k)
    if (numel[k] == 0) return fail(ZERO_EINVAL, "%s: tensor %u has 0 elements", who, k);
  if (n_live > 0 && !live) return fail(ZERO_EINVAL, "%s: live is NULL", who);
  for (uint32_t i = 0; i < n_live; ++i) {
    if (live[i] >= n_tensors) return fail(ZERO_EINVAL, "%s: live tensor %u out of range", who, live[i]);
    for (uint32_t j = 0; j < i; ++j)
      if (live[j] == live[i]) return fail(ZERO_EINVAL, "%s: live tensor %u listed twice", who, live[i]);
  }
  return ZERO_OK;
}

uint64_t shard_of(uint64_t n, uint32_t ranks) { return n / ranks + (n % ranks != 0); }

// Totals of a stage-3 layout in 128 bits: elements of all tensors, of one
// rank's shard buffer, and of the live tensors' gathered buffers.  ERANGE when
// any of them (and so any offset inside them) exceeds 64 bits.
int stage3_totals(const uint64_t* numel, uint32_t n_tensors, uint32_t ranks, const uint32_t* live,
                  uint32_t n_live, const char* who, u128* dense, u128* resident, u128* gathered) {
  u128 d = 0, res = 0, gat = 0;
  for (uint32_t k = 0; k < n_tensors; ++k) {
    d += numel[k];
    res += shard_of(numel[k], ranks);
  }
  for (uint32_t i = 0; i < n_live; ++i) gat += (u128)shard_of(numel[live[i]], ranks) * ranks;
  if (d > (u128)UINT64_MAX || res > (u128)UINT64_MAX || gat > (u128)UINT64_MAX)
    return fail(ZERO_ERANGE, "%s: counts exceed 64 bits", who);
  if (dense) *dense = d;
  if (resident) *resident = res;
  if (gathered) *gathered = gat;
  return ZERO_OK;
}

// Append [src, src+len) -> [dst, dst+len) of buffer `buf`, cut into pieces of at most C.
void add_spans(uint64_t src, uint64_t dst, uint64_t len, uint32_t buf, uint64_t C, zero_copy_span* out,
               uint64_t capacity, uint64_t* count) {
  while (len > 0) {
    const uint64_t piece = len < C ? len : C;
    if (out && *count < capacity) {
      out[*count].src = src;
      out[*count].dst = dst;
      out[*count].len = (uint32_t)piece;
      out[*count].buf = buf;
    }
    ++*count;
    src += piece;
    dst += piece;
    len -= piece;
  }
}

int finish_spans(zero_copy_span* out, uint64_t capacity, uint64_t count, uint64_t* n_spans,
                 const char* who) {
  *n_spans = count;
  if (out == nullptr && capacity == 0) return ZERO_OK;
  if (count > capacity)
    return fail(ZERO_ERANGE, "%s: %llu spans needed, capacity %llu", who, (unsigned long long)count,
                (unsigned long long)capacity);
  return ZERO_OK;
}
}  // namespace

extern "C" int zero3_storage(const uint64_t* numel, uint32_t n_tensors, uint32_t ranks,
                             const uint32_t* live, uint32_t n_live, uint64_t* shard_numel,
                             uint64_t* resident, uint64_t* gathered) {
  zs::clear_error();
  static const char* who = "zero3_storage";
  int rc = check_stage3(numel, n_tensors, ranks, live, n_live, who);
  if (rc) return rc;
  if (!resident || !gathered) return fail(ZERO_EINVAL, "%s: NULL output", who);
  u128 res = 0, gat = 0;
  if ((rc = stage3_totals(numel, n_tensors, ranks, live, n_live, who, nullptr, &res, &gat))) return rc;
  if (shard_numel)
    for (uint32_t k = 0; k < n_tensors; ++k) shard_numel[k] = shard_of(numel[k], ranks);
  *resident = (uint64_t)res;
  *gathered = (uint64_t)gat;
  return ZERO_OK;
}

extern "C" int zero3_gather_spans(const uint64_t* numel, uint32_t n_tensors, uint32_t ranks,
                                  const uint32_t* live, uint32_t n_live, uint32_t max_span,
                                  zero_copy_span* out, uint64_t capacity, uint64_t* n_spans) {
  zs::clear_error();
  static const char* who = "zero3_gather_spans";
  int rc = check_stage3(numel, n_tensors, ranks, live, n_live, who);
  if (rc) return rc;
  if (!n_spans) return fail(ZERO_EINVAL, "%s: n_spans is NULL", who);
  if (max_span == 0) return fail(ZERO_EINVAL, "%s: max_span must be >= 1", who);
  if (capacity > 0 && !out) return fail(ZERO_EINVAL, "%s: out is NULL", who);
  // every offset below is bounded by the shard-buffer or gathered total
  if ((rc = stage3_totals(numel, n_tensors, ranks, live, n_live, who, nullptr, nullptr, nullptr)))
    return rc;
  std::vector<uint64_t> so(n_tensors);  // shard offset of each tensor
  for (uint64_t k = 0, acc = 0; k < n_tensors; ++k) {
    so[k] = acc;
    acc += shard_of(numel[k], ranks);
  }
  uint64_t count = 0, gbase = 0;
  for (uint32_t i = 0; i < n_live; ++i) {
    const uint32_t k = live[i];
    const uint64_t s = shard_of(numel[k], ranks);
    for (uint32_t r = 0; r < ranks; ++r)
      add_spans(so[k], gbase + (uint64_t)r * s, s, r, max_span, out, capacity, &count);
    gbase += (uint64_t)ranks * s;
  }
  return finish_spans(out, capacity, count, n_spans, who);
}

extern "C" int zero3_partition_spans(const uint64_t* numel, uint32_t n_tensors, uint32_t ranks,
                                     uint32_t rank, uint32_t max_span, zero_copy_span* out,
                                     uint64_t capacity, uint64_t* n_spans) {
  zs::clear_error();
  static const char* who = "zero3_partition_spans";
  int rc = check_stage3(numel, n_tensors, ranks, nullptr, 0, who);
  if (rc) return rc;
  if (!n_spans) return fail(ZERO_EINVAL, "%s: n_spans is NULL", who);
  if (rank >= ranks) return fail(ZERO_EINVAL, "%s: rank %u >= ranks %u", who, rank, ranks);
  if (max_span == 0) return fail(ZERO_EINVAL, "%s: max_span must be >= 1", who);
  if (capacity > 0 && !out) return fail(ZERO_EINVAL, "%s: out is NULL", who);
  if ((rc = stage3_totals(numel, n_tensors, ranks, nullptr, 0, who, nullptr, nullptr, nullptr))) return rc;
  uint64_t count = 0, so = 0, dense = 0;
  for (uint32_t k = 0; k < n_tensors; ++k) {
    const uint64_t s = shard_of(numel[k], ranks);
    const uint64_t first = (uint64_t)rank * s;
    if (first < numel[k]) {
      const uint64_t len = numel[k] - first < s ? numel[k] - first : s;
      add_spans(dense + first, so, len, 0, max_span, out, capacity, &count);
    }
    so += s;
    dense += numel[k];
  }
  return finish_spans(out, capacity, count, n_spans, who);
}
