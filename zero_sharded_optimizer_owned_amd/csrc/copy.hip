// Copy kernels of libzero_shard and their C entry points:
//   * export and import of fp32 shard data between an owner's shard and the
//     dense per-tensor layout (over the owner's chunk table);
//   * span-table copies: the stage-3 gather of a live working set from the
//     ranks' shard buffers, and the partition of dense tensors into a shard.
#include <hip/hip_runtime.h>

#include <cstring>

#include "internal.h"
#include "launch.h"
#include "scan.h"

namespace zs {
namespace {

// ---------------------------------------------------------------------------
// Export / import between an owner's shard and the dense per-tensor layout.
// ---------------------------------------------------------------------------
struct DenseArgs {
  const zero_chunk* chunks;
  uint64_t n_chunks;
  const uint64_t* groups;  // [n_groups + 1] first chunk of each block's work, or NULL
  uint64_t n_groups;
  uint64_t begin, end;
  const uint64_t* tensor_offset;  // [n_tensors] flat start of each tensor
  const uint64_t* dense_offset;   // [n_tensors] dense start of each tensor
  uint32_t n_tensors;
  float* owner;                   // element f - owner_base
  uint64_t owner_base;
  float* dense;                   // [dense_total]
  uint64_t dense_total;
};

// One block per chunk (grid stride past the grid): consecutive threads copy
// consecutive elements on both sides, four per thread in flight.  Chunks
// whose tensor index or position disagrees with the tables are skipped, and
// no dense index at or past dense_total is touched.
template <bool TO_DENSE>
__device__ __forceinline__ void dense_one(const DenseArgs& a, const zero_chunk ch, uint64_t t) {
  if (ch.tensor >= a.n_tensors) return;
  const uint64_t toff = a.tensor_offset[ch.tensor];
  const uint64_t doff = a.dense_offset[ch.tensor];
  const uint64_t f0 = max(max(ch.flat, a.begin), toff);
  const uint64_t f1 = min(ch.flat + ch.len, a.end);
  for (uint64_t f = f0 + t; f < f1; f += 4 * kBlock) {
    float x[4];
    uint64_t d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t fj = f + kBlock * j;
      d[j] = fj < f1 ? doff + (fj - toff) : a.dense_total;
      if (d[j] < a.dense_total) x[j] = TO_DENSE ? a.owner[fj - a.owner_base] : a.dense[d[j]];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (d[j] < a.dense_total) {
        if (TO_DENSE) a.dense[d[j]] = x[j];
        else a.owner[f + kBlock * j - a.owner_base] = x[j];
      }
    }
  }
}

template <bool TO_DENSE>
__global__ void __launch_bounds__(kBlock) dense_kernel(const DenseArgs a) {
  for (uint64_t c = blockIdx.x; c < a.n_chunks; c += gridDim.x) dense_one<TO_DENSE>(a, a.chunks[c], threadIdx.x);
}

// Several short chunks by one block: the block's threads take the elements of
// all its chunks together (thread t on elements t, t + kBlock, ...), finding
// an element's chunk by binary search over the prefix sums of the chunk
// lengths (chunks taken kBlock at a time).
template <bool TO_DENSE>
__device__ void dense_packed(const DenseArgs& a, uint64_t c0, uint64_t c1, uint32_t t) {
  __shared__ uint64_t s_f0[kBlock], s_shift[kBlock];
  __shared__ uint64_t s_pre[kBlock + 1];
  __shared__ uint64_t s_wave[kWavesPerBlock];
  for (uint64_t s0 = c0; s0 < c1; s0 += kBlock) {
    const uint32_t m = (uint32_t)min((uint64_t)kBlock, c1 - s0);
    uint64_t len = 0;
    if (t < m) {
      const zero_chunk ch = a.chunks[s0 + t];
      if (ch.tensor < a.n_tensors) {
        const uint64_t toff = a.tensor_offset[ch.tensor];
        const uint64_t f0 = max(max(ch.flat, a.begin), toff);
        const uint64_t f1 = max(f0, min(ch.flat + ch.len, a.end));
        s_f0[t] = f0;
        s_shift[t] = a.dense_offset[ch.tensor] - toff;  // dense index of f = f + shift (wrapping)
        len = f1 - f0;
      }
    }
    s_pre[t + 1] = block_inclusive_scan(len, s_wave);
    if (t == 0) s_pre[0] = 0;
    __syncthreads();
    const uint64_t total = s_pre[m];
    for (uint64_t e = t; e < total; e += kBlock) {
      uint32_t lo = 0, hi = m;
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (s_pre[mid] <= e) lo = mid;
        else hi = mid;
      }
      const uint64_t f = s_f0[lo] + (e - s_pre[lo]);
      const uint64_t d = f + s_shift[lo];
      if (d < a.dense_total) {
        if (TO_DENSE) a.dense[d] = a.owner[f - a.owner_base];
        else a.owner[f - a.owner_base] = a.dense[d];
      }
    }
    __syncthreads();
  }
}

template <bool TO_DENSE>
__global__ void __launch_bounds__(kBlock) dense_group_kernel(const DenseArgs a) {
  const uint32_t t = threadIdx.x;
  for (uint64_t w = blockIdx.x; w < a.n_groups; w += gridDim.x) {
    const uint64_t c0 = a.groups[w];
    const uint64_t c1 = min(a.groups[w + 1], a.n_chunks);
    if (c1 <= c0) continue;
    if (c1 - c0 == 1) dense_one<TO_DENSE>(a, a.chunks[c0], t);
    else dense_packed<TO_DENSE>(a, c0, c1, t);
  }
}

// ---------------------------------------------------------------------------
// Span-table copies.
// ---------------------------------------------------------------------------
struct SpanArgs {
  const zero_copy_span* spans;
  uint64_t n_spans;
  const uint64_t* groups;  // [n_groups + 1] first span of each block's work, or NULL
  uint64_t n_groups;
  const void* src[ZERO_MAX_COPY_SOURCES];
  uint64_t src_numel[ZERO_MAX_COPY_SOURCES];
  uint32_t n_srcs;
  void* dst;
  uint64_t dst_numel;
};

// Whether a span lies inside its source and the destination.
__device__ __forceinline__ bool span_fits(const SpanArgs& a, const zero_copy_span& sp) {
  if (sp.buf >= a.n_srcs) return false;
  const uint64_t len = sp.len, sn = a.src_numel[sp.buf];
  return !(sp.src > sn || len > sn - sp.src || sp.dst > a.dst_numel || len > a.dst_numel - sp.dst);
}

// d[i + j * kBlock] = s[i + j * kBlock] for j = 0..3 below n, one element at a
// time: each load completes before its store, so a thread has one load in
// flight.  (Four loads issued before the stores ran 4% slower on the stage-3
// gather; the same loop over an array of four had kept the array in scratch
// memory once inlined into the group kernel.)
template <typename E>
__device__ __forceinline__ void copy4(const E* s, E* d, uint64_t i, uint64_t n) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (i + kBlock * j < n) d[i + kBlock * j] = s[i + kBlock * j];
}

// One span by one block.  When source and destination share their phase
// within a 16-byte vector, the body moves as 128-bit vectors (consecutive
// threads on consecutive vectors, up to four per thread and pass of copy4)
// between scalar head and tail pieces; otherwise threads copy single
// elements.  Spans that do not fit their buffers are skipped.
template <typename T>
__device__ __forceinline__ void span_one(const SpanArgs& a, const zero_copy_span sp, uint64_t t) {
  constexpr uint64_t V = 16 / sizeof(T);
  if (!span_fits(a, sp)) return;
  const uint64_t len = sp.len;
  const T* s = static_cast<const T*>(a.src[sp.buf]) + sp.src;
  T* d = static_cast<T*>(a.dst) + sp.dst;
  if ((sp.src - sp.dst) % V == 0) {
    const uint64_t head = min(len, (V - sp.dst % V) % V);
    const uint64_t body = (len - head) / V;
    const uint64_t tail0 = head + body * V;
    if (t < head) d[t] = s[t];
    if (t < len - tail0) d[tail0 + t] = s[tail0 + t];
    const uint4* sv = reinterpret_cast<const uint4*>(s + head);
    uint4* dv = reinterpret_cast<uint4*>(d + head);
    for (uint64_t v = t; v < body; v += 4 * kBlock) copy4<uint4>(sv, dv, v, body);
  } else {
    for (uint64_t i = t; i < len; i += 4 * kBlock) copy4<T>(s, d, i, len);
  }
}

// One block per span (grid stride past the grid).
template <typename T>
__global__ void __launch_bounds__(kBlock) span_kernel(const SpanArgs a) {
  for (uint64_t c = blockIdx.x; c < a.n_spans; c += gridDim.x) span_one<T>(a, a.spans[c], threadIdx.x);
}

// Several short spans by one block.  Each span is cut into work units --
// scalar head elements, 128-bit vectors, scalar tail elements; a span whose
// source and destination phases differ is all scalar units -- and the
// block's threads take the units of all its spans together, finding a unit's
// span by binary search over the prefix sums of the unit counts (spans taken
// kBlock at a time).
template <typename T>
__device__ void span_packed(const SpanArgs& a, uint64_t c0, uint64_t c1, uint32_t t) {
  constexpr uint64_t V = 16 / sizeof(T);
  __shared__ const T* s_src[kBlock];
  __shared__ T* s_dst[kBlock];
  __shared__ uint64_t s_head[kBlock], s_nvec[kBlock];
  __shared__ uint64_t s_pre[kBlock + 1];
  __shared__ uint64_t s_wave[kWavesPerBlock];
  for (uint64_t s0 = c0; s0 < c1; s0 += kBlock) {
    const uint32_t m = (uint32_t)min((uint64_t)kBlock, c1 - s0);
    uint64_t units = 0;
    if (t < m) {
      const zero_copy_span sp = a.spans[s0 + t];
      if (span_fits(a, sp)) {
        const uint64_t len = sp.len;
        s_src[t] = static_cast<const T*>(a.src[sp.buf]) + sp.src;
        s_dst[t] = static_cast<T*>(a.dst) + sp.dst;
        uint64_t head = len, nvec = 0;
        if ((sp.src - sp.dst) % V == 0) {
          head = min(len, (V - sp.dst % V) % V);
          nvec = (len - head) / V;
        }
        s_head[t] = head;
        s_nvec[t] = nvec;
        units = len - nvec * (V - 1);
      }
    }
    s_pre[t + 1] = block_inclusive_scan(units, s_wave);
    if (t == 0) s_pre[0] = 0;
    __syncthreads();
    const uint64_t total = s_pre[m];
    for (uint64_t u = t; u < total; u += kBlock) {
      uint32_t lo = 0, hi = m;
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (s_pre[mid] <= u) lo = mid;
        else hi = mid;
      }
      const uint64_t r = u - s_pre[lo];
      const uint64_t head = s_head[lo], nvec = s_nvec[lo];
      const T* src = s_src[lo];
      T* dst = s_dst[lo];
      if (r < head) {
        dst[r] = src[r];
      } else if (r < head + nvec) {
        const uint64_t e = head + V * (r - head);
        *reinterpret_cast<uint4*>(dst + e) = *reinterpret_cast<const uint4*>(src + e);
      } else {
        const uint64_t e = head + V * nvec + (r - head - nvec);
        dst[e] = src[e];
      }
    }
    __syncthreads();
  }
}

// One block per group of the span group table: one long span, or several
// short ones packed together.
template <typename T>
__global__ void __launch_bounds__(kBlock) span_group_kernel(const SpanArgs a) {
  const uint32_t t = threadIdx.x;
  for (uint64_t w = blockIdx.x; w < a.n_groups; w += gridDim.x) {
    const uint64_t c0 = a.groups[w];
    const uint64_t c1 = min(a.groups[w + 1], a.n_spans);
    if (c1 <= c0) continue;
    if (c1 - c0 == 1) span_one<T>(a, a.spans[c0], t);
    else span_packed<T>(a, c0, c1, t);
  }
}

}  // namespace
}  // namespace zs

using namespace zs;

namespace {
int dense_copy(bool to_dense, const zero_chunk* chunks, uint64_t n_chunks, const uint64_t* groups,
               uint64_t n_groups, uint64_t begin, uint64_t end, const uint64_t* tensor_offset,
               const uint64_t* dense_offset, uint32_t n_tensors, float* owner, uint64_t owner_base,
               float* dense, uint64_t dense_total, hipStream_t stream, const char* who) {
  clear_error();
  if (begin > end) return fail(ZERO_EINVAL, "%s: begin > end", who);
  if (!groups && n_groups != 0) return fail(ZERO_EINVAL, "%s: n_groups given without a group table", who);
  if (n_chunks > 0 && (!chunks || !tensor_offset || !dense_offset || !owner || !dense))
    return fail(ZERO_EINVAL, "%s: NULL pointer argument", who);
  if (n_tensors == 0 && n_chunks > 0) return fail(ZERO_EINVAL, "%s: no tensors", who);
  if (owner_base > begin) return fail(ZERO_EINVAL, "%s: owner_base lies above begin", who);
  if ((reinterpret_cast<uintptr_t>(owner) | reinterpret_cast<uintptr_t>(dense)) & 3u)
    return fail(ZERO_EINVAL, "%s: fp32 buffers must be 4-byte aligned", who);
  if (n_chunks == 0 || begin == end || (groups && n_groups == 0)) return ZERO_OK;
  int rc = begin_launch();
  if (rc) return rc;
  DenseArgs a;
  a.chunks = chunks;
  a.n_chunks = n_chunks;
  a.groups = groups;
  a.n_groups = groups ? n_groups : 0;
  a.begin = begin;
  a.end = end;
  a.tensor_offset = tensor_offset;
  a.dense_offset = dense_offset;
  a.n_tensors = n_tensors;
  a.owner = owner;
  a.owner_base = owner_base;
  a.dense = dense;
  a.dense_total = dense_total;
  if (groups) {
    if (to_dense) hipLaunchKernelGGL(dense_group_kernel<true>, chunk_grid(n_groups, 0), kBlock, 0, stream, a);
    else hipLaunchKernelGGL(dense_group_kernel<false>, chunk_grid(n_groups, 0), kBlock, 0, stream, a);
  } else if (to_dense) {
    hipLaunchKernelGGL(dense_kernel<true>, chunk_grid(n_chunks, 0), kBlock, 0, stream, a);
  } else {
    hipLaunchKernelGGL(dense_kernel<false>, chunk_grid(n_chunks, 0), kBlock, 0, stream, a);
  }
  return launch_status(who);
}
}  // namespace

extern "C" int zero_owner_to_dense(const zero_chunk* chunks, uint64_t n_chunks, const uint64_t* groups,
                                   uint64_t n_groups, uint64_t begin, uint64_t end,
                                   const uint64_t* tensor_offset, const uint64_t* dense_offset,
                                   uint32_t n_tensors, const float* owner, uint64_t owner_base,
                                   float* dense, uint64_t dense_total, hipStream_t stream) {
  return dense_copy(true, chunks, n_chunks, groups, n_groups, begin, end, tensor_offset, dense_offset,
                    n_tensors, const_cast<float*>(owner), owner_base, dense, dense_total, stream,
                    "zero_owner_to_dense");
}

extern "C" int zero_dense_to_owner(const zero_chunk* chunks, uint64_t n_chunks, const uint64_t* groups,
                                   uint64_t n_groups, uint64_t begin, uint64_t end,
                                   const uint64_t* tensor_offset, const uint64_t* dense_offset,
                                   uint32_t n_tensors, const float* dense, uint64_t dense_total,
                                   float* owner, uint64_t owner_base, hipStream_t stream) {
  return dense_copy(false, chunks, n_chunks, groups, n_groups, begin, end, tensor_offset, dense_offset,
                    n_tensors, owner, owner_base, const_cast<float*>(dense), dense_total, stream,
                    "zero_dense_to_owner");
}

extern "C" int zero_copy_spans(const zero_copy_span* spans, uint64_t n_spans, const void* const* srcs,
                               const uint64_t* src_numel, uint32_t n_srcs, void* dst,
                               uint64_t dst_numel, uint32_t elem_bytes, const uint64_t* groups,
                               uint64_t n_groups, hipStream_t stream) {
  static const char* who = "zero_copy_spans";
  clear_error();
  if (elem_bytes != 2 && elem_bytes != 4) return fail(ZERO_EINVAL, "%s: elem_bytes must be 2 or 4", who);
  if (!groups && n_groups != 0) return fail(ZERO_EINVAL, "%s: n_groups given without a group table", who);
  if (n_spans == 0 || (groups && n_groups == 0)) return ZERO_OK;
  if (!spans || !dst) return fail(ZERO_EINVAL, "%s: NULL spans or dst", who);
  if (n_srcs == 0 || n_srcs > ZERO_MAX_COPY_SOURCES)
    return fail(ZERO_EINVAL, "%s: n_srcs = %u outside [1, %d]", who, n_srcs, ZERO_MAX_COPY_SOURCES);
  if (!srcs || !src_numel) return fail(ZERO_EINVAL, "%s: NULL source arrays", who);
  if (!aligned16(dst)) return fail(ZERO_EINVAL, "%s: dst is not 16-byte aligned", who);
  SpanArgs a;
  std::memset(&a, 0, sizeof a);
  for (uint32_t i = 0; i < n_srcs; ++i) {
    if (!srcs[i]) return fail(ZERO_EINVAL, "%s: source %u is NULL", who, i);
    if (!aligned16(srcs[i])) return fail(ZERO_EINVAL, "%s: source %u is not 16-byte aligned", who, i);
    a.src[i] = srcs[i];
    a.src_numel[i] = src_numel[i];
  }
  a.spans = spans;
  a.n_spans = n_spans;
  a.n_srcs = n_srcs;
  a.dst = dst;
  a.dst_numel = dst_numel;
  a.groups = groups;
  a.n_groups = groups ? n_groups : 0;
  int rc = begin_launch();
  if (rc) return rc;
  if (groups) {
    if (elem_bytes == 2)
      hipLaunchKernelGGL(span_group_kernel<uint16_t>, chunk_grid(n_groups, 0), kBlock, 0, stream, a);
    else
      hipLaunchKernelGGL(span_group_kernel<uint32_t>, chunk_grid(n_groups, 0), kBlock, 0, stream, a);
  } else if (elem_bytes == 2) {
    hipLaunchKernelGGL(span_kernel<uint16_t>, chunk_grid(n_spans, 0), kBlock, 0, stream, a);
  } else {
    hipLaunchKernelGGL(span_kernel<uint32_t>, chunk_grid(n_spans, 0), kBlock, 0, stream, a);
  }
  return launch_status(who);
}
