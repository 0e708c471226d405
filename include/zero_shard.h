/*
 * zero_shard.h -- C ABI of libzero_shard.so: the ZeRO owner-shard optimizer
 * step on one MI355X (gfx950).
 *
 * In ZeRO stages 1-3 each data-parallel rank owns one contiguous slice of the
 * flattened parameter buffer and keeps the fp32 master weights and Adam
 * moments for that slice only.  At an optimizer boundary the owner reduces
 * the ranks' gradients for its slice (equally weighted mean), applies
 * Adam/AdamW once to the reduced gradient and writes the 16-bit compute copy
 * of its updated weights.  This library performs that step inside one GPU's
 * memory: the R ranks' gradients for the owned slice are R device buffers.
 *
 * Sources, cited by page title and section:
 *   [ZeRO-3 docs]  DeepSpeed ZeRO API documentation (zero3.rst): the stage
 *                  list; the JSON examples (AdamW, fp16).
 *   [ZeRO Q&A]     "How does DeepSpeed ZeRO stage 1, 2, and 3 partition
 *                  optimizer states, gradients, and parameters?":
 *                  "Memory Footprint Reduction Matrix".
 *   [Deep dive]    "Deep dive: DeepSpeed" (leetllm): "Count state before
 *                  choosing a stage", "Reduce first, then update the owned
 *                  slice", "Let the engine own the microstep".
 *
 * Conventions for every call:
 *   - Return 0 (ZERO_OK) or a negative ZERO_E* code; zero_last_error() then
 *     gives a message (thread-local, valid until the next call on the thread).
 *     No exceptions escape, nothing exits the process.
 *   - The caller owns every buffer.  The library allocates no memory and
 *     keeps no state between calls apart from a read-only cache of each
 *     device's LDS sizes, and, for zero_reduce_owned_noalloc only, its
 *     static device scratch array and that array's address on each device
 *     (see there).  Arguments are validated before anything is
 *     launched; a call that fails validation launches nothing and writes
 *     nothing.  Buffer extents cannot be seen through plain pointers: the
 *     caller guarantees the sizes stated for each argument.
 *   - Device calls are asynchronous on `stream`; errors of the running
 *     kernels surface at the caller's next synchronisation of the stream.
 *   - Device pointers must be 16-byte aligned.  Flat index f of a buffer with
 *     base index B lives at element f - B; every base index is a multiple
 *     of 8 so that 128-bit vectors of all streams start at the same flat
 *     indices.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

enum zero_status {
  ZERO_OK = 0,
  ZERO_EINVAL = -1, /* bad argument: nothing launched, nothing written */
  ZERO_ERANGE = -2, /* output capacity too small, or an integer result above 2^64 - 1 */
  ZERO_EHIP = -3    /* HIP runtime or launch error */
};

enum zero_dtype {
  ZERO_NONE = 0, /* no 16-bit write-back (fp32 model) */
  ZERO_F16 = 1,  /* IEEE binary16 */
  ZERO_BF16 = 2, /* bfloat16 */
  ZERO_F32 = 3   /* IEEE binary32 */
};

/* Most rank buffers one reduce can read (pointers travel as kernel arguments). */
#define ZERO_MAX_RANKS 256

/* Message for the last failed call on this thread ("" if none). */
const char *zero_last_error(void);

/* ----------------------------------------------------------------------------
 * zero_shard_layout -- flattened, padded buffer and contiguous ownership.
 *
 * [Deep dive] "Reduce first, then update the owned slice": owner r of R holds
 * the contiguous range [floor(P*r/R), floor(P*(r+1)/R)); owners may be empty
 * when R exceeds P.  The pages do not give the padding; here every tensor,
 * the last included, is padded up to a multiple of `align_elems` elements
 * (tensor k starts at the sum of the padded sizes before it) and ownership is
 * taken over the padded total P.  Padding is owned, but the fused step and
 * the copies never read or write it (they walk the chunk table); the flat
 * reduce works on a flat range and treats padding like any other element,
 * so rank gradient buffers hold zeros there (no parameter, no gradient).
 *
 * numel[n_tensors]          in : element count of each tensor, all > 0
 * ranks, align_elems        in : R >= 1, alignment in elements >= 1
 * tensor_offset[n_tensors]  out: flat index of each tensor's first element
 * padded_total              out: P
 * owner_begin/end[ranks]    out: owner ranges (128-bit intermediate products)
 * Errors: EINVAL for zero counts or NULL pointers; ERANGE if P overflows 64 bits.
 * -------------------------------------------------------------------------- */
int zero_shard_layout(const uint64_t *numel, uint32_t n_tensors, uint32_t ranks,
                      uint32_t align_elems, uint64_t *tensor_offset, uint64_t *padded_total,
                      uint64_t *owner_begin, uint64_t *owner_end);

/* One piece of an owner's work: `len` real elements from flat index `flat`.
 * `tensor` holds the first of them; the piece may run on into the following
 * tensors when no padding separates them.  16 bytes; the device calls read an
 * array of these. */
typedef struct {
  uint64_t flat;
  uint32_t len;
  uint32_t tensor;
} zero_chunk;

/* ----------------------------------------------------------------------------
 * zero_chunk_table -- the owner's real elements as a list of chunks.
 *
 * The real elements of [begin, end) are the union over tensors of
 * [tensor_offset[k], tensor_offset[k] + numel[k]) intersected with it (the
 * padding after each tensor is skipped).  Maximal runs of real elements --
 * consecutive tensors with no padding between them count as one run, so many
 * small tensors still make full-size chunks -- are cut at the flat multiples
 * of `max_chunk_elems`, so interior cuts fall on 128-bit vector boundaries.
 * Chunks come out in increasing flat order and cover every real element of
 * the range exactly once.  Padding follows the reading stated at
 * zero_shard_layout (the pages leave it open): every tensor, the last one
 * included, is padded to the alignment, and the padding belongs to no chunk.
 *
 * numel, tensor_offset [n_tensors] in: as from zero_shard_layout (offsets
 *                      increasing, tensors not overlapping)
 * max_chunk_elems      in : a multiple of 8, at least 8
 * out[capacity]        out: the chunks; with out == NULL and capacity == 0 only
 *                      the count is computed (returns ZERO_OK)
 * n_chunks             out: number of chunks needed, also on ERANGE
 * Errors: EINVAL (bad sizes, overlapping tensors, begin > end, bad chunk size);
 *         ERANGE when capacity < *n_chunks (the first `capacity` are written).
 * -------------------------------------------------------------------------- */
int zero_chunk_table(const uint64_t *numel, const uint64_t *tensor_offset, uint32_t n_tensors,
                     uint64_t begin, uint64_t end, uint32_t max_chunk_elems, zero_chunk *out,
                     uint64_t capacity, uint64_t *n_chunks);

/* ----------------------------------------------------------------------------
 * zero_dense_offsets -- where each tensor starts in the dense layout.
 *
 * [Deep dive] "Resume training and export weights separately": exporting
 * consolidates the fp32 weights into per-tensor form, without the flat
 * buffer's padding.  dense_offset[k] = numel[0] + ... + numel[k-1]; the
 * dense buffer holds dense_total = numel[0] + ... + numel[n_tensors-1]
 * elements.  These are the offsets zero_owner_to_dense / zero_dense_to_owner
 * take (as a device table) to address the dense buffer.
 *
 * numel[n_tensors]         in : element counts, all > 0
 * dense_offset[n_tensors]  out: caller-owned host array
 * dense_total              out
 * Errors: EINVAL for a zero count or NULL pointers; ERANGE if the total
 * exceeds 64 bits (nothing is written then).
 * -------------------------------------------------------------------------- */
int zero_dense_offsets(const uint64_t *numel, uint32_t n_tensors, uint64_t *dense_offset,
                       uint64_t *dense_total);

/* Exact byte count num/den, reduced to lowest terms. */
typedef struct {
  uint64_t num;
  uint64_t den;
} zero_ratio;

/* ----------------------------------------------------------------------------
 * zero_state_bytes -- idealised persistent bytes per rank.
 *
 * [Deep dive] "Count state before choosing a stage" and [ZeRO Q&A] "Memory
 * Footprint Reduction Matrix": with p, g, o bytes per parameter for the
 * compute weights, gradients and optimizer state (master + moments),
 *   out[0] DP     = P (p + g + o)
 *   out[1] ZeRO-1 = P (p + g) + P o / R
 *   out[2] ZeRO-2 = P p + P (g + o) / R
 *   out[3] ZeRO-3 = P (p + g + o) / R
 * Errors: EINVAL if any count or width is 0 or out is NULL; ERANGE if a
 * numerator does not fit 64 bits.
 * -------------------------------------------------------------------------- */
int zero_state_bytes(uint64_t params, uint64_t ranks, uint32_t param_bytes, uint32_t grad_bytes,
                     uint32_t optim_bytes, zero_ratio out[4]);

/* ----------------------------------------------------------------------------
 * zero_reduce_owned -- the owner's reduced gradient, in fp32.
 *
 * [Deep dive] "Reduce first, then update the owned slice": the owner's
 * share of a reduce-scatter, i.e. the equally weighted mean over ranks,
 * formed only at the indices it owns.  For every flat index f in [begin, begin + n), with
 * o = out[f - out_base]:
 *   s = (accumulate == 1 ? o : +0.0f);
 *   for r = 0 .. R-1:  s = s + (float) rank_grads[r][f - grad_base];   (fp32)
 *   s = s / divisor;                                                    (IEEE fp32)
 *   out[f - out_base] = (accumulate == 2 ? o + s : s);                  (fp32)
 * accumulate: 0 overwrite; 1 start the sum from the output; 2 add the
 * reduced mean to the output -- the per-backward schedule of [Deep dive]
 * "Communication volume isn't elapsed time" (ZeRO-2/3 reduce and keep the
 * owned slice on every backward call; Adam runs at the boundary).
 * The order is fixed, so results are identical run to run and bit-exact
 * against a sequential fp32 loop.  A loss scale is folded into `divisor`
 * (e.g. R * 65536).  R = 1, divisor = 1, accumulate = 1 is fp32 gradient
 * accumulation (acc += g) of one microstep.  The range may span the padding
 * between tensors; it is reduced like real elements, so with zeros in the
 * rank buffers' padding the check below equals the check over the real
 * elements alone.
 *
 * rank_grads  host array [R] of device pointers; buffer r holds at least
 *             begin + n - grad_base elements of `grad_dtype` (F16, BF16, F32)
 * out         device fp32, at least begin + n - out_base elements
 * d_overflow, d_sumsq: both NULL, or both device pointers; then the pass also
 *             computes the overflow flag and squared norm of the values it
 *             writes, exactly as zero_grad_check does (needs `workspace`:
 *             device, 256-byte aligned, at least zero_check_workspace_bytes(n)
 *             bytes).
 * n == 0 launches nothing (the check outputs are then left untouched).
 * Errors: EINVAL (R out of [1, ZERO_MAX_RANKS], bad dtype, misaligned pointer
 *         or base, begin below a base, divisor not finite and > 0, accumulate
 *         not 0, 1 or 2, workspace missing or too small); EHIP.
 * -------------------------------------------------------------------------- */
int zero_reduce_owned(const void *const *rank_grads, uint32_t R, int grad_dtype, uint64_t grad_base,
                      uint64_t begin, uint64_t n, float divisor, int accumulate, float *out,
                      uint64_t out_base, int32_t *d_overflow, double *d_sumsq, void *workspace,
                      size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * zero_reduce_owned_noalloc -- zero_reduce_owned without a workspace argument.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as zero_reduce_owned, minus workspace and
 * ws_bytes; it calls no allocating routine.  The check's per-block partials
 * go to a 16 MiB array that the library keeps on every GPU it runs on until
 * the process ends, so a check covers at most about 2.8e9 elements (larger n
 * with a check: ERANGE, nothing launched).  Without the check outputs it is
 * zero_reduce_owned itself.  All calls on one GPU share that array: calls
 * that overlap on one GPU (different streams, host threads) race and must
 * be ordered by the caller.  The first call on a device looks the array up
 * once (EHIP if that fails); make that first call outside graph capture.
 * -------------------------------------------------------------------------- */
int zero_reduce_owned_noalloc(const void *const *rank_grads, uint32_t R, int grad_dtype,
                              uint64_t grad_base, uint64_t begin, uint64_t n, float divisor,
                              int accumulate, float *out, uint64_t out_base, int32_t *d_overflow,
                              double *d_sumsq, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * zero_check_workspace_bytes -- device workspace a check over n elements needs
 * (zero_grad_check, or zero_reduce_owned with the check outputs): the
 * per-block partial sums and flags of the first stage (one block per 2048
 * elements) and of the fold after it.  Host only; grows linearly with n
 * (about 6 bytes per 1000 elements).
 * Errors: EINVAL (bytes NULL).
 * -------------------------------------------------------------------------- */
int zero_check_workspace_bytes(uint64_t n, uint64_t *bytes);

/* ----------------------------------------------------------------------------
 * zero_grad_check -- overflow flag and squared norm of an fp32 gradient.
 *
 * *d_overflow = 1 if any g[i] is infinite or NaN, else 0.
 * *d_sumsq    = sum of g[i]^2, each square and the sum in fp64 (a fixed
 *               reduction tree: per-thread sums, wavefront shuffles, an LDS
 *               block stage, then the per-block partials folded in fixed
 *               contiguous slices), so the result is identical run to run on
 *               one device.  When the
 *               flag is set the sum is meaningless.
 * The pages name no overflow handling; with a loss scale the caller skips the
 * step when the flag is set, and clips with zero_clip_coef otherwise.
 * g          device fp32 [n];  workspace: device, 256-byte aligned, at least
 *            zero_check_workspace_bytes(n) bytes (per-block partials).
 * n == 0 writes flag 0 and sum 0.
 * Errors: EINVAL (NULL outputs, workspace too small, misaligned); EHIP.
 * -------------------------------------------------------------------------- */
int zero_grad_check(const float *g, uint64_t n, int32_t *d_overflow, double *d_sumsq,
                    void *workspace, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * zero_clip_coef -- host scalar of a global-norm clip:
 *   *coef = (float) min(1, max_norm / (sqrt(sumsq) + eps))   (fp64, one rounding)
 * The pages give no clipping rule; this is the common clip_grad_norm_ form.
 * Errors: EINVAL for a negative or non-finite sumsq, max_norm <= 0, eps < 0.
 * -------------------------------------------------------------------------- */
int zero_clip_coef(double sumsq, double max_norm, double eps, float *coef);

/* ----------------------------------------------------------------------------
 * zero_step_decision -- the host half of an overflow-checked, clipped step
 * over several owners.
 *
 * The pages give neither the overflow skip nor the clip (see zero_clip_coef
 * for the clip's form).  Every owner checks only its own slice, so the
 * decision needs all of them: the step is skipped when any owner's flag is
 * set; otherwise the global squared norm is the sum of the owners' partials,
 * added in owner order in fp64, and the clip factor follows from it.  Every
 * owner then takes the same decision and the same factor, which is what the
 * unsharded step would do.  With one owner the partial is the whole norm.
 *
 * overflow[n_owners], sumsq[n_owners]  in : host arrays, one entry per owner
 *                                           (what zero_reduce_owned's check or
 *                                           zero_grad_check left on the device)
 * max_norm, eps                        in : as for zero_clip_coef
 * update                               out: 1 to apply the step, 0 to skip it
 *                                           (the step count then stays)
 * coef                                 out: the clip factor (0 when skipped)
 * Errors: EINVAL for NULL pointers, n_owners == 0, a negative or non-finite
 *         partial (only looked at when no flag is set), or bad max_norm / eps.
 * -------------------------------------------------------------------------- */
int zero_step_decision(const int32_t *overflow, const double *sumsq, uint32_t n_owners,
                       double max_norm, double eps, int32_t *update, float *coef);

/* ----------------------------------------------------------------------------
 * zero_chunk_groups -- packs runs of short chunks into groups that one block
 * of zero_adam_step processes together (host only; a layout aid, not a step
 * of the method).  Walking the chunks in order, a group is either one chunk,
 * or consecutive chunks whose work units -- scalar head elements, 128-bit
 * vectors and scalar tail elements -- number at most 256 in all and whose
 * elements number at most max_group_elems.  Tensors whose padding breaks the
 * runs of real elements (e.g. 100-element tensors padded to 128) otherwise
 * give one almost idle block each.
 *
 * chunks[n_chunks]     in : a host copy of the chunk table
 * max_group_elems      in : > 0 (the chunk size is the natural choice)
 * out[capacity]        out: the first chunk of each group, then n_chunks as a
 *                      sentinel (n_groups + 1 entries); out == NULL with
 *                      capacity == 0 only counts
 * n_groups             out: number of groups, also on ERANGE
 * Errors: EINVAL (NULL pointers, max_group_elems 0); ERANGE (capacity below
 * n_groups + 1).
 * -------------------------------------------------------------------------- */
int zero_chunk_groups(const zero_chunk *chunks, uint64_t n_chunks, uint32_t max_group_elems,
                      uint64_t *out, uint64_t capacity, uint64_t *n_groups);

/* Arguments of zero_adam_step. */
typedef struct {
  /* The owner's work: device chunk table (from zero_chunk_table) and the owner
   * range [begin, end); chunk pieces outside the range are ignored. */
  const zero_chunk *chunks;
  uint64_t n_chunks;
  /* Optional device group table from zero_chunk_groups (n_groups + 1 entries):
   * one block per group instead of one per chunk.  NULL (and n_groups 0): one
   * block per chunk.  The results are the same either way. */
  const uint64_t *groups;
  uint64_t n_groups;
  uint64_t begin, end;
  /* Gradient source: either R rank buffers (reduced here, as zero_reduce_owned,
   * then multiplied by clip_coef) or, with reduced_g != NULL, an owner-local
   * fp32 reduced gradient (reduced_g[f - local_base]) multiplied by clip_coef. */
  const void *const *rank_grads; /* host array [R] of device pointers, or NULL */
  uint32_t R;
  int32_t grad_dtype;
  uint64_t grad_base;
  float divisor;
  const float *reduced_g;
  /* fp32 master weights and moments of the owner: element f - local_base,
   * each at least end - local_base elements. */
  float *master, *exp_avg, *exp_avg_sq;
  uint64_t local_base;
  /* 16-bit compute copy: param16[f - param_base] (F16 or BF16), or ZERO_NONE. */
  void *param16;
  int32_t param_dtype;
  uint64_t param_base;
  /* Optimizer: step >= 1 counts completed updates including this one. */
  double lr, beta1, beta2, eps, weight_decay;
  int32_t adamw; /* 1: decoupled decay (AdamW); 0: classic Adam, wd added to g */
  uint64_t step;
  double clip_coef; /* 1.0 when not clipping */
  uint32_t grid_blocks; /* 0: one block per chunk or group (the library
                           default); else that many blocks, each taking chunks
                           or groups with a grid stride (same results for
                           every grid) */
} zero_adam_args;

/* ----------------------------------------------------------------------------
 * zero_adam_step -- fused reduce + Adam/AdamW + 16-bit write-back.
 *
 * [Deep dive] "Reduce first, then update the owned slice": for every real
 * element f of the chunk table (one pass; each byte read and written once):
 *   g  = reduced gradient (bit-identical to zero_reduce_owned) * clip_coef
 *   (adamw == 0 and weight_decay != 0: g += weight_decay * w)
 *   m  = beta1 m + (1 - beta1) g
 *   v  = beta2 v + (1 - beta2) g^2                 (uncentred)
 *   w  = w (1 - lr wd [adamw only]) - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *   param16[f] = round-to-nearest-even 16-bit copy of w
 * [ZeRO-3 docs] configuration examples name AdamW with weight_decay; the
 * pages give no formula, and the decoupled form is used.  Arithmetic is fp32
 * with constants derived on the host in fp64.
 * Errors: EINVAL (NULL args, step 0, bad dtype/R/alignment/bases, hyper-
 * parameters out of range: lr, wd, eps >= 0, betas in [0, 1), divisor > 0,
 * clip_coef >= 0, all finite; n_groups without a group table); EHIP.
 * n_chunks == 0, begin == end, or a group table with n_groups == 0 is a no-op.
 * -------------------------------------------------------------------------- */
int zero_adam_step(const zero_adam_args *args, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * zero_owner_to_dense / zero_dense_to_owner -- export and import of fp32 shard
 * data (master weights or moments) between one owner's shard and the dense
 * per-tensor layout (every tensor's elements in order, tensors concatenated,
 * no padding).
 *
 * [Deep dive] "Resume training and export weights separately": exporting a
 * model consolidates the fp32 weights from the owners' shards; a weights-only
 * restore loads them back with fresh moments (and resumes a different
 * trajectory than a full-state restore).  Calling zero_owner_to_dense for
 * every owner of a layout fills the whole dense buffer.
 *
 * For every real element f of the chunk table within [begin, end), with k the
 * tensor that holds f:  dense[dense_offset[k] + f - tensor_offset[k]]  <->
 * owner[f - owner_base].  (A chunk runs across tensors only where no padding
 * separates them; there, with dense_offset as below, its first tensor gives
 * the same dense index for every element, and that is how the kernel
 * computes it.)
 * chunks[n_chunks]            device: the owner's chunk table
 * groups, n_groups            optional device group table from zero_chunk_groups
 *                             (n_groups + 1 entries): one block per group, the
 *                             short chunks of a group copied together; NULL
 *                             and 0 for one block per chunk
 * tensor_offset, dense_offset device uint64 [n_tensors]: flat and dense start of
 *                             each tensor (dense_offset[k] = sum of numel[j<k])
 * owner                       device fp32, at least end - owner_base elements
 * dense                       device fp32 [dense_total]
 * Chunks naming a tensor >= n_tensors, and dense indices >= dense_total, are
 * skipped.  Errors: EINVAL (NULL pointers with work to do, begin > end,
 * owner_base > begin, misaligned fp32 pointers, n_groups without a group
 * table); EHIP.
 * -------------------------------------------------------------------------- */
int zero_owner_to_dense(const zero_chunk *chunks, uint64_t n_chunks, const uint64_t *groups,
                        uint64_t n_groups, uint64_t begin, uint64_t end,
                        const uint64_t *tensor_offset, const uint64_t *dense_offset,
                        uint32_t n_tensors, const float *owner, uint64_t owner_base, float *dense,
                        uint64_t dense_total, hipStream_t stream);
int zero_dense_to_owner(const zero_chunk *chunks, uint64_t n_chunks, const uint64_t *groups,
                        uint64_t n_groups, uint64_t begin, uint64_t end,
                        const uint64_t *tensor_offset, const uint64_t *dense_offset,
                        uint32_t n_tensors, const float *dense, uint64_t dense_total, float *owner,
                        uint64_t owner_base, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * ZeRO-3 per-tensor partitioning and the gathered working set.
 *
 * [Deep dive] "Stage 3 needs a live working set": each tensor k of n_k
 * elements is cut into R shards of s_k = ceil(n_k / R) elements (rank r holds
 * elements [r s_k, (r+1) s_k), zero past the end of the tensor).  A rank's
 * shard buffer holds its shards of all tensors in tensor order (tensor k at
 * so_k = sum of s_j, j < k).  Using a tensor gathers all R shards into a
 * separate full buffer of R s_k elements, in rank order; the tensor is its
 * first n_k elements.  Live tensors' buffers follow each other in the order
 * the live list gives.
 *
 * zero3_storage: resident = sum_k s_k elements per rank, gathered = sum over
 *   live tensors of R s_k; shard_numel[k] = s_k (shard_numel may be NULL).
 * zero3_gather_spans: the copy spans that assemble the live tensors' buffers
 *   from the R shard buffers (span.buf = source rank).
 * zero3_partition_spans: the copy spans that cut rank `rank`'s shard buffer
 *   out of the dense tensors (tensors concatenated, no padding); the padding
 *   past each tensor's end is not written, so the shard buffer should start
 *   zeroed.
 * Span tables follow zero_chunk_table's conventions: spans of at most
 * max_span elements; out == NULL with capacity == 0 only counts; ERANGE when
 * capacity is short (the first `capacity` spans are written).
 * Errors: EINVAL for ranks 0, a 0-element tensor, a live index out of range
 * or listed twice, rank >= ranks, max_span 0; ERANGE for counts above 2^64.
 * -------------------------------------------------------------------------- */
typedef struct {
  uint64_t src;  /* first element in source buffer `buf` */
  uint64_t dst;  /* first element in the destination */
  uint32_t len;  /* elements */
  uint32_t buf;  /* source buffer index */
} zero_copy_span;

int zero3_storage(const uint64_t *numel, uint32_t n_tensors, uint32_t ranks, const uint32_t *live,
                  uint32_t n_live, uint64_t *shard_numel, uint64_t *resident, uint64_t *gathered);
int zero3_gather_spans(const uint64_t *numel, uint32_t n_tensors, uint32_t ranks,
                       const uint32_t *live, uint32_t n_live, uint32_t max_span,
                       zero_copy_span *out, uint64_t capacity, uint64_t *n_spans);
int zero3_partition_spans(const uint64_t *numel, uint32_t n_tensors, uint32_t ranks,
                          uint32_t rank, uint32_t max_span, zero_copy_span *out,
                          uint64_t capacity, uint64_t *n_spans);

/* Most source buffers one zero_copy_spans call can read. */
#define ZERO_MAX_COPY_SOURCES 128

/* ----------------------------------------------------------------------------
 * zero_span_groups -- packs runs of short spans into groups that one block of
 * zero_copy_spans copies together (host only; a layout aid).  As
 * zero_chunk_groups, with a span's work units being its scalar head
 * elements, 16-byte vectors and scalar tail elements when source and
 * destination share their 16-byte phase, else one unit per element, and at
 * most 2048 units (eight per thread) in a group of several spans.  Small
 * tensors give short shards (a 4096-element norm over 8 ranks: 512-element
 * spans), one almost idle block each without groups.
 * spans[n_spans] in: a host copy of the span table; elem_bytes 2 or 4;
 * max_group_elems > 0; out/capacity/n_groups as in zero_chunk_groups.
 * Errors: EINVAL (NULL pointers, bad elem_bytes, max_group_elems 0); ERANGE.
 * -------------------------------------------------------------------------- */
int zero_span_groups(const zero_copy_span *spans, uint64_t n_spans, uint32_t elem_bytes,
                     uint32_t max_group_elems, uint64_t *out, uint64_t capacity, uint64_t *n_groups);

/* ----------------------------------------------------------------------------
 * zero_copy_spans -- dst[span.dst + i] = srcs[span.buf][span.src + i] for every
 * span of a device span table, in one multi-span launch.  The
 * device side of the stage-3 gather (and partition) on one GPU.
 * spans[n_spans]      device table (from the builders above)
 * srcs, src_numel     host arrays [n_srcs] of device pointers and their
 *                     element counts; n_srcs <= ZERO_MAX_COPY_SOURCES
 * dst, dst_numel      device destination and its element count
 * elem_bytes          2 (fp16/bf16) or 4 (fp32)
 * groups, n_groups    optional device group table from zero_span_groups
 *                     (n_groups + 1 entries): one block per group instead of
 *                     one per span; NULL and 0 for one block per span.  The
 *                     copies are the same either way.
 * Spans whose buffer index or extent falls outside these counts are skipped.
 * Errors: EINVAL (NULL pointers with work, bad elem_bytes, n_srcs out of
 * range, pointers not 16-byte aligned, n_groups without a group table); EHIP.
 * -------------------------------------------------------------------------- */
int zero_copy_spans(const zero_copy_span *spans, uint64_t n_spans, const void *const *srcs,
                    const uint64_t *src_numel, uint32_t n_srcs, void *dst, uint64_t dst_numel,
                    uint32_t elem_bytes, const uint64_t *groups, uint64_t n_groups,
                    hipStream_t stream);

/* ----------------------------------------------------------------------------
 * Measurement.
 * -------------------------------------------------------------------------- */

/* Most source (and most destination) streams of one zero_stream_probe call. */
#define ZERO_MAX_PROBE_STREAMS 64

/* ----------------------------------------------------------------------------
 * zero_stream_probe -- the bandwidth probe against which the optimizer kernels
 * are measured (no part of the optimizer step; the pages define no such
 * operation).  Every destination receives the bytewise XOR of all sources,
 * streamed with 16-byte loads and stores, one block per 256-thread piece.
 * A stream's width w (1 or 2) is the number of consecutive 16-byte vectors
 * each thread touches: width 1 is how the kernels stream 16-bit data (8
 * elements, 16 bytes per thread), width 2 how they stream fp32 data (8
 * elements, 32 bytes), so a probe can copy a kernel's exact stream structure.
 * With `bytes` per width unit, thread i of the grid (i < bytes / 16) reads
 * vectors [w i, w i + w) of every source, XORs them all into one vector and
 * writes it to vectors [w i, w i + w) of every destination; a stream of width
 * w spans w * bytes bytes, and one launch moves the sum of all of them.  One
 * source and one destination of width 1 is a plain copy; no destinations
 * reads only, no sources writes zeros.
 * srcs[n_src], dsts[n_dst]  host arrays of device pointers, each 16-byte
 *                           aligned; n_src, n_dst <= ZERO_MAX_PROBE_STREAMS,
 *                           not both 0 (an empty array may be NULL)
 * src_widths, dst_widths    host arrays of 1 or 2 per stream, or NULL (all 1)
 * bytes                     bytes per width unit, a multiple of 16 (0: no launch)
 * order                     0: block b takes piece b (blocks are dealt to the
 *                           8 XCDs in turn); 1: each XCD takes one contiguous
 *                           run of pieces.  Which is faster depends on the
 *                           number of streams.
 * A destination that overlaps a source or another destination gives
 * unspecified contents (no fault: every access stays inside the streams).
 * Errors: EINVAL (stream counts, NULL or misaligned pointers, a width other
 * than 1 or 2, bytes not a multiple of 16, order not 0 or 1); EHIP.
 * -------------------------------------------------------------------------- */
int zero_stream_probe(const void *const *srcs, const uint8_t *src_widths, uint32_t n_src,
                      void *const *dsts, const uint8_t *dst_widths, uint32_t n_dst, uint64_t bytes,
                      int order, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
