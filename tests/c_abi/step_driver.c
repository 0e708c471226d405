/*
 * A plain C caller of libzero_shard: one owner step through the C ABI alone,
 * with device memory from hipMalloc and a stream of its own (no torch, no
 * Python).  Test infrastructure: tests/test_gpu_c_driver.py writes the
 * inputs, runs this program and checks what it writes against the oracle.
 *
 * Usage: step_driver <inputs> <outputs>
 *
 * Inputs (little-endian):
 *   u64  magic "ZSTEPIN1", n_tensors, R, align, owner, grad_dtype, param_dtype,
 *        step, adamw
 *   f64  lr, beta1, beta2, eps, weight_decay
 *   u64  numel[n_tensors]
 *   R rank gradient buffers of padded_total elements (grad_dtype), then the
 *   owner-local master, m and v, (end - local_base) fp32 values each.
 * Outputs: master, m, v after the fused step; the 16-bit copy
 *   (padded_total values, zero before the step); the reduced gradient of a
 *   separate checked reduce (end - local_base fp32, zero outside the owner
 *   range); its overflow flag (i32) and squared norm (f64); the step decision
 *   for this owner alone with max_norm 1 and eps 1e-6 (update i32, clip
 *   factor f32); the dense layout (dense_total u64, then dense_offset u64
 *   [n_tensors]).
 *
 * The program also checks, on its own: the error convention (a call with
 * step 0 must return ZERO_EINVAL with a message); that the allocation-free
 * checked reduce gives the same bits, flag and norm as the workspace form;
 * and that the decision's factor equals zero_clip_coef of the same norm.
 * Exit status 0 on success, 1 on any failure (with a message on stderr).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_shard.h"

#define FAIL(...)                     \
  do {                                \
    fprintf(stderr, __VA_ARGS__);     \
    fputc('\n', stderr);              \
    exit(1);                          \
  } while (0)

#define HIP(call)                                                              \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_));        \
  } while (0)

#define ZS(call)                                                               \
  do {                                                                         \
    int rc_ = (call);                                                          \
    if (rc_ != ZERO_OK) FAIL("%s: %d %s", #call, rc_, zero_last_error());      \
  } while (0)

static void read_all(FILE* f, void* p, size_t bytes, const char* what) {
  if (bytes && fread(p, 1, bytes, f) != bytes) FAIL("short read: %s", what);
}

static void write_all(FILE* f, const void* p, size_t bytes) {
  if (bytes && fwrite(p, 1, bytes, f) != bytes) FAIL("short write");
}

static void* dev_copy(const void* host, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) FAIL("usage: %s <inputs> <outputs>", argv[0]);
  FILE* in = fopen(argv[1], "rb");
  if (!in) FAIL("cannot open %s", argv[1]);
  uint64_t hdr[9];
  double hp[5];
  read_all(in, hdr, sizeof hdr, "header");
  if (memcmp(&hdr[0], "ZSTEPIN1", 8) != 0) FAIL("bad magic");
  const uint64_t n_tensors = hdr[1], R = hdr[2], align = hdr[3], owner = hdr[4];
  const int gdt = (int)hdr[5], pdt = (int)hdr[6];
  const uint64_t step = hdr[7], adamw = hdr[8];
  read_all(in, hp, sizeof hp, "hyperparameters");
  if (n_tensors == 0 || n_tensors > 100000 || R == 0 || R > ZERO_MAX_RANKS || owner >= R)
    FAIL("bad sizes");
  if ((gdt != ZERO_F16 && gdt != ZERO_BF16 && gdt != ZERO_F32) ||
      (pdt != ZERO_F16 && pdt != ZERO_BF16))
    FAIL("bad dtypes");
  uint64_t* numel = malloc(n_tensors * sizeof *numel);
  read_all(in, numel, n_tensors * sizeof *numel, "numel");

  /* layout and the owner's chunk table, on the host */
  uint64_t* offs = malloc(n_tensors * sizeof *offs);
  uint64_t* obeg = malloc(R * sizeof *obeg);
  uint64_t* oend = malloc(R * sizeof *oend);
  uint64_t total = 0;
  ZS(zero_shard_layout(numel, (uint32_t)n_tensors, (uint32_t)R, (uint32_t)align, offs, &total, obeg, oend));
  const uint64_t begin = obeg[owner], end = oend[owner], lb = begin & ~(uint64_t)7;
  uint64_t n_chunks = 0;
  ZS(zero_chunk_table(numel, offs, (uint32_t)n_tensors, begin, end, 2048, NULL, 0, &n_chunks));
  zero_chunk* chunks = malloc((n_chunks ? n_chunks : 1) * sizeof *chunks);
  ZS(zero_chunk_table(numel, offs, (uint32_t)n_tensors, begin, end, 2048, chunks, n_chunks, &n_chunks));

  /* inputs to the device */
  const size_t gsz = gdt == ZERO_F32 ? 4 : 2, nloc = (size_t)(end - lb);
  void* h_grad = malloc(total * gsz > 0 ? total * gsz : 1);
  const void** d_grads = malloc(R * sizeof *d_grads);
  for (uint64_t r = 0; r < R; ++r) {
    read_all(in, h_grad, total * gsz, "rank gradients");
    d_grads[r] = dev_copy(h_grad, total * gsz);
  }
  float* h_state = malloc(3 * nloc * sizeof(float) + 1);
  read_all(in, h_state, 3 * nloc * sizeof(float), "state");
  fclose(in);
  float* d_w = dev_copy(h_state, nloc * 4);
  float* d_m = dev_copy(h_state + nloc, nloc * 4);
  float* d_v = dev_copy(h_state + 2 * nloc, nloc * 4);
  void* d_chunks = dev_copy(chunks, n_chunks * sizeof *chunks);
  void* d_p16 = NULL;
  HIP(hipMalloc(&d_p16, total * 2 + 16));
  HIP(hipMemset(d_p16, 0, total * 2 + 16));
  float* d_g = NULL;
  HIP(hipMalloc((void**)&d_g, nloc * 4 + 16));
  HIP(hipMemset(d_g, 0, nloc * 4 + 16));
  uint64_t ws_bytes = 0;
  ZS(zero_check_workspace_bytes(end - begin, &ws_bytes));
  void* d_ws = NULL;
  int32_t* d_flag = NULL;
  double* d_sumsq = NULL;
  HIP(hipMalloc(&d_ws, ws_bytes));
  HIP(hipMalloc((void**)&d_flag, sizeof(int32_t)));
  HIP(hipMalloc((void**)&d_sumsq, sizeof(double)));
  hipStream_t stream;
  HIP(hipStreamCreate(&stream));

  zero_adam_args a;
  memset(&a, 0, sizeof a);
  a.chunks = (const zero_chunk*)d_chunks;
  a.n_chunks = n_chunks;
  a.begin = begin;
  a.end = end;
  a.rank_grads = d_grads;
  a.R = (uint32_t)R;
  a.grad_dtype = gdt;
  a.grad_base = 0;
  a.divisor = (float)R;
  a.master = d_w;
  a.exp_avg = d_m;
  a.exp_avg_sq = d_v;
  a.local_base = lb;
  a.param16 = d_p16;
  a.param_dtype = pdt;
  a.param_base = 0;
  a.lr = hp[0];
  a.beta1 = hp[1];
  a.beta2 = hp[2];
  a.eps = hp[3];
  a.weight_decay = hp[4];
  a.adamw = (int32_t)adamw;
  a.clip_coef = 1.0;

  /* the error convention first: step 0 is rejected before any launch */
  a.step = 0;
  if (zero_adam_step(&a, stream) != ZERO_EINVAL || zero_last_error()[0] == '\0')
    FAIL("step 0 was not rejected with a message");
  a.step = step;
  ZS(zero_adam_step(&a, stream));
  ZS(zero_reduce_owned((const void* const*)d_grads, (uint32_t)R, gdt, 0, begin, end - begin, (float)R, 0,
                       d_g, lb, d_flag, d_sumsq, d_ws, (size_t)ws_bytes, stream));
  /* the same checked reduce without a workspace: identical bits, flag and norm */
  float* d_g2 = NULL;
  int32_t* d_flag2 = NULL;
  double* d_sumsq2 = NULL;
  HIP(hipMalloc((void**)&d_g2, nloc * 4 + 16));
  HIP(hipMemset(d_g2, 0, nloc * 4 + 16));
  HIP(hipMalloc((void**)&d_flag2, sizeof(int32_t)));
  HIP(hipMalloc((void**)&d_sumsq2, sizeof(double)));
  ZS(zero_reduce_owned_noalloc((const void* const*)d_grads, (uint32_t)R, gdt, 0, begin, end - begin, (float)R, 0,
                               d_g2, lb, d_flag2, d_sumsq2, stream));
  HIP(hipStreamSynchronize(stream));

  FILE* out = fopen(argv[2], "wb");
  if (!out) FAIL("cannot open %s", argv[2]);
  float* h_f = malloc(nloc * 4 + 1);
  float* dst[4] = {d_w, d_m, d_v, NULL};
  for (int k = 0; k < 3; ++k) {
    HIP(hipMemcpy(h_f, dst[k], nloc * 4, hipMemcpyDeviceToHost));
    write_all(out, h_f, nloc * 4);
  }
  uint16_t* h_p = malloc(total * 2 + 1);
  HIP(hipMemcpy(h_p, d_p16, total * 2, hipMemcpyDeviceToHost));
  write_all(out, h_p, total * 2);
  HIP(hipMemcpy(h_f, d_g, nloc * 4, hipMemcpyDeviceToHost));
  write_all(out, h_f, nloc * 4);
  int32_t flag = -1;
  double sumsq = -1.0;
  HIP(hipMemcpy(&flag, d_flag, sizeof flag, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&sumsq, d_sumsq, sizeof sumsq, hipMemcpyDeviceToHost));
  write_all(out, &flag, sizeof flag);
  write_all(out, &sumsq, sizeof sumsq);

  float* h_f2 = malloc(nloc * 4 + 1);
  int32_t flag2 = -1;
  double sumsq2 = -1.0;
  HIP(hipMemcpy(h_f2, d_g2, nloc * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&flag2, d_flag2, sizeof flag2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&sumsq2, d_sumsq2, sizeof sumsq2, hipMemcpyDeviceToHost));
  if (memcmp(h_f, h_f2, nloc * 4) != 0) FAIL("the allocation-free reduce differs from the workspace form");
  if (flag2 != flag || memcmp(&sumsq2, &sumsq, sizeof sumsq) != 0)
    FAIL("the allocation-free check differs: flag %d/%d, sumsq %.17g/%.17g", flag2, flag, sumsq2, sumsq);

  int32_t update = -1;
  float coef = -1.0f, coef1 = -2.0f;
  ZS(zero_step_decision(&flag, &sumsq, 1, 1.0, 1e-6, &update, &coef));
  if (!flag) {
    ZS(zero_clip_coef(sumsq, 1.0, 1e-6, &coef1));
    if (update != 1 || coef != coef1) FAIL("decision (%d, %.9g) against zero_clip_coef %.9g", update, coef, coef1);
  }
  write_all(out, &update, sizeof update);
  write_all(out, &coef, sizeof coef);

  uint64_t* dense = malloc(n_tensors * sizeof *dense);
  uint64_t dense_total = 0;
  ZS(zero_dense_offsets(numel, (uint32_t)n_tensors, dense, &dense_total));
  write_all(out, &dense_total, sizeof dense_total);
  write_all(out, dense, n_tensors * sizeof *dense);
  if (fclose(out) != 0) FAIL("cannot write %s", argv[2]);

  HIP(hipStreamDestroy(stream));
  for (uint64_t r = 0; r < R; ++r) HIP(hipFree((void*)d_grads[r]));
  HIP(hipFree(d_w));
  HIP(hipFree(d_m));
  HIP(hipFree(d_v));
  HIP(hipFree(d_chunks));
  HIP(hipFree(d_p16));
  HIP(hipFree(d_g));
  HIP(hipFree(d_ws));
  HIP(hipFree(d_flag));
  HIP(hipFree(d_sumsq));
  HIP(hipFree(d_g2));
  HIP(hipFree(d_flag2));
  HIP(hipFree(d_sumsq2));
  free(numel), free(offs), free(obeg), free(oend), free(chunks), free(h_grad), free(d_grads);
  free(h_state), free(h_f), free(h_f2), free(h_p), free(dense);
  printf("step_driver ok: owner %llu of %llu, %llu chunks\n", (unsigned long long)owner,
         (unsigned long long)R, (unsigned long long)n_chunks);
  return 0;
}
