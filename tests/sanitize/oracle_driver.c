/* Sanitizer driver for the oracle (test infrastructure): calls every oracle
 * function on small random inputs -- random bit patterns, so NaN, infinities
 * and subnormals occur -- and on ragged owner layouts, so that an
 * AddressSanitizer / UndefinedBehaviorSanitizer build reports any
 * out-of-bounds access or undefined operation.  Exit status 0 = clean run. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
  int32_t adamw;
  uint64_t step;
  double clip_coef;
} oracle_hyper;

uint16_t oracle_f32_to_f16(float x);
uint16_t oracle_f32_to_bf16(float x);
double oracle_f16_value(uint16_t b);
double oracle_bf16_value(uint16_t b);
void oracle_encode16(const float *x, uint64_t n, int dtype, uint16_t *out);
void oracle_reduce(uint32_t R, int dtype, const void *const *grads, uint64_t n, float divisor,
                   int accumulate, float *out);
void oracle_reduce_add(uint32_t R, int dtype, const void *const *grads, uint64_t n, float divisor,
                       float *out);
void oracle_accumulate(int dtype, const void *g, uint64_t n, int first, float *acc);
void oracle_grad_check(const float *g, uint64_t n, int32_t *overflow, double *sumsq);
double oracle_clip_coef(double sumsq, double max_norm, double eps);
void oracle_adam_f64(uint64_t n, const double *g, double *w, double *m, double *v,
                     const oracle_hyper *h);
void oracle_adam_f32(uint64_t n, const float *g, float *w, float *m, float *v, const oracle_hyper *h);
void oracle_owner_step(uint32_t R, int gdtype, const void *const *grads, uint64_t grad_base,
                       const float *reduced_g, float divisor, uint64_t n_ranges,
                       const uint64_t *range_begin, const uint64_t *range_end, float *w, float *m,
                       float *v, uint64_t local_base, void *p16, int pdtype, uint64_t param_base,
                       const oracle_hyper *h);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static uint64_t below(uint64_t n) { return n ? next() % n : 0; }

/* `n` elements of dtype 1 (f16), 2 (bf16) or 3 (f32) with random bits, exactly sized. */
static void *random_buf(int dtype, uint64_t n) {
  const size_t w = dtype == 3 ? 4 : 2;
  unsigned char *p = malloc(n * w + 1);
  for (uint64_t i = 0; i < n * w; ++i) p[i] = (unsigned char)next();
  return p;
}

static float *random_f32(uint64_t n, int finite) {
  float *p = malloc(n * sizeof(float) + 1);
  for (uint64_t i = 0; i < n; ++i) {
    if (finite) {
      p[i] = (float)((double)(int64_t)(next() >> 11) / 9.0e15);
    } else {
      uint32_t u = (uint32_t)next();
      memcpy(&p[i], &u, 4);
    }
  }
  return p;
}

int main(void) {
  for (int trial = 0; trial < 300; ++trial) {
    const uint32_t R = 1 + (uint32_t)below(9);
    const int dtype = 1 + (int)below(3);
    const uint64_t n = below(300);
    const void *grads[9];
    for (uint32_t r = 0; r < R; ++r) grads[r] = random_buf(dtype, n);
    float *out = random_f32(n, trial & 1);
    const float divisors[] = {1.0f, 3.0f, 4.0f, 65536.0f * 8.0f};
    const float d = divisors[below(4)];
    oracle_reduce(R, dtype, grads, n, d, 0, out);
    oracle_reduce(R, dtype, grads, n, d, 1, out);
    oracle_reduce_add(R, dtype, grads, n, d, out);
    oracle_accumulate(dtype, grads[0], n, trial & 2, out);
    int32_t ov = 0;
    double ss = 0.0;
    oracle_grad_check(out, n, &ov, &ss);
    (void)oracle_clip_coef(ss, 1.0, 1e-6);
    uint16_t *o16 = malloc(n * 2 + 1);
    oracle_encode16(out, n, 1 + (int)below(2), o16);
    for (uint64_t i = 0; i < n; ++i) {
      (void)oracle_f16_value(o16[i]);
      (void)oracle_bf16_value(o16[i]);
    }

    oracle_hyper h = {1e-3, 0.8, 0.999, 1e-8, 3e-7, (int32_t)(trial & 1), 1 + below(20), 0.5};
    float *g = random_f32(n, 1), *w = random_f32(n, 1), *m = random_f32(n, 1), *v = random_f32(n, 1);
    for (uint64_t i = 0; i < n; ++i) v[i] = v[i] < 0 ? -v[i] : v[i];
    oracle_adam_f32(n, g, w, m, v, &h);
    double *gd = malloc(n * sizeof(double) + 1), *wd = malloc(n * sizeof(double) + 1);
    double *md = malloc(n * sizeof(double) + 1), *vd = malloc(n * sizeof(double) + 1);
    for (uint64_t i = 0; i < n; ++i) {
      gd[i] = g[i];
      wd[i] = w[i];
      md[i] = m[i];
      vd[i] = v[i];
    }
    oracle_adam_f64(n, gd, wd, md, vd, &h);

    /* An owner range [begin, end) of a flat buffer, several real ranges inside
     * it, rank buffers based at grad_base and the 16-bit copy at param_base. */
    const uint64_t begin = 8 + below(40), end = begin + below(200);
    const uint64_t local_base = begin & ~7ull, grad_base = local_base, param_base = below(2) ? 0 : local_base;
    const uint64_t L = end - local_base;
    uint64_t rb[4], re[4], nr = 0, f = begin;
    while (f < end && nr < 4) {
      const uint64_t b = f + below(end - f + 1), e = b + below(end - b + 1);
      rb[nr] = b;
      re[nr] = e;
      ++nr;
      f = e;
    }
    const void *og[9];
    for (uint32_t r = 0; r < R; ++r) og[r] = random_buf(dtype, end - grad_base);
    float *ow = random_f32(L, 1), *om = random_f32(L, 1), *ovv = random_f32(L, 1);
    for (uint64_t i = 0; i < L; ++i) ovv[i] = ovv[i] < 0 ? -ovv[i] : ovv[i];
    uint16_t *p16 = malloc((end - param_base) * 2 + 1);
    float *rg = random_f32(L, 1);
    oracle_owner_step(R, dtype, og, grad_base, NULL, d, nr, rb, re, ow, om, ovv, local_base, p16,
                      1 + (int)below(2), param_base, &h);
    oracle_owner_step(0, 0, NULL, 0, rg, 1.0f, nr, rb, re, ow, om, ovv, local_base, p16, 0, param_base,
                      &h);

    for (uint32_t r = 0; r < R; ++r) {
      free((void *)grads[r]);
      free((void *)og[r]);
    }
    free(out);
    free(o16);
    free(g);
    free(w);
    free(m);
    free(v);
    free(gd);
    free(wd);
    free(md);
    free(vd);
    free(ow);
    free(om);
    free(ovv);
    free(p16);
    free(rg);
  }
  puts("oracle driver: clean");
  return 0;
}
