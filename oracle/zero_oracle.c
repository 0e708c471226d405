/*
 * ORACLE -- test infrastructure, not a product path.
 *
 * A plain, slow, scalar CPU definition of the ZeRO owner-shard optimizer step.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library.  It shares no code with the HIP library: its own
 * 16-bit decoders and encoders, its own loops, fp64 optimizer arithmetic.
 *
 * Sources ("the pages"):
 *   [ZeRO-3 docs]    DeepSpeed "ZeRO" API documentation (zero3.rst), the
 *                    stage list and the AdamW configuration examples.
 *   [ZeRO Q&A]       "How does DeepSpeed ZeRO stage 1, 2, and 3 partition
 *                    optimizer states, gradients, and parameters?", section
 *                    "Memory Footprint Reduction Matrix".
 *   [Deep dive]      "Deep dive: DeepSpeed" lesson (leetllm), sections "Count
 *                    state before choosing a stage", "Reduce first, then update
 *                    the owned slice", "Let the engine own the microstep".
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp (no fast-math), so that
 * every float operation below is one IEEE operation in the type written.
 * OpenMP only splits independent elements across threads; no result depends
 * on the thread count.  The squared-norm sum runs on one thread.
 *
 * Parity pins: every function here is pinned by CPU tests against values the
 * pages print, closed forms, library routines (numpy fp16 casts, torch bf16
 * casts, torch.optim.Adam / AdamW in float64) or exact rational arithmetic.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3 };

/* ------------------------------------------------------------------------ */
/* 16-bit formats, written from the IEEE-754 binary16 and bfloat16 layouts. */
/* ------------------------------------------------------------------------ */

/* Value of a 16-bit pattern with `mbits` mantissa bits and exponent bias
 * `bias` (binary16: 10, 15; bfloat16: 7, 127).  Exact in double. */
static double decode16(uint16_t bits, int mbits, int bias) {
  const int ebits = 15 - mbits;
  const int sign = bits >> 15;
  const int e = (bits >> mbits) & ((1 << ebits) - 1);
  const int frac = bits & ((1 << mbits) - 1);
  double mag;
  if (e == (1 << ebits) - 1) {
    mag = frac ? NAN : INFINITY;
  } else if (e == 0) {
    mag = ldexp((double)frac, 1 - bias - mbits); /* subnormal */
  } else {
    mag = ldexp((double)((1 << mbits) + frac), e - bias - mbits);
  }
  return sign ? -mag : mag;
}

/* Nearest 16-bit pattern to x, ties to even, overflow to infinity, NaN to a
 * quiet NaN.  x is a double holding an fp32 value, so the scaling by powers
 * of two and the integer rounding below are exact apart from the one
 * rounding being defined. */
static uint16_t encode16(double x, int mbits, int bias) {
  const int ebits = 15 - mbits;
  const int emax = (1 << ebits) - 2 - bias;             /* largest normal exponent */
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  const uint16_t inf = (uint16_t)(((1 << ebits) - 1) << mbits);
  if (isnan(x)) return (uint16_t)(sign | inf | (1u << (mbits - 1)));
  double a = fabs(x);
  if (isinf(a)) return (uint16_t)(sign | inf);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);           /* a = f * 2^e2 with f in [0.5, 1) */
  int e = e2 - 1;          /* a in [2^e, 2^(e+1)) */
  if (e < 1 - bias) e = 1 - bias; /* subnormal range shares the smallest quantum */
  const double q = ldexp(1.0, e - mbits);  /* spacing of representable values near a */
  double k = a / q;                          /* exact */
  double kr = floor(k);
  const double rem = k - kr;
  if (rem > 0.5 || (rem == 0.5 && fmod(kr, 2.0) != 0.0)) kr += 1.0;
  /* kr * q is the rounded magnitude; re-normalise a carry into the next binade. */
  if (kr >= (double)(2 << mbits)) {
    kr /= 2.0;
    e += 1;
  }
  if (e > emax) return (uint16_t)(sign | inf);
  if (kr < (double)(1 << mbits)) {
    /* subnormal (only possible when e is the smallest normal exponent) */
    return (uint16_t)(sign | (uint16_t)kr);
  }
  const int field = e + bias;
  return (uint16_t)(sign | (uint16_t)(field << mbits) | (uint16_t)((int)kr - (1 << mbits)));
}

uint16_t oracle_f32_to_f16(float x) { return encode16((double)x, 10, 15); }
uint16_t oracle_f32_to_bf16(float x) { return encode16((double)x, 7, 127); }
double oracle_f16_value(uint16_t b) { return decode16(b, 10, 15); }
double oracle_bf16_value(uint16_t b) { return decode16(b, 7, 127); }

void oracle_encode16(const float *x, uint64_t n, int dtype, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = dtype == OR_F16 ? oracle_f32_to_f16(x[i]) : oracle_f32_to_bf16(x[i]);
}

/* Element i of a gradient buffer, widened to fp32 (exact for all three formats). */
static float widen(const void *buf, int dtype, uint64_t i) {
  if (dtype == OR_F32) return ((const float *)buf)[i];
  const uint16_t b = ((const uint16_t *)buf)[i];
  return (float)(dtype == OR_F16 ? decode16(b, 10, 15) : decode16(b, 7, 127));
}

/* ------------------------------------------------------------------------ */
/* Owner reduce.                                                            */
/* [Deep dive] "Reduce first, then update the owned slice": the owner's     */
/* gradient is the equally weighted mean over ranks of their gradients for  */
/* the owned indices.  The sum runs in fp32, rank 0 first, starting from    */
/* +0 (or from the accumulator), then one fp32 division by the divisor.     */
/* ------------------------------------------------------------------------ */
static float reduce_one(uint32_t R, int dtype, const void *const *grads, uint64_t i, float start,
                        float divisor) {
  float s = start;
  for (uint32_t r = 0; r < R; ++r) s = s + widen(grads[r], dtype, i);
  return s / divisor;
}

/* out[i] = (start_i + g_0[i] + ... + g_{R-1}[i]) / divisor, i in [0, n);
 * start_i = out[i] if accumulate else +0. */
void oracle_reduce(uint32_t R, int dtype, const void *const *grads, uint64_t n, float divisor,
                   int accumulate, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = reduce_one(R, dtype, grads, (uint64_t)i, accumulate ? out[i] : 0.0f, divisor);
}

/* Per-backward reduce-and-accumulate ([Deep dive] "Communication volume isn't
 * elapsed time": by default ZeRO-2 and ZeRO-3 reduce and partition gradients
 * on every backward call and keep only the owned slice until the optimizer
 * step).  Each microstep's owned gradient is reduced first, rounded to fp32,
 * then added to the accumulator in fp32:
 *   out[i] = out[i] + (g_0[i] + ... + g_{R-1}[i]) / divisor. */
void oracle_reduce_add(uint32_t R, int dtype, const void *const *grads, uint64_t n, float divisor,
                       float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    const float reduced = reduce_one(R, dtype, grads, (uint64_t)i, 0.0f, divisor);
    out[i] = out[i] + reduced;
  }
}

/* Gradient accumulation in an fp32 array ([Deep dive] "Count state before
 * choosing a stage" and "Let the engine own the microstep": a four-byte
 * accumulation buffer replaces the two-byte gradient).  first != 0 starts the
 * window: acc = +0 + g; otherwise acc = acc + g.  No 1/GAS factor. */
void oracle_accumulate(int dtype, const void *g, uint64_t n, int first, float *acc) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    const float base = first ? 0.0f : acc[i];
    acc[i] = base + widen(g, dtype, (uint64_t)i);
  }
}

/* ------------------------------------------------------------------------ */
/* Overflow flag and squared norm of the owner's reduced gradient.          */
/* ------------------------------------------------------------------------ */
void oracle_grad_check(const float *g, uint64_t n, int32_t *overflow, double *sumsq) {
  int32_t flag = 0;
  double sum = 0.0, comp = 0.0; /* Neumaier compensated summation */
  for (uint64_t i = 0; i < n; ++i) {
    const double x = (double)g[i];
    if (!isfinite(x)) flag = 1;
    const double sq = x * x; /* exact: a 24-bit significand squared fits in 53 bits */
    const double t = sum + sq;
    if (fabs(sum) >= fabs(sq))
      comp += (sum - t) + sq;
    else
      comp += (sq - t) + sum;
    sum = t;
  }
  *overflow = flag;
  *sumsq = sum + comp;
}

/* Global-norm clip factor: min(1, max_norm / (sqrt(sumsq) + eps)). */
double oracle_clip_coef(double sumsq, double max_norm, double eps) {
  const double c = max_norm / (sqrt(sumsq) + eps);
  return c < 1.0 ? c : 1.0;
}

/* ------------------------------------------------------------------------ */
/* Adam / AdamW on one element, in fp64.                                    */
/* [Deep dive] "Reduce first, then update the owned slice": first moment    */
/* m = b1*m + (1-b1)*g, uncentred second moment v = b2*v + (1-b2)*g^2, both */
/* divided by (1 - b^t), step lr * mhat / (sqrt(vhat) + eps), t from 1.     */
/* [ZeRO-3 docs] configuration examples: type AdamW with weight_decay.      */
/* Decoupled decay scales the weight by (1 - lr*wd) before the Adam step;   */
/* with adamw == 0 a non-zero wd is classic L2 (wd*w added to g).           */
/* The gradient is first multiplied by the clip coefficient.                */
/* ------------------------------------------------------------------------ */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
  int32_t adamw;
  uint64_t step;
  double clip_coef;
} oracle_hyper;

static void adam_one(double g, double *w, double *m, double *v, const oracle_hyper *h) {
  double grad = g * h->clip_coef;
  double weight = *w;
  if (!h->adamw && h->weight_decay != 0.0) grad = grad + h->weight_decay * weight;
  const double first = h->beta1 * (*m) + (1.0 - h->beta1) * grad;
  const double second = h->beta2 * (*v) + (1.0 - h->beta2) * grad * grad;
  const double mhat = first / (1.0 - pow(h->beta1, (double)h->step));
  const double vhat = second / (1.0 - pow(h->beta2, (double)h->step));
  if (h->adamw) weight = weight * (1.0 - h->lr * h->weight_decay);
  weight = weight - h->lr * mhat / (sqrt(vhat) + h->eps);
  *w = weight;
  *m = first;
  *v = second;
}

/* fp64 state, fp64 gradient: the pages' scalar arithmetic. */
void oracle_adam_f64(uint64_t n, const double *g, double *w, double *m, double *v,
                     const oracle_hyper *h) {
  for (uint64_t i = 0; i < n; ++i) adam_one(g[i], &w[i], &m[i], &v[i], h);
}

/* fp32 stored state and gradient, fp64 arithmetic, one rounding on store. */
void oracle_adam_f32(uint64_t n, const float *g, float *w, float *m, float *v,
                     const oracle_hyper *h) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    double ww = w[i], mm = m[i], vv = v[i];
    adam_one((double)g[i], &ww, &mm, &vv, h);
    w[i] = (float)ww;
    m[i] = (float)mm;
    v[i] = (float)vv;
  }
}

/* ------------------------------------------------------------------------ */
/* The whole owner step over a list of flat index ranges (the owner's real  */
/* elements): reduce (or read a stored reduced gradient), Adam/AdamW, write */
/* the 16-bit compute copy of the updated master weight.                    */
/*                                                                          */
/* Indexing: flat index f lives at grads[r][f - grad_base],                 */
/* reduced_g / w / m / v [f - local_base], p16[f - param_base].             */
/* reduced_g != NULL: use it instead of the rank buffers.                    */
/* p16 == NULL or pdtype == 0: no write-back.                               */
/* ------------------------------------------------------------------------ */
void oracle_owner_step(uint32_t R, int gdtype, const void *const *grads, uint64_t grad_base,
                       const float *reduced_g, float divisor, uint64_t n_ranges,
                       const uint64_t *range_begin, const uint64_t *range_end, float *w, float *m,
                       float *v, uint64_t local_base, void *p16, int pdtype, uint64_t param_base,
                       const oracle_hyper *h) {
  for (uint64_t k = 0; k < n_ranges; ++k) {
    const int64_t b = (int64_t)range_begin[k], e = (int64_t)range_end[k];
#pragma omp parallel for schedule(static)
    for (int64_t f = b; f < e; ++f) {
      const uint64_t li = (uint64_t)f - local_base;
      float g;
      if (reduced_g) {
        g = reduced_g[li];
      } else {
        g = reduce_one(R, gdtype, grads, (uint64_t)f - grad_base, 0.0f, divisor);
      }
      double ww = w[li], mm = m[li], vv = v[li];
      adam_one((double)g, &ww, &mm, &vv, h);
      w[li] = (float)ww;
      m[li] = (float)mm;
      v[li] = (float)vv;
      if (p16 && pdtype) {
        const float wf = (float)ww;
        ((uint16_t *)p16)[(uint64_t)f - param_base] =
            pdtype == OR_F16 ? oracle_f32_to_f16(wf) : oracle_f32_to_bf16(wf);
      }
    }
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
