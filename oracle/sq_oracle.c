/*
 * sq_oracle.c -- plain, slow CPU reference for the SmoothQuant W8A8 linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this code;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header or constant with the GPU library.
 *
 * Every function is the plain definition of one step of the method, written
 * as loops in IEEE fp32 (the precision the pages' own code computes the
 * quantizer in) or fp64 where noted.  Build with -ffp-contract=off so that no
 * multiply-add is fused.  OpenMP only splits independent rows or columns.
 *
 * Steps and where they are defined:
 *   rms_rscale     RMSNorm reciprocal scale; the norm in front of q/k/v and
 *                  gate/up ("SmoothQuant and W8A8", The trick).  The pages give
 *                  no formula: r = 1/sqrt(mean(h^2) + eps), mean in fp64.
 *   act_absmax     a_j = max_t |X[t,j]| over calibration tokens ("Taming the
 *                  Outliers", System Architecture step C2 and calibrate()).
 *   weight_absmax  w_j = max_n |W[j,n]|, j = input channel ("06 -- SmoothQuant",
 *                  section 3).
 *   smooth_factor  s_j = a_j^alpha / w_j^(1-alpha), clamped at 1e-5
 *                  ("06 -- SmoothQuant", section 3; "SmoothQuant and W8A8",
 *                  The trick; "Taming the Outliers", calibrate()).
 *   fold           gamma'_j = gamma_j / s_j and W^[j,n] = s_j * W[j,n]
 *                  ("06 -- SmoothQuant", sections 2 and 7).
 *   quant_weight   one symmetric scale per output channel, Delta = amax/127,
 *                  codes = round-half-even(W^/Delta) ("06 -- SmoothQuant",
 *                  section 7; "Taming the Outliers", the quantization equation).
 *   quant_act      one dynamic symmetric scale per token, same quantizer
 *                  ("06 -- SmoothQuant", section 7).
 *   static_scale   one activation step for the whole tensor, from the
 *                  calibration tokens' maximum ("SmoothQuant and W8A8", One
 *                  layer, measured; "06 -- SmoothQuant", section 7: per-token
 *                  or per-tensor activation scales).
 *   quant_act_static  the same quantizer with that fixed step: values past the
 *                  calibrated maximum clip to +-127 ("SmoothQuant and W8A8",
 *                  Gotchas: a static scale clips what calibration never saw).
 *   e4m3_*, *_fp8  the FP8 E4M3 variant of the same path ("SmoothQuant and
 *                  W8A8", One layer, measured: weights per output channel,
 *                  activations per token, in FP8 E4M3): step = amax / 448
 *                  (448 is E4M3's largest finite value), code = the E4M3
 *                  value nearest fp32(x / step), ties to even; products summed
 *                  exactly (fp64) in place of the int64 sum.
 *   ln_*           the LayerNorm form of the smoothed norm ("SmoothQuant:
 *                  Weight-Only vs W8A8", Integration with Transformers: S^-1
 *                  folds into the LayerNorm's gamma and beta).  The pages give
 *                  no formula: mean and variance over the row in fp64,
 *                  r = 1/sqrt(var + eps), LN(h) = fp32(fp32(fp32(h - mean) * r)
 *                  * gamma) + beta, every step rounded to fp32.
 *   fold_prev      1/s folded into the output columns of the linear in front
 *                  ("06 -- SmoothQuant", section 7).
 *   int_gemm       acc = sum_k q[t,k] * qw[n,k] in int64 ("06 -- SmoothQuant",
 *                  section 7: INT8 x INT8 -> INT32).
 *   epilogue       y = (Delta_t * Delta_n) * acc + bias ("06 -- SmoothQuant",
 *                  section 7; "Taming the Outliers", step I6).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* element i of an fp32 (is_bf16 == 0) or bf16 (is_bf16 == 1) array */
static float elem(const void *p, int is_bf16, int64_t i) {
  return is_bf16 ? bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

/* symmetric INT8 code of the quotient v = x / Delta: nearest integer, ties to
   even (the default rounding mode), clamped to [-127, 127]. */
static int8_t code_of(float v) {
  float r = nearbyintf(v);
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

int oracle_version(void) { return 1; }

/* threads an OpenMP parallel region of the oracle uses */
int oracle_max_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

/* r[t] = fp32( 1 / sqrt( (sum_k h[t,k]^2) / K + eps ) ), sum and root in fp64 */
void oracle_rms_rscale(const void *h, int is_bf16, int64_t T, int64_t K, int64_t ld,
                       float eps, float *r) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double v = (double)elem(h, is_bf16, t * ld + k);
      acc += v * v;
    }
    double ms = acc / (double)K;
    r[t] = (float)(1.0 / sqrt(ms + (double)eps));
  }
}

/* a[j] = max_t |x[t,j]|; in norm mode the calibration activation is the
   linear's input x = fp32(fp32(h * r_t) * gamma_j).  accumulate != 0 keeps a
   running maximum across calls. */
void oracle_act_absmax(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld,
                       int norm, const float *gamma, float eps, int accumulate, float *a) {
  float *r = NULL;
  if (norm) {
    r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    oracle_rms_rscale(x, is_bf16, T, K, ld, eps, r);
  }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < K; ++j) {
    float m = accumulate ? a[j] : 0.0f;
    for (int64_t t = 0; t < T; ++t) {
      float v = elem(x, is_bf16, t * ld + j);
      if (norm) {
        float hr = v * r[t];
        v = hr * (gamma ? gamma[j] : 1.0f);
      }
      m = fmaxf(m, fabsf(v));
    }
    a[j] = m;
  }
  free(r);
}

/* wmax[j] = max_n |W[j,n]|, W row-major [K,N] with leading dimension ld */
void oracle_weight_absmax(const void *w, int is_bf16, int64_t K, int64_t N, int64_t ld,
                          float *wmax) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < K; ++j) {
    float m = 0.0f;
    for (int64_t n = 0; n < N; ++n) m = fmaxf(m, fabsf(elem(w, is_bf16, j * ld + n)));
    wmax[j] = m;
  }
}

/* s[j] = max( fp32( a_j^alpha / w_j^(1-alpha) ), 1e-5 ), quotient in fp64;
   an all-zero weight row (w_j == 0) gets s_j = 1. */
void oracle_smooth_factor(const float *a, const float *wmax, int64_t K, float alpha,
                          float *s) {
  double al = (double)alpha;
  for (int64_t j = 0; j < K; ++j) {
    if (wmax[j] == 0.0f) {
      s[j] = 1.0f;
      continue;
    }
    double q = pow((double)a[j], al) / pow((double)wmax[j], 1.0 - al);
    float f = (float)q;
    s[j] = f < 1e-5f ? 1e-5f : f;
  }
}

/* gamma_out[j] = gamma_j / s_j (gamma NULL -> 1); w_hat[j,n] = W[j,n] * s_j
   (fp32, row-major [K,N], leading dimension N); either output may be NULL. */
void oracle_fold(const float *s, int64_t K, const float *gamma, float *gamma_out,
                 const void *w, int is_bf16, int64_t N, int64_t ldw, float *w_hat) {
  if (gamma_out)
    for (int64_t j = 0; j < K; ++j) gamma_out[j] = (gamma ? gamma[j] : 1.0f) / s[j];
  if (w_hat && w) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < K; ++j)
      for (int64_t n = 0; n < N; ++n) w_hat[j * N + n] = elem(w, is_bf16, j * ldw + n) * s[j];
  }
}

/* Per-output-channel symmetric INT8 of W^ [K,N] (fp32, leading dimension ld):
   w_scale[n] = max_j |W^[j,n]| / 127;  qw[n*K + j] = code(W^[j,n] / w_scale[n]).
   The codes are stored transposed, [N,K] with K contiguous. */
void oracle_quant_weight(const float *w_hat, int64_t K, int64_t N, int64_t ld, int8_t *qw,
                         float *w_scale) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    float amax = 0.0f;
    for (int64_t j = 0; j < K; ++j) amax = fmaxf(amax, fabsf(w_hat[j * ld + n]));
    float d = amax / 127.0f;
    w_scale[n] = d;
    for (int64_t j = 0; j < K; ++j)
      qw[n * K + j] = (d == 0.0f) ? (int8_t)0 : code_of(w_hat[j * ld + n] / d);
  }
}

/* Per-token dynamic symmetric INT8 of the smoothed activation.
     norm == 0:  x^[t,k] = fp32(x[t,k] * gamma_f[k])
     norm == 1:  x^[t,k] = fp32(fp32(h[t,k] * r_t) * gamma_f[k]),
                 r_t from r_in if given, else computed as in oracle_rms_rscale
   gamma_f NULL means 1.  x_scale[t] = max_k |x^| / 127; q = code(x^ / x_scale).
   r_out (nullable) receives the r_t used. */
void oracle_quant_act(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld, int norm,
                      const float *r_in, float eps, const float *gamma_f, int8_t *q,
                      float *x_scale, float *r_out) {
  float *r = NULL;
  if (norm) {
    r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    if (r_in)
      memcpy(r, r_in, sizeof(float) * (size_t)T);
    else
      oracle_rms_rscale(x, is_bf16, T, K, ld, eps, r);
    if (r_out) memcpy(r_out, r, sizeof(float) * (size_t)T);
  }
#pragma omp parallel
  {
    float *xh = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      float amax = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        float v = elem(x, is_bf16, t * ld + k);
        if (norm) v = v * r[t];
        xh[k] = v * (gamma_f ? gamma_f[k] : 1.0f);
        amax = fmaxf(amax, fabsf(xh[k]));
      }
      float d = amax / 127.0f;
      x_scale[t] = d;
      for (int64_t k = 0; k < K; ++k)
        q[t * K + k] = (d == 0.0f) ? (int8_t)0 : code_of(xh[k] / d);
    }
    free(xh);
  }
  free(r);
}

/* x^[t,k] of one element, as the activation quantizer forms it */
static float smoothed(const void *x, int is_bf16, int64_t i, int norm, float r, const float *gamma_f,
                      int64_t k) {
  float v = elem(x, is_bf16, i);
  if (norm) v = v * r;
  return v * (gamma_f ? gamma_f[k] : 1.0f);
}

/* max over every calibration token t and channel k of |x^[t,k]|, with x^
   formed exactly as in oracle_quant_act */
static float static_amax(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld, int norm,
                         float eps, const float *gamma_f) {
  float *r = NULL;
  if (norm) {
    r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    oracle_rms_rscale(x, is_bf16, T, K, ld, eps, r);
  }
  float amax = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : amax)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t k = 0; k < K; ++k)
      amax = fmaxf(amax, fabsf(smoothed(x, is_bf16, t * ld + k, norm, norm ? r[t] : 1.0f,
                                        gamma_f, k)));
  free(r);
  return amax;
}

/* x^ of every element, as the activation quantizer forms it (r_in: the RMSNorm
   factors to use in norm mode, NULL: computed as in oracle_rms_rscale); out is
   fp32 [T, K].  GPTQ's Hessian is taken over these values. */
void oracle_smoothed_act(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld, int norm,
                         const float *r_in, float eps, const float *gamma_f, float *out) {
  float *r = NULL;
  if (norm) {
    r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    if (r_in)
      memcpy(r, r_in, sizeof(float) * (size_t)T);
    else
      oracle_rms_rscale(x, is_bf16, T, K, ld, eps, r);
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t k = 0; k < K; ++k)
      out[t * K + k] = smoothed(x, is_bf16, t * ld + k, norm, norm ? r[t] : 1.0f, gamma_f, k);
  free(r);
}

/* Static per-tensor step: Delta = fp32( max over every calibration token t and
   channel k of |x^[t,k]| / 127 ). */
float oracle_static_scale(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld, int norm,
                          float eps, const float *gamma_f) {
  return static_amax(x, is_bf16, T, K, ld, norm, eps, gamma_f) / 127.0f;
}

/* Static quantization with a fixed step `delta` for every token:
   q = code(x^ / delta), clamped to [-127, 127] (code_of), so values past the
   calibrated maximum clip; x_scale[t] = delta.  delta == 0 gives codes 0.
   r_in / r_out as in oracle_quant_act. */
void oracle_quant_act_static(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld,
                             int norm, const float *r_in, float eps, const float *gamma_f,
                             float delta, int8_t *q, float *x_scale, float *r_out) {
  float *r = NULL;
  if (norm) {
    r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    if (r_in)
      memcpy(r, r_in, sizeof(float) * (size_t)T);
    else
      oracle_rms_rscale(x, is_bf16, T, K, ld, eps, r);
    if (r_out) memcpy(r_out, r, sizeof(float) * (size_t)T);
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    x_scale[t] = delta;
    for (int64_t k = 0; k < K; ++k) {
      float v = smoothed(x, is_bf16, t * ld + k, norm, norm ? r[t] : 1.0f, gamma_f, k);
      q[t * K + k] = (delta == 0.0f) ? (int8_t)0 : code_of(v / delta);
    }
  }
  free(r);
}

/* ---------------------------------------------------------------------------
 * FP8 E4M3 (the OCP "fn" encoding): sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; no infinities; 0x7F / 0xFF are NaN, so the largest finite
 * magnitude is 1.75 * 2^8 = 448.  Exponent field 0 holds the subnormals
 * m * 2^-9, m = 0..7.
 * ------------------------------------------------------------------------- */

/* value of an E4M3 code (NaN codes decode to NaN) */
float oracle_e4m3_decode(uint8_t c) {
  const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return sign ? -v : v;
}

/* nearest E4M3 value to a finite v, ties to even (even mantissa field);
   magnitudes past 448 saturate to 448 (the quantizers never produce them:
   their quotients are at most 448 up to one fp32 rounding) */
uint8_t oracle_e4m3_encode(float v) {
  const uint8_t sign = (v < 0.0f || (v == 0.0f && signbit(v))) ? 0x80 : 0x00;
  const double a = fabs((double)v);
  if (a == 0.0) return sign;
  if (a >= 448.0) return sign | 0x7E;
  int e;
  frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
  int ex = e - 1;          /* a in [2^ex, 2^(ex+1)) */
  if (ex < -6) {           /* subnormal range: multiples of 2^-9 */
    const double q = nearbyint(a * 512.0);      /* exact scaling, ties to even */
    return sign | (uint8_t)q;                   /* q = 8 is the smallest normal, 0x08 */
  }
  const double f = nearbyint((a / ldexp(1.0, ex) - 1.0) * 8.0);   /* 0..8 */
  int m = (int)f;
  if (m == 8) { m = 0; ex += 1; }
  if (ex > 8 || (ex == 8 && m == 7)) return sign | 0x7E;
  return sign | (uint8_t)(((ex + 7) << 3) | m);
}

void oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_array(const uint8_t *c, int64_t n, float *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* Per-output-channel E4M3 of W^ [K,N]: w_scale[n] = max_j |W^[j,n]| / 448,
   code = e4m3(fp32(W^[j,n] / w_scale[n])), stored transposed [N,K]. */
void oracle_quant_weight_fp8(const float *w_hat, int64_t K, int64_t N, int64_t ld, uint8_t *qw,
                             float *w_scale) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    float amax = 0.0f;
    for (int64_t j = 0; j < K; ++j) amax = fmaxf(amax, fabsf(w_hat[j * ld + n]));
    float d = amax / 448.0f;
    w_scale[n] = d;
    for (int64_t j = 0; j < K; ++j)
      qw[n * K + j] = (d == 0.0f) ? (uint8_t)0 : oracle_e4m3_encode(w_hat[j * ld + n] / d);
  }
}

/* Per-token E4M3 of the smoothed activation, x^ formed as in
   oracle_quant_act: x_scale[t] = max_k |x^| / 448, code = e4m3(fp32(x^ / x_scale[t])). */
void oracle_quant_act_fp8(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld, int norm,
                          const float *r_in, float eps, const float *gamma_f, uint8_t *q,
                          float *x_scale, float *r_out) {
  float *r = NULL;
  if (norm) {
    r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    if (r_in)
      memcpy(r, r_in, sizeof(float) * (size_t)T);
    else
      oracle_rms_rscale(x, is_bf16, T, K, ld, eps, r);
    if (r_out) memcpy(r_out, r, sizeof(float) * (size_t)T);
  }
#pragma omp parallel
  {
    float *xh = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      float amax = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        xh[k] = smoothed(x, is_bf16, t * ld + k, norm, norm ? r[t] : 1.0f, gamma_f, k);
        amax = fmaxf(amax, fabsf(xh[k]));
      }
      float d = amax / 448.0f;
      x_scale[t] = d;
      for (int64_t k = 0; k < K; ++k)
        q[t * K + k] = (d == 0.0f) ? (uint8_t)0 : oracle_e4m3_encode(xh[k] / d);
    }
    free(xh);
  }
  free(r);
}

/* Static per-tensor E4M3 step: Delta = fp32( max over every calibration token
   and channel of |x^| / 448 ). */
float oracle_static_scale_fp8(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld,
                              int norm, float eps, const float *gamma_f) {
  return static_amax(x, is_bf16, T, K, ld, norm, eps, gamma_f) / 448.0f;
}

/* Static E4M3 quantization with a fixed step `delta` for every token:
   code = e4m3(clip(fp32(x^ / delta), -448, 448)), so values past the
   calibrated maximum clip to the largest finite magnitude; x_scale[t] = delta;
   delta == 0 gives codes 0.  r_in / r_out as in oracle_quant_act. */
void oracle_quant_act_static_fp8(const void *x, int is_bf16, int64_t T, int64_t K, int64_t ld,
                                 int norm, const float *r_in, float eps, const float *gamma_f,
                                 float delta, uint8_t *q, float *x_scale, float *r_out) {
  float *r = NULL;
  if (norm) {
    r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
    if (r_in)
      memcpy(r, r_in, sizeof(float) * (size_t)T);
    else
      oracle_rms_rscale(x, is_bf16, T, K, ld, eps, r);
    if (r_out) memcpy(r_out, r, sizeof(float) * (size_t)T);
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    x_scale[t] = delta;
    for (int64_t k = 0; k < K; ++k) {
      float v = smoothed(x, is_bf16, t * ld + k, norm, norm ? r[t] : 1.0f, gamma_f, k);
      if (delta == 0.0f) {
        q[t * K + k] = 0;
        continue;
      }
      float y = v / delta;
      if (y > 448.0f) y = 448.0f;
      if (y < -448.0f) y = -448.0f;
      q[t * K + k] = oracle_e4m3_encode(y);
    }
  }
  free(r);
}

/* acc[t,n] = sum_k e4m3(q[t,k]) * e4m3(qw[n,k]), summed in fp64 (every product
   and every partial sum of 4-bit-significand values is exact there for
   K <= 65536), returned in fp64 [T,N]. */
void oracle_gemm_fp8(const uint8_t *q, const uint8_t *qw, int64_t T, int64_t K, int64_t N,
                     double *acc) {
  double lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = (double)oracle_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += lut[q[t * K + k]] * lut[qw[n * K + k]];
      acc[t * N + n] = s;
    }
}

/* ---------------------------------------------------------------------------
 * LayerNorm form ("SmoothQuant: Weight-Only vs W8A8", Integration with
 * Transformers) and the fold into the previous linear ("06 -- SmoothQuant",
 * section 7).
 * ------------------------------------------------------------------------- */

/* Row statistics: mean[t] = fp32(mu), r[t] = fp32(1 / sqrt(var + eps)) with
   mu = (sum_k h) / K and var = (sum_k (h - mu)^2) / K, both sums in fp64 in
   index order (mu kept in fp64 for the variance). */
void oracle_ln_stats(const void *h, int is_bf16, int64_t T, int64_t K, int64_t ld, float eps,
                     float *mean, float *r) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double s1 = 0.0;
    for (int64_t k = 0; k < K; ++k) s1 += (double)elem(h, is_bf16, t * ld + k);
    const double mu = s1 / (double)K;
    double s2 = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double d = (double)elem(h, is_bf16, t * ld + k) - mu;
      s2 += d * d;
    }
    mean[t] = (float)mu;
    r[t] = (float)(1.0 / sqrt(s2 / (double)K + (double)eps));
  }
}

/* one LayerNorm output element with per-channel gamma, beta (NULL: 1, 0) */
static float ln_elem(float h, float m, float r, const float *gamma, const float *beta, int64_t k) {
  const float c = h - m;
  const float n = c * r;
  const float g = n * (gamma ? gamma[k] : 1.0f);
  return g + (beta ? beta[k] : 0.0f);
}

/* a[j] = max_t |LN(h)[t,j]| with the norm's own gamma and beta: the
   calibration absmax of the linear's input in LayerNorm mode. */
void oracle_act_absmax_ln(const void *h, int is_bf16, int64_t T, int64_t K, int64_t ld,
                          const float *gamma, const float *beta, float eps, float *a) {
  float *m = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  float *r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  oracle_ln_stats(h, is_bf16, T, K, ld, eps, m, r);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < K; ++j) {
    float mx = 0.0f;
    for (int64_t t = 0; t < T; ++t)
      mx = fmaxf(mx, fabsf(ln_elem(elem(h, is_bf16, t * ld + j), m[t], r[t], gamma, beta, j)));
    a[j] = mx;
  }
  free(m);
  free(r);
}

/* gamma'_j = fp32(gamma_j / s_j), beta'_j = fp32(beta_j / s_j) (NULL gamma:
   1; NULL beta: beta' = 0) */
void oracle_fold_ln(const float *s, int64_t K, const float *gamma, const float *beta,
                    float *gamma_out, float *beta_out) {
  for (int64_t j = 0; j < K; ++j) {
    gamma_out[j] = (gamma ? gamma[j] : 1.0f) / s[j];
    beta_out[j] = (beta ? beta[j] : 0.0f) / s[j];
  }
}

/* Per-token dynamic symmetric INT8 of the smoothed LayerNorm output
   x^ = LN(h; gamma_f, beta_f); mean/r from mean_in/r_in if given, else as in
   oracle_ln_stats; mean_out/r_out (nullable) receive them. */
void oracle_quant_act_ln(const void *h, int is_bf16, int64_t T, int64_t K, int64_t ld,
                         const float *mean_in, const float *r_in, float eps,
                         const float *gamma_f, const float *beta_f, int8_t *q, float *x_scale,
                         float *mean_out, float *r_out) {
  float *m = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  float *r = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  oracle_ln_stats(h, is_bf16, T, K, ld, eps, m, r);
  if (mean_in) memcpy(m, mean_in, sizeof(float) * (size_t)T);
  if (r_in) memcpy(r, r_in, sizeof(float) * (size_t)T);
  if (mean_out) memcpy(mean_out, m, sizeof(float) * (size_t)T);
  if (r_out) memcpy(r_out, r, sizeof(float) * (size_t)T);
#pragma omp parallel
  {
    float *xh = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      float amax = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        xh[k] = ln_elem(elem(h, is_bf16, t * ld + k), m[t], r[t], gamma_f, beta_f, k);
        amax = fmaxf(amax, fabsf(xh[k]));
      }
      const float d = amax / 127.0f;
      x_scale[t] = d;
      for (int64_t k = 0; k < K; ++k)
        q[t * K + k] = (d == 0.0f) ? (int8_t)0 : code_of(xh[k] / d);
    }
    free(xh);
  }
  free(m);
  free(r);
}

/* The previous linear's output channel j is the next linear's input channel
   j: w_out[i, j] = fp32(W_prev[i, j] / s_j) for W_prev [K_prev, K] (leading
   dimension ld, output [K_prev, K] dense) and bias_out[j] = fp32(b_j / s_j)
   (bias NULL: bias_out untouched). */
void oracle_fold_prev(const float *s, int64_t K, const void *w_prev, int is_bf16, int64_t K_prev,
                      int64_t ld, float *w_out, const float *bias, float *bias_out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < K_prev; ++i)
    for (int64_t j = 0; j < K; ++j) w_out[i * K + j] = elem(w_prev, is_bf16, i * ld + j) / s[j];
  if (bias && bias_out)
    for (int64_t j = 0; j < K; ++j) bias_out[j] = bias[j] / s[j];
}

/* acc[t,n] = sum_k q[t,k] * qw[n,k] in int64; q is [T,K], qw is [N,K].
   Returns the number of sums that do not fit in int32 (those are clamped). */
int64_t oracle_int_gemm(const int8_t *q, const int8_t *qw, int64_t T, int64_t K, int64_t N,
                        int32_t *acc) {
  int64_t overflow = 0;
#pragma omp parallel for schedule(static) reduction(+ : overflow)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t n = 0; n < N; ++n) {
      int64_t s = 0;
      for (int64_t k = 0; k < K; ++k) s += (int64_t)q[t * K + k] * (int64_t)qw[n * K + k];
      if (s > INT32_MAX) { s = INT32_MAX; ++overflow; }
      if (s < INT32_MIN) { s = INT32_MIN; ++overflow; }
      acc[t * N + n] = (int32_t)s;
    }
  }
  return overflow;
}

/* y[t,n] = fp32( fp32(x_scale[t] * w_scale[n]) * fp32(acc[t,n]) ) + bias[n]
   (bias NULL -> no add), fp32 out [T,N]. */
void oracle_epilogue(const int32_t *acc, const float *x_scale, const float *w_scale,
                     const float *bias, int64_t T, int64_t N, float *y) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n) {
      float sc = x_scale[t] * w_scale[n];
      float v = sc * (float)acc[t * N + n];
      y[t * N + n] = bias ? v + bias[n] : v;
    }
}

/* fp32 -> bf16 bits, round to nearest, ties to even (finite inputs) */
void oracle_f32_to_bf16(const float *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &x[i], sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
  }
}
