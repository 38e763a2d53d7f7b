/*
 * sanitize_driver.c -- runs every oracle step once on small, exactly sized
 * heap buffers (ragged shapes, bf16 and fp32, norm and plain modes) so that a
 * build with -fsanitize=address,undefined catches any out-of-bounds access or
 * undefined arithmetic in the oracle.  Test infrastructure: built and run by
 * tests/test_oracle_sanitizers.py only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_rms_rscale(const void *, int, int64_t, int64_t, int64_t, float, float *);
void oracle_act_absmax(const void *, int, int64_t, int64_t, int64_t, int, const float *, float,
                       int, float *);
void oracle_weight_absmax(const void *, int, int64_t, int64_t, int64_t, float *);
void oracle_smooth_factor(const float *, const float *, int64_t, float, float *);
void oracle_fold(const float *, int64_t, const float *, float *, const void *, int, int64_t,
                 int64_t, float *);
void oracle_quant_weight(const float *, int64_t, int64_t, int64_t, int8_t *, float *);
void oracle_quant_act(const void *, int, int64_t, int64_t, int64_t, int, const float *, float,
                      const float *, int8_t *, float *, float *);
void oracle_smoothed_act(const void *, int, int64_t, int64_t, int64_t, int, const float *, float,
                         const float *, float *);
float oracle_static_scale(const void *, int, int64_t, int64_t, int64_t, int, float,
                          const float *);
void oracle_quant_act_static(const void *, int, int64_t, int64_t, int64_t, int, const float *,
                             float, const float *, float, int8_t *, float *, float *);
void oracle_e4m3_encode_array(const float *, int64_t, uint8_t *);
void oracle_e4m3_decode_array(const uint8_t *, int64_t, float *);
void oracle_quant_weight_fp8(const float *, int64_t, int64_t, int64_t, uint8_t *, float *);
void oracle_quant_act_fp8(const void *, int, int64_t, int64_t, int64_t, int, const float *,
                          float, const float *, uint8_t *, float *, float *);
float oracle_static_scale_fp8(const void *, int, int64_t, int64_t, int64_t, int, float,
                              const float *);
void oracle_quant_act_static_fp8(const void *, int, int64_t, int64_t, int64_t, int,
                                 const float *, float, const float *, float, uint8_t *, float *,
                                 float *);
void oracle_gemm_fp8(const uint8_t *, const uint8_t *, int64_t, int64_t, int64_t, double *);
void oracle_ln_stats(const void *, int, int64_t, int64_t, int64_t, float, float *, float *);
void oracle_act_absmax_ln(const void *, int, int64_t, int64_t, int64_t, const float *,
                          const float *, float, float *);
void oracle_fold_ln(const float *, int64_t, const float *, const float *, float *, float *);
void oracle_quant_act_ln(const void *, int, int64_t, int64_t, int64_t, const float *,
                         const float *, float, const float *, const float *, int8_t *, float *,
                         float *, float *);
void oracle_fold_prev(const float *, int64_t, const void *, int, int64_t, int64_t, float *,
                      const float *, float *);
int64_t oracle_int_gemm(const int8_t *, const int8_t *, int64_t, int64_t, int64_t, int32_t *);
void oracle_epilogue(const int32_t *, const float *, const float *, const float *, int64_t,
                     int64_t, float *);
void oracle_f32_to_bf16(const float *, int64_t, uint16_t *);

static void *xalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) exit(2);
  return p;
}

static float frand(uint64_t *s) {   /* xorshift64*, in [-1, 1) */
  *s ^= *s >> 12;
  *s ^= *s << 25;
  *s ^= *s >> 27;
  return (float)((*s * 2685821657736338717ULL) >> 40) / (float)(1 << 24) * 2.0f - 1.0f;
}

static void run(int64_t T, int64_t K, int64_t N, int bf16, uint64_t seed) {
  uint64_t s = seed;
  const int64_t ld = K + 3;           /* a leading dimension past K */
  float *xf = xalloc(sizeof(float) * T * ld), *wf = xalloc(sizeof(float) * K * N);
  for (int64_t i = 0; i < T * ld; ++i) xf[i] = frand(&s) * (i % 7 == 0 ? 30.0f : 1.0f);
  for (int64_t i = 0; i < K * N; ++i) wf[i] = frand(&s) * 0.05f;
  uint16_t *xb = xalloc(sizeof(uint16_t) * T * ld), *wb = xalloc(sizeof(uint16_t) * K * N);
  oracle_f32_to_bf16(xf, T * ld, xb);
  oracle_f32_to_bf16(wf, K * N, wb);
  const void *x = bf16 ? (const void *)xb : (const void *)xf;
  const void *w = bf16 ? (const void *)wb : (const void *)wf;
  float *g = xalloc(sizeof(float) * K), *b = xalloc(sizeof(float) * K);
  for (int64_t k = 0; k < K; ++k) {
    g[k] = 0.5f + 0.5f * (frand(&s) + 1.0f);
    b[k] = 0.1f * frand(&s);
  }
  float *r = xalloc(sizeof(float) * T), *m = xalloc(sizeof(float) * T);
  float *a = xalloc(sizeof(float) * K), *wm = xalloc(sizeof(float) * K), *sf = xalloc(sizeof(float) * K);
  float *gp = xalloc(sizeof(float) * K), *bp = xalloc(sizeof(float) * K);
  float *what = xalloc(sizeof(float) * K * N), *ws = xalloc(sizeof(float) * N);
  float *xs = xalloc(sizeof(float) * T), *xh = xalloc(sizeof(float) * T * K);
  int8_t *qw = xalloc((size_t)N * K), *q = xalloc((size_t)T * K);
  uint8_t *qw8 = xalloc((size_t)N * K), *q8 = xalloc((size_t)T * K);
  int32_t *acc = xalloc(sizeof(int32_t) * T * N);
  double *acc8 = xalloc(sizeof(double) * T * N);
  float *y = xalloc(sizeof(float) * T * N), *wout = xalloc(sizeof(float) * K * K);
  float *dec = xalloc(sizeof(float) * T * K);

  for (int norm = 0; norm < 2; ++norm) {
    oracle_rms_rscale(x, bf16, T, K, ld, 1e-6f, r);
    oracle_act_absmax(x, bf16, T, K, ld, norm, g, 1e-6f, 0, a);
    oracle_act_absmax(x, bf16, T, K, ld, norm, g, 1e-6f, 1, a);
    oracle_weight_absmax(w, bf16, K, N, N, wm);
    oracle_smooth_factor(a, wm, K, 0.5f, sf);
    oracle_fold(sf, K, norm ? g : NULL, gp, w, bf16, N, N, what);
    oracle_quant_weight(what, K, N, N, qw, ws);
    oracle_quant_act(x, bf16, T, K, ld, norm, NULL, 1e-6f, gp, q, xs, norm ? r : NULL);
    oracle_smoothed_act(x, bf16, T, K, ld, norm, NULL, 1e-6f, gp, xh);
    const float d = oracle_static_scale(x, bf16, T, K, ld, norm, 1e-6f, gp);
    oracle_quant_act_static(x, bf16, T, K, ld, norm, NULL, 1e-6f, gp, d, q, xs, r);
    oracle_int_gemm(q, qw, T, K, N, acc);
    oracle_epilogue(acc, xs, ws, b, T, N, y);
    oracle_quant_weight_fp8(what, K, N, N, qw8, ws);
    oracle_quant_act_fp8(x, bf16, T, K, ld, norm, NULL, 1e-6f, gp, q8, xs, r);
    const float d8 = oracle_static_scale_fp8(x, bf16, T, K, ld, norm, 1e-6f, gp);
    oracle_quant_act_static_fp8(x, bf16, T, K, ld, norm, NULL, 1e-6f, gp, d8, q8, xs, r);
    oracle_gemm_fp8(q8, qw8, T, K, N, acc8);
    oracle_e4m3_decode_array(q8, T * K, dec);
    oracle_e4m3_encode_array(dec, T * K, q8);
  }
  oracle_ln_stats(x, bf16, T, K, ld, 1e-5f, m, r);
  oracle_act_absmax_ln(x, bf16, T, K, ld, g, b, 1e-5f, a);
  oracle_fold_ln(sf, K, g, b, gp, bp);
  oracle_quant_act_ln(x, bf16, T, K, ld, NULL, NULL, 1e-5f, gp, bp, q, xs, m, r);
  oracle_quant_act_ln(x, bf16, T, K, ld, m, r, 1e-5f, gp, bp, q, xs, NULL, NULL);
  oracle_fold_prev(sf, K, x, bf16, T < K ? T : K, ld, wout, b, bp);

  free(xf); free(wf); free(xb); free(wb); free(g); free(b); free(r); free(m); free(a);
  free(wm); free(sf); free(gp); free(bp); free(what); free(ws); free(xs); free(xh); free(qw);
  free(q); free(qw8); free(q8); free(acc); free(acc8); free(y); free(wout); free(dec);
}

int main(void) {
  const int64_t shapes[][3] = {{1, 64, 8}, {7, 128, 24}, {33, 192, 40}, {64, 256, 72}};
  for (int i = 0; i < 4; ++i)
    for (int bf16 = 0; bf16 < 2; ++bf16)
      run(shapes[i][0], shapes[i][1], shapes[i][2], bf16, 0x9E3779B97F4A7C15ULL + i * 2 + bf16);
  printf("oracle sanitizer run ok\n");
  return 0;
}
