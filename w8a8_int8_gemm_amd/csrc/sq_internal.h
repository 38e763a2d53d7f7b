// sq_internal.h -- launchers of the gfx950 kernels, called by the C ABI layer
// (sq_w8a8.hip) after it has validated the arguments.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace sqk {

// k_calib.hip
void launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
// out[c] = max(out[c], max_r |m[r,c] * row_scale[r]| / qdiv) (row_scale NULL = 1)
void launch_col_absmax(const void* m, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                       const float* row_scale, float qdiv, float* out, hipStream_t st);
void launch_rms_act_absmax(const void* h, bool bf16, int64_t rows, int64_t K, int64_t ld,
                           const float* gamma, float eps, float* out, hipStream_t st);
void launch_ln_act_absmax(const void* h, bool bf16, int64_t rows, int64_t K, int64_t ld,
                          const float* gamma, const float* beta, float eps, float* out,
                          hipStream_t st);
void launch_wrow_absmax_s(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                          const float* a, float alpha, float* wmax, float* s, hipStream_t st);

// k_weight.hip
void launch_fold_gamma(const float* s, const float* gamma, float* gout, int64_t K, hipStream_t st);
void launch_fold_w(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld, const float* s,
                   float* wout, hipStream_t st);
void launch_fold_beta(const float* s, const float* beta, float* bout, int64_t K, hipStream_t st);
void launch_fold_prev(const void* w, bool bf16, int64_t Kp, int64_t K, int64_t ld, const float* s,
                      float* wout, int64_t ldo, hipStream_t st);
// one launch: steps and codes of a bf16 weight with K <= 4096 (quant_weight_strip_ok)
bool quant_weight_strip_ok(bool bf16, int64_t K, int64_t N);
void launch_quant_weight_strip(const void* w, int64_t K, int64_t N, int64_t ld, const float* s,
                               float* wscale, int8_t* wq, hipStream_t st);
void launch_quant_weight_strip_fp8(const void* w, int64_t K, int64_t N, int64_t ld,
                                   const float* s, float* wscale, uint8_t* wq, hipStream_t st);
void launch_quant_weight_t(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                           const float* s, const float* wscale, int8_t* wq, hipStream_t st);
void launch_quant_weight_t_fp8(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                               const float* s, const float* wscale, uint8_t* wq, hipStream_t st);

// k_actquant.hip
// static_scale NULL: per-token step; else the device scalar per-tensor step
void launch_quant_act(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld, bool norm,
                      const float* gamma_f, float eps, const float* static_scale, int8_t* xq,
                      float* xscale, float* rrow, hipStream_t st);
// FP8 E4M3 codes; static_scale NULL: per-token step amax / 448, else the
// device scalar per-tensor step (quotients clip to +-448)
void launch_quant_act_fp8(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld, bool norm,
                          const float* gamma_f, float eps, const float* static_scale, uint8_t* xq,
                          float* xscale, float* rrow, hipStream_t st);
// out[0] = max_j fp32(a[j] * |gamma_f[j]|) / qmax
// LayerNorm form, per-token INT8; gamma_f and beta_f non-NULL
void launch_quant_act_ln(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld,
                         const float* gamma_f, const float* beta_f, float eps, int8_t* xq,
                         float* xscale, float* mrow, float* rrow, hipStream_t st);
void launch_static_scale(const float* a, const float* gamma_f, int64_t K, float qmax, float* out,
                         hipStream_t st);

// k_gptq.hip: GPTQ rounding of W^ = W * s with the Hessian of the calibration x^
size_t gptq_workspace_bytes(int64_t T, int64_t K, int64_t N);
void launch_gptq(const void* x, bool xbf16, int64_t T, int64_t ldx, bool norm,
                 const float* gamma_f, float eps, const void* w, bool wbf16, int64_t K, int64_t N,
                 int64_t ldw, const float* s, float damp, int8_t* wq, float* wscale,
                 float* rrow_out, void* workspace, hipStream_t st);

// compute units of the current device (k_gemm.hip)
int cu_count();

// k_gemm.hip / k_gemm_decode.hip; out: 0 = bf16, 1 = fp32, 2 = int32 accumulators
void launch_gemm(const int8_t* xq, const float* xs, int64_t T, int64_t K, const int8_t* wq,
                 const float* ws, int64_t N, const float* bias, void* y, int64_t ldy, int out,
                 hipStream_t st);
void launch_gemm_fp8(const uint8_t* xq, const float* xs, int64_t T, int64_t K, const uint8_t* wq,
                     const float* ws, int64_t N, const float* bias, void* y, int64_t ldy, int out,
                     hipStream_t st);
void launch_gemm_decode(const int8_t* xq, const float* xs, int64_t T, int64_t K, const int8_t* wq,
                        const float* ws, int64_t N, const float* bias, void* y, int64_t ldy,
                        int out, hipStream_t st);

}  // namespace sqk
