// sq_w8a8.hip -- the C ABI of libsqw8a8.so (declared in include/sq_w8a8.h).
// Host side only: argument checks, then stream-ordered kernel launches.  The
// library allocates nothing; its only state is the per-device address of the
// scratch array behind sq_w8a8_linear_noalloc.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "sq_internal.h"
#include "sq_w8a8.h"

namespace {

constexpr int64_t kMaxK = 65536;
constexpr int64_t kMaxRows = int64_t(1) << 24;   // tokens (T) and output channels (N) per call
constexpr int64_t kMaxGptqK = 16384;   // the K x K fp64 Hessian and its factor: 2 GiB each

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool is_fp(sq_dtype d) { return d == SQ_F32 || d == SQ_BF16; }
inline int64_t esize(sq_dtype d) { return d == SQ_F32 ? 4 : d == SQ_BF16 ? 2 : d == SQ_I32 ? 4 : 1; }
inline int64_t round256(int64_t b) { return (b + 255) & ~int64_t(255); }

// K rules shared by every call
inline sq_status check_k(int64_t k) {
  if (k <= 0) return SQ_ERR_SHAPE;
  if (k % 64 != 0 || k > kMaxK) return SQ_ERR_UNSUPPORTED;
  return SQ_OK;
}

// a row-major matrix of `rows` x `cols` elements with leading dimension ld
inline sq_status check_mat(const void* p, sq_dtype dt, int64_t rows, int64_t cols, int64_t ld) {
  if (p == nullptr) return SQ_ERR_NULL;
  if (!is_fp(dt)) return SQ_ERR_DTYPE;
  if (rows < 0 || cols < 0 || ld < cols) return SQ_ERR_SHAPE;
  if (!aligned16(p) || (ld * esize(dt)) % 16 != 0) return SQ_ERR_UNSUPPORTED;
  return SQ_OK;
}

inline sq_status hip_status() {
  return hipGetLastError() == hipSuccess ? SQ_OK : SQ_ERR_HIP;
}

#define SQ_TRY(expr)                 \
  do {                               \
    const sq_status st__ = (expr);   \
    if (st__ != SQ_OK) return st__;  \
  } while (0)

sq_status check_act(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx, sq_norm norm,
                    float eps) {
  SQ_TRY(check_k(k));
  SQ_TRY(check_mat(x, x_dt, t, k, ldx));
  if (t > kMaxRows) return SQ_ERR_UNSUPPORTED;
  if (norm != SQ_NORM_NONE && norm != SQ_NORM_RMS) return SQ_ERR_UNSUPPORTED;
  if (norm == SQ_NORM_RMS && !(eps >= 0.0f && isfinite(eps))) return SQ_ERR_SHAPE;
  return SQ_OK;
}

sq_status check_gemm(const int8_t* xq, const float* xs, int64_t t, int64_t k, const int8_t* wq,
                     const float* ws, int64_t n, void* y, sq_dtype y_dt, int64_t ldy,
                     const int32_t* acc_out) {
  SQ_TRY(check_k(k));
  if (xq == nullptr || wq == nullptr) return SQ_ERR_NULL;
  if (t < 0 || n < 0) return SQ_ERR_SHAPE;
  if (t > kMaxRows || n > kMaxRows) return SQ_ERR_UNSUPPORTED;
  // launch grids stay far below 2^32 work-items
  if (((t + 127) / 128) * ((n + 127) / 128) > (int64_t(1) << 22)) return SQ_ERR_UNSUPPORTED;
  if (!aligned16(xq) || !aligned16(wq)) return SQ_ERR_UNSUPPORTED;
  if (acc_out != nullptr) {
    if (!aligned16(acc_out)) return SQ_ERR_UNSUPPORTED;
    return SQ_OK;
  }
  if (xs == nullptr || ws == nullptr || y == nullptr) return SQ_ERR_NULL;
  if (!is_fp(y_dt)) return SQ_ERR_DTYPE;
  if (ldy < n) return SQ_ERR_SHAPE;
  if (ldy > INT32_MAX) return SQ_ERR_UNSUPPORTED;
  if (!aligned16(y) || (ldy * esize(y_dt)) % 16 != 0) return SQ_ERR_UNSUPPORTED;
  return SQ_OK;
}

inline int gemm_out(sq_dtype y_dt, const int32_t* acc_out) {
  return acc_out != nullptr ? 2 : (y_dt == SQ_BF16 ? 0 : 1);
}

}  // namespace

extern "C" {

int sq_abi_version(void) { return 1; }

const char* sq_status_string(sq_status status) {
  switch (status) {
    case SQ_OK: return "SQ_OK";
    case SQ_ERR_NULL: return "SQ_ERR_NULL: a required pointer is NULL";
    case SQ_ERR_SHAPE: return "SQ_ERR_SHAPE: negative size or leading dimension too small";
    case SQ_ERR_DTYPE: return "SQ_ERR_DTYPE: dtype not accepted for this argument";
    case SQ_ERR_ALPHA: return "SQ_ERR_ALPHA: alpha must be a finite value in [0, 1]";
    case SQ_ERR_UNSUPPORTED:
      return "SQ_ERR_UNSUPPORTED: shape or alignment outside the supported set";
    case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE: workspace missing or too small";
    case SQ_ERR_HIP: return "SQ_ERR_HIP: the HIP runtime reported an error";
  }
  return "unknown sq_status";
}

sq_status sq_calibrate(const void* x_cal, sq_dtype x_dt, int64_t t_cal, int64_t k, int64_t ldx,
                       sq_norm norm, const float* gamma, float eps, const void* w, sq_dtype w_dt,
                       int64_t n, int64_t ldw, float alpha, unsigned flags, float* a, float* wmax,
                       float* s, hipStream_t stream) {
  SQ_TRY(check_k(k));
  if (a == nullptr) return SQ_ERR_NULL;
  if ((flags & ~(SQ_CALIB_ACCUMULATE | SQ_CALIB_SKIP_ACT)) != 0u) return SQ_ERR_UNSUPPORTED;
  const bool act = (flags & SQ_CALIB_SKIP_ACT) == 0u;
  if (act) {
    SQ_TRY(check_act(x_cal, x_dt, t_cal, k, ldx, norm, eps));
  }
  if (w != nullptr) {
    SQ_TRY(check_mat(w, w_dt, k, n, ldw));
    if (wmax == nullptr || s == nullptr) return SQ_ERR_NULL;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ALPHA;
  }
  if (!act && w == nullptr) return SQ_OK;
  if (act) {
    if ((flags & SQ_CALIB_ACCUMULATE) == 0u) sqk::launch_fill_f32(a, k, 0.0f, stream);
    if (norm == SQ_NORM_RMS)
      sqk::launch_rms_act_absmax(x_cal, x_dt == SQ_BF16, t_cal, k, ldx, gamma, eps, a, stream);
    else
      sqk::launch_col_absmax(x_cal, x_dt == SQ_BF16, t_cal, k, ldx, nullptr, 1.0f, a, stream);
  }
  if (w != nullptr)
    sqk::launch_wrow_absmax_s(w, w_dt == SQ_BF16, k, n, ldw, a, alpha, wmax, s, stream);
  return hip_status();
}

sq_status sq_smooth_fold(const float* s, int64_t k, const float* gamma, float* gamma_out,
                         const void* w, sq_dtype w_dt, int64_t n, int64_t ldw, float* w_out,
                         hipStream_t stream) {
  SQ_TRY(check_k(k));
  if (s == nullptr) return SQ_ERR_NULL;
  const bool do_w = (w != nullptr && w_out != nullptr);
  if (do_w) {
    SQ_TRY(check_mat(w, w_dt, k, n, ldw));
    if (!aligned16(w_out)) return SQ_ERR_UNSUPPORTED;
  }
  if (gamma_out == nullptr && !do_w) return SQ_OK;
  if (gamma_out != nullptr) sqk::launch_fold_gamma(s, gamma, gamma_out, k, stream);
  if (do_w) sqk::launch_fold_w(w, w_dt == SQ_BF16, k, n, ldw, s, w_out, stream);
  return hip_status();
}

sq_status sq_quant_weight(const void* w, sq_dtype w_dt, int64_t k, int64_t n, int64_t ldw,
                          const float* s, int8_t* wq, float* w_scale, hipStream_t stream) {
  SQ_TRY(check_k(k));
  SQ_TRY(check_mat(w, w_dt, k, n, ldw));
  if (wq == nullptr || w_scale == nullptr) return SQ_ERR_NULL;
  if (!aligned16(wq)) return SQ_ERR_UNSUPPORTED;
  if (n == 0) return SQ_OK;
  if (sqk::quant_weight_strip_ok(w_dt == SQ_BF16, k, n)) {
    sqk::launch_quant_weight_strip(w, k, n, ldw, s, w_scale, wq, stream);
    return hip_status();
  }
  sqk::launch_fill_f32(w_scale, n, 0.0f, stream);
  sqk::launch_col_absmax(w, w_dt == SQ_BF16, k, n, ldw, s, 127.0f, w_scale, stream);
  sqk::launch_quant_weight_t(w, w_dt == SQ_BF16, k, n, ldw, s, w_scale, wq, stream);
  return hip_status();
}

sq_status sq_quant_weight_fp8(const void* w, sq_dtype w_dt, int64_t k, int64_t n, int64_t ldw,
                              const float* s, uint8_t* wq, float* w_scale, hipStream_t stream) {
  SQ_TRY(check_k(k));
  SQ_TRY(check_mat(w, w_dt, k, n, ldw));
  if (wq == nullptr || w_scale == nullptr) return SQ_ERR_NULL;
  if (!aligned16(wq)) return SQ_ERR_UNSUPPORTED;
  if (n == 0) return SQ_OK;
  if (sqk::quant_weight_strip_ok(w_dt == SQ_BF16, k, n)) {
    sqk::launch_quant_weight_strip_fp8(w, k, n, ldw, s, w_scale, wq, stream);
    return hip_status();
  }
  sqk::launch_fill_f32(w_scale, n, 0.0f, stream);
  sqk::launch_col_absmax(w, w_dt == SQ_BF16, k, n, ldw, s, 448.0f, w_scale, stream);
  sqk::launch_quant_weight_t_fp8(w, w_dt == SQ_BF16, k, n, ldw, s, w_scale, wq, stream);
  return hip_status();
}

sq_status sq_quant_act_fp8(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                           sq_norm norm, const float* gamma_f, float eps, uint8_t* xq,
                           float* x_scale, float* row_rscale, hipStream_t stream) {
  SQ_TRY(check_act(x, x_dt, t, k, ldx, norm, eps));
  if (xq == nullptr || x_scale == nullptr) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_UNSUPPORTED;
  if (t == 0) return SQ_OK;
  sqk::launch_quant_act_fp8(x, x_dt == SQ_BF16, t, k, ldx, norm == SQ_NORM_RMS, gamma_f, eps,
                            nullptr, xq, x_scale, norm == SQ_NORM_RMS ? row_rscale : nullptr,
                            stream);
  return hip_status();
}

sq_status sq_act_static_scale_fp8(const float* a, const float* gamma_f, int64_t k,
                                  float* x_scale_static, hipStream_t stream) {
  SQ_TRY(check_k(k));
  if (a == nullptr || x_scale_static == nullptr) return SQ_ERR_NULL;
  sqk::launch_static_scale(a, gamma_f, k, 448.0f, x_scale_static, stream);
  return hip_status();
}

sq_status sq_quant_act_static_fp8(const void* x, sq_dtype x_dt, int64_t t, int64_t k,
                                  int64_t ldx, sq_norm norm, const float* gamma_f, float eps,
                                  const float* x_scale_static, uint8_t* xq, float* x_scale,
                                  float* row_rscale, hipStream_t stream) {
  SQ_TRY(check_act(x, x_dt, t, k, ldx, norm, eps));
  if (x_scale_static == nullptr || xq == nullptr || x_scale == nullptr) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_UNSUPPORTED;
  if (t == 0) return SQ_OK;
  sqk::launch_quant_act_fp8(x, x_dt == SQ_BF16, t, k, ldx, norm == SQ_NORM_RMS, gamma_f, eps,
                            x_scale_static, xq, x_scale,
                            norm == SQ_NORM_RMS ? row_rscale : nullptr, stream);
  return hip_status();
}

sq_status sq_gemm_fp8(const uint8_t* xq, const float* x_scale, int64_t t, int64_t k,
                      const uint8_t* wq, const float* w_scale, int64_t n, const float* bias,
                      void* y, sq_dtype y_dt, int64_t ldy, float* acc_out, hipStream_t stream) {
  SQ_TRY(check_gemm(reinterpret_cast<const int8_t*>(xq), x_scale, t, k,
                    reinterpret_cast<const int8_t*>(wq), w_scale, n, y, y_dt, ldy,
                    reinterpret_cast<const int32_t*>(acc_out)));
  if (t == 0 || n == 0) return SQ_OK;
  void* out = acc_out != nullptr ? (void*)acc_out : y;
  sqk::launch_gemm_fp8(xq, x_scale, t, k, wq, w_scale, n, bias, out, acc_out ? n : ldy,
                       gemm_out(y_dt, reinterpret_cast<const int32_t*>(acc_out)), stream);
  return hip_status();
}

sq_status sq_quant_act(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                       sq_norm norm, const float* gamma_f, float eps, int8_t* xq, float* x_scale,
                       float* row_rscale, hipStream_t stream) {
  SQ_TRY(check_act(x, x_dt, t, k, ldx, norm, eps));
  if (xq == nullptr || x_scale == nullptr) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_UNSUPPORTED;
  if (t == 0) return SQ_OK;
  sqk::launch_quant_act(x, x_dt == SQ_BF16, t, k, ldx, norm == SQ_NORM_RMS, gamma_f, eps, nullptr,
                        xq, x_scale, norm == SQ_NORM_RMS ? row_rscale : nullptr, stream);
  return hip_status();
}

sq_status sq_act_static_scale(const float* a, const float* gamma_f, int64_t k,
                              float* x_scale_static, hipStream_t stream) {
  SQ_TRY(check_k(k));
  if (a == nullptr || x_scale_static == nullptr) return SQ_ERR_NULL;
  sqk::launch_static_scale(a, gamma_f, k, 127.0f, x_scale_static, stream);
  return hip_status();
}

sq_status sq_quant_act_static(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                              sq_norm norm, const float* gamma_f, float eps,
                              const float* x_scale_static, int8_t* xq, float* x_scale,
                              float* row_rscale, hipStream_t stream) {
  SQ_TRY(check_act(x, x_dt, t, k, ldx, norm, eps));
  if (x_scale_static == nullptr || xq == nullptr || x_scale == nullptr) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_UNSUPPORTED;
  if (t == 0) return SQ_OK;
  sqk::launch_quant_act(x, x_dt == SQ_BF16, t, k, ldx, norm == SQ_NORM_RMS, gamma_f, eps,
                        x_scale_static, xq, x_scale, norm == SQ_NORM_RMS ? row_rscale : nullptr,
                        stream);
  return hip_status();
}

sq_status sq_gemm_w8a8(const int8_t* xq, const float* x_scale, int64_t t, int64_t k,
                       const int8_t* wq, const float* w_scale, int64_t n, const float* bias,
                       void* y, sq_dtype y_dt, int64_t ldy, int32_t* acc_out,
                       hipStream_t stream) {
  SQ_TRY(check_gemm(xq, x_scale, t, k, wq, w_scale, n, y, y_dt, ldy, acc_out));
  if (t == 0 || n == 0) return SQ_OK;
  void* out = acc_out != nullptr ? (void*)acc_out : y;
  sqk::launch_gemm(xq, x_scale, t, k, wq, w_scale, n, bias, out, acc_out ? n : ldy,
                   gemm_out(y_dt, acc_out), stream);
  return hip_status();
}

size_t sq_linear_workspace_bytes(int64_t t, int64_t k) {
  if (t <= 0 || k <= 0) return 0;
  return (size_t)(round256(t * k) + round256(t * 4));
}

}  // extern "C"

// The workspace of sq_w8a8_linear_noalloc (codes and per-token steps): one
// copy on each GPU the library runs on, for the life of the process.  Host
// code never uses this name as an address -- on the host it is a stand-in --
// only the device address hipGetSymbolAddress returns for it.
static __device__ __align__(256) int8_t scratch[SQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// the current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept
sq_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SQ_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return SQ_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SQ_OK;
}

}  // namespace

namespace {

// the forward of sq_w8a8_linear (static_scale NULL), sq_w8a8_linear_static and
// their FP8 forms (fp8)
// LayerNorm form: the norm's beta' and the optional mean output
struct LnArgs {
  const float* beta_f;
  float* row_mean;
};

sq_status linear_impl(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                      sq_norm norm, const float* gamma_f, float eps, const float* static_scale,
                      bool fp8, const int8_t* wq, const float* w_scale, int64_t n,
                      const float* bias, void* y, sq_dtype y_dt, int64_t ldy, void* workspace,
                      size_t ws_bytes, const sq_debug_out* dbg, hipStream_t stream,
                      const LnArgs* ln = nullptr) {
  SQ_TRY(check_act(x, x_dt, t, k, ldx, norm, eps));
  if (t == 0) return wq == nullptr ? SQ_ERR_NULL : SQ_OK;   // nothing to compute
  int8_t* xq = dbg ? dbg->xq : nullptr;
  float* xs = dbg ? dbg->x_scale : nullptr;
  int32_t* acc = dbg ? dbg->acc : nullptr;
  float* rrow = dbg ? dbg->row_rscale : nullptr;
  if (xq == nullptr || xs == nullptr) {
    if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0 ||
        ws_bytes < sq_linear_workspace_bytes(t, k))
      return SQ_ERR_WORKSPACE;
    int8_t* wsb = static_cast<int8_t*>(workspace);
    if (xq == nullptr) xq = wsb;
    if (xs == nullptr) xs = reinterpret_cast<float*>(wsb + round256(t * k));
  }
  // the GEMM's own checks, with the codes and scales that will exist by then
  if (w_scale == nullptr && acc == nullptr) return SQ_ERR_NULL;
  SQ_TRY(check_gemm(xq, xs, t, k, wq, w_scale, n, y, y_dt, ldy, acc));
  if (ln != nullptr)
    sqk::launch_quant_act_ln(x, x_dt == SQ_BF16, t, k, ldx, gamma_f, ln->beta_f, eps, xq, xs,
                             ln->row_mean, rrow, stream);
  else if (fp8)
    sqk::launch_quant_act_fp8(x, x_dt == SQ_BF16, t, k, ldx, norm == SQ_NORM_RMS, gamma_f, eps,
                              static_scale, reinterpret_cast<uint8_t*>(xq), xs,
                              norm == SQ_NORM_RMS ? rrow : nullptr, stream);
  else
    sqk::launch_quant_act(x, x_dt == SQ_BF16, t, k, ldx, norm == SQ_NORM_RMS, gamma_f, eps,
                          static_scale, xq, xs, norm == SQ_NORM_RMS ? rrow : nullptr, stream);
  SQ_TRY(hip_status());
  if (n == 0) return SQ_OK;
  void* out = acc != nullptr ? (void*)acc : y;
  if (fp8)
    sqk::launch_gemm_fp8(reinterpret_cast<const uint8_t*>(xq), xs, t, k,
                         reinterpret_cast<const uint8_t*>(wq), w_scale, n, bias, out,
                         acc ? n : ldy, gemm_out(y_dt, acc), stream);
  else
    sqk::launch_gemm(xq, xs, t, k, wq, w_scale, n, bias, out, acc ? n : ldy, gemm_out(y_dt, acc),
                     stream);
  return hip_status();
}

}  // namespace

extern "C" {

sq_status sq_w8a8_linear(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                         sq_norm norm, const float* gamma_f, float eps, const int8_t* wq,
                         const float* w_scale, int64_t n, const float* bias, void* y,
                         sq_dtype y_dt, int64_t ldy, void* workspace, size_t ws_bytes,
                         const sq_debug_out* dbg, hipStream_t stream) {
  return linear_impl(x, x_dt, t, k, ldx, norm, gamma_f, eps, nullptr, false, wq, w_scale, n, bias,
                     y, y_dt, ldy, workspace, ws_bytes, dbg, stream);
}

sq_status sq_w8a8_linear_noalloc(const void* x, sq_dtype x_dt, int64_t t, int64_t k,
                                 int64_t ldx, sq_norm norm, const float* gamma_f, float eps,
                                 const int8_t* wq, const float* w_scale, int64_t n,
                                 const float* bias, void* y, sq_dtype y_dt, int64_t ldy,
                                 const sq_debug_out* dbg, hipStream_t stream) {
  // the activation's own checks first, so that a bad call touches no device state
  SQ_TRY(check_act(x, x_dt, t, k, ldx, norm, eps));
  const bool own_codes = dbg != nullptr && dbg->xq != nullptr && dbg->x_scale != nullptr;
  if (!own_codes && sq_linear_workspace_bytes(t, k) > SQ_NOALLOC_SCRATCH_BYTES)
    return SQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (t > 0) SQ_TRY(scratch_ptr(&ws));
  return linear_impl(x, x_dt, t, k, ldx, norm, gamma_f, eps, nullptr, false, wq, w_scale, n, bias,
                     y, y_dt, ldy, ws, SQ_NOALLOC_SCRATCH_BYTES, dbg, stream);
}

sq_status sq_w8a8_linear_fp8(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                             sq_norm norm, const float* gamma_f, float eps, const uint8_t* wq,
                             const float* w_scale, int64_t n, const float* bias, void* y,
                             sq_dtype y_dt, int64_t ldy, void* workspace, size_t ws_bytes,
                             const sq_debug_out* dbg, hipStream_t stream) {
  return linear_impl(x, x_dt, t, k, ldx, norm, gamma_f, eps, nullptr, true,
                     reinterpret_cast<const int8_t*>(wq), w_scale, n, bias, y, y_dt, ldy,
                     workspace, ws_bytes, dbg, stream);
}

sq_status sq_w8a8_linear_static(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                                sq_norm norm, const float* gamma_f, float eps,
                                const float* x_scale_static, const int8_t* wq,
                                const float* w_scale, int64_t n, const float* bias, void* y,
                                sq_dtype y_dt, int64_t ldy, void* workspace, size_t ws_bytes,
                                const sq_debug_out* dbg, hipStream_t stream) {
  if (x_scale_static == nullptr) return SQ_ERR_NULL;
  return linear_impl(x, x_dt, t, k, ldx, norm, gamma_f, eps, x_scale_static, false, wq, w_scale,
                     n, bias, y, y_dt, ldy, workspace, ws_bytes, dbg, stream);
}

sq_status sq_w8a8_linear_static_fp8(const void* x, sq_dtype x_dt, int64_t t, int64_t k,
                                    int64_t ldx, sq_norm norm, const float* gamma_f, float eps,
                                    const float* x_scale_static, const uint8_t* wq,
                                    const float* w_scale, int64_t n, const float* bias, void* y,
                                    sq_dtype y_dt, int64_t ldy, void* workspace,
                                    size_t ws_bytes, const sq_debug_out* dbg,
                                    hipStream_t stream) {
  if (x_scale_static == nullptr) return SQ_ERR_NULL;
  return linear_impl(x, x_dt, t, k, ldx, norm, gamma_f, eps, x_scale_static, true,
                     reinterpret_cast<const int8_t*>(wq), w_scale, n, bias, y, y_dt, ldy,
                     workspace, ws_bytes, dbg, stream);
}

// --- GPTQ on the migrated weight -----------------------------------------------

size_t sq_gptq_workspace_bytes(int64_t t_cal, int64_t k, int64_t n) {
  if (t_cal <= 0 || k <= 0 || n <= 0) return 0;
  return sqk::gptq_workspace_bytes(t_cal, k, n);
}

sq_status sq_quant_weight_gptq(const void* x_cal, sq_dtype x_dt, int64_t t_cal, int64_t ldx,
                               sq_norm norm, const float* gamma_f, float eps, const void* w,
                               sq_dtype w_dt, int64_t k, int64_t n, int64_t ldw, const float* s,
                               float damp, int8_t* wq, float* w_scale, float* row_rscale,
                               void* workspace, size_t ws_bytes, hipStream_t stream) {
  SQ_TRY(check_act(x_cal, x_dt, t_cal, k, ldx, norm, eps));
  SQ_TRY(check_mat(w, w_dt, k, n, ldw));
  if (wq == nullptr || w_scale == nullptr) return SQ_ERR_NULL;
  if (t_cal == 0 || n == 0) return SQ_ERR_SHAPE;
  if (k > kMaxGptqK || !aligned16(wq)) return SQ_ERR_UNSUPPORTED;
  if (!(damp >= 0.0f && isfinite(damp))) return SQ_ERR_SHAPE;
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0 ||
      ws_bytes < sqk::gptq_workspace_bytes(t_cal, k, n))
    return SQ_ERR_WORKSPACE;
  sqk::launch_gptq(x_cal, x_dt == SQ_BF16, t_cal, ldx, norm == SQ_NORM_RMS, gamma_f, eps, w,
                   w_dt == SQ_BF16, k, n, ldw, s, damp, wq, w_scale,
                   norm == SQ_NORM_RMS ? row_rscale : nullptr, workspace, stream);
  return hip_status();
}

// --- LayerNorm form and the fold into the previous linear --------------------

sq_status sq_calibrate_ln(const void* x_cal, sq_dtype x_dt, int64_t t_cal, int64_t k, int64_t ldx,
                          const float* gamma, const float* beta, float eps, const void* w,
                          sq_dtype w_dt, int64_t n, int64_t ldw, float alpha, unsigned flags,
                          float* a, float* wmax, float* s, hipStream_t stream) {
  SQ_TRY(check_k(k));
  if (a == nullptr) return SQ_ERR_NULL;
  if ((flags & ~(SQ_CALIB_ACCUMULATE | SQ_CALIB_SKIP_ACT)) != 0u) return SQ_ERR_UNSUPPORTED;
  const bool act = (flags & SQ_CALIB_SKIP_ACT) == 0u;
  if (act) {
    SQ_TRY(check_act(x_cal, x_dt, t_cal, k, ldx, SQ_NORM_RMS, eps));
  }
  if (w != nullptr) {
    SQ_TRY(check_mat(w, w_dt, k, n, ldw));
    if (wmax == nullptr || s == nullptr) return SQ_ERR_NULL;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ALPHA;
  }
  if (!act && w == nullptr) return SQ_OK;
  if (act) {
    if ((flags & SQ_CALIB_ACCUMULATE) == 0u) sqk::launch_fill_f32(a, k, 0.0f, stream);
    sqk::launch_ln_act_absmax(x_cal, x_dt == SQ_BF16, t_cal, k, ldx, gamma, beta, eps, a, stream);
  }
  if (w != nullptr)
    sqk::launch_wrow_absmax_s(w, w_dt == SQ_BF16, k, n, ldw, a, alpha, wmax, s, stream);
  return hip_status();
}

sq_status sq_smooth_fold_ln(const float* s, int64_t k, const float* gamma, const float* beta,
                            float* gamma_out, float* beta_out, hipStream_t stream) {
  SQ_TRY(check_k(k));
  if (s == nullptr || gamma_out == nullptr || beta_out == nullptr) return SQ_ERR_NULL;
  sqk::launch_fold_gamma(s, gamma, gamma_out, k, stream);
  sqk::launch_fold_beta(s, beta, beta_out, k, stream);
  return hip_status();
}

sq_status sq_quant_act_ln(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                          const float* gamma_f, const float* beta_f, float eps, int8_t* xq,
                          float* x_scale, float* row_mean, float* row_rscale,
                          hipStream_t stream) {
  SQ_TRY(check_act(x, x_dt, t, k, ldx, SQ_NORM_RMS, eps));
  if (gamma_f == nullptr || beta_f == nullptr || xq == nullptr || x_scale == nullptr)
    return SQ_ERR_NULL;
  if (!aligned16(xq) || !aligned16(gamma_f) || !aligned16(beta_f)) return SQ_ERR_UNSUPPORTED;
  if (t == 0) return SQ_OK;
  sqk::launch_quant_act_ln(x, x_dt == SQ_BF16, t, k, ldx, gamma_f, beta_f, eps, xq, x_scale,
                           row_mean, row_rscale, stream);
  return hip_status();
}

sq_status sq_w8a8_linear_ln(const void* x, sq_dtype x_dt, int64_t t, int64_t k, int64_t ldx,
                            const float* gamma_f, const float* beta_f, float eps,
                            const int8_t* wq, const float* w_scale, int64_t n, const float* bias,
                            void* y, sq_dtype y_dt, int64_t ldy, void* workspace, size_t ws_bytes,
                            const sq_debug_out* dbg, float* row_mean, hipStream_t stream) {
  if (gamma_f == nullptr || beta_f == nullptr) return SQ_ERR_NULL;
  if (!aligned16(gamma_f) || !aligned16(beta_f)) return SQ_ERR_UNSUPPORTED;
  const LnArgs ln{beta_f, row_mean};
  return linear_impl(x, x_dt, t, k, ldx, SQ_NORM_RMS, gamma_f, eps, nullptr, false, wq, w_scale, n,
                     bias, y, y_dt, ldy, workspace, ws_bytes, dbg, stream, &ln);
}

sq_status sq_fold_prev_linear(const float* s, int64_t k, const void* w_prev, sq_dtype w_dt,
                              int64_t k_prev, int64_t ldw, float* w_out, int64_t ldo,
                              const float* bias, float* bias_out, hipStream_t stream) {
  SQ_TRY(check_k(k));
  if (s == nullptr || w_out == nullptr) return SQ_ERR_NULL;
  SQ_TRY(check_mat(w_prev, w_dt, k_prev, k, ldw));
  if (ldo < k) return SQ_ERR_SHAPE;
  if (!aligned16(w_out) || ldo % 4 != 0 || !aligned16(s)) return SQ_ERR_UNSUPPORTED;
  if (bias != nullptr && bias_out == nullptr) return SQ_ERR_NULL;
  sqk::launch_fold_prev(w_prev, w_dt == SQ_BF16, k_prev, k, ldw, s, w_out, ldo, stream);
  if (bias != nullptr) sqk::launch_fold_beta(s, bias, bias_out, k, stream);   // b_j / s_j
  return hip_status();
}

}  // extern "C"
