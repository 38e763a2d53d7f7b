// k_actquant.hip -- fused RMSNorm -> smooth -> per-token dynamic INT8
// quantization for gfx950.
//
// Per token t ("06 -- SmoothQuant", section 7: one scale per token; the
// smoothing 1/s is already folded into gamma_f, "SmoothQuant and W8A8", The
// trick):
//   x^ = fp32(fp32(h * r_t) * gamma_f)     (norm)   or   fp32(x * gamma_f)
//   Delta_t = fp32(max|x^| / 127);  code = round-half-even(fp32(x^ / Delta_t))
//
// Exact codes without a division per element.  With rc = fp32(1/Delta) and
// y = fp32(x^ * rc), |y - x^/Delta| <= 2^-23 * |x^/Delta| and the correctly
// rounded quotient q* is within 2^-24 * |x^/Delta| of x^/Delta; |x^/Delta| <= 128,
// so |y - q*| < 2.3e-5.  When y is farther than 2^-15 from every half-integer,
// q* rounds to the same integer as y.  Chunks of 8 where some y is within
// 2^-15 of a half-integer (including exact ties) are redone with the IEEE
// division.  The result equals round-half-even of the correctly rounded
// quotient, bit for bit.
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

constexpr float kTieBand = 0.5f - 0x1p-15f;

// codes of 8 values of one token; `d` > 0, `rc` = fp32(1/d) finite
__device__ __forceinline__ u32x2 quant8(const float (&xh)[8], float d, float rc) {
  float q[8];
  float dm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = xh[i] * rc;
    const float r = rintf(y);
    dm = fmaxf(dm, fabsf(y - r));
    q[i] = r;
  }
  if (dm > kTieBand) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = rintf(xh[i] / d);
  }
  u32x2 out;
  out[0] = 0u;
  out[1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = fminf(fmaxf(q[i], -127.0f), 127.0f);
    out[i >> 2] |= code_byte(c) << (8 * (i & 3));
  }
  return out;
}

// exact path for every element (Delta so small that 1/Delta overflows)
__device__ __forceinline__ u32x2 quant8_div(const float (&xh)[8], float d) {
  u32x2 out;
  out[0] = 0u;
  out[1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = fminf(fmaxf(rintf(xh[i] / d), -127.0f), 127.0f);
    out[i >> 2] |= code_byte(c) << (8 * (i & 3));
  }
  return out;
}

// ---------------------------------------------------------------------------
// K <= 8192: one wave per token.  Lane l owns the 8-element chunks
// l, l+64, ... (NV of them); the row is held in VGPRs between the max and the
// quantize pass, so HBM is read once and written once.  GREG keeps gamma_f in
// VGPRs across the rows a wave visits.
// ---------------------------------------------------------------------------
template <class In, int NV, bool NORM, bool GREG>
__global__ __launch_bounds__(256) void k_quant_act(const typename In::elem* __restrict__ x,
                                                   int64_t T, int64_t K, int64_t ld,
                                                   const float* __restrict__ gamma_f, float eps,
                                                   int8_t* __restrict__ xq,
                                                   float* __restrict__ xscale,
                                                   float* __restrict__ rrow) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nchunk = K >> 3;
  float g[GREG ? NV : 1][8];
  if (GREG) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t ch = (int64_t)j * 64 + lane;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        g[GREG ? j : 0][i] = (ch < nchunk) ? (gamma_f ? gamma_f[ch * 8 + i] : 1.0f) : 0.0f;
    }
  }
  const double deps = (double)eps;
  const double dK = (double)K;
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < T; r += (int64_t)gridDim.x * 4) {
    const typename In::elem* row = x + r * ld;
    typename In::Raw raw[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t ch = (int64_t)j * 64 + lane;
      raw[j] = In::raw8(row + (ch < nchunk ? ch : 0) * 8);
    }
    float rt = 1.0f;
    if (NORM) {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int64_t ch = (int64_t)j * 64 + lane;
        float v[8];
        In::widen(raw[j], v);
        if (ch < nchunk) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const double dv = (double)v[i];
            ss = fma(dv, dv, ss);   // exact square, so same as mul + add
          }
        }
      }
      ss = wave_sum(ss);
      rt = (float)(1.0 / sqrt(ss / dK + deps));
      if (rrow != nullptr && lane == 0) rrow[r] = rt;
    }
    float xh[NV][8];
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t ch = (int64_t)j * 64 + lane;
      float v[8];
      In::widen(raw[j], v);
      float gj[8];
      if (GREG) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gj[i] = g[GREG ? j : 0][i];
      } else {
        if (ch < nchunk && gamma_f != nullptr) {
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma_f + ch * 8);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma_f + ch * 8 + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gj[i] = g0[i];
            gj[4 + i] = g1[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) gj[i] = (ch < nchunk) ? 1.0f : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = NORM ? v[i] * rt : v[i];
        xh[j][i] = (ch < nchunk) ? t * gj[i] : 0.0f;
        am = fmaxf(am, fabsf(xh[j][i]));
      }
    }
    am = wave_max(am);
    const float d = am / 127.0f;
    if (lane == 0) xscale[r] = d;
    const float rc = 1.0f / d;
    int8_t* qrow = xq + r * K;
    if (d > 0.0f && rc <= 3.0e38f) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int64_t ch = (int64_t)j * 64 + lane;
        if (ch < nchunk) *reinterpret_cast<u32x2*>(qrow + ch * 8) = quant8(xh[j], d, rc);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int64_t ch = (int64_t)j * 64 + lane;
        u32x2 z;
        z[0] = 0u;
        z[1] = 0u;
        if (ch < nchunk)
          *reinterpret_cast<u32x2*>(qrow + ch * 8) = (d > 0.0f) ? quant8_div(xh[j], d) : z;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K > 8192: one workgroup per token, three passes over the row (sum of
// squares, max, quantize); the re-reads hit L2.
// ---------------------------------------------------------------------------
template <class In, bool NORM>
__global__ __launch_bounds__(256) void k_quant_act_wide(const typename In::elem* __restrict__ x,
                                                        int64_t T, int64_t K, int64_t ld,
                                                        const float* __restrict__ gamma_f,
                                                        float eps, int8_t* __restrict__ xq,
                                                        float* __restrict__ xscale,
                                                        float* __restrict__ rrow) {
  __shared__ double red_d[4];
  __shared__ float red_f[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nchunk = K >> 3;
  const int64_t r = blockIdx.x;
  const typename In::elem* row = x + r * ld;
  float rt = 1.0f;
  if (NORM) {
    double ss = 0.0;
    for (int64_t ch = threadIdx.x; ch < nchunk; ch += 256) {
      float v[8];
      In::load8(row + ch * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double dv = (double)v[i];
        ss = fma(dv, dv, ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red_d[wave] = ss;
    __syncthreads();
    ss = (red_d[0] + red_d[1]) + (red_d[2] + red_d[3]);
    rt = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    if (rrow != nullptr && threadIdx.x == 0) rrow[r] = rt;
  }
  float am = 0.0f;
  for (int64_t ch = threadIdx.x; ch < nchunk; ch += 256) {
    float v[8];
    In::load8(row + ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = NORM ? v[i] * rt : v[i];
      am = fmaxf(am, fabsf(t * (gamma_f ? gamma_f[ch * 8 + i] : 1.0f)));
    }
  }
  am = wave_max(am);
  if (lane == 0) red_f[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  const float d = am / 127.0f;
  if (threadIdx.x == 0) xscale[r] = d;
  const float rc = 1.0f / d;
  const bool fast = d > 0.0f && rc <= 3.0e38f;
  for (int64_t ch = threadIdx.x; ch < nchunk; ch += 256) {
    float v[8], xh[8];
    In::load8(row + ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = NORM ? v[i] * rt : v[i];
      xh[i] = t * (gamma_f ? gamma_f[ch * 8 + i] : 1.0f);
    }
    u32x2 c;
    c[0] = 0u;
    c[1] = 0u;
    if (fast) c = quant8(xh, d, rc);
    else if (d > 0.0f) c = quant8_div(xh, d);
    *reinterpret_cast<u32x2*>(xq + r * K + ch * 8) = c;
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------

template <class In, int NV, bool NORM>
static void quant_act_nv(const void* x, int64_t T, int64_t K, int64_t ld, const float* gamma_f,
                         float eps, int8_t* xq, float* xscale, float* rrow, hipStream_t st) {
  constexpr bool kGreg = NV <= 8;
  // about 2 rows per wave at T = 8192; gamma_f stays in VGPRs between rows
  int64_t blocks = (T + 3) / 4;
  const int64_t cap = kGreg ? 1024 : 2048;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((k_quant_act<In, NV, NORM, kGreg>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const typename In::elem*)x, T, K, ld, gamma_f, eps, xq, xscale, rrow);
}

template <class In, bool NORM>
static void quant_act_t(const void* x, int64_t T, int64_t K, int64_t ld, const float* gamma_f,
                        float eps, int8_t* xq, float* xscale, float* rrow, hipStream_t st) {
  const int64_t nv = (K + 511) / 512;
  if (nv <= 1) quant_act_nv<In, 1, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nv <= 2) quant_act_nv<In, 2, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nv <= 4) quant_act_nv<In, 4, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nv <= 8) quant_act_nv<In, 8, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nv <= 16) quant_act_nv<In, 16, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else
    hipLaunchKernelGGL((k_quant_act_wide<In, NORM>), dim3((unsigned)T), dim3(256), 0, st,
                       (const typename In::elem*)x, T, K, ld, gamma_f, eps, xq, xscale, rrow);
}

void launch_quant_act(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld, bool norm,
                      const float* gamma_f, float eps, int8_t* xq, float* xscale, float* rrow,
                      hipStream_t st) {
  if (T <= 0) return;
  if (bf16) {
    if (norm) quant_act_t<Bf16In, true>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
    else quant_act_t<Bf16In, false>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  } else {
    if (norm) quant_act_t<F32In, true>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
    else quant_act_t<F32In, false>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  }
}

}  // namespace sqk
