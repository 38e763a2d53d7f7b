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
//
// No clamp to [-127, 127] is needed: |x^| <= max|x^| = 127 * Delta * (1 + e)
// with |e| <= 2^-24, so |x^ / Delta| and its rounded forms stay below 127.5 and
// round to at most 127 in magnitude.
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

constexpr float kTieBand = 0.5f - 0x1p-15f;

// codes of 8 values of one token by the reciprocal; `d` > 0, `rc` = fp32(1/d)
// finite.  `near_tie` is set when some quotient is within 2^-15 of a
// half-integer: those 8 codes must then be recomputed with quant8_div.
__device__ __forceinline__ u32x2 quant8(const float (&xh)[8], float rc, bool& near_tie) {
  u32x2 out;
  out[0] = 0u;
  out[1] = 0u;
  float dm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = xh[i] * rc;
    const float r = rintf(y);
    dm = fmaxf(dm, fabsf(y - r));
    out[i >> 2] |= code_byte(r) << (8 * (i & 3));
  }
  near_tie = dm > kTieBand;
  return out;
}

// exact path for every element (Delta so small that 1/Delta overflows)
__device__ __forceinline__ u32x2 quant8_div(const float (&xh)[8], float d) {
  u32x2 out;
  out[0] = 0u;
  out[1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i >> 2] |= code_byte(rintf(xh[i] / d)) << (8 * (i & 3));
  return out;
}

// ---------------------------------------------------------------------------
// K <= 8192: one token per WPR waves (WPR = 1, 2 or 4 of the workgroup's 4
// waves, so 4/WPR tokens per workgroup pass).  Thread i of a token's 64*WPR
// threads owns the 8-element chunks i, i + 64*WPR, ... (NV of them), so every
// load and store of a wave is 1 KiB / 512 B contiguous.  The token's values
// stay in VGPRs between the max and the quantize pass (HBM is read once and
// written once); the per-token maximum (and the RMSNorm sum of squares) is
// combined across the token's waves through LDS.  gamma_f stays in VGPRs for
// all the tokens a workgroup visits.
// ---------------------------------------------------------------------------
template <class In, int NV, int WPR, bool NORM>
__global__ __launch_bounds__(256) void k_quant_act(const typename In::elem* __restrict__ x,
                                                   int64_t T, int64_t K, int64_t ld,
                                                   const float* __restrict__ gamma_f, float eps,
                                                   int8_t* __restrict__ xq,
                                                   float* __restrict__ xscale,
                                                   float* __restrict__ rrow) {
  constexpr int RPB = 4 / WPR;   // tokens per workgroup pass
  __shared__ float red_m[2][4];
  __shared__ double red_s[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rloc = wave / WPR;
  const int tl = (wave % WPR) * 64 + lane;
  const int nchunk = (int)(K >> 3);   // <= 1024 on this path
  float g[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int ch = j * 64 * WPR + tl;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      g[j][i] = (ch < nchunk) ? (gamma_f ? gamma_f[ch * 8 + i] : 1.0f) : 0.0f;
  }
  const double deps = (double)eps;
  const double dK = (double)K;
  const int Ti = (int)T;   // T < 2^31 (checked by the caller)
  const int step = gridDim.x * RPB;
  auto load = [&](int rb, typename In::Raw (&raw)[NV]) {
    const int r = rb + rloc;
    const typename In::elem* row = x + (int64_t)(r < Ti ? r : 0) * ld;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int ch = j * 64 * WPR + tl;
      raw[j] = In::raw8(row + (ch < nchunk ? ch : 0) * 8);
    }
  };
  int par = 0;
  auto process = [&](int rb, const typename In::Raw (&raw)[NV]) {
    const int r = rb + rloc;
    const bool ok = r < Ti;
    float rt = 1.0f;
    if (NORM) {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int ch = j * 64 * WPR + tl;
        float v[8];
        In::widen(raw[j], v);
        if (ch < nchunk) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const double dv = (double)v[i];
            ss = fma(dv, dv, ss);   // exact square, so the same as mul + add
          }
        }
      }
      ss = wave_sum(ss);
      if (WPR > 1) {
        if (lane == 0) red_s[wave] = ss;
        __syncthreads();
        ss = red_s[rloc * WPR];
#pragma unroll
        for (int w = 1; w < WPR; ++w) ss += red_s[rloc * WPR + w];
      }
      rt = (float)(1.0 / sqrt(ss / dK + deps));
      if (rrow != nullptr && ok && tl == 0) rrow[r] = rt;
    }
    float xh[NV][8];
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[8];
      In::widen(raw[j], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = NORM ? v[i] * rt : v[i];
        xh[j][i] = t * g[j][i];   // g is 0 on chunks past K
        am = fmaxf(am, fabsf(xh[j][i]));
      }
    }
    am = wave_max(am);
    if (WPR > 1) {
      // two buffers, so the next token's writes cannot race this token's reads
      if (lane == 0) red_m[par][wave] = am;
      __syncthreads();
      float m = red_m[par][rloc * WPR];
#pragma unroll
      for (int w = 1; w < WPR; ++w) m = fmaxf(m, red_m[par][rloc * WPR + w]);
      am = m;
      par ^= 1;
    }
    const float d = am / 127.0f;
    const float rc = 1.0f / d;
    // d == 0: every x^ is 0 and rc = 0 gives code 0.  1/d overflowing (d tiny):
    // every chunk is redone by IEEE division below.
    const bool fast = rc <= 3.0e38f;
    const float rcu = fast ? rc : 0.0f;
    if (ok) {
      if (tl == 0) xscale[r] = d;
      int8_t* qrow = xq + (int64_t)r * K;
      uint32_t redo = (!fast && d > 0.0f) ? ~0u : 0u;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int ch = j * 64 * WPR + tl;
        bool tie;
        const u32x2 c = quant8(xh[j], rcu, tie);
        redo |= (tie ? 1u : 0u) << j;
        if (ch < nchunk) *reinterpret_cast<u32x2*>(qrow + ch * 8) = c;
      }
      // rare: chunks with a quotient near a rounding tie, by IEEE division
      if (redo != 0u) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int ch = j * 64 * WPR + tl;
          if (((redo >> j) & 1u) && ch < nchunk)
            *reinterpret_cast<u32x2*>(qrow + ch * 8) = quant8_div(xh[j], d);
        }
      }
    }
  };
  // one token ahead: the next pass's loads are in flight while this one is
  // reduced, quantized and stored
  typename In::Raw ra[NV], rb2[NV];
  int rb = blockIdx.x * RPB;
  if (rb < Ti) load(rb, ra);
  while (rb < Ti) {
    if (rb + step < Ti) load(rb + step, rb2);
    process(rb, ra);
    rb += step;
    if (rb >= Ti) break;
    if (rb + step < Ti) load(rb + step, ra);
    process(rb, rb2);
    rb += step;
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
    bool tie = true;
    if (fast) c = quant8(xh, rc, tie);
    if (d > 0.0f && tie) c = quant8_div(xh, d);
    *reinterpret_cast<u32x2*>(xq + r * K + ch * 8) = c;
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------

template <class In, int NV, int WPR, bool NORM>
static void quant_act_nv(const void* x, int64_t T, int64_t K, int64_t ld, const float* gamma_f,
                         float eps, int8_t* xq, float* xscale, float* rrow, hipStream_t st) {
  constexpr int RPB = 4 / WPR;
  // up to 2048 workgroups; each visits the tokens blockIdx*RPB + i*gridDim*RPB
  int64_t blocks = (T + RPB - 1) / RPB;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL((k_quant_act<In, NV, WPR, NORM>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const typename In::elem*)x, T, K, ld, gamma_f, eps, xq, xscale, rrow);
}

template <class In, bool NORM>
static void quant_act_t(const void* x, int64_t T, int64_t K, int64_t ld, const float* gamma_f,
                        float eps, int8_t* xq, float* xscale, float* rrow, hipStream_t st) {
  const int64_t nchunk = K / 8;
  if (nchunk <= 64) quant_act_nv<In, 1, 1, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nchunk <= 128) quant_act_nv<In, 1, 2, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nchunk <= 256) quant_act_nv<In, 1, 4, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nchunk <= 512) quant_act_nv<In, 2, 4, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
  else if (nchunk <= 1024) quant_act_nv<In, 4, 4, NORM>(x, T, K, ld, gamma_f, eps, xq, xscale, rrow, st);
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
