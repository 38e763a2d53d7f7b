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
// The reciprocal path needs no clamp to [-127, 127]: it runs only while
// 1/Delta is finite (Delta >= 2^-128), where Delta = fp32(max|x^| / 127) keeps
// at least 21 significant bits, so |x^ / Delta| and its rounded forms stay
// below 127.5 and round to at most 127 in magnitude.  Below that a subnormal
// step can be rounded by far more (max|x^| = 2e-43 gives Delta = 1e-45 and a
// quotient of 143), so the division path clamps, as the definition does.
//
// Static per-tensor step ("SmoothQuant and W8A8", One layer, measured: one
// scale per tensor from the calibration tokens' maximum): Delta is given, the
// same for every token, and the codes are clamped to [-127, 127] -- values past
// the calibrated maximum clip (same page, Gotchas).  The tie argument above
// holds for every quotient below 128 in magnitude; at and above 128 the
// rounded value clamps to +-127 whichever way it rounds.
#include "sq_common.h"
#include "sq_norm.h"
#include "sq_internal.h"

namespace sqk {

// codes of 8 values of one token by the reciprocal; `d` > 0, `rc` = fp32(1/d)
// finite.  `near_tie` is set when some quotient is within 2^-15 of a
// half-integer: those 8 codes must then be recomputed with quant8_div.
// CLAMP: clamp the rounded quotient to [-127, 127] (static step only).
template <bool CLAMP>
__device__ __forceinline__ float clamp127(float r) {
  return CLAMP ? fminf(fmaxf(r, -127.0f), 127.0f) : r;
}

//
// The rounding adds and subtracts 1.5 * 2^23: for |y| < 2^22 the sum's unit
// in the last place is 1, so the addition rounds y to an integer, ties to
// even, exactly as rintf, and the sum's low byte is that integer's two's
// complement byte (its significand is 2^22 + rint(y)); v_perm_b32 packs four
// such bytes per dword.  The static step can see quotients of any size: they
// are first clamped to [-128, 128], which changes no code (every quotient at
// or past 127.5 in magnitude ends at +-127) and no near-tie decision below
// 128.  Against rintf and a shift-and-or per code: 8192 x 4096 23.1 -> 22.0
// us, 16 x 8192 8.4 -> 7.6 us, identical codes.
template <bool CLAMP = false>
__device__ __forceinline__ u32x2 quant8(const float (&xh)[8], float rc, bool& near_tie) {
  constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
  float t[8];
  float dm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y = xh[i] * rc;
    if (CLAMP) y = fminf(fmaxf(y, -128.0f), 128.0f);
    t[i] = y + kMagic;
    const float r = t[i] - kMagic;
    dm = fmaxf(dm, fabsf(y - r));
    if (CLAMP) t[i] = fminf(fmaxf(t[i], kMagic - 127.0f), kMagic + 127.0f);
  }
  near_tie = dm > kTieBand;
  u32x2 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // bytes 0 of t[4h], t[4h+1] into bytes 0, 1; of t[4h+2], t[4h+3] into 2, 3
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t[4 * h + 1]),
                                              __float_as_uint(t[4 * h]), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t[4 * h + 3]),
                                              __float_as_uint(t[4 * h + 2]), 0x04000c0cu);
    out[h] = lo | hi;
  }
  return out;
}

// exact path for every element (near-ties, and Delta so small that 1/Delta
// overflows); always clamped: a deep subnormal step can leave quotients above
// 127.5 even for the per-token step
template <bool CLAMP = false>
__device__ __forceinline__ u32x2 quant8_div(const float (&xh)[8], float d) {
  u32x2 out;
  out[0] = 0u;
  out[1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i >> 2] |= code_byte(clamp127<true>(rintf(xh[i] / d))) << (8 * (i & 3));
  return out;
}

// FP8 E4M3 codes of 8 values: the fp32 quotient x^ / d (IEEE division), then
// v_cvt_pk_fp8_f32, which rounds to the nearest E4M3 value, ties to even.
// With d = amax / 448 every quotient is at most 448 up to one rounding, inside
// the format's finite range -- unless d is a deep subnormal rounded far from
// amax / 448 -- and a static step (CLAMP) can see larger quotients: every
// quotient clips to +-448 first (the largest finite code, which the
// definition gives for anything at or past it; the conversion would give NaN
// from 480 up).  d == 0 (an all-zero token, or a zero static step) gives
// codes 0.
template <bool CLAMP = false>
__device__ __forceinline__ u32x2 quant8_fp8(const float (&xh)[8], float d) {
  u32x2 out;
  out[0] = 0u;
  out[1] = 0u;
  if (d == 0.0f) return out;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[i] = fminf(fmaxf(xh[i] / d, -448.0f), 448.0f);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h], y[4 * h + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2], y[4 * h + 3], w, true);
    out[h] = (uint32_t)w;
  }
  return out;
}

// FP8 E4M3 codes of 8 values by the reciprocal.  With rc = fp32(1/d) finite,
// rlo = fp32(rc * (1 - 2^-20)) and rhi = fp32(rc * (1 + 2^-20)), the products
// x^ * rlo and x^ * rhi miss x^ * (1 -+ 2^-20) / d by under 3 * 2^-24
// relative, so they bracket both x^ / d and its correctly rounded fp32 value.
// The conversion is monotonic: where the two ends give the same code, that is
// quant8_fp8's code.  `split` is set when some pair differs (a quotient near
// a point where the E4M3 rounding changes, about 4e-5 of them): those 8 codes
// must then come from quant8_fp8.  CLAMP as there.
template <bool CLAMP = false>
__device__ __forceinline__ u32x2 quant8_fp8_rc(const float (&xh)[8], float rlo, float rhi,
                                               bool& split) {
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo[i] = xh[i] * rlo;
    hi[i] = xh[i] * rhi;
    if (CLAMP) {
      lo[i] = fminf(fmaxf(lo[i], -448.0f), 448.0f);
      hi[i] = fminf(fmaxf(hi[i], -448.0f), 448.0f);
    }
  }
  u32x2 a, b;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(lo[4 * h], lo[4 * h + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(lo[4 * h + 2], lo[4 * h + 3], w, true);
    a[h] = (uint32_t)w;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(hi[4 * h], hi[4 * h + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(hi[4 * h + 2], hi[4 * h + 3], w, true);
    b[h] = (uint32_t)w;
  }
  split = ((a[0] ^ b[0]) | (a[1] ^ b[1])) != 0u;
  return a;
}

enum { QF_INT8 = 0, QF_FP8 = 1 };

// ---------------------------------------------------------------------------
// K <= 8192 (bf16: K <= 16384, 128 VGPRs of raw values and 64 KiB of LDS
// for gamma at NV = 32): one token per wave, WPB tokens per workgroup.  Lane
// l owns the
// 8-element chunks l, l + 64, ... (NV of them), so every load of a wave is
// 1 KiB contiguous and every store 512 B.  The token's raw values stay in
// VGPRs from the load to the store (HBM is read once and written once) and
// every reduction stays inside the wave: no workgroup barrier between load
// and store, so each wave streams on its own.  gamma_f is staged once per
// workgroup in LDS and read there by both passes (the max pass and the
// quantize pass recompute x^ with the same fp32 operations).
// ---------------------------------------------------------------------------
constexpr int kWavesPerBlock = 8;
// Up to 16 raw bytes per lane-chunk-slot (bf16 with K <= 4096, fp32 with
// K <= 2048) the kernel fits 64 VGPRs: ask for 8 waves per SIMD there (6 for
// the FP8 codes).
template <class In, int NV, int QF>
constexpr int quant_act_min_waves() {
  return In::kBytes * NV <= 16 ? (QF == 1 ? 6 : 8) : 1;   // FP8: 8 quotients live per chunk
}

// (x is not __restrict__: that would let the compiler move the token loads
// past the barrier that the gamma_f staging needs, serializing them again)
template <class In, int NV, bool NORM, bool STATIC, int QF>
__global__ __launch_bounds__(64 * kWavesPerBlock, (quant_act_min_waves<In, NV, QF>())) void k_quant_act(
    const typename In::elem* x, int64_t T, int64_t K, int64_t ld,
    const float* __restrict__ gamma_f, float eps, const float* __restrict__ static_scale,
    int8_t* __restrict__ xq, float* __restrict__ xscale, float* __restrict__ rrow) {
  // gamma_f of chunk c: elements 0-3 at gs[c], 4-7 at gs[NV * 64 + c] (1
  // without gamma, 0 past K)
  __shared__ __attribute__((aligned(1024))) f32x4 gs[NV * 64 * 2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunk = (int)(K >> 3);   // <= 64 * NV
  // gamma_f goes to LDS by direct-to-LDS loads (no VGPRs), issued before
  // this wave's token loads; the wait below covers only those gamma loads
  // (loads complete in order), so the token's loads are in flight during the
  // staging and the barrier: the two memory latencies overlap instead of
  // adding up, which is what sets the time at a few thousand tokens.
  // Positions past K read as 0 (outside the buffer resource).
  if (gamma_f != nullptr) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t gr =
        __builtin_amdgcn_make_buffer_rsrc((void*)gamma_f, 0, (int)(K * 4), 0x00020000);
    for (int base = wave * 64; base < NV * 64 * 2; base += 64 * kWavesPerBlock) {
      const int i = base + lane;
      const int ch = i % (NV * 64), half = i / (NV * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          gr, (__attribute__((address_space(3))) void*)&gs[base], 16, (ch * 8 + half * 4) * 4, 0,
          0, 0);
    }
#endif
  } else {
    for (int i = threadIdx.x; i < NV * 64 * 2; i += 64 * kWavesPerBlock) {
      const float one = (i % (NV * 64)) < nchunk ? 1.0f : 0.0f;
      gs[i] = f32x4{one, one, one, one};
    }
  }
  const int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const bool live = r < T;
  const typename In::elem* row = x + (live ? r : T - 1) * ld;
  typename In::Raw raw[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int ch = j * 64 + lane;
    raw[j] = In::raw8_nt(row + (ch < nchunk ? ch : 0) * 8);   // read once
  }
  // keep the token's loads here, ahead of the barrier (the scheduler would
  // otherwise sink them below it); they (NV for bf16, 2 NV for fp32) may
  // still fly
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(NV * In::kBytes / 2) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const uint32_t gaddr = lds_addr(&gs[lane]);
  if (!live) return;
  float rt = 1.0f;
  if (NORM) {
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[8];
      In::widen(raw[j], v);
      if (j * 64 + lane < nchunk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double dv = (double)v[i];
          ss = fma(dv, dv, ss);   // exact square, so the same as mul + add
        }
      }
    }
    ss = wave_sum(ss);
    rt = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    if (rrow != nullptr && lane == 0) rrow[r] = rt;
#pragma unroll
    for (int j = 0; j < NV; ++j) In::opaque(raw[j]);
  }
  // x^ of chunk j, the same fp32 operations in both passes.  gamma is read
  // from LDS chunk by chunk, with the wait in the same asm block: the
  // compiler cannot then hoist every chunk's gamma into VGPRs at once.  The
  // outputs are early-clobber: the first read's data may land before the
  // second read has taken its address, so no output may share the address
  // register.
  auto smooth = [&](auto jc, float (&xh)[8]) {
    constexpr int j = decltype(jc)::value;
    float v[8];
    In::widen(raw[j], v);
    f32x4 g0, g1;
    asm volatile("ds_read_b128 %0, %2 offset:%3\n\tds_read_b128 %1, %2 offset:%4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(g0), "=&v"(g1)
                 : "v"(gaddr), "n"(j * 1024), "n"(NV * 1024 + j * 1024)
                 : "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = NORM ? v[i] * rt : v[i];
      xh[i] = t * (i < 4 ? g0[i] : g1[i - 4]);   // gamma is 0 past K
    }
  };
  float am = 0.0f;
  if (!STATIC) {
    static_for<NV>([&](auto jc) {
      float xh[8];
      smooth(jc, xh);
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(xh[i]));
    });
    am = wave_max(am);
  }
  // Keep only the raw values alive between the passes: the quantize pass
  // widens them again and re-reads gamma from LDS (the compiler would otherwise
  // keep every chunk's x^ in VGPRs and quarter the occupancy).
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < NV; ++j) In::opaque(raw[j]);
  const float d = STATIC ? static_scale[0] : am / (QF == QF_FP8 ? 448.0f : 127.0f);
  const float rc = 1.0f / d;
  // d == 0: every x^ is 0 (or, for a static step, every code is 0) and rc = 0
  // gives code 0.  1/d overflowing (d tiny): every chunk takes the IEEE
  // division below.
  const bool fast = rc <= 3.0e38f;
  const float rcu = fast ? rc : 0.0f;
  const float rlo = rcu * (1.0f - 0x1p-20f), rhi = rcu * (1.0f + 0x1p-20f);
  if (lane == 0) xscale[r] = d;
  int8_t* qrow = xq + r * K;
  // exact path for the whole row when 1/d overflows
  const bool all_div = !fast && d > 0.0f;
  static_for<NV>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int ch = j * 64 + lane;
    float xh[8];
    smooth(jc, xh);
    u32x2 c;
    if constexpr (QF == QF_FP8) {
      bool split = true;
      if (fast) c = quant8_fp8_rc<STATIC>(xh, rlo, rhi, split);
      // rare: near an E4M3 rounding point; d == 0 or 1/d overflowing: all
      if (split) c = quant8_fp8<STATIC>(xh, d);
    } else {
      bool tie;
      c = quant8<STATIC>(xh, rcu, tie);
      // rare: a quotient near a rounding tie; redo the chunk by IEEE division
      if (tie || all_div) c = quant8_div<STATIC>(xh, d);
    }
    if (ch < nchunk) *reinterpret_cast<u32x2*>(qrow + ch * 8) = c;
  });
}

// ---------------------------------------------------------------------------
// K > 16384: one workgroup per token, three passes over the row (sum of
// squares, max, quantize); the re-reads hit L2.
// ---------------------------------------------------------------------------
template <class In, bool NORM, bool STATIC, int QF>
__global__ __launch_bounds__(256) void k_quant_act_wide(const typename In::elem* __restrict__ x,
                                                        int64_t T, int64_t K, int64_t ld,
                                                        const float* __restrict__ gamma_f,
                                                        float eps,
                                                        const float* __restrict__ static_scale,
                                                        int8_t* __restrict__ xq,
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
  if (!STATIC) {
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
  }
  const float d = STATIC ? static_scale[0] : am / (QF == QF_FP8 ? 448.0f : 127.0f);
  if (threadIdx.x == 0) xscale[r] = d;
  const float rc = 1.0f / d;
  const bool fast = d > 0.0f && rc <= 3.0e38f;
  const float rlo = rc * (1.0f - 0x1p-20f), rhi = rc * (1.0f + 0x1p-20f);
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
    if constexpr (QF == QF_FP8) {
      bool split = true;
      if (fast) c = quant8_fp8_rc<STATIC>(xh, rlo, rhi, split);
      if (split) c = quant8_fp8<STATIC>(xh, d);
    } else {
      bool tie = true;
      if (fast) c = quant8<STATIC>(xh, rc, tie);
      if (d > 0.0f && tie) c = quant8_div<STATIC>(xh, d);
    }
    *reinterpret_cast<u32x2*>(xq + r * K + ch * 8) = c;
  }
}

// ---------------------------------------------------------------------------
// Rows of 512-2048 chunks (4096-16384 values) at up to 4096 tokens, and wider
// rows up to 2048 chunks that the one-wave kernel does not take: one workgroup
// of 256 threads per token with the row in registers, NC chunks per thread
// (chunk c * 256 + thread), every load of the row and of gamma_f issued at
// once; x^ is formed once, and the maximum and the codes come from those
// registers.  The same fp32 operations per element as the kernels above.
// ---------------------------------------------------------------------------
template <class In, int NC, bool NORM, bool STATIC, int QF>
__global__ __launch_bounds__(256) void k_quant_act_row(const typename In::elem* __restrict__ x,
                                                       int64_t T, int64_t K, int64_t ld,
                                                       const float* __restrict__ gamma_f,
                                                       float eps,
                                                       const float* __restrict__ static_scale,
                                                       int8_t* __restrict__ xq,
                                                       float* __restrict__ xscale,
                                                       float* __restrict__ rrow) {
  __shared__ double red_d[4];
  __shared__ float red_f[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = (int)(K >> 3);   // <= 256 * NC
  const int64_t r = blockIdx.x;
  const typename In::elem* row = x + r * ld;
  typename In::Raw raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = c * 256 + threadIdx.x;
    raw[c] = In::raw8_nt(row + (ch < nchunk ? ch : 0) * 8);   // read once
  }
  // gamma_f of the thread's chunks, two 16-byte loads each, in flight with
  // the row (read element by element, each load waited for in turn, they
  // cost 2048 x 4096 19.8 -> 7.0 us)
  f32x4 gv[NC][2];
  if (gamma_f != nullptr) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = c * 256 + threadIdx.x;
      const float* gp = gamma_f + (ch < nchunk ? ch : 0) * 8;
      gv[c][0] = *reinterpret_cast<const f32x4*>(gp);
      gv[c][1] = *reinterpret_cast<const f32x4*>(gp + 4);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) gv[c][0] = gv[c][1] = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
  }
  // (keep every load here, ahead of their first use)
  __builtin_amdgcn_sched_barrier(0);
  float rt = 1.0f;
  if (NORM) {
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float v[8];
      In::widen(raw[c], v);
      if (c * 256 + (int)threadIdx.x < nchunk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double dv = (double)v[i];
          ss = fma(dv, dv, ss);   // exact square, so the same as mul + add
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) red_d[wave] = ss;
    __syncthreads();
    ss = (red_d[0] + red_d[1]) + (red_d[2] + red_d[3]);
    rt = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    if (rrow != nullptr && threadIdx.x == 0) rrow[r] = rt;
  }
  float xh[NC][8];
  float am = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = c * 256 + threadIdx.x;
    float v[8];
    In::widen(raw[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = NORM ? v[i] * rt : v[i];
      xh[c][i] = t * (i < 4 ? gv[c][0][i] : gv[c][1][i - 4]);   // exact when gamma_f is NULL
    }
    if (ch < nchunk)
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(xh[c][i]));
  }
  if (!STATIC) {
    am = wave_max(am);
    if (lane == 0) red_f[wave] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  }
  const float d = STATIC ? static_scale[0] : am / (QF == QF_FP8 ? 448.0f : 127.0f);
  if (threadIdx.x == 0) xscale[r] = d;
  const float rc = 1.0f / d;
  const bool fast = d > 0.0f && rc <= 3.0e38f;
  const float rlo = rc * (1.0f - 0x1p-20f), rhi = rc * (1.0f + 0x1p-20f);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = c * 256 + threadIdx.x;
    if (ch >= nchunk) continue;
    u32x2 q;
    q[0] = 0u;
    q[1] = 0u;
    if constexpr (QF == QF_FP8) {
      bool split = true;
      if (fast) q = quant8_fp8_rc<STATIC>(xh[c], rlo, rhi, split);
      if (split) q = quant8_fp8<STATIC>(xh[c], d);
    } else {
      bool tie = true;
      if (fast) q = quant8<STATIC>(xh[c], rc, tie);
      if (d > 0.0f && tie) q = quant8_div<STATIC>(xh[c], d);
    }
    *reinterpret_cast<u32x2*>(xq + r * K + ch * 8) = q;
  }
}

// ---------------------------------------------------------------------------
// LayerNorm form ("SmoothQuant: Weight-Only vs W8A8", Integration with
// Transformers: 1/s folded into the LayerNorm's gamma and beta):
//   m_t = fp32(mean), r_t = fp32(1/sqrt(var + eps)) (one pass of fp64 sums
//   shifted by the row's first element, ln_stats), x^ =
//   fp32(fp32(fp32(h - m_t) * r_t) * gamma'_k) +
//   beta'_k, then the per-token INT8 quantizer above.
// K <= 2048: one token per wave, the row's raw values in
// VGPRs from the load to the store; gamma' and beta' come through the caches
// (every token reads the same K floats).  Wider rows: k_quant_act_ln_row.
// ---------------------------------------------------------------------------
template <class In, int NV>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_quant_act_ln(
    const typename In::elem* __restrict__ x, int64_t T, int64_t K, int64_t ld,
    const float* __restrict__ gamma_f, const float* __restrict__ beta_f, float eps,
    int8_t* __restrict__ xq, float* __restrict__ xscale, float* __restrict__ mrow,
    float* __restrict__ rrow) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = (int)(K >> 3);
  const int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (r >= T) return;
  const typename In::elem* row = x + r * ld;
  typename In::Raw raw[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int ch = j * 64 + lane;
    raw[j] = In::raw8_nt(row + (ch < nchunk ? ch : 0) * 8);   // read once
  }
  // the norm's statistics in one pass, shifted by the row's first element
  // (ln_stats)
  double c;
  {
    float v0[8];
    In::widen(raw[0], v0);
    c = (double)__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v0[0])));
  }
  double s1 = 0.0, s2 = 0.0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float v[8];
    In::widen(raw[j], v);
    if (j * 64 + lane < nchunk)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double d = (double)v[i] - c;
        s1 += d;
        s2 = fma(d, d, s2);
      }
  }
  float mt, rt;
  ln_stats(c, wave_sum(s1), wave_sum(s2), K, eps, mt, rt);
  if (lane == 0) {
    if (mrow != nullptr) mrow[r] = mt;
    if (rrow != nullptr) rrow[r] = rt;
  }
  auto smooth = [&](int j, float (&xh)[8]) {
    const int ch = j * 64 + lane;
    float v[8];
    In::widen(raw[j], v);
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma_f + ch * 8);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma_f + ch * 8 + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(beta_f + ch * 8);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(beta_f + ch * 8 + 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float n = (v[i] - mt) * rt;
      xh[i] = n * (i < 4 ? g0[i] : g1[i - 4]) + (i < 4 ? b0[i] : b1[i - 4]);
    }
  };
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    if (j * 64 + lane < nchunk) {
      float xh[8];
      smooth(j, xh);
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(xh[i]));
    }
  }
  am = wave_max(am);
  const float d = am / 127.0f;
  const float rc = 1.0f / d;
  const bool fast = rc <= 3.0e38f;
  const float rcu = fast ? rc : 0.0f;
  const bool all_div = !fast && d > 0.0f;
  if (lane == 0) xscale[r] = d;
  int8_t* qrow = xq + r * K;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int ch = j * 64 + lane;
    if (ch < nchunk) {
      float xh[8];
      smooth(j, xh);
      bool tie;
      u32x2 c = quant8(xh, rcu, tie);
      if (tie || all_div) c = quant8_div(xh, d);
      *reinterpret_cast<u32x2*>(qrow + ch * 8) = c;
    }
  }
}

// K > 4096: one workgroup per token, four passes over the row (sum, squared
// deviations, maximum, quantize); the re-reads hit L2.
template <class In>
__global__ __launch_bounds__(256) void k_quant_act_ln_wide(
    const typename In::elem* __restrict__ x, int64_t T, int64_t K, int64_t ld,
    const float* __restrict__ gamma_f, const float* __restrict__ beta_f, float eps,
    int8_t* __restrict__ xq, float* __restrict__ xscale, float* __restrict__ mrow,
    float* __restrict__ rrow) {
  __shared__ double red_d[4];
  __shared__ float red_f[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nchunk = K >> 3;
  const int64_t r = blockIdx.x;
  const typename In::elem* row = x + r * ld;
  auto block_sum = [&](double v) {
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red_d[wave] = v;
    __syncthreads();
    return (red_d[0] + red_d[1]) + (red_d[2] + red_d[3]);
  };
  // the norm's statistics in one pass, shifted by the row's first element
  // (ln_stats)
  double c;
  {
    float v0[8];
    In::load8(row, v0);
    c = (double)v0[0];
  }
  double s1 = 0.0, s2 = 0.0;
  for (int64_t ch = threadIdx.x; ch < nchunk; ch += 256) {
    float v[8];
    In::load8(row + ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double dd = (double)v[i] - c;
      s1 += dd;
      s2 = fma(dd, dd, s2);
    }
  }
  s1 = block_sum(s1);
  s2 = block_sum(s2);
  float mt, rt;
  ln_stats(c, s1, s2, K, eps, mt, rt);
  if (threadIdx.x == 0) {
    if (mrow != nullptr) mrow[r] = mt;
    if (rrow != nullptr) rrow[r] = rt;
  }
  auto smooth = [&](int64_t ch, float (&xh)[8]) {
    float v[8];
    In::load8(row + ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) xh[i] = (v[i] - mt) * rt * gamma_f[ch * 8 + i] + beta_f[ch * 8 + i];
  };
  float am = 0.0f;
  for (int64_t ch = threadIdx.x; ch < nchunk; ch += 256) {
    float xh[8];
    smooth(ch, xh);
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(xh[i]));
  }
  am = wave_max(am);
  if (lane == 0) red_f[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  const float d = am / 127.0f;
  const float rc = 1.0f / d;
  const bool fast = rc <= 3.0e38f;
  if (threadIdx.x == 0) xscale[r] = d;
  for (int64_t ch = threadIdx.x; ch < nchunk; ch += 256) {
    float xh[8];
    smooth(ch, xh);
    u32x2 c;
    c[0] = 0u;
    c[1] = 0u;
    bool tie = true;
    if (fast) c = quant8(xh, rc, tie);
    if (d > 0.0f && tie) c = quant8_div(xh, d);
    *reinterpret_cast<u32x2*>(xq + r * K + ch * 8) = c;
  }
}

// LayerNorm rows of 4097-16384 values: one workgroup of 256 threads per
// token with the row in registers (chunk c * 256 + thread, NC per thread, all
// loads issued at once); the same operations and sum orders per thread as
// k_quant_act_ln_wide, without its re-reads.
template <class In, int NC>
__global__ __launch_bounds__(256) void k_quant_act_ln_row(
    const typename In::elem* __restrict__ x, int64_t T, int64_t K, int64_t ld,
    const float* __restrict__ gamma_f, const float* __restrict__ beta_f, float eps,
    int8_t* __restrict__ xq, float* __restrict__ xscale, float* __restrict__ mrow,
    float* __restrict__ rrow) {
  __shared__ double red_d[4];
  __shared__ float red_f[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = (int)(K >> 3);   // <= 256 * NC
  const int64_t r = blockIdx.x;
  const typename In::elem* row = x + r * ld;
  typename In::Raw raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = c * 256 + threadIdx.x;
    raw[c] = In::raw8_nt(row + (ch < nchunk ? ch : 0) * 8);   // read once
  }
  // (every row load issued before the first is used: otherwise the scheduler
  // waits for each chunk before issuing the next; 8192 x 4096 33.1 -> 32.0 us)
  __builtin_amdgcn_sched_barrier(0);
  auto block_sum = [&](double v) {
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red_d[wave] = v;
    __syncthreads();
    return (red_d[0] + red_d[1]) + (red_d[2] + red_d[3]);
  };
  // the norm's statistics in one pass, shifted by the row's first element
  // (ln_stats)
  double sh;
  {
    float v0[8];
    In::load8(row, v0);
    sh = (double)v0[0];
  }
  double s1 = 0.0, s2 = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float v[8];
    In::widen(raw[c], v);
    if (c * 256 + (int)threadIdx.x < nchunk)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double dd = (double)v[i] - sh;
        s1 += dd;
        s2 = fma(dd, dd, s2);
      }
  }
  s1 = block_sum(s1);
  s2 = block_sum(s2);
  float mt, rt;
  ln_stats(sh, s1, s2, K, eps, mt, rt);
  if (threadIdx.x == 0) {
    if (mrow != nullptr) mrow[r] = mt;
    if (rrow != nullptr) rrow[r] = rt;
  }
  float xh[NC][8];
  float am = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = c * 256 + threadIdx.x;
    const int cs = ch < nchunk ? ch : 0;
    float v[8];
    In::widen(raw[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xh[c][i] = (v[i] - mt) * rt * gamma_f[cs * 8 + i] + beta_f[cs * 8 + i];
    if (ch < nchunk)
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(xh[c][i]));
  }
  am = wave_max(am);
  if (lane == 0) red_f[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  const float d = am / 127.0f;
  const float rc = 1.0f / d;
  const bool fast = rc <= 3.0e38f;
  if (threadIdx.x == 0) xscale[r] = d;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = c * 256 + threadIdx.x;
    if (ch >= nchunk) continue;
    u32x2 q;
    q[0] = 0u;
    q[1] = 0u;
    bool tie = true;
    if (fast) q = quant8(xh[c], rc, tie);
    if (d > 0.0f && tie) q = quant8_div(xh[c], d);
    *reinterpret_cast<u32x2*>(xq + r * K + ch * 8) = q;
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------

template <class In, int NV, bool NORM, bool STATIC, int QF>
static void quant_act_nv(const void* x, int64_t T, int64_t K, int64_t ld, const float* gamma_f,
                         float eps, const float* sscale, int8_t* xq, float* xscale, float* rrow,
                         hipStream_t st) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((k_quant_act<In, NV, NORM, STATIC, QF>), dim3((unsigned)blocks),
                     dim3(64 * kWavesPerBlock), 0, st, (const typename In::elem*)x, T, K, ld,
                     gamma_f, eps, sscale, xq, xscale, rrow);
}

template <class In, bool NORM, bool STATIC, int QF>
static void quant_act_t(const void* x, int64_t T, int64_t K, int64_t ld, const float* gamma_f,
                        float eps, const float* sscale, int8_t* xq, float* xscale, float* rrow,
                        hipStream_t st) {
  const int64_t nchunk = K / 8;
#define SQ_QAR(NC)                                                                            \
  hipLaunchKernelGGL((k_quant_act_row<In, NC, NORM, STATIC, QF>), dim3((unsigned)T), dim3(256), \
                     0, st, (const typename In::elem*)x, T, K, ld, gamma_f, eps, sscale, xq,   \
                     xscale, rrow)
  // Up to 4096 tokens of 4096-16384 values: a workgroup per token (four
  // waves share the row, gamma_f through the caches) instead of a wave per
  // token, which leaves much of the chip idle at few tokens and gives each
  // wave a long serial row (µs, one wave / workgroup per token: 16 x 8192
  // 6.5 / 4.2, 512 x 4096 RMSNorm 7.3 / 4.5, 1024 x 4096 6.6 / 4.5, 2048 x
  // 4096 7.6 / 7.0, 4096 x 4096 12.3 / 12.1, 1024 x 14336 RMSNorm 23.0 /
  // 13.9); at 8192 tokens the wave per token, which stages gamma_f once per
  // eight tokens, wins (8192 x 4096 20.5 / 21.2)
  if (T <= 4096 && nchunk >= 512 && nchunk <= 2048) {
    if (nchunk <= 512) SQ_QAR(2);
    else if (nchunk <= 1024) SQ_QAR(4);
    else if (nchunk <= 1536) SQ_QAR(6);
    else SQ_QAR(8);
    return;
  }
#define SQ_QA(NV) \
  quant_act_nv<In, NV, NORM, STATIC, QF>(x, T, K, ld, gamma_f, eps, sscale, xq, xscale, rrow, st)
  if (nchunk <= 64) SQ_QA(1);
  else if (nchunk <= 128) SQ_QA(2);
  else if (nchunk <= 256) SQ_QA(4);
  else if (nchunk <= 512) SQ_QA(8);
  else if (nchunk <= 1024) SQ_QA(16);
  else if (In::kBytes == 2 && nchunk <= 2048 && gamma_f != nullptr) {
    // past 4096 tokens, bf16 rows up to 16384 in VGPRs with gamma_f staged in
    // LDS once per eight tokens, rather than read per token through the
    // caches; with no gamma_f the workgroup per token below
    if constexpr (In::kBytes == 2) SQ_QA(32);
  } else if (nchunk <= 2048) {
    // a workgroup per token with the row in registers, chunks per thread
    // sized to the row
    if (nchunk <= 1536) SQ_QAR(6);
    else SQ_QAR(8);
  } else
    hipLaunchKernelGGL((k_quant_act_wide<In, NORM, STATIC, QF>), dim3((unsigned)T), dim3(256), 0, st,
                       (const typename In::elem*)x, T, K, ld, gamma_f, eps, sscale, xq, xscale,
                       rrow);
#undef SQ_QA
#undef SQ_QAR
}

template <class In, bool NORM>
static void quant_act_s(const void* x, int64_t T, int64_t K, int64_t ld, const float* gamma_f,
                        float eps, const float* sscale, bool fp8, int8_t* xq, float* xscale,
                        float* rrow, hipStream_t st) {
  if (fp8 && sscale)
    quant_act_t<In, NORM, true, QF_FP8>(x, T, K, ld, gamma_f, eps, sscale, xq, xscale, rrow, st);
  else if (fp8)
    quant_act_t<In, NORM, false, QF_FP8>(x, T, K, ld, gamma_f, eps, sscale, xq, xscale, rrow, st);
  else if (sscale)
    quant_act_t<In, NORM, true, QF_INT8>(x, T, K, ld, gamma_f, eps, sscale, xq, xscale, rrow, st);
  else
    quant_act_t<In, NORM, false, QF_INT8>(x, T, K, ld, gamma_f, eps, sscale, xq, xscale, rrow, st);
}

static void quant_act_any(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld, bool norm,
                          const float* gamma_f, float eps, const float* sscale, bool fp8,
                          int8_t* xq, float* xscale, float* rrow, hipStream_t st) {
  if (T <= 0) return;
  if (bf16) {
    if (norm) quant_act_s<Bf16In, true>(x, T, K, ld, gamma_f, eps, sscale, fp8, xq, xscale, rrow, st);
    else quant_act_s<Bf16In, false>(x, T, K, ld, gamma_f, eps, sscale, fp8, xq, xscale, rrow, st);
  } else {
    if (norm) quant_act_s<F32In, true>(x, T, K, ld, gamma_f, eps, sscale, fp8, xq, xscale, rrow, st);
    else quant_act_s<F32In, false>(x, T, K, ld, gamma_f, eps, sscale, fp8, xq, xscale, rrow, st);
  }
}

void launch_quant_act(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld, bool norm,
                      const float* gamma_f, float eps, const float* static_scale, int8_t* xq,
                      float* xscale, float* rrow, hipStream_t st) {
  quant_act_any(x, bf16, T, K, ld, norm, gamma_f, eps, static_scale, false, xq, xscale, rrow, st);
}

void launch_quant_act_fp8(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld, bool norm,
                          const float* gamma_f, float eps, const float* static_scale, uint8_t* xq,
                          float* xscale, float* rrow, hipStream_t st) {
  quant_act_any(x, bf16, T, K, ld, norm, gamma_f, eps, static_scale, true,
                reinterpret_cast<int8_t*>(xq), xscale, rrow, st);
}

template <class In, int NV>
static void quant_act_ln_nv(const void* x, int64_t T, int64_t K, int64_t ld, const float* g,
                            const float* b, float eps, int8_t* xq, float* xscale, float* mrow,
                            float* rrow, hipStream_t st) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((k_quant_act_ln<In, NV>), dim3((unsigned)blocks), dim3(64 * kWavesPerBlock),
                     0, st, (const typename In::elem*)x, T, K, ld, g, b, eps, xq, xscale, mrow,
                     rrow);
}

template <class In>
static void quant_act_ln_t(const void* x, int64_t T, int64_t K, int64_t ld, const float* g,
                           const float* b, float eps, int8_t* xq, float* xscale, float* mrow,
                           float* rrow, hipStream_t st) {
  const int64_t nchunk = K / 8;
#define SQ_LNR(NC)                                                                            \
  hipLaunchKernelGGL((k_quant_act_ln_row<In, NC>), dim3((unsigned)T), dim3(256), 0, st,      \
                     (const typename In::elem*)x, T, K, ld, g, b, eps, xq, xscale, mrow, rrow)
  // Rows of 2049-4096 values: a workgroup per token (gamma' and beta' come
  // through the caches either way, and four waves share each row's chain).
  // µs, wave / workgroup per token, 4096 values: 16 tokens 8.3 / 4.7, 256
  // 8.5 / 5.1, 1024 9.1 / 6.3, 2048 10.7 / 9.5, 8192 34.7 / 30.5.
  if (nchunk > 256 && nchunk <= 512) {
    SQ_LNR(2);
    return;
  }
  if (nchunk <= 64) quant_act_ln_nv<In, 1>(x, T, K, ld, g, b, eps, xq, xscale, mrow, rrow, st);
  else if (nchunk <= 128) quant_act_ln_nv<In, 2>(x, T, K, ld, g, b, eps, xq, xscale, mrow, rrow, st);
  else if (nchunk <= 256) quant_act_ln_nv<In, 4>(x, T, K, ld, g, b, eps, xq, xscale, mrow, rrow, st);
  else if (nchunk <= 512) quant_act_ln_nv<In, 8>(x, T, K, ld, g, b, eps, xq, xscale, mrow, rrow, st);
  else if (nchunk <= 2048) {   // wider rows: a workgroup per token, chunks per
                               // thread sized to the row
    const int nc = (int)((nchunk + 255) / 256);
    if (nc <= 3) SQ_LNR(3);
    else if (nc == 4) SQ_LNR(4);
    else if (nc <= 6) SQ_LNR(6);
    else SQ_LNR(8);
  } else
    hipLaunchKernelGGL((k_quant_act_ln_wide<In>), dim3((unsigned)T), dim3(256), 0, st,
                       (const typename In::elem*)x, T, K, ld, g, b, eps, xq, xscale, mrow, rrow);
#undef SQ_LNR
}

void launch_quant_act_ln(const void* x, bool bf16, int64_t T, int64_t K, int64_t ld,
                         const float* gamma_f, const float* beta_f, float eps, int8_t* xq,
                         float* xscale, float* mrow, float* rrow, hipStream_t st) {
  if (T <= 0) return;
  if (bf16)
    quant_act_ln_t<Bf16In>(x, T, K, ld, gamma_f, beta_f, eps, xq, xscale, mrow, rrow, st);
  else
    quant_act_ln_t<F32In>(x, T, K, ld, gamma_f, beta_f, eps, xq, xscale, mrow, rrow, st);
}

// ---------------------------------------------------------------------------
// Static step from channel maxima: out[0] = fp32( max_j fp32(a[j] * |g[j]|) /
// qmax ), g NULL = 1, qmax 127 (INT8) or 448 (FP8 E4M3).  Rounding is monotone and sign symmetric, so with a[j] the
// channel maximum of |x| (of |fp32(h * r_t)| in norm mode) this is the maximum
// of |x^| over every calibration token and channel.  One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_static_scale(const float* __restrict__ a,
                                                      const float* __restrict__ g, int64_t K,
                                                      float qmax, float* __restrict__ out) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int64_t j = threadIdx.x; j < K; j += 256) m = fmaxf(m, a[j] * (g ? fabsf(g[j]) : 1.0f));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / qmax;
}

void launch_static_scale(const float* a, const float* gamma_f, int64_t K, float qmax, float* out,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_static_scale, dim3(1), dim3(256), 0, st, a, gamma_f, K, qmax, out);
}

}  // namespace sqk
