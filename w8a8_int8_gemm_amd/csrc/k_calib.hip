// k_calib.hip -- calibration kernels for gfx950.
//
//  * k_col_absmax: out[c] = max(out[c], max_r |M[r, c] * rs[r]| / qdiv) over
//    a row-major matrix -- the per-input-channel activation absmax over
//    calibration tokens ("Taming the Outliers", System Architecture step C2,
//    qdiv = 1) and, with rs = s, the per-output-channel step of the smoothed
//    weight (qdiv = 127 or 448).  Division by a positive constant rounds
//    monotonically, so the maximum of the rounded quotients is the rounded
//    quotient of the maximum: the step comes out exact with no extra pass.
//  * k_rms_act_absmax: the same absmax taken of an RMSNorm output computed on
//    the fly (the smoothed linears read a norm's output: "SmoothQuant and
//    W8A8", The trick).
//  * k_ln_act_absmax: the same for a LayerNorm output ("SmoothQuant:
//    Weight-Only vs W8A8", Integration with Transformers), gamma and beta
//    included.
//  * k_wrow_absmax_s: per-input-channel weight absmax and the smoothing
//    factor s_j = a_j^alpha / w_j^(1-alpha) ("06 -- SmoothQuant", section 3).
//
// All three stream HBM once with 16-byte loads; maxima are reduced inside the
// wave, then across the workgroup, then with one unsigned atomic max per
// column (max is order-free, so the result is exact and deterministic).
#include "sq_common.h"
#include "sq_norm.h"
#include "sq_internal.h"

namespace sqk {

__global__ void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Column absmax.  Workgroup = 4 waves over one strip of 512 columns (each lane
// owns 8 consecutive columns = one 16-byte bf16 load per row).  Wave w of
// workgroup (x, y) visits rows y*4 + w, stepping by 4*gridDim.y, U rows per
// step so that U loads are in flight per lane.
// ---------------------------------------------------------------------------
template <class In, bool kRowScale, int U>
__global__ __launch_bounds__(256) void k_col_absmax(const typename In::elem* __restrict__ m,
                                                    int64_t rows, int64_t cols, int64_t ld,
                                                    const float* __restrict__ rs,
                                                    float qdiv, float* __restrict__ out) {
  __shared__ float red[4][512];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t c0 = (int64_t)blockIdx.x * 512 + lane * 8;
  const int64_t nv = cols - c0;   // columns of this lane's 8 that exist
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mx[i] = 0.0f;

  const int64_t step = (int64_t)gridDim.y * 4;
  int64_t r = (int64_t)blockIdx.y * 4 + wave;
  if (nv > 0 && nv < 8) {
    // the ragged end of the rows: the missing columns read as 0; U rows in
    // flight, rows past the end re-read row r and count with scale 0
    const typename In::elem* base = m + c0;
    for (; r < rows; r += U * step) {
      typename In::Raw raw[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = r + u * step < rows;
        const int64_t rr = in ? r + u * step : r;
        raw[u] = In::raw8_part(base + rr * ld, (int)nv);
        sc[u] = in ? (kRowScale ? rs[rr] : 1.0f) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[8];
        In::widen(raw[u], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(v[i] * sc[u]));
      }
    }
  } else if (nv > 0) {
    const typename In::elem* base = m + c0;
    for (; r + (U - 1) * step < rows; r += U * step) {
      // the U rows' loads (and their row scales) all in flight before any use
      typename In::Raw raw[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // the calibration set is read once (non-temporal); a weight with its
        // row scale is read again by the quantizer that follows
        raw[u] = kRowScale ? In::raw8(base + (r + u * step) * ld)
                           : In::raw8_nt(base + (r + u * step) * ld);
        sc[u] = kRowScale ? rs[r + u * step] : 1.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[8];
        In::widen(raw[u], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(kRowScale ? v[i] * sc[u] : v[i]));
      }
    }
    if (r < rows) {
      // the last, partial batch: every remaining row's load in flight at once;
      // rows past the end re-read row r and count with scale 0
      typename In::Raw raw[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = r + u * step < rows;
        const int64_t rr = in ? r + u * step : r;
        raw[u] = kRowScale ? In::raw8(base + rr * ld) : In::raw8_nt(base + rr * ld);
        sc[u] = in ? (kRowScale ? rs[rr] : 1.0f) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[8];
        In::widen(raw[u], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(v[i] * sc[u]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = mx[i];
  __syncthreads();
  // 256 threads fold the 4 waves' partial maxima of 512 columns: 2 columns each
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x + h * 256;
    const int64_t col = (int64_t)blockIdx.x * 512 + c;
    if (col < cols) {
      const float v = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
      atomic_max_nonneg(out + col, v / qdiv);
    }
  }
}

// ---------------------------------------------------------------------------
// Norm-mode calibration absmax.  One wave per row: lane l owns the 8-element
// chunks l, l+64, l+128, ... (NV of them), so a row is NV coalesced 1 KiB
// loads per wave.  Per row: r_t from the fp64 sum of squares, then the running
// maximum of |fp32(h * r_t)| per column.  Rounding is monotone and sign
// symmetric, so max_t |fp32(fp32(h*r_t) * gamma_j)| = fp32(max_t |fp32(h*r_t)|
// * |gamma_j|): gamma is applied once per column at the end, exactly.
// ---------------------------------------------------------------------------
template <class In, int NV>
__global__ __launch_bounds__(256) void k_rms_act_absmax(const typename In::elem* __restrict__ h,
                                                        int64_t rows, int64_t K, int64_t ld,
                                                        const float* __restrict__ gamma, float eps,
                                                        float* __restrict__ out) {
  extern __shared__ unsigned int lmax[];   // [K] running maxima (float bits)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nchunk = K >> 3;
  for (int64_t c = threadIdx.x; c < K; c += 256) lmax[c] = 0u;

  float mx[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) mx[j][i] = 0.0f;
  const double deps = (double)eps;
  const double dK = (double)K;
  const int64_t rstep = (int64_t)gridDim.x * 4;
  int64_t r = (int64_t)blockIdx.x * 4 + wave;
  // K <= 2048: the next row's values are loaded while this row is reduced
  // (60.5 -> 52.6 us over 65536 x 2048 bf16; no gain at K = 4096, and above
  // that the second copy no longer fits the register budget)
  constexpr bool kPrefetch = NV <= 4;
  typename In::Raw nxt[kPrefetch ? NV : 1];
  auto load_row = [&](int64_t rr, typename In::Raw* dst) {
    const typename In::elem* row = h + (rr < rows ? rr : rows - 1) * ld;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t ch = (int64_t)j * 64 + lane;
      dst[j] = In::raw8_nt(row + (ch < nchunk ? ch : 0) * 8);   // read once
    }
  };
  if (kPrefetch && r < rows) load_row(r, nxt);
  for (; r < rows; r += rstep) {
    typename In::Raw raw[NV];
    if (kPrefetch) {
#pragma unroll
      for (int j = 0; j < NV; ++j) raw[j] = nxt[kPrefetch ? j : 0];
      if (r + rstep < rows) load_row(r + rstep, nxt);
    } else {
      load_row(r, raw);
    }
    // squares of bf16/fp32 values are exact in fp64, so fma == mul + add here
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t ch = (int64_t)j * 64 + lane;
      float v[8];
      In::widen(raw[j], v);
      if (ch < nchunk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double d = (double)v[i];
          ss = fma(d, d, ss);
        }
      }
    }
    ss = wave_sum(ss);
    const float rt = (float)(1.0 / sqrt(ss / dK + deps));
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[8];
      In::widen(raw[j], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[j][i] = fmaxf(mx[j][i], fabsf(v[i] * rt));
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t ch = (int64_t)j * 64 + lane;
    if (ch < nchunk)
#pragma unroll
      for (int i = 0; i < 8; ++i) atomicMax(&lmax[ch * 8 + i], __float_as_uint(mx[j][i]));
  }
  __syncthreads();
  for (int64_t c = threadIdx.x; c < K; c += 256) {
    const float g = gamma ? fabsf(gamma[c]) : 1.0f;
    atomic_max_nonneg(out + c, __uint_as_float(lmax[c]) * g);
  }
}

// ---------------------------------------------------------------------------
// LayerNorm-mode calibration absmax, K <= 4096.  Same row-per-wave layout.
// Per row: the fp64 mean and variance (one pass of sums shifted by the row's
// first element, ln_stats), m_t = fp32(mean) and r_t = fp32(1/sqrt(var +
// eps)); then every element's
// norm output x = fp32(fp32(fp32(h - m_t) * r_t) * gamma_j) + beta_j, exactly
// as the norm forms it, and the running maximum of |x| per column -- one
// value per column in registers (tracking the maximum and minimum of the
// normalized value and applying gamma and beta at the end needs two, and
// twice the registers).  gamma and beta are staged once per workgroup in LDS
// and read there chunk by chunk.  Wider rows take k_ln_act_absmax_wide.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned int ordered_bits(float f) {
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(unsigned int o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <class In, int NV>
__global__ __launch_bounds__(256) void k_ln_act_absmax(const typename In::elem* __restrict__ h,
                                                       int64_t rows, int64_t K, int64_t ld,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, float eps,
                                                       float* __restrict__ out) {
  // gamma and beta of chunk c: elements 0-3 at [c], 4-7 at [NV * 64 + c]
  __shared__ f32x4 gsm[NV * 64 * 2];
  __shared__ f32x4 bsm[NV * 64 * 2];
  __shared__ unsigned int lmax[NV * 512];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = (int)(K >> 3);
  for (int i = threadIdx.x; i < NV * 64 * 2; i += 256) {
    const int ch = i % (NV * 64), half = i / (NV * 64);
    f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f}, bt = g;
    if (ch < nchunk) {
      g = gamma ? *reinterpret_cast<const f32x4*>(gamma + ch * 8 + half * 4)
                : f32x4{1.0f, 1.0f, 1.0f, 1.0f};
      if (beta) bt = *reinterpret_cast<const f32x4*>(beta + ch * 8 + half * 4);
    }
    gsm[i] = g;
    bsm[i] = bt;
  }
  for (int c = threadIdx.x; c < NV * 512; c += 256) lmax[c] = 0u;
  __syncthreads();
  const uint32_t gaddr = lds_addr(&gsm[lane]);
  const uint32_t baddr = lds_addr(&bsm[lane]);
  float mx[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) mx[j][i] = 0.0f;
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < rows; r += (int64_t)gridDim.x * 4) {
    typename In::Raw raw[NV];
    const typename In::elem* row = h + r * ld;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int ch = j * 64 + lane;
      raw[j] = In::raw8_nt(row + (ch < nchunk ? ch : 0) * 8);   // read once
    }
    // one pass of shifted fp64 sums (ln_stats), shifted by the row's first
    // element; against sums about the mean in a second pass: 16384 x 4096
    // 52.7 -> 44.9 us, 65536 x 4096 153.6 -> 126.5 us, same maxima
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
#pragma unroll
    for (int j = 0; j < NV; ++j) In::opaque(raw[j]);
    static_for<NV>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      float v[8];
      In::widen(raw[j], v);
      // gamma and beta of this chunk from LDS, the wait in the same asm block
      // (the compiler cannot then hoist every chunk's values into VGPRs);
      // early-clobber outputs, so that no read's data can land in a register
      // that a later read still takes its address from
      f32x4 g0, g1, b0, b1;
      asm volatile(
          "ds_read_b128 %0, %4 offset:%6\n\tds_read_b128 %1, %4 offset:%7\n\t"
          "ds_read_b128 %2, %5 offset:%6\n\tds_read_b128 %3, %5 offset:%7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(g0), "=&v"(g1), "=&v"(b0), "=&v"(b1)
          : "v"(gaddr), "v"(baddr), "n"(j * 1024), "n"(NV * 1024 + j * 1024)
          : "memory");
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float n = (v[i] - mt) * rt;
        const float x = n * (i < 4 ? g0[i] : g1[i - 4]) + (i < 4 ? b0[i] : b1[i - 4]);
        mx[j][i] = fmaxf(mx[j][i], fabsf(x));
      }
    });
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int ch = j * 64 + lane;
    if (ch < nchunk)
#pragma unroll
      for (int i = 0; i < 8; ++i) atomicMax(&lmax[ch * 8 + i], __float_as_uint(mx[j][i]));
  }
  __syncthreads();
  for (int c = threadIdx.x; c < K; c += 256) atomic_max_nonneg(out + c, __uint_as_float(lmax[c]));
}

// ---------------------------------------------------------------------------
// Wide rows (K > 8192) in norm mode: the column maxima no longer fit in
// registers, so they live in LDS.  A workgroup owns a slice of CS columns
// (the slices of one row range run as blockIdx.y); each wave takes one row at
// a time, reads it whole for the norm's statistics (fp64 sums, as the narrow
// kernels), then reads its slice again -- from L2, the row is a few tens of
// KiB -- and raises the slice maxima with LDS atomics.  Column c of the slice
// sits at index c + c/64, so the 64 lanes' stride-8 updates fall on 64
// different banks.
// ---------------------------------------------------------------------------
constexpr int kWideCS = 16384;   // columns per slice
constexpr int kWideLds = kWideCS + kWideCS / 64;

__device__ __forceinline__ int wide_idx(int c) { return c + (c >> 6); }

// fp64 sum over the row of f(v) for every element v (chunks of 8, 4 loads in
// flight per lane), reduced across the wave
template <class In, class F>
__device__ __forceinline__ double wide_row_sum(const typename In::elem* row, int64_t nchunk,
                                               int lane, F f) {
  double acc = 0.0;
  int64_t ch = lane;
  for (; ch + 3 * 64 < nchunk; ch += 4 * 64) {
    typename In::Raw raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[u] = In::raw8(row + (ch + u * 64) * 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float v[8];
      In::widen(raw[u], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += f((double)v[i]);
    }
  }
  for (; ch < nchunk; ch += 64) {
    float v[8];
    In::load8(row + ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += f((double)v[i]);
  }
  return wave_sum(acc);
}

// the LayerNorm statistics' shifted sums over the row (ln_stats): s1 =
// sum(v - c), s2 = sum((v - c)^2), in one pass with the same load pattern
template <class In>
__device__ __forceinline__ void wide_row_shifted_sums(const typename In::elem* row, int64_t nchunk,
                                                      int lane, double c, double& s1,
                                                      double& s2) {
  double a1 = 0.0, a2 = 0.0;
  auto add8 = [&](const float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double d = (double)v[i] - c;
      a1 += d;
      a2 = fma(d, d, a2);
    }
  };
  int64_t ch = lane;
  for (; ch + 3 * 64 < nchunk; ch += 4 * 64) {
    typename In::Raw raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[u] = In::raw8(row + (ch + u * 64) * 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float v[8];
      In::widen(raw[u], v);
      add8(v);
    }
  }
  for (; ch < nchunk; ch += 64) {
    float v[8];
    In::load8(row + ch * 8, v);
    add8(v);
  }
  s1 = wave_sum(a1);
  s2 = wave_sum(a2);
}

template <class In>
__global__ __launch_bounds__(512) void k_rms_act_absmax_wide(const typename In::elem* __restrict__ h,
                                                             int64_t rows, int64_t K, int64_t ld,
                                                             const float* __restrict__ gamma,
                                                             float eps, float* __restrict__ out) {
  __shared__ unsigned int lmax[kWideLds];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c_lo = (int64_t)blockIdx.y * kWideCS;
  const int cw = (int)min((int64_t)kWideCS, K - c_lo);   // a multiple of 64
  for (int c = threadIdx.x; c < kWideLds; c += 512) lmax[c] = 0u;
  __syncthreads();
  const int64_t nchunk = K >> 3;
  const double dK = (double)K;
  for (int64_t r = (int64_t)blockIdx.x * 8 + wave; r < rows; r += (int64_t)gridDim.x * 8) {
    const typename In::elem* row = h + r * ld;
    // squares of bf16/fp32 values are exact in fp64
    const double ss = wide_row_sum<In>(row, nchunk, lane, [](double d) { return d * d; });
    const float rt = (float)(1.0 / sqrt(ss / dK + (double)eps));
    for (int ch = lane; ch < (cw >> 3); ch += 64) {
      float v[8];
      In::load8(row + c_lo + (int64_t)ch * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        atomicMax(&lmax[wide_idx(ch * 8 + i)], __float_as_uint(fabsf(v[i] * rt)));
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < cw; c += 512) {
    const float g = gamma ? fabsf(gamma[c_lo + c]) : 1.0f;
    atomic_max_nonneg(out + c_lo + c, __uint_as_float(lmax[wide_idx(c)]) * g);
  }
}

// LayerNorm form of the wide path: the mean and variance (one pass of shifted
// fp64 sums over the row, ln_stats), then the slice's running maximum and
// minimum of n = fp32(fp32(h - m_t) * r_t) as ordered bits in LDS; gamma and
// beta are applied once per column at the end (f(n) monotone, as in
// k_ln_act_absmax).
constexpr int kWideCSLn = 8192;
constexpr int kWideLdsLn = kWideCSLn + kWideCSLn / 64;

template <class In>
__global__ __launch_bounds__(512) void k_ln_act_absmax_wide(const typename In::elem* __restrict__ h,
                                                            int64_t rows, int64_t K, int64_t ld,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta,
                                                            float eps, float* __restrict__ out) {
  __shared__ unsigned int lmax[kWideLdsLn];
  __shared__ unsigned int lmin[kWideLdsLn];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c_lo = (int64_t)blockIdx.y * kWideCSLn;
  const int cw = (int)min((int64_t)kWideCSLn, K - c_lo);
  for (int c = threadIdx.x; c < kWideLdsLn; c += 512) {
    lmax[c] = 0u;            // below every ordered value
    lmin[c] = 0xffffffffu;   // above every ordered value
  }
  __syncthreads();
  const int64_t nchunk = K >> 3;
  bool any = false;
  for (int64_t r = (int64_t)blockIdx.x * 8 + wave; r < rows; r += (int64_t)gridDim.x * 8) {
    any = true;
    const typename In::elem* row = h + r * ld;
    // the norm's statistics in one pass, shifted by the row's first element
    float v0[8];
    In::load8(row, v0);
    double s1, s2;
    wide_row_shifted_sums<In>(row, nchunk, lane, (double)v0[0], s1, s2);
    float mt, rt;
    ln_stats((double)v0[0], s1, s2, K, eps, mt, rt);
    for (int ch = lane; ch < (cw >> 3); ch += 64) {
      float v[8];
      In::load8(row + c_lo + (int64_t)ch * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned int o = ordered_bits((v[i] - mt) * rt);
        atomicMax(&lmax[wide_idx(ch * 8 + i)], o);
        atomicMin(&lmin[wide_idx(ch * 8 + i)], o);
      }
    }
  }
  __syncthreads();
  if (!__syncthreads_or(any)) return;   // this workgroup saw no row
  for (int c = threadIdx.x; c < cw; c += 512) {
    const float g = gamma ? gamma[c_lo + c] : 1.0f;
    const float b = beta ? beta[c_lo + c] : 0.0f;
    const float hi = from_ordered_bits(lmax[wide_idx(c)]) * g + b;
    const float lo = from_ordered_bits(lmin[wide_idx(c)]) * g + b;
    atomic_max_nonneg(out + c_lo + c, fmaxf(fabsf(hi), fabsf(lo)));
  }
}

// ---------------------------------------------------------------------------
// Weight row absmax and smoothing factor.  A workgroup of 4 waves takes 16
// input channels (rows j of the [K, N] weight); each wave streams 4 rows at
// once, U 16-byte loads per row in flight.  s_j = fp32(a_j^alpha /
// w_j^(1-alpha)) in fp64, floored at 1e-5; s_j = 1 for an all-zero row.  The
// fp64 powers run one lane per row, 16 rows at a time, after the maxima meet
// in LDS: a serial power per row would hold a whole wave for each row.
// ---------------------------------------------------------------------------
template <class In, int U>
__global__ __launch_bounds__(256) void k_wrow_absmax_s(const typename In::elem* __restrict__ w,
                                                       int64_t K, int64_t N, int64_t ld,
                                                       const float* __restrict__ a, float alpha,
                                                       float* __restrict__ wmax,
                                                       float* __restrict__ s) {
  __shared__ float rmax[16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t j0 = (int64_t)blockIdx.x * 16 + wave * 4;   // K % 16 == 0: all 4 rows exist
  float mx[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int64_t c = (int64_t)lane * 8;
  for (; c + (U - 1) * 512 + 8 <= N; c += U * 512) {
    typename In::Raw raw[4][U];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < U; ++u) raw[q][u] = In::raw8(w + (j0 + q) * ld + c + u * 512);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[8];
        In::widen(raw[q][u], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx[q] = fmaxf(mx[q], fabsf(v[i]));
      }
  }
  for (; c < N; c += 512) {   // the rest, the ragged end of the rows read as 0
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[8];
      In::widen(raw8_upto<In>(w + (j0 + q) * ld + c, N - c), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[q] = fmaxf(mx[q], fabsf(v[i]));
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) mx[q] = wave_max(mx[q]);
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) rmax[wave * 4 + q] = mx[q];
  __syncthreads();
  if (threadIdx.x < 16) {
    const int64_t j = (int64_t)blockIdx.x * 16 + threadIdx.x;
    const float m = rmax[threadIdx.x];
    wmax[j] = m;
    float sj = 1.0f;
    if (m != 0.0f) {
      const double al = (double)alpha;
      const double q = pow((double)a[j], al) / pow((double)m, 1.0 - al);
      const float f = (float)q;
      sj = f < 1e-5f ? 1e-5f : f;
    }
    s[j] = sj;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

void launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
}

// One workgroup (4 waves, 8 rows in flight per wave) per compute unit at most,
// so every unit streams the same number of rows to within one workgroup, and
// at least 8 rows per wave.  Measured on bf16 inputs rotated past the
// Infinity Cache (us, this rule / about 2048 workgroups of 8 rows per wave):
// 8192 x 4096 14.7 / 17.2; 65536 x 4096 83.1 / 94.8; 262144 x 8192 619 / 729
// (6.9 TB/s); 4096 x 28672 38.1 / 45.2.  Two workgroups per unit, or 16 rows
// in flight per wave, were slower at every shape but 4096 x 14336: the
// memory system serves fewer, longer streams better than the whole matrix
// requested at once.
static int col_absmax_grid_y(int64_t rows, int64_t gx) {
  int64_t gy = (int64_t)cu_count() / gx;
  const int64_t max_gy = (rows + 31) / 32;
  if (gy > max_gy) gy = max_gy;
  if (gy < 1) gy = 1;
  if (gy > 65535) gy = 65535;
  return (int)gy;
}

void launch_col_absmax(const void* m, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                       const float* rs, float qdiv, float* out, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return;
  const int64_t gx = (cols + 511) / 512;
  const dim3 grid((unsigned)gx, (unsigned)col_absmax_grid_y(rows, gx));
  if (bf16) {
    if (rs)
      hipLaunchKernelGGL((k_col_absmax<Bf16In, true, 8>), grid, dim3(256), 0, st,
                         (const uint16_t*)m, rows, cols, ld, rs, qdiv, out);
    else
      hipLaunchKernelGGL((k_col_absmax<Bf16In, false, 8>), grid, dim3(256), 0, st,
                         (const uint16_t*)m, rows, cols, ld, rs, qdiv, out);
  } else {
    if (rs)
      hipLaunchKernelGGL((k_col_absmax<F32In, true, 4>), grid, dim3(256), 0, st,
                         (const float*)m, rows, cols, ld, rs, qdiv, out);
    else
      hipLaunchKernelGGL((k_col_absmax<F32In, false, 4>), grid, dim3(256), 0, st,
                         (const float*)m, rows, cols, ld, rs, qdiv, out);
  }
}

template <class In, int NV>
static void rms_absmax_nv(const void* h, int64_t rows, int64_t K, int64_t ld, const float* gamma,
                          float eps, float* out, hipStream_t st) {
  // 4 waves per workgroup; enough workgroups for ~2 waves per SIMD
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 512) blocks = 512;   // 1024 measured slower at K = 2048 .. 8192
  hipLaunchKernelGGL((k_rms_act_absmax<In, NV>), dim3((unsigned)blocks), dim3(256),
                     (size_t)K * sizeof(float), st, (const typename In::elem*)h, rows, K, ld,
                     gamma, eps, out);
}

template <class In>
static void rms_absmax_t(const void* h, int64_t rows, int64_t K, int64_t ld, const float* gamma,
                         float eps, float* out, hipStream_t st) {
  const int64_t nv = (K + 511) / 512;
  if (nv <= 1) rms_absmax_nv<In, 1>(h, rows, K, ld, gamma, eps, out, st);
  else if (nv <= 2) rms_absmax_nv<In, 2>(h, rows, K, ld, gamma, eps, out, st);
  else if (nv <= 4) rms_absmax_nv<In, 4>(h, rows, K, ld, gamma, eps, out, st);
  else if (nv <= 8) rms_absmax_nv<In, 8>(h, rows, K, ld, gamma, eps, out, st);
  else rms_absmax_nv<In, 16>(h, rows, K, ld, gamma, eps, out, st);
}

// wide rows: 256 row blocks of 8 rows per column slice (2 workgroups per CU)
static dim3 wide_grid(int64_t rows, int64_t K, int cs) {
  int64_t gx = (rows + 7) / 8;
  if (gx > 256) gx = 256;
  return dim3((unsigned)gx, (unsigned)((K + cs - 1) / cs));
}

void launch_rms_act_absmax(const void* h, bool bf16, int64_t rows, int64_t K, int64_t ld,
                           const float* gamma, float eps, float* out, hipStream_t st) {
  if (rows <= 0 || K <= 0) return;
  if (K > 8192) {
    const dim3 g = wide_grid(rows, K, kWideCS);
    if (bf16)
      hipLaunchKernelGGL(k_rms_act_absmax_wide<Bf16In>, g, dim3(512), 0, st, (const uint16_t*)h,
                         rows, K, ld, gamma, eps, out);
    else
      hipLaunchKernelGGL(k_rms_act_absmax_wide<F32In>, g, dim3(512), 0, st, (const float*)h, rows,
                         K, ld, gamma, eps, out);
    return;
  }
  if (bf16) rms_absmax_t<Bf16In>(h, rows, K, ld, gamma, eps, out, st);
  else rms_absmax_t<F32In>(h, rows, K, ld, gamma, eps, out, st);
}

template <class In, int NV>
static void ln_absmax_nv(const void* h, int64_t rows, int64_t K, int64_t ld, const float* gamma,
                         const float* beta, float eps, float* out, hipStream_t st) {
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 512) blocks = 512;
  hipLaunchKernelGGL((k_ln_act_absmax<In, NV>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const typename In::elem*)h, rows, K, ld, gamma, beta, eps, out);
}

template <class In>
static void ln_absmax_t(const void* h, int64_t rows, int64_t K, int64_t ld, const float* gamma,
                        const float* beta, float eps, float* out, hipStream_t st) {
  const int64_t nv = (K + 511) / 512;   // K <= 4096 here
  if (nv <= 1) ln_absmax_nv<In, 1>(h, rows, K, ld, gamma, beta, eps, out, st);
  else if (nv <= 2) ln_absmax_nv<In, 2>(h, rows, K, ld, gamma, beta, eps, out, st);
  else if (nv <= 4) ln_absmax_nv<In, 4>(h, rows, K, ld, gamma, beta, eps, out, st);
  else ln_absmax_nv<In, 8>(h, rows, K, ld, gamma, beta, eps, out, st);
}

void launch_ln_act_absmax(const void* h, bool bf16, int64_t rows, int64_t K, int64_t ld,
                          const float* gamma, const float* beta, float eps, float* out,
                          hipStream_t st) {
  if (rows <= 0 || K <= 0) return;
  // above 4096 columns the per-column maxima in LDS beat those in registers
  // (16384 x 8192 bf16: 136 against 327 us)
  if (K > 4096) {
    const dim3 g = wide_grid(rows, K, kWideCSLn);
    if (bf16)
      hipLaunchKernelGGL(k_ln_act_absmax_wide<Bf16In>, g, dim3(512), 0, st, (const uint16_t*)h,
                         rows, K, ld, gamma, beta, eps, out);
    else
      hipLaunchKernelGGL(k_ln_act_absmax_wide<F32In>, g, dim3(512), 0, st, (const float*)h, rows,
                         K, ld, gamma, beta, eps, out);
    return;
  }
  if (bf16) ln_absmax_t<Bf16In>(h, rows, K, ld, gamma, beta, eps, out, st);
  else ln_absmax_t<F32In>(h, rows, K, ld, gamma, beta, eps, out, st);
}

void launch_wrow_absmax_s(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                          const float* a, float alpha, float* wmax, float* s, hipStream_t st) {
  if (K <= 0) return;
  const dim3 grid((unsigned)(K / 16));   // K % 64 == 0
  if (bf16)
    hipLaunchKernelGGL((k_wrow_absmax_s<Bf16In, 8>), grid, dim3(256), 0, st, (const uint16_t*)w,
                       K, N, ld, a, alpha, wmax, s);
  else
    hipLaunchKernelGGL((k_wrow_absmax_s<F32In, 4>), grid, dim3(256), 0, st, (const float*)w, K, N,
                       ld, a, alpha, wmax, s);
}

}  // namespace sqk
