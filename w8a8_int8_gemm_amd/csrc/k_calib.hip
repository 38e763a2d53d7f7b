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
  const bool active = c0 < cols;   // cols % 8 == 0, so a lane is all-in or all-out
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mx[i] = 0.0f;

  const int64_t step = (int64_t)gridDim.y * 4;
  int64_t r = (int64_t)blockIdx.y * 4 + wave;
  if (active) {
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
    for (; r < rows; r += step) {
      float v[8];
      In::load8(base + r * ld, v);
      const float sc = kRowScale ? rs[r] : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(kRowScale ? v[i] * sc : v[i]));
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
// LayerNorm-mode calibration absmax.  Same row-per-wave layout.  Per row: the
// fp64 mean, the fp64 sum of squared deviations from it, m_t = fp32(mean) and
// r_t = fp32(1/sqrt(var + eps)); then per column the running maximum and
// minimum of n = fp32(fp32(h - m_t) * r_t).  f(n) = fp32(fp32(n * gamma_j) +
// beta_j) is monotone in n (fp32 multiply and add round monotonically), so
// max_t |f(n_t)| = max(|f(max_t n)|, |f(min_t n)|): gamma and beta are applied
// once per column at the end, exactly.  Maxima and minima are combined across
// waves in LDS through an order-preserving map of the float bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned int ordered_bits(float f) {
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(unsigned int o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <class In, int NV, int SPLIT>
__global__ __launch_bounds__(256) void k_ln_act_absmax(const typename In::elem* __restrict__ h,
                                                       int64_t rows, int64_t K, int64_t ld,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, float eps,
                                                       float* __restrict__ out) {
  // SPLIT waves share a row: each takes the whole row for the statistics and
  // keeps the running maximum and minimum of its own NV / SPLIT chunks.
  constexpr int NM = NV / SPLIT;
  constexpr int RPB = 4 / SPLIT;           // rows per workgroup pass
  extern __shared__ unsigned int lmm[];   // [K] maxima, then [K] minima (ordered bits)
  unsigned int* lmax = lmm;
  unsigned int* lmin = lmm + K;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slice = wave % SPLIT;
  const int64_t nchunk = K >> 3;
  for (int64_t c = threadIdx.x; c < K; c += 256) {
    lmax[c] = 0u;            // below every ordered value
    lmin[c] = 0xffffffffu;   // above every ordered value
  }
  float mx[NM][8], mn[NM][8];
#pragma unroll
  for (int j = 0; j < NM; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mx[j][i] = -INFINITY;
      mn[j][i] = INFINITY;
    }
  const double dK = (double)K;
  bool any = false;
  for (int64_t r = (int64_t)blockIdx.x * RPB + wave / SPLIT; r < rows;
       r += (int64_t)gridDim.x * RPB) {
    any = true;
    typename In::Raw raw[NV];
    const typename In::elem* row = h + r * ld;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t ch = (int64_t)j * 64 + lane;
      raw[j] = In::raw8_nt(row + (ch < nchunk ? ch : 0) * 8);   // read once
    }
    double s1 = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[8];
      In::widen(raw[j], v);
      if ((int64_t)j * 64 + lane < nchunk)
#pragma unroll
        for (int i = 0; i < 8; ++i) s1 += (double)v[i];
    }
    const double mu = wave_sum(s1) / dK;
    double s2 = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[8];
      In::widen(raw[j], v);
      if ((int64_t)j * 64 + lane < nchunk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double d = (double)v[i] - mu;
          s2 += d * d;
        }
    }
    s2 = wave_sum(s2);
    const float mt = (float)mu;
    const float rt = (float)(1.0 / sqrt(s2 / dK + (double)eps));
#pragma unroll
    for (int jj = 0; jj < NM; ++jj) {
      float v[8];
      In::widen(raw[slice * NM + jj], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float n = (v[i] - mt) * rt;
        mx[jj][i] = fmaxf(mx[jj][i], n);
        mn[jj][i] = fminf(mn[jj][i], n);
      }
    }
  }
  __syncthreads();
  if (any) {
#pragma unroll
    for (int jj = 0; jj < NM; ++jj) {
      const int64_t ch = (int64_t)(slice * NM + jj) * 64 + lane;
      if (ch < nchunk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          atomicMax(&lmax[ch * 8 + i], ordered_bits(mx[jj][i]));
          atomicMin(&lmin[ch * 8 + i], ordered_bits(mn[jj][i]));
        }
    }
  }
  __syncthreads();
  for (int64_t c = threadIdx.x; c < K; c += 256) {
    if (lmax[c] == 0u) continue;   // this workgroup saw no row
    const float g = gamma ? gamma[c] : 1.0f;
    const float b = beta ? beta[c] : 0.0f;
    const float hi = from_ordered_bits(lmax[c]) * g + b;
    const float lo = from_ordered_bits(lmin[c]) * g + b;
    atomic_max_nonneg(out + c, fmaxf(fabsf(hi), fabsf(lo)));
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
  for (; c + (U - 1) * 512 < N; c += U * 512) {
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
  for (; c < N; c += 512) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[8];
      In::load8(w + (j0 + q) * ld + c, v);
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

static int col_absmax_grid_y(int64_t rows, int64_t gx) {
  // about 2048 workgroups in all, but at least 8 rows per wave
  int64_t gy = (2048 + gx - 1) / gx;
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

void launch_rms_act_absmax(const void* h, bool bf16, int64_t rows, int64_t K, int64_t ld,
                           const float* gamma, float eps, float* out, hipStream_t st) {
  if (rows <= 0 || K <= 0) return;
  if (bf16) rms_absmax_t<Bf16In>(h, rows, K, ld, gamma, eps, out, st);
  else rms_absmax_t<F32In>(h, rows, K, ld, gamma, eps, out, st);
}

template <class In, int NV>
static void ln_absmax_nv(const void* h, int64_t rows, int64_t K, int64_t ld, const float* gamma,
                         const float* beta, float eps, float* out, hipStream_t st) {
  // a lane holds the row's raw chunks plus 16 floats of maxima and minima per
  // chunk it tracks: wider rows share the tracking among 2 or 4 waves
  constexpr int SPLIT = NV >= 16 ? 4 : (NV >= 8 && In::kBytes == 4) ? 2 : 1;
  int64_t blocks = (rows + 4 / SPLIT - 1) / (4 / SPLIT);
  if (blocks > 512) blocks = 512;
  hipLaunchKernelGGL((k_ln_act_absmax<In, NV, SPLIT>), dim3((unsigned)blocks), dim3(256),
                     (size_t)K * 2 * sizeof(unsigned int), st, (const typename In::elem*)h, rows,
                     K, ld, gamma, beta, eps, out);
}

template <class In>
static void ln_absmax_t(const void* h, int64_t rows, int64_t K, int64_t ld, const float* gamma,
                        const float* beta, float eps, float* out, hipStream_t st) {
  const int64_t nv = (K + 511) / 512;
  if (nv <= 1) ln_absmax_nv<In, 1>(h, rows, K, ld, gamma, beta, eps, out, st);
  else if (nv <= 2) ln_absmax_nv<In, 2>(h, rows, K, ld, gamma, beta, eps, out, st);
  else if (nv <= 4) ln_absmax_nv<In, 4>(h, rows, K, ld, gamma, beta, eps, out, st);
  else if (nv <= 8) ln_absmax_nv<In, 8>(h, rows, K, ld, gamma, beta, eps, out, st);
  else ln_absmax_nv<In, 16>(h, rows, K, ld, gamma, beta, eps, out, st);
}

void launch_ln_act_absmax(const void* h, bool bf16, int64_t rows, int64_t K, int64_t ld,
                          const float* gamma, const float* beta, float eps, float* out,
                          hipStream_t st) {
  if (rows <= 0 || K <= 0) return;
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
