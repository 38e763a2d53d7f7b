// k_weight.hip -- offline fold and per-output-channel INT8 weight quantization
// for gfx950.
//
//  * k_fold_gamma: gamma'_j = gamma_j / s_j -- 1/s folded into the preceding
//    norm's weight ("06 -- SmoothQuant", section 7; "SmoothQuant and W8A8",
//    The trick).
//  * k_fold_w: W^[j, n] = W[j, n] * s_j -- s folded into the weight's input
//    rows ("06 -- SmoothQuant", section 2).
//  * k_fold_beta: beta'_j = beta_j / s_j, the LayerNorm bias taking its share
//    of 1/s ("SmoothQuant: Weight-Only vs W8A8", Integration with
//    Transformers).
//  * k_fold_prev: W_prev'[i, j] = W_prev[i, j] / s_j -- 1/s folded into the
//    output columns of the linear whose output is this linear's input ("06 --
//    SmoothQuant", section 7), with its bias b'_j = b_j / s_j.
//  * k_quant_weight_t: codes = round-half-even(W^ / Delta_n) (INT8, rounded
//    by the reciprocal of the step with the IEEE division for near-ties, as
//    k_quant_weight_strip; or the nearest E4M3 value for FP8), written
//    transposed to the [N, K] K-contiguous layout the GEMM streams.
//  * k_quant_weight_strip: the per-output-channel step and the codes of a
//    bf16 weight with K <= 4096 in one launch, one workgroup per 16 output
//    channels (where it beats the path below: quant_weight_strip_ok).
// Otherwise the per-output-channel step between fold and quant is
// k_col_absmax with the row scale s and the divisor 127 (the symmetric 8-bit
// step, "Taming the Outliers", The Problem) or 448 (FP8 E4M3), in
// k_calib.hip, followed by k_quant_weight_t; either way W^ is never
// materialised.
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

__global__ void k_fold_gamma(const float* __restrict__ s, const float* __restrict__ gamma,
                             float* __restrict__ gout, int64_t K) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < K) gout[j] = (gamma ? gamma[j] : 1.0f) / s[j];
}

__global__ void k_fold_beta(const float* __restrict__ s, const float* __restrict__ beta,
                            float* __restrict__ bout, int64_t K) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < K) bout[j] = (beta ? beta[j] : 0.0f) / s[j];
}

// 8 consecutive output columns of one row of W_prev [Kp, K] per thread (the
// bias folds like a LayerNorm beta, k_fold_beta)
template <class In>
__global__ __launch_bounds__(256) void k_fold_prev(const typename In::elem* __restrict__ w,
                                                   int64_t Kp, int64_t K, int64_t ld,
                                                   const float* __restrict__ s,
                                                   float* __restrict__ wout, int64_t ldo) {
  const int64_t chunks_per_row = K >> 3;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= Kp * chunks_per_row) return;
  const int64_t i = c / chunks_per_row;
  const int64_t j0 = (c - i * chunks_per_row) * 8;
  float v[8];
  In::load8(w + i * ld + j0, v);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s + j0);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + j0 + 4);
  f32x4 o0, o1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o0[e] = v[e] / s0[e];
    o1[e] = v[4 + e] / s1[e];
  }
  *reinterpret_cast<f32x4*>(wout + i * ldo + j0) = o0;
  *reinterpret_cast<f32x4*>(wout + i * ldo + j0 + 4) = o1;
}

// 8 consecutive elements of one row per thread (fewer at the ragged end of a
// row; the output rows are 16-byte aligned only when N % 4 == 0)
template <class In>
__global__ __launch_bounds__(256) void k_fold_w(const typename In::elem* __restrict__ w,
                                                int64_t K, int64_t N, int64_t ld,
                                                const float* __restrict__ s,
                                                float* __restrict__ wout) {
  const int64_t chunks_per_row = (N + 7) >> 3;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= K * chunks_per_row) return;
  const int64_t j = c / chunks_per_row;
  const int64_t n0 = (c - j * chunks_per_row) * 8;
  const int64_t nv = N - n0;
  float v[8];
  In::widen(raw8_upto<In>(w + j * ld + n0, nv), v);
  const float sj = s[j];
  if (nv >= 8 && (N & 3) == 0) {
    f32x4 o0, o1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o0[i] = v[i] * sj;
      o1[i] = v[4 + i] * sj;
    }
    *reinterpret_cast<f32x4*>(wout + j * N + n0) = o0;
    *reinterpret_cast<f32x4*>(wout + j * N + n0 + 4) = o1;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nv) wout[j * N + n0 + i] = v[i] * sj;
  }
}

// Tile of 128 input channels (k) x 64 output channels (n).  Thread (tx, ty),
// tx = tid % 8, ty = tid / 8: columns n0 + 8*tx .. +7 of rows k0 + 4*ty .. +3.
// Each thread packs its 4 codes per column (4 consecutive k) into one dword of
// the LDS tile [n][k]; the tile is then written out 32 bytes per thread along k.
template <class In, bool kRowScale, bool F8>
__global__ __launch_bounds__(256) void k_quant_weight_t(const typename In::elem* __restrict__ w,
                                                        int64_t K, int64_t N, int64_t ld,
                                                        const float* __restrict__ s,
                                                        const float* __restrict__ wscale,
                                                        int8_t* __restrict__ wq) {
  constexpr int KT = 128, NT = 64, LDT = KT + 4;   // padded row of the [n][k] tile
  __shared__ uint32_t tile[NT * LDT / 4];
  const int tid = threadIdx.x;
  const int tx = tid & 7, ty = tid >> 3;
  const int64_t n0 = (int64_t)blockIdx.x * NT;
  const int64_t k0 = (int64_t)blockIdx.y * KT;
  const int64_t nb = n0 + tx * 8;
  const bool ncol = nb < N;
  const int64_t nv = ncol ? N - nb : 8;   // columns of the thread's 8 that exist

  float d[8];
  F32In::widen(ncol ? raw8_upto<F32In>(wscale + nb, nv) : F32In::raw8_part(wscale, 0), d);

  // all four rows' loads in flight at once (rows past K read row K-1 and
  // are dropped; columns past N read column 0 and are dropped)
  typename In::Raw raw[4];
  float sk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t k = min(k0 + ty * 4 + r, K - 1);
    raw[r] = raw8_upto<In>(w + k * ld + (ncol ? nb : 0), nv);
    sk[r] = kRowScale ? s[k] : 1.0f;
  }
  uint32_t packed[8];
  // W^ (0 for rows past K and columns past N, whose codes are never written)
  float wh[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t k = k0 + ty * 4 + r;
    float v[8];
    In::widen(raw[r], v);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      wh[r][i] = (ncol && k < K) ? (kRowScale ? v[i] * sk[r] : v[i]) : 0.0f;
  }
  if (F8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // the IEEE quotient, then the nearest E4M3, ties to even; |quotient|
      // <= 448 up to one rounding except for a deep subnormal step, so it
      // clips to the largest finite code first
      float q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        q[r] = d[i] != 0.0f ? fminf(fmaxf(wh[r][i] / d[i], -448.0f), 448.0f) : 0.0f;
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
      packed[i] = (uint32_t)w;
    }
  } else {
    // rounding by the reciprocal, as k_quant_weight_strip: y + 1.5 * 2^23
    // rounds y to an integer (ties to even) with the code in its low byte;
    // near-ties, zero steps and overflowing reciprocals take the division
    constexpr float kMagic = 12582912.0f;
    float rc[8];
    bool slow = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rc[i] = 1.0f / d[i];
      slow |= !(rc[i] < INFINITY);
    }
    float dm = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t tb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float y = wh[r][i] * rc[i];
        const float tq = y + kMagic;
        dm = fmaxf(dm, fabsf(y - (tq - kMagic)));
        tb[r] = __float_as_uint(tq);
      }
      const uint32_t lo = __builtin_amdgcn_perm(tb[1], tb[0], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(tb[3], tb[2], 0x04000c0cu);
      packed[i] = lo | hi;
    }
    if (slow || !(dm <= kTieBand)) {
      // rare: the division for only the values near a tie (every value when
      // a reciprocal overflowed); a wave runs a value's division only if one
      // of its lanes needs it
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // y recomputed (rc made opaque, so the fast pass keeps no y alive)
          float rci = rc[i];
          asm volatile("" : "+v"(rci));
          const float y = wh[r][i] * rci;   // rint(y) = tq - 1.5 * 2^23 of the fast pass
          if (slow || !(fabsf(y - rintf(y)) <= kTieBand)) {
            const float q = d[i] != 0.0f ? rintf(wh[r][i] / d[i]) : 0.0f;
            packed[i] = (packed[i] & ~(0xffu << (8 * r))) |
                        (code_byte(fminf(fmaxf(q, -127.0f), 127.0f)) << (8 * r));
          }
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) tile[((tx * 8 + i) * LDT + ty * 4) / 4] = packed[i];
  __syncthreads();
  // write out: 64 rows (n) x 128 bytes (k); thread -> row tid/4, 32 bytes at (tid%4)*32
  const int nr = tid >> 2;
  const int seg = (tid & 3) * 32;
  const int64_t n = n0 + nr;
  if (n < N && k0 + seg < K) {
    const uint32_t* src = &tile[(nr * LDT + seg) / 4];
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = src[i];
      b[i] = src[4 + i];
    }
    int8_t* dst = wq + n * K + k0 + seg;
    *reinterpret_cast<u32x4*>(dst) = a;
    *reinterpret_cast<u32x4*>(dst + 16) = b;
  }
}

// ---------------------------------------------------------------------------
// One-launch quantization of a bf16 weight with K <= 4096.  A workgroup of NT
// threads owns a strip of 16 output channels (columns n0 .. n0+15 of the
// [K, N] weight) and holds the whole strip in registers as W^ = W * s: thread
// t = 2*rt + h has the 8 columns n0 + 8h .. +7 of the rows 4*(rt + RT*m) + r
// (RT = NT/2 row threads, m < M, r < 4), all loads in flight at once.  The
// column maxima of |W^| are reduced across the workgroup and written as the
// steps directly: the strip is the only writer of its columns, so there is
// no fill and no atomic.  The codes are packed four rows to a dword into an
// LDS tile [16][2048 bytes] and written out K-contiguous, 2048 values of k at
// a time.  Strips go to the XCDs in contiguous runs, so the four strips that
// share the 128-byte lines of a row share one L2.
//
// INT8 rounding by the reciprocal of the step (kTieBand): the bound there
// holds since |W^ / Delta| <= 127 / (1 - 2^-24) < 128 whenever 1/Delta is
// finite (Delta > 2^-128, so its own rounding error is below 2^-22 of it).
// y + 1.5 * 2^23 rounds y to an integer, ties to even, and leaves that integer
// in the low bits of the sum: its low byte is the code, and subtracting the
// constant back gives rint(y) exactly for the tie check.  |y| < 127.5, so no
// clamp is needed on this path.  FP8 takes the IEEE quotient and the
// hardware's nearest-E4M3 conversion, as k_quant_weight_t does.
// ---------------------------------------------------------------------------
template <int NT, int M, bool kRowScale, bool F8>
__global__ __launch_bounds__(NT) void k_quant_weight_strip(const uint16_t* __restrict__ w,
                                                           int64_t K, int64_t N, int64_t ld,
                                                           const float* __restrict__ s,
                                                           float qdiv, float* __restrict__ wscale,
                                                           int8_t* __restrict__ wq, int nstrips) {
  constexpr int RT = NT / 2;       // row threads; 4*RT rows per m
  constexpr int NW = NT / kWave;
  constexpr int TW = 512;          // tile width in dwords: 2048 k
  constexpr int MPP = TW / RT;     // m groups per tile
  constexpr int LDT = TW + 4;      // padded tile row: the two 8-column halves on other banks
  static_assert(MPP >= 1 && TW % RT == 0, "tile covers whole m groups");
  __shared__ uint32_t tile[16 * LDT];
  __shared__ float red[NW][16];
  __shared__ float dsh[16];
  const int t = threadIdx.x;
  const int h = t & 1, rt = t >> 1;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int b = blockIdx.x;
  const int strip = (nstrips & 7) == 0 ? (b & 7) * (nstrips >> 3) + (b >> 3) : b;
  const int64_t n0 = (int64_t)strip * 16;
  const int64_t nb = n0 + 8 * h;
  const bool ncol = nb < N;
  const int64_t nv = ncol ? N - nb : 8;   // columns of the thread's 8 that exist
  const int64_t kq = K >> 2;  // groups of 4 rows (K % 64 == 0)

  // The whole strip.  Rows past K read row K-1 again (a duplicate cannot
  // change a maximum); a thread wholly past N reads column 0 and one at the
  // ragged end of the rows reads 0 past N (those values belong to no
  // column); neither is ever written out.
  float wh[M][4][8];
  {
    Bf16In::Raw raw[M][4];
    float sk[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t k = min(4 * ((int64_t)rt + RT * m) + r, K - 1);
        raw[m][r] = raw8_upto<Bf16In>(w + k * ld + (ncol ? nb : 0), nv);
        sk[m][r] = kRowScale ? s[k] : 1.0f;
      }
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v[8];
        Bf16In::widen(raw[m][r], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) wh[m][r][i] = kRowScale ? v[i] * sk[m][r] : v[i];
      }
  }
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mx[i] = 0.0f;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(wh[m][r][i]));
  // lanes of equal h first, then the waves through LDS
#pragma unroll
  for (int off = 2; off < kWave; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], off, kWave));
  if (lane < 2)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = mx[i];
  __syncthreads();
  if (t < 16) {
    float v = red[0][t];
#pragma unroll
    for (int j = 1; j < NW; ++j) v = fmaxf(v, red[j][t]);
    const float d = v / qdiv;
    if (n0 + t < N) wscale[n0 + t] = d;
    dsh[t] = d;
  }
  __syncthreads();
  float d[8], rc[8];
  bool slow = false;   // a zero step (all-zero column) or one whose reciprocal overflows
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    d[i] = dsh[h * 8 + i];
    rc[i] = 1.0f / d[i];
    slow |= !(rc[i] < INFINITY);
  }

#pragma unroll
  for (int p = 0; p < (M + MPP - 1) / MPP; ++p) {
    if (p > 0) __syncthreads();   // the previous tile has been written out
#pragma unroll
    for (int mm = 0; mm < MPP; ++mm) {
      const int m = MPP * p + mm;
      if (m >= M) break;
      const int64_t g = (int64_t)rt + RT * m;
      if (!ncol || g >= kq) continue;
      uint32_t pk[8];
      if (F8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float q[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            q[r] = d[i] != 0.0f ? fminf(fmaxf(wh[m][r][i] / d[i], -448.0f), 448.0f) : 0.0f;
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], x, true);
          pk[i] = (uint32_t)x;
        }
      } else {
        constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
        float dm = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t tb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float y = wh[m][r][i] * rc[i];
            const float tq = y + kMagic;
            dm = fmaxf(dm, fabsf(y - (tq - kMagic)));
            tb[r] = __float_as_uint(tq);
          }
          // low bytes of tb[0..3] -> one dword, tb[0] in the lowest byte
          const uint32_t lo = __builtin_amdgcn_perm(tb[1], tb[0], 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm(tb[3], tb[2], 0x04000c0cu);
          pk[i] = lo | hi;
        }
        if (slow || !(dm <= kTieBand)) {
          // rare: redo by IEEE division only the values near a tie (or every
          // value when 1/Delta overflowed); a wave runs a value's division
          // only if one of its lanes needs it
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // y recomputed (rc made opaque, so the fast pass keeps no y alive)
              float rci = rc[i];
              asm volatile("" : "+v"(rci));
              const float y = wh[m][r][i] * rci;   // rint(y) = tq - 1.5 * 2^23 of the fast pass
              if (slow || !(fabsf(y - rintf(y)) <= kTieBand)) {
                const float q = d[i] != 0.0f ? rintf(wh[m][r][i] / d[i]) : 0.0f;
                pk[i] = (pk[i] & ~(0xffu << (8 * r))) |
                        (code_byte(fminf(fmaxf(q, -127.0f), 127.0f)) << (8 * r));
              }
            }
        }
      }
      const int col = (int)(g - TW * p);
#pragma unroll
      for (int i = 0; i < 8; ++i) tile[(h * 8 + i) * LDT + col] = pk[i];
    }
    __syncthreads();
    // this tile: 16 rows x kspan bytes, 16 bytes per thread per pass
    const int64_t k0 = (int64_t)4 * TW * p;
    const int64_t kspan = min(K - k0, (int64_t)4 * TW);
    const int segs = (int)(kspan >> 4);
    for (int q = t; q < 16 * segs; q += NT) {
      const int n = q / segs;
      const int sg = q - n * segs;
      if (n0 + n < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&tile[n * LDT + 4 * sg]);
        *reinterpret_cast<u32x4*>(wq + (n0 + n) * K + k0 + 16 * sg) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

void launch_fold_gamma(const float* s, const float* gamma, float* gout, int64_t K, hipStream_t st) {
  if (K <= 0) return;
  hipLaunchKernelGGL(k_fold_gamma, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, s, gamma,
                     gout, K);
}

void launch_fold_beta(const float* s, const float* beta, float* bout, int64_t K, hipStream_t st) {
  if (K <= 0) return;
  hipLaunchKernelGGL(k_fold_beta, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, s, beta,
                     bout, K);
}

void launch_fold_prev(const void* w, bool bf16, int64_t Kp, int64_t K, int64_t ld, const float* s,
                      float* wout, int64_t ldo, hipStream_t st) {
  const int64_t chunks = Kp * (K >> 3);
  if (chunks <= 0) return;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(k_fold_prev<Bf16In>, grid, dim3(256), 0, st, (const uint16_t*)w, Kp, K, ld,
                       s, wout, ldo);
  else
    hipLaunchKernelGGL(k_fold_prev<F32In>, grid, dim3(256), 0, st, (const float*)w, Kp, K, ld, s,
                       wout, ldo);
}

void launch_fold_w(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld, const float* s,
                   float* wout, hipStream_t st) {
  const int64_t chunks = K * ((N + 7) >> 3);
  if (chunks <= 0) return;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(k_fold_w<Bf16In>, grid, dim3(256), 0, st, (const uint16_t*)w, K, N, ld, s,
                       wout);
  else
    hipLaunchKernelGGL(k_fold_w<F32In>, grid, dim3(256), 0, st, (const float*)w, K, N, ld, s, wout);
}

template <bool F8>
static void quant_weight_f(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                           const float* s, const float* wscale, int8_t* wq, hipStream_t st) {
  if (K <= 0 || N <= 0) return;
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((K + 127) / 128));
  if (bf16) {
    if (s)
      hipLaunchKernelGGL((k_quant_weight_t<Bf16In, true, F8>), grid, dim3(256), 0, st,
                         (const uint16_t*)w, K, N, ld, s, wscale, wq);
    else
      hipLaunchKernelGGL((k_quant_weight_t<Bf16In, false, F8>), grid, dim3(256), 0, st,
                         (const uint16_t*)w, K, N, ld, s, wscale, wq);
  } else {
    if (s)
      hipLaunchKernelGGL((k_quant_weight_t<F32In, true, F8>), grid, dim3(256), 0, st,
                         (const float*)w, K, N, ld, s, wscale, wq);
    else
      hipLaunchKernelGGL((k_quant_weight_t<F32In, false, F8>), grid, dim3(256), 0, st,
                         (const float*)w, K, N, ld, s, wscale, wq);
  }
}

void launch_quant_weight_t(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                           const float* s, const float* wscale, int8_t* wq, hipStream_t st) {
  quant_weight_f<false>(w, bf16, K, N, ld, s, wscale, wq, st);
}

// The strip kernel takes a whole compute unit per workgroup once K > 2048, so
// its rounds of cu_count() strips run one after another with no overlap of
// one strip's loads and another's arithmetic: about 20 us per round at K =
// 4096, where the three-launch path streams 32 MiB in about 18 us once its
// fixed costs are paid.  It wins by skipping those costs only with at most two
// rounds, the last nearly full (measured at K = 4096: N = 4096 20.1 vs 28.8
// us, 8192 34.5 vs 39.1; N = 1024, 2048, 6144, 14336, 28672 lose).  With
// K <= 2048 it won at every shape measured (N = 4096: 8.6 vs 13.4 us at
// K = 1024, 12.1 vs 17.0 at K = 2048).
bool quant_weight_strip_ok(bool bf16, int64_t K, int64_t N) {
  if (!(bf16 && K > 0 && K <= 4096 && K % 64 == 0 && N > 0)) return false;
  const int64_t strips = (N + 15) / 16;
  if (K <= 2048) return strips <= (int64_t)INT32_MAX;
  const int64_t cu = cu_count();
  const int64_t rounds = (strips + cu - 1) / cu;
  return rounds <= 2 && 10 * strips >= 9 * rounds * cu;
}

// NT threads per strip: 1024 (4 waves per SIMD, to hide the quantization's
// dependency chains) once K > 1024, else 512
template <int NT, int M, bool F8>
static void strip_m(const uint16_t* w, int64_t K, int64_t N, int64_t ld, const float* s,
                    float qdiv, float* wscale, int8_t* wq, hipStream_t st) {
  const int nstrips = (int)((N + 15) / 16);
  if (s)
    hipLaunchKernelGGL((k_quant_weight_strip<NT, M, true, F8>), dim3((unsigned)nstrips), dim3(NT),
                       0, st, w, K, N, ld, s, qdiv, wscale, wq, nstrips);
  else
    hipLaunchKernelGGL((k_quant_weight_strip<NT, M, false, F8>), dim3((unsigned)nstrips), dim3(NT),
                       0, st, w, K, N, ld, s, qdiv, wscale, wq, nstrips);
}

template <bool F8>
static void strip_f(const void* w, int64_t K, int64_t N, int64_t ld, const float* s,
                    float* wscale, int8_t* wq, hipStream_t st) {
  const float qdiv = F8 ? 448.0f : 127.0f;
  const uint16_t* wb = (const uint16_t*)w;
  const int64_t groups = K >> 2;   // groups of 4 rows
  if (groups <= 256) strip_m<512, 1, F8>(wb, K, N, ld, s, qdiv, wscale, wq, st);
  else if (groups <= 512) strip_m<1024, 1, F8>(wb, K, N, ld, s, qdiv, wscale, wq, st);
  else strip_m<1024, 2, F8>(wb, K, N, ld, s, qdiv, wscale, wq, st);
}

void launch_quant_weight_strip(const void* w, int64_t K, int64_t N, int64_t ld, const float* s,
                               float* wscale, int8_t* wq, hipStream_t st) {
  strip_f<false>(w, K, N, ld, s, wscale, wq, st);
}

void launch_quant_weight_strip_fp8(const void* w, int64_t K, int64_t N, int64_t ld,
                                   const float* s, float* wscale, uint8_t* wq, hipStream_t st) {
  strip_f<true>(w, K, N, ld, s, wscale, reinterpret_cast<int8_t*>(wq), st);
}

void launch_quant_weight_t_fp8(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                               const float* s, const float* wscale, uint8_t* wq, hipStream_t st) {
  quant_weight_f<true>(w, bf16, K, N, ld, s, wscale, reinterpret_cast<int8_t*>(wq), st);
}

}  // namespace sqk
