// k_gemm_decode.hip -- the W8A8 GEMM for a handful of tokens (T <= 64) on
// gfx950.  The same contraction and epilogue as k_gemm.hip, but the weight is
// read exactly once and nothing else matters: decode time is set by the weight
// bytes ("SmoothQuant and W8A8", The full model, served).
//
//  * v_mfma_i32_16x16x64_i8 with the weight rows as the A operand (16 output
//    channels) and up to 16 tokens as the B operand; a lane's 4 accumulators
//    are 4 consecutive output channels of one token.
//  * Workgroup = 8 waves over 16*NB output channels (NB = 1 or 2, chosen per
//    shape); the K steps are split over the 8 waves and each wave streams its
//    slice of the weight rows straight into VGPRs (no LDS staging: nothing is
//    reused), U steps in flight.  The 8 partial int32 sums are added through LDS -- integer adds,
//    so the result is exact in any order.
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

enum { D_OUT_BF16 = 0, D_OUT_F32 = 1, D_OUT_I32 = 2 };

template <int TB, int NB, int U, int OUT>
__global__ __launch_bounds__(512) void k_gemm_decode(const int8_t* __restrict__ xq,
                                                     const float* __restrict__ xs, int T, int K,
                                                     const int8_t* __restrict__ wq,
                                                     const float* __restrict__ ws, int N,
                                                     const float* __restrict__ bias,
                                                     void* __restrict__ yout, int ldy) {
  constexpr int NW = 8;
  __shared__ v4i part[NW][NB][TB][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * (16 * NB);
  const int r16 = lane & 15, kq = (lane >> 4) * 16;

  const int nsteps = K >> 6;
  const int spw = (nsteps + NW - 1) / NW;
  const int s0 = wave * spw;
  const int s1 = min(nsteps, s0 + spw);

  const int8_t* wrow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) wrow[b] = wq + (int64_t)min(n0 + b * 16 + r16, N - 1) * K + kq;
  const int8_t* xrow[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) xrow[tb] = xq + (int64_t)min(tb * 16 + r16, T - 1) * K + kq;

  v4i acc[NB][TB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[b][tb] = v4i{0, 0, 0, 0};

  int s = s0;
  for (; s + U <= s1; s += U) {
    v4i a[U][NB], x[U][TB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (int64_t)(s + u) * 64;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        a[u][b] = *reinterpret_cast<const v4i*>(wrow[b] + off);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) x[u][tb] = *reinterpret_cast<const v4i*>(xrow[tb] + off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          acc[b][tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][b], x[u][tb], acc[b][tb], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const int64_t off = (int64_t)s * 64;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const v4i a = *reinterpret_cast<const v4i*>(wrow[b] + off);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const v4i x = *reinterpret_cast<const v4i*>(xrow[tb] + off);
        acc[b][tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, x, acc[b][tb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) part[wave][b][tb][lane] = acc[b][tb];
  __syncthreads();

  // one thread per (channel block, token block, lane) sums the 8 partials
  const int item = threadIdx.x;
  if (item >= NB * TB * 64) return;
  const int b = item / (TB * 64);
  const int tb = (item / 64) % TB;
  const int l = item & 63;
  v4i sum = part[0][b][tb][l];
#pragma unroll
  for (int w = 1; w < NW; ++w) sum += part[w][b][tb][l];
  const int t = tb * 16 + (l & 15);
  const int n = n0 + b * 16 + (l >> 4) * 4;
  if (t >= T || n >= N) return;
  const bool full = n + 3 < N;
  if (OUT == D_OUT_I32) {
    int32_t* dst = reinterpret_cast<int32_t*>(yout) + (int64_t)t * N + n;
    if (full && (N & 3) == 0) {
      *reinterpret_cast<v4i*>(dst) = sum;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) dst[e] = sum[e];
    }
    return;
  }
  const float xst = xs[t];
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int nn = min(n + e, N - 1);
    const float sc = xst * ws[nn];
    const float v = sc * (float)sum[e];
    o[e] = bias ? v + bias[nn] : v;
  }
  if (OUT == D_OUT_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(yout) + (int64_t)t * ldy + n;
    if (full) {
      u32x2 p;
      p[0] = pack_bf16x2(o[0], o[1]);
      p[1] = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<u32x2*>(dst) = p;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) dst[e] = (uint16_t)(pack_bf16x2(o[e], 0.0f) & 0xffffu);
    }
  } else {
    float* dst = reinterpret_cast<float*>(yout) + (int64_t)t * ldy + n;
    if (full) {
      f32x4 p;
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = o[e];
      *reinterpret_cast<f32x4*>(dst) = p;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) dst[e] = o[e];
    }
  }
}

template <int TB, int NB, int U>
static void decode_tb(const int8_t* xq, const float* xs, int T, int K, const int8_t* wq,
                      const float* ws, int N, const float* bias, void* y, int ldy, int out,
                      hipStream_t st) {
  const dim3 grid((unsigned)((N + 16 * NB - 1) / (16 * NB))), block(512);
  if (out == 0)
    hipLaunchKernelGGL((k_gemm_decode<TB, NB, U, D_OUT_BF16>), grid, block, 0, st, xq, xs, T, K, wq,
                       ws, N, bias, y, ldy);
  else if (out == 1)
    hipLaunchKernelGGL((k_gemm_decode<TB, NB, U, D_OUT_F32>), grid, block, 0, st, xq, xs, T, K, wq,
                       ws, N, bias, y, ldy);
  else
    hipLaunchKernelGGL((k_gemm_decode<TB, NB, U, D_OUT_I32>), grid, block, 0, st, xq, xs, T, K, wq,
                       ws, N, bias, y, ldy);
}

// Channels per workgroup: 32 (NB = 2) share each token load between two
// channel blocks, which pays with more than 8 tokens when N / 32 workgroups
// still cover every compute unit; otherwise 16 (NB = 1, 8 k-steps in flight)
// keep twice as many workgroups streaming.  Measured at 16 tokens: K = N =
// 8192 17.5 us (NB = 2) vs 19.6 us; N = 4096: K = 4096 6.4 us vs 8.0 us,
// K = 14336 18.0 us vs 24.7 us; one token, K = N = 8192: 15.1 us vs 17.5 us.
void launch_gemm_decode(const int8_t* xq, const float* xs, int64_t T, int64_t K, const int8_t* wq,
                        const float* ws, int64_t N, const float* bias, void* y, int64_t ldy,
                        int out, hipStream_t st) {
  const int it = (int)T, ik = (int)K, in = (int)N, il = (int)ldy;
  if (T <= 16) {
    if (T > 8 && (N + 31) / 32 >= cu_count())
      decode_tb<1, 2, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
    else
      decode_tb<1, 1, 8>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  } else if (T <= 32) {
    decode_tb<2, 2, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  } else if (T <= 48) {
    decode_tb<3, 2, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  } else {
    decode_tb<4, 2, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  }
}

}  // namespace sqk
