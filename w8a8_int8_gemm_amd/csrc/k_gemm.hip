// k_gemm.hip -- INT8 x INT8 -> INT32 GEMM on the gfx950 matrix cores with the
// fused dequantization epilogue ("06 -- SmoothQuant", section 7: the matmul is
// a straight INT8 x INT8 -> INT32 product followed by
// Y = scale_x * scale_w * Y_int32; "Taming the Outliers", step I6: add bias
// and dequantize).
//
//   acc[t, n] = sum_k xq[t, k] * wq[n, k]     (xq [T, K], wq [N, K], K contiguous)
//   y[t, n]   = fp32(fp32(xs[t] * ws[n]) * fp32(acc)) + bias[n]  -> bf16 / fp32
//
// Design (CDNA4):
//  * v_mfma_i32_32x32x32_i8: 16 int8 of K per lane per operand, int32
//    accumulators.  The weight tile is the MFMA's A operand (rows = output
//    channels) and the activation tile its B operand (columns = tokens), so a
//    lane's 4 consecutive accumulator rows are 4 consecutive output channels
//    of one token -- one 8-byte bf16 store instead of four 2-byte ones.
//  * Workgroup tile BT tokens x BN channels, 4 waves in a 2 x 2 grid, each
//    wave (BT/2) x (BN/2) = (BT/64) x (BN/64) MFMA tiles of 32 x 32.
//  * K is staged through LDS 128 bytes at a time, double buffered, with
//    global_load_lds_dwordx4 (HBM/L2 -> LDS without VGPRs).  A 1 KiB load
//    instruction fills 8 rows of 128 bytes; the 16-byte chunk c of row r is
//    stored at chunk position c ^ swz(r), so the 32 rows an MFMA operand read
//    touches spread over all LDS banks.
//  * Tiles are ordered so that the workgroups that share an XCD (the
//    hardware deals workgroup ids round-robin over the 8 XCDs) take one
//    contiguous range of tiles, grouped GROUP_T token panels at a time: they
//    share activation and weight panels in their XCD's L2.
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

typedef __attribute__((address_space(3))) void lds_void;

template <int SWZ>
__device__ __forceinline__ int swz(int row) {
  if (SWZ == 1) return row & 7;
  if (SWZ == 2) return (row >> 1) & 7;
  return 0;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Bijective workgroup -> tile map.  Workgroup b runs on XCD b % 8; the
// workgroups of XCD x get the contiguous tile range that precedes the ranges
// of XCDs x+1..7.  Inside the range, tiles go GROUP_T token panels at a time.
__device__ __forceinline__ void tile_of(int bid, int nt_t, int nt_n, int group_t, int& pid_t,
                                        int& pid_n) {
  const int ntiles = nt_t * nt_n;
  const int x = bid & 7;
  const int idx = bid >> 3;
  const int q = ntiles >> 3, r = ntiles & 7;
  const int tile = (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
  const int in_group = group_t * nt_n;
  const int g = tile / in_group;
  const int first_t = g * group_t;
  const int gsize = min(nt_t - first_t, group_t);
  const int local = tile - g * in_group;
  pid_t = first_t + local % gsize;
  pid_n = local / gsize;
}

enum { OUT_BF16 = 0, OUT_F32 = 1, OUT_I32 = 2 };

template <int BT, int BN, int SWZ, int OUT>
__global__ __launch_bounds__(256) void k_gemm_w8a8(const int8_t* __restrict__ xq,
                                                   const float* __restrict__ xs, int T, int K,
                                                   const int8_t* __restrict__ wq,
                                                   const float* __restrict__ ws, int N,
                                                   const float* __restrict__ bias,
                                                   void* __restrict__ yout, int ldy,
                                                   int group_t) {
  constexpr int BK = 128;                   // bytes of K per stage
  constexpr int NTT = BT / 64;              // 32x32 tiles per wave along tokens
  constexpr int NTN = BN / 64;              // ... along output channels
  constexpr int XS = BT * BK, WS = BN * BK; // bytes per stage
  __shared__ __attribute__((aligned(1024))) int8_t smem[2 * (XS + WS)];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wt = wave & 1, wn = wave >> 1;
  const int nt_t = (T + BT - 1) / BT, nt_n = (N + BN - 1) / BN;
  int pid_t, pid_n;
  tile_of(blockIdx.x, nt_t, nt_n, group_t, pid_t, pid_n);
  const int t0 = pid_t * BT, n0 = pid_n * BN;

  int8_t* xs_l = smem;              // [2][BT][BK]
  int8_t* ws_l = smem + 2 * XS;     // [2][BN][BK]

  // --- global -> LDS: lane l of a 1 KiB block fills row 8b + l/8, chunk l%8
  const int lrow = lane >> 3, lchunk = lane & 7;
  auto issue = [&](int stage, int k0, bool tail) {
#pragma unroll
    for (int bb = 0; bb < BT / 32; ++bb) {
      const int b = bb * 4 + wave;
      const int row = b * 8 + lrow;
      int c = lchunk ^ swz<SWZ>(row);
      if (tail && k0 + c * 16 >= K) c -= 4;   // half stage at the K tail: stay in bounds
      const int grow = min(t0 + row, T - 1);
      const int8_t* src = xq + (int64_t)grow * K + k0 + c * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(xs_l + stage * XS + b * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int bb = 0; bb < BN / 32; ++bb) {
      const int b = bb * 4 + wave;
      const int row = b * 8 + lrow;
      int c = lchunk ^ swz<SWZ>(row);
      if (tail && k0 + c * 16 >= K) c -= 4;
      const int grow = min(n0 + row, N - 1);
      const int8_t* src = wq + (int64_t)grow * K + k0 + c * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(ws_l + stage * WS + b * 1024), 16, 0, 0);
    }
  };

  v16i acc[NTN][NTT];
#pragma unroll
  for (int i = 0; i < NTN; ++i)
#pragma unroll
    for (int j = 0; j < NTT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  // --- MFMA over one stage: KS k-steps of 32 bytes
  const int frow = lane & 31, fhalf = lane >> 5;
  auto compute = [&](int stage, auto ks_tag) {
    constexpr int KS = decltype(ks_tag)::value;
    const int8_t* wb = ws_l + stage * WS;
    const int8_t* xb = xs_l + stage * XS;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      v4i a[NTN], b[NTT];
      const int c = kk * 2 + fhalf;
#pragma unroll
      for (int i = 0; i < NTN; ++i) {
        const int row = wn * (BN / 2) + i * 32 + frow;
        a[i] = *reinterpret_cast<const v4i*>(wb + row * BK + ((c ^ swz<SWZ>(row)) << 4));
      }
#pragma unroll
      for (int j = 0; j < NTT; ++j) {
        const int row = wt * (BT / 2) + j * 32 + frow;
        b[j] = *reinterpret_cast<const v4i*>(xb + row * BK + ((c ^ swz<SWZ>(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < NTN; ++i)
#pragma unroll
        for (int j = 0; j < NTT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nfull = K / BK;
  const bool has_tail = (K % BK) != 0;
  const int nst = nfull + (has_tail ? 1 : 0);
  issue(0, 0, has_tail && nfull == 0);
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < nfull; ++it) {
    const int cur = it & 1;
    if (it + 1 < nst) issue(cur ^ 1, (it + 1) * BK, has_tail && it + 1 == nfull);
    compute(cur, std::integral_constant<int, 4>());
    wait_vmem();
    __syncthreads();
  }
  if (has_tail) {
    compute(nfull & 1, std::integral_constant<int, 2>());
    __syncthreads();
  }

  // --- epilogue.  Lane l of tile (i, j): token t = .. + l%32; channels
  // n = .. + 8g + 4(l/32) + e for g, e in 0..3 hold acc[i][j][4g + e].
  // The tile's scales and bias are staged in LDS (the operand buffers are
  // free now) so each lane reads them 4 channels at a time.
  float* s_xs = reinterpret_cast<float*>(smem);   // [BT]
  float* s_ws = s_xs + BT;                         // [BN]
  float* s_b = s_ws + BN;                          // [BN]
  const bool has_bias = bias != nullptr;
  if (OUT != OUT_I32) {
    for (int i = threadIdx.x; i < BT; i += 256) s_xs[i] = (t0 + i < T) ? xs[t0 + i] : 0.0f;
    for (int i = threadIdx.x; i < BN; i += 256) {
      s_ws[i] = (n0 + i < N) ? ws[n0 + i] : 0.0f;
      s_b[i] = (has_bias && n0 + i < N) ? bias[n0 + i] : 0.0f;
    }
    __syncthreads();
  }
  const bool full_tile = (t0 + BT <= T) && (n0 + BN <= N) && (OUT != OUT_I32 || (N & 3) == 0);
#pragma unroll
  for (int j = 0; j < NTT; ++j) {
    const int tl = wt * (BT / 2) + j * 32 + frow;
    const int t = t0 + tl;
    const float xst = (OUT == OUT_I32) ? 0.0f : s_xs[tl];
#pragma unroll
    for (int i = 0; i < NTN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * (BN / 2) + i * 32 + g * 8 + fhalf * 4;
        const int n = n0 + nl;
        if (OUT == OUT_I32) {
          int32_t* dst = reinterpret_cast<int32_t*>(yout) + (int64_t)t * N + n;
          v4i o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * g + e];
          if (full_tile) {
            *reinterpret_cast<v4i*>(dst) = o;
          } else if (t < T) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) dst[e] = o[e];
          }
        } else {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(s_ws + nl);
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(s_b + nl);
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sc = xst * w4[e];
            const float v = sc * (float)acc[i][j][4 * g + e];
            o[e] = has_bias ? v + b4[e] : v;
          }
          if (OUT == OUT_BF16) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(yout) + (int64_t)t * ldy + n;
            u32x2 p;
            p[0] = pack_bf16x2(o[0], o[1]);
            p[1] = pack_bf16x2(o[2], o[3]);
            if (full_tile || (t < T && n + 3 < N)) {
              *reinterpret_cast<u32x2*>(dst) = p;
            } else if (t < T) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = (uint16_t)((p[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
          } else {
            float* dst = reinterpret_cast<float*>(yout) + (int64_t)t * ldy + n;
            if (full_tile || (t < T && n + 3 < N)) {
              f32x4 p;
#pragma unroll
              for (int e = 0; e < 4; ++e) p[e] = o[e];
              *reinterpret_cast<f32x4*>(dst) = p;
            } else if (t < T) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = o[e];
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------

template <int BT, int BN, int SWZ>
static void gemm_tile(const int8_t* xq, const float* xs, int T, int K, const int8_t* wq,
                      const float* ws, int N, const float* bias, void* y, int ldy, int out,
                      hipStream_t st) {
  const int ntiles = ((T + BT - 1) / BT) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)ntiles), block(256);
  const int group_t = 4;
  if (out == OUT_BF16)
    hipLaunchKernelGGL((k_gemm_w8a8<BT, BN, SWZ, OUT_BF16>), grid, block, 0, st, xq, xs, T, K, wq,
                       ws, N, bias, y, ldy, group_t);
  else if (out == OUT_F32)
    hipLaunchKernelGGL((k_gemm_w8a8<BT, BN, SWZ, OUT_F32>), grid, block, 0, st, xq, xs, T, K, wq,
                       ws, N, bias, y, ldy, group_t);
  else
    hipLaunchKernelGGL((k_gemm_w8a8<BT, BN, SWZ, OUT_I32>), grid, block, 0, st, xq, xs, T, K, wq,
                       ws, N, bias, y, ldy, group_t);
}

void launch_gemm(const int8_t* xq, const float* xs, int64_t T, int64_t K, const int8_t* wq,
                 const float* ws, int64_t N, const float* bias, void* y, int64_t ldy, int out,
                 hipStream_t st) {
  if (T <= 0 || N <= 0) return;
  if (T <= 64) {
    launch_gemm_decode(xq, xs, T, K, wq, ws, N, bias, y, ldy, out, st);
    return;
  }
  const int it = (int)T, ik = (int)K, in = (int)N, il = (int)ldy;
  // 256 x 256 tiles fill the chip when there are at least ~2 per CU;
  // otherwise smaller tiles trade reuse for occupancy.
  const int64_t t256 = ((T + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 384)
    gemm_tile<256, 256, 1>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  else if (((T + 255) / 256) * ((N + 127) / 128) >= 256)
    gemm_tile<256, 128, 1>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  else
    gemm_tile<128, 128, 1>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
}

}  // namespace sqk
