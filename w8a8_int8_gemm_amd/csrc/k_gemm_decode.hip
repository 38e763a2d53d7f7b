// k_gemm_decode.hip -- the W8A8 GEMM for a handful of tokens (T <= 64) on
// gfx950.  The same contraction and epilogue as k_gemm.hip, but the weight is
// read exactly once and nothing else matters: decode time is set by the weight
// bytes ("SmoothQuant and W8A8", The full model, served).
//
//  * v_mfma_i32_16x16x64_i8 with 16 weight rows as the A operand and up to 16
//    tokens per B operand; a lane's 4 accumulators are 4 consecutive output
//    channels of one token.
//  * Workgroup = NW waves over NB blocks of 16 output channels; the waves
//    split K.  Each wave streams its slice of those rows into its own LDS
//    ring with direct-to-LDS buffer loads that read C contiguous bytes of a
//    row per 16 lanes (256-byte runs) instead of 64-byte pieces of 16 rows,
//    the pattern the MFMA operand layout would dictate; the operand reads
//    then take each row's 16-byte chunks in MFMA order from LDS.  A wave owns
//    its ring, so the K loop has no barrier.  Token operands come from L2
//    straight into registers, one 16x64-byte load per k-step and token block,
//    shared by the NB row blocks.
//  * The partial int32 sums of the waves are added through LDS -- integer
//    adds, so the result is exact in any order.
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

typedef __attribute__((address_space(3))) void lds_void_d;

enum { D_OUT_BF16 = 0, D_OUT_F32 = 1, D_OUT_I32 = 2 };

// y[t, n .. n+3] from the int32 sums of one lane: int32 (OUT = D_OUT_I32), or
// fp32(fp32(xs[t] * ws[n]) * fp32(acc)) + bias[n] in fp32 or bf16
template <int OUT>
__device__ __forceinline__ void store_out(const v4i sum, int t, int n, int N,
                                          const float* __restrict__ xs,
                                          const float* __restrict__ ws,
                                          const float* __restrict__ bias, void* __restrict__ yout,
                                          int ldy) {
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

template <int TB, int NB, int C, int NW, int OUT>
__global__ __launch_bounds__(64 * NW) void k_gemm_decode(const int8_t* __restrict__ xq,
                                                         const float* __restrict__ xs, int T,
                                                         int K, const int8_t* __restrict__ wq,
                                                         const float* __restrict__ ws, int N,
                                                         const float* __restrict__ bias,
                                                         void* __restrict__ yout, int ldy) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(C >= 256 && C <= 1024 && (C & (C - 1)) == 0, "segment bytes");
  constexpr int STEPS = C / 64;          // MFMA k-steps per stage
  constexpr int R = 1024 / C;            // rows per 1 KiB load
  constexpr int CPR = C / 16;            // 16-byte chunks per row segment
  constexpr int RB = 16 * NB;            // weight rows of the workgroup
  constexpr int LW = RB / R;             // weight loads per stage
  constexpr int LX = TB * STEPS;         // token loads per stage
  constexpr int LPS = LW + LX;
  constexpr int SB = RB * C;             // stage bytes
  constexpr int kOff = 1 << 30;          // an offset past every resource
  constexpr int RING = NW * 2 * SB;
  constexpr int PART = NW * NB * TB * 64 * 16;
  __shared__ __attribute__((aligned(1024))) int8_t smem[RING > PART ? RING : PART];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * RB;
  int8_t* ring = smem + wave * 2 * SB;

  // rows past N and tokens past T lie outside the resources and read as 0
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wq + (int64_t)n0 * K), 0, min(RB, N - n0) * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)xq, 0, T * K, 0x00020000);

  // this wave's K bytes [kw0, kw1), whole 64-byte steps
  const int nsteps = K >> 6;
  const int spw = (nsteps + NW - 1) / NW;
  const int kw0 = min(nsteps, wave * spw) * 64;
  const int kw1 = min(nsteps, (wave + 1) * spw) * 64;
  const int ns = (kw1 - kw0 + C - 1) / C;   // stages

  // load j of a stage: lane l fills LDS bytes j*1024 + 16 l = row j*R + l/CPR,
  // position p = l % CPR, with the row's global chunk p ^ (row & 15).
  int wbase[LW], wchunk[LW];
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int row = j * R + lane / CPR;
    const int g = (lane % CPR) ^ (row & 15);
    wbase[j] = row * K + g * 16;
    wchunk[j] = g * 16;
  }
  const int i16 = lane & 15, q = lane >> 4;
  int xbase[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) xbase[tb] = (tb * 16 + i16) * K + q * 16;
  // operand read of k-step s, row block b: row 16b + i16's global chunk 4s + q
  int rbase[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
    rbase[s] = (i16 / R) * 1024 + (i16 % R) * C + (((4 * s + q) ^ i16) << 4);
  constexpr int BB = 16 * C;   // bytes between row blocks (16 rows)

  v4i x0[STEPS][TB], x1[STEPS][TB];
  auto issue = [&](int st, int8_t* slot, v4i (&x)[STEPS][TB]) {
    const int kst = kw0 + st * C;
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      const int off = (kst + wchunk[j] < kw1) ? wbase[j] + kst : kOff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_d*)(slot + j * 1024), 16, off, 0, 0,
                                               0);
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int k = kst + s * 64;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        x[s][tb] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(xr, k < kw1 ? xbase[tb] + k : kOff, 0, 0));
    }
  };
  v4i acc[NB][TB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[b][tb] = v4i{0, 0, 0, 0};
  auto compute = [&](const int8_t* slot, v4i (&x)[STEPS][TB]) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const v4i a = *reinterpret_cast<const v4i*>(slot + b * BB + rbase[s]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          acc[b][tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, x[s][tb], acc[b][tb], 0, 0, 0);
      }
    }
  };
  // A stage is LPS loads: its LW direct-to-LDS weight loads, then its LX token
  // loads into registers, all buffer loads.  Loads of one wave complete in
  // issue order, so "at most LPS loads in flight" means every load of all
  // but the newest stage has landed.
  int8_t* slot0 = ring;
  int8_t* slot1 = ring + SB;
  // stages 0 and 1 (a stage past ns is all outside: zeros, no traffic)
  issue(0, slot0, x0);
  issue(1, slot1, x1);
  int st = 0;
  for (; st + 3 < ns; st += 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
    compute(slot0, x0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(st + 2, slot0, x0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
    compute(slot1, x1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(st + 3, slot1, x1);
  }
  const int rem = ns - st;   // 0 .. 3 stages left; two of them are in flight
  if (rem == 3) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
    compute(slot0, x0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(st + 2, slot0, x0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
    compute(slot1, x1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    compute(slot0, x0);
  } else if (rem == 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
    compute(slot0, x0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    compute(slot1, x1);
  } else if (rem == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
    compute(slot0, x0);
  }
  // every load has landed and every ring read is done before the ring turns
  // into the partial sums
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  v4i* part = reinterpret_cast<v4i*>(smem);   // [NW][NB * TB][64]
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) part[((wave * NB + b) * TB + tb) * 64 + lane] = acc[b][tb];
  __syncthreads();

  // one thread per (row block, token block, lane) sums the NW partials
  for (int item = threadIdx.x; item < NB * TB * 64; item += 64 * NW) {
    const int bt = item / 64;          // b * TB + tb
    const int l = item & 63;
    v4i sum = part[bt * 64 + l];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += part[(w * NB * TB + bt) * 64 + l];
    const int t = (bt % TB) * 16 + (l & 15);
    const int n = n0 + (bt / TB) * 16 + (l >> 4) * 4;
    if (t < T && n < N) store_out<OUT>(sum, t, n, N, xs, ws, bias, yout, ldy);
  }
#endif
}

template <int TB, int NB, int C, int NW>
static void decode_tb(const int8_t* xq, const float* xs, int T, int K, const int8_t* wq,
                      const float* ws, int N, const float* bias, void* y, int ldy, int out,
                      hipStream_t st) {
  const dim3 grid((unsigned)((N + 16 * NB - 1) / (16 * NB))), block(64 * NW);
  if (out == 0)
    hipLaunchKernelGGL((k_gemm_decode<TB, NB, C, NW, D_OUT_BF16>), grid, block, 0, st, xq, xs, T,
                       K, wq, ws, N, bias, y, ldy);
  else if (out == 1)
    hipLaunchKernelGGL((k_gemm_decode<TB, NB, C, NW, D_OUT_F32>), grid, block, 0, st, xq, xs, T,
                       K, wq, ws, N, bias, y, ldy);
  else
    hipLaunchKernelGGL((k_gemm_decode<TB, NB, C, NW, D_OUT_I32>), grid, block, 0, st, xq, xs, T,
                       K, wq, ws, N, bias, y, ldy);
}

// Shapes (measured at T = 1 .. 64 against weights past the Infinity Cache):
// 32 channels per workgroup (NB = 2) share each token load between two row
// blocks and win when N / 32 workgroups cover every compute unit, or when
// K <= 4096 keeps each wave's slice short; otherwise 16 channels (NB = 1) with
// 8 waves keep more waves streaming.  A ring of two 256-byte stages per wave
// beat 512- and 1024-byte segments and deeper rings.
void launch_gemm_decode(const int8_t* xq, const float* xs, int64_t T, int64_t K, const int8_t* wq,
                        const float* ws, int64_t N, const float* bias, void* y, int64_t ldy,
                        int out, hipStream_t st) {
  const int it = (int)T, ik = (int)K, in = (int)N, il = (int)ldy;
  const bool nb2 = (N + 31) / 32 >= cu_count() || K <= 4096;
  if (T <= 4) {
    decode_tb<1, 1, 256, 8>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  } else if (T <= 16) {
    if (nb2) decode_tb<1, 2, 256, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
    else decode_tb<1, 1, 256, 8>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  } else if (T <= 32) {
    decode_tb<2, 2, 256, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  } else if (T <= 48) {
    decode_tb<3, 2, 256, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  } else {
    decode_tb<4, 2, 256, 4>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  }
}

}  // namespace sqk
