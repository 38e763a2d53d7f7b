// k_gemm.hip -- INT8 x INT8 -> INT32 GEMM on the gfx950 matrix cores with the
// fused dequantization epilogue ("06 -- SmoothQuant", section 7: the matmul is
// a straight INT8 x INT8 -> INT32 product followed by
// Y = scale_x * scale_w * Y_int32; "Taming the Outliers", step I6: add bias
// and dequantize), and the same kernel for FP8 E4M3 operands with fp32
// accumulation ("SmoothQuant and W8A8", One layer, measured: FP8 E4M3).
//
//   acc[t, n] = sum_k xq[t, k] * wq[n, k]     (xq [T, K], wq [N, K], K contiguous)
//   y[t, n]   = fp32(fp32(xs[t] * ws[n]) * fp32(acc)) + bias[n]  -> bf16 / fp32
//
// Design (CDNA4):
//  * v_mfma_i32_32x32x32_i8 (INT8) / v_mfma_f32_32x32x64_f8f6f4 (FP8).  The
//    weight tile is the MFMA's A operand (rows = output channels) and the
//    activation tile its B operand (columns = tokens), so a lane's 4
//    consecutive accumulator rows are 4 consecutive output channels of one
//    token -- 8 contiguous output bytes.
//  * Workgroup tile BT tokens x BN channels; WGT x WGN waves, each a
//    (BT/WGT) x (BN/WGN) grid of 32 x 32 MFMA tiles.  The large-T tile is
//    256 x 256 with 8 waves of 128 x 64 (2 waves per SIMD).
//  * K is staged through LDS 64 bytes at a time in 4 buffers, loads issued 3-4
//    stages ahead with buffer_load_dwordx4 ... lds (HBM/L2 -> LDS without
//    VGPRs).  A 1 KiB load instruction fills 16 rows of 64 bytes; the 16-byte
//    chunk c of row r is stored at chunk position c ^ swz(r), so the rows an
//    MFMA operand read touches spread over all 64 LDS banks.
//  * Operand reads of the next k-step are interleaved one-for-one with the
//    MFMAs; one workgroup barrier per stage.
//  * Tiles are ordered so that the workgroups that share an XCD (the
//    hardware deals workgroup ids round-robin over the 8 XCDs) take one
//    contiguous range of tiles, grouped GROUP_T token panels at a time: they
//    share activation and weight panels in their XCD's L2.
//  * The bf16 epilogue stages each wave's tile in LDS and writes whole
//    128-byte row segments.
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk permutation of an LDS row of 64 bytes.  An MFMA operand read
// (ds_read_b128) is served 16 lanes at a time, i.e. 16 consecutive rows at one
// logical chunk; with 64 four-byte banks a pass covers 256 bytes = 16 chunk
// slots, and row r starts at slot 4*(r % 4).  (r >> 2) & 3 moves the 4 rows
// that share a start slot onto 4 different chunk slots: no two lanes of a pass
// share a bank.  (r & 3) would suit a 32-bank LDS that serves 8 lanes a pass.
template <int SWZ>
__device__ __forceinline__ int swz(int row) {
  if (SWZ == 1) return row & 3;
  if (SWZ == 2) return (row >> 2) & 3;
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

// L loads of 1 KiB (64 lanes x 16 bytes) from a buffer resource into LDS:
// load bb of this wave fills the 1 KiB block (bb * NW + wave) of `dst`, lane l
// taking the bytes at voffset off[bb] (+ k0 in the scalar offset).
#if defined(__HIP_DEVICE_COMPILE__)
template <int L, int NW>
__device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t r, int8_t* dst, const int (&off)[L],
                                           int wave, int k0) {
#pragma unroll
  for (int bb = 0; bb < L; ++bb)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (bb * NW + wave) * 1024), 16,
                                             off[bb], k0, 0, 0);
}
#endif

// F8: the operands are FP8 E4M3 codes (same bytes, same staging) multiplied
// by v_mfma_f32_32x32x64_f8f6f4 into fp32 accumulators; else INT8 codes into
// int32 accumulators.  The FP8 instruction sums its products in groups of 8
// consecutive k (MFMA order, which keeps 16-byte K runs together here), each
// aligned to the group's largest product with the bits below 2^-13 of it
// dropped, then adds the group sums in fp32.
template <int BT, int BN, int WGT, int WGN, int SWZ, int OUT, bool F8>
__global__ __launch_bounds__(64 * WGT * WGN) void k_gemm_w8a8(const int8_t* __restrict__ xq,
                                                   const float* __restrict__ xs, int T, int K,
                                                   const int8_t* __restrict__ wq,
                                                   const float* __restrict__ ws, int N,
                                                   const float* __restrict__ bias,
                                                   void* __restrict__ yout, int ldy,
                                                   int group_t) {
  // The body uses buffer-resource types that exist only for the GPU target;
  // the host pass needs nothing but the signature for the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BK = 64;                    // bytes of K per stage
  constexpr int NS = 4;                     // LDS stages (loads run 3-4 stages ahead)
  constexpr int NW = WGT * WGN;             // waves: WGT along tokens x WGN along channels
  constexpr int NTH = 64 * NW;
  constexpr int WTT = BT / WGT, WTN = BN / WGN;  // wave tile
  constexpr int NTT = WTT / 32;             // 32x32 tiles per wave along tokens
  constexpr int NTN = WTN / 32;             // ... along output channels
  constexpr int XS = BT * BK, WS = BN * BK; // bytes per stage
  constexpr int XL = BT / (16 * NW), WL = BN / (16 * NW);  // 1 KiB loads per wave per stage
  constexpr int LPS = XL + WL;              // loads per wave per stage
  constexpr int OPB = NS * (XS + WS);       // operand stages
  constexpr int EPS = WTN * 2 + 16;         // epilogue: bytes per staged output row
  constexpr int EPB = NW * WTT * EPS;       // epilogue: the waves' bf16 tiles
  constexpr int SCO = OPB > EPB ? OPB : EPB;  // scales live after both
  __shared__ __attribute__((aligned(1024))) int8_t smem[SCO + (BT + 2 * BN) * 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wt = wave % WGT, wn = wave / WGT;
  const int nt_t = (T + BT - 1) / BT, nt_n = (N + BN - 1) / BN;
  int pid_t, pid_n;
  tile_of(blockIdx.x, nt_t, nt_n, group_t, pid_t, pid_n);
  const int t0 = pid_t * BT, n0 = pid_n * BN;

  int8_t* xs_l = smem;              // [NS][BT][BK]
  int8_t* ws_l = smem + NS * XS;    // [NS][BN][BK]

  // --- global -> LDS through buffer resources based at the tile's first row.
  // Rows past T (or N) are outside the resource's range and read as zeros.
  // Lane l of a 1 KiB load fills row 16b + l/4, chunk position l%4, which holds
  // the row's 16-byte K chunk (l%4) ^ swz(row); k0 goes in the scalar offset.
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(xq + (int64_t)t0 * K), 0, min(BT, T - t0) * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wq + (int64_t)n0 * K), 0, min(BN, N - n0) * K, 0x00020000);
  const int lrow = lane >> 2, lchunk = lane & 3;
  int xoff[XL], woff[WL];
#pragma unroll
  for (int bb = 0; bb < XL; ++bb) {
    const int row = (bb * NW + wave) * 16 + lrow;
    xoff[bb] = row * K + ((lchunk ^ swz<SWZ>(row)) << 4);
  }
#pragma unroll
  for (int bb = 0; bb < WL; ++bb) {
    const int row = (bb * NW + wave) * 16 + lrow;
    woff[bb] = row * K + ((lchunk ^ swz<SWZ>(row)) << 4);
  }
  auto issue = [&](int stage) {   // K stage `stage` -> LDS buffer stage % NS
    const int buf = stage & (NS - 1);
    issue_rows<XL, NW>(xr, xs_l + buf * XS, xoff, wave, stage * BK);
    issue_rows<WL, NW>(wr, ws_l + buf * WS, woff, wave, stage * BK);
  };

  // the tile's scales and bias, staged once in their own LDS region (read
  // after the K loop, whose barriers make them visible)
  float* s_xs = reinterpret_cast<float*>(smem + SCO);   // [BT]
  float* s_ws = s_xs + BT;                               // [BN]
  float* s_b = s_ws + BN;                                // [BN]
  const bool has_bias = bias != nullptr;
  if (OUT != OUT_I32) {
    for (int i = threadIdx.x; i < BT; i += NTH) s_xs[i] = (t0 + i < T) ? xs[t0 + i] : 0.0f;
    for (int i = threadIdx.x; i < BN; i += NTH) {
      s_ws[i] = (n0 + i < N) ? ws[n0 + i] : 0.0f;
      s_b[i] = (has_bias && n0 + i < N) ? bias[n0 + i] : 0.0f;
    }
  }

  typedef typename std::conditional<F8, v16f, v16i>::type AccT;
  AccT acc[NTN][NTT];
#pragma unroll
  for (int i = 0; i < NTN; ++i)
#pragma unroll
    for (int j = 0; j < NTT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  // --- MFMA operands of k-step kk (32 bytes of K) of a stage
  const int frow = lane & 31, fhalf = lane >> 5;
  auto frags = [&](int stage, int kk, v4i (&a)[NTN], v4i (&b)[NTT]) {
    const int buf = stage & (NS - 1);
    const int8_t* wb = ws_l + buf * WS;
    const int8_t* xb = xs_l + buf * XS;
    const int c = kk * 2 + fhalf;
#pragma unroll
    for (int i = 0; i < NTN; ++i) {
      const int row = wn * WTN + i * 32 + frow;
      a[i] = *reinterpret_cast<const v4i*>(wb + row * BK + ((c ^ swz<SWZ>(row)) << 4));
    }
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int row = wt * WTT + j * 32 + frow;
      b[j] = *reinterpret_cast<const v4i*>(xb + row * BK + ((c ^ swz<SWZ>(row)) << 4));
    }
  };
  auto mfmas = [&](const v4i (&a)[NTN], const v4i (&b)[NTT]) {
    if constexpr (!F8) {
#pragma unroll
      for (int i = 0; i < NTN; ++i)
#pragma unroll
        for (int j = 0; j < NTT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // --- pipeline.  Stage s lives in LDS buffer s % 4.  In iteration s the
  // operands of k-step 1 are read while k-step 0 multiplies; then every wave
  // waits for stage s+1 to land (its own loads; the barrier makes them
  // everyone's) and for its reads of stage s to finish, so after the barrier
  // buffer s % 4 is free: the loads of stage s+4 go there, and k-step 0 of
  // stage s+1 is read while k-step 1 of stage s multiplies.
  const int nst = K / BK;
  issue(0);
  if (nst > 1) issue(1);
  if (nst > 2) issue(2);
  if (nst > 3) issue(3);
  // stage 0 landed: at most min(nst-1, 3) later stages still in flight
  if (nst >= 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LPS) : "memory");
  else if (nst == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPS) : "memory");
  else if (nst == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (F8) {
    // FP8: one v_mfma_f32_32x32x64_f8f6f4 per 32x32 tile per stage.  A lane's
    // 32 operand bytes are its two 16-byte chunks of the INT8 layout (k-steps
    // 0 and 1): the A and B operands take the same K positions, so the sum is
    // over the stage's 64 K values in a permuted order.  Iteration s: wait for
    // stage s+1 and for this wave's reads of stage s (issued last iteration),
    // barrier, loads of stage s+4 into the buffer stage s vacated, then the
    // MFMAs of stage s column by column, each column's B operands of stage s+1
    // read as soon as its MFMAs have consumed stage s's.
    typedef int v8i_t __attribute__((ext_vector_type(8)));
    auto cat = [](const v4i& lo, const v4i& hi) -> v8i_t {
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto fa = [&](int stage, int i, v4i& lo, v4i& hi) {
      const int8_t* wb = ws_l + (stage & (NS - 1)) * WS;
      const int row = wn * WTN + i * 32 + frow;
      lo = *reinterpret_cast<const v4i*>(wb + row * BK + ((fhalf ^ swz<SWZ>(row)) << 4));
      hi = *reinterpret_cast<const v4i*>(wb + row * BK + (((2 + fhalf) ^ swz<SWZ>(row)) << 4));
    };
    auto fb = [&](int stage, int j, v4i& lo, v4i& hi) {
      const int8_t* xb = xs_l + (stage & (NS - 1)) * XS;
      const int row = wt * WTT + j * 32 + frow;
      lo = *reinterpret_cast<const v4i*>(xb + row * BK + ((fhalf ^ swz<SWZ>(row)) << 4));
      hi = *reinterpret_cast<const v4i*>(xb + row * BK + (((2 + fhalf) ^ swz<SWZ>(row)) << 4));
    };
    // A1/B1 are written before they are read whenever a next stage exists; the
    // zeros only keep the optimizer from treating them as undefined.
    v4i A0[NTN][2], B0[NTT][2], A1[NTN][2], B1[NTT][2];
#pragma unroll
    for (int i = 0; i < NTN; ++i) A1[i][0] = A1[i][1] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < NTT; ++j) B1[j][0] = B1[j][1] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NTN; ++i) fa(0, i, A0[i][0], A0[i][1]);
#pragma unroll
    for (int j = 0; j < NTT; ++j) fb(0, j, B0[j][0], B0[j][1]);
    auto step8 = [&](int st, v4i (&ca)[NTN][2], v4i (&cb)[NTT][2], v4i (&na)[NTN][2],
                     v4i (&nb)[NTT][2]) {
      const int left = nst - 1 - st;          // stages after st
      if (left >= 3) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * LPS) : "memory");
      else if (left == 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LPS) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
      if (st + NS < nst) issue(st + NS);
      const bool more = left >= 1;
#pragma unroll
      for (int j = 0; j < NTT; ++j) {
#pragma unroll
        for (int i = 0; i < NTN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              cat(ca[i][0], ca[i][1]), cat(cb[j][0], cb[j][1]), acc[i][j], 0, 0, 0, 0, 0, 0);
        if (more) fb(st + 1, j, nb[j][0], nb[j][1]);
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < NTN; ++i) fa(st + 1, i, na[i][0], na[i][1]);
      }
    };
    int st = 0;
    for (; st + 1 < nst; st += 2) {
      step8(st, A0, B0, A1, B1);
      step8(st + 1, A1, B1, A0, B0);
    }
    if (st < nst) step8(st, A0, B0, A1, B1);
  } else {
  v4i a0[NTN], b0[NTT], a1[NTN], b1[NTT];
  frags(0, 0, a0, b0);
  // one iteration; FLY = stages still in flight after stage s+1 has landed
  // (-1: s is the last stage), ISSUE: the loads of stage s+4 exist.  One wave
  // per SIMD means nothing else can issue while this wave is busy with
  // non-MFMA work, so the operand reads and global loads are interleaved
  // one-for-one with the MFMAs (sched_group_barrier) and run under them:
  //   A: MFMAs of k-step 0 of stage s   | LDS reads of k-step 1 of stage s
  //   wait: stage s+1 landed, own reads of stage s done; workgroup barrier
  //   B: MFMAs of k-step 1 of stage s   | LDS reads of k-step 0 of stage s+1,
  //                                     | then the loads of stage s+4 into the
  //                                     | buffer stage s just vacated
  // The steady state has no branch inside, so nothing forces a full wait.
  auto iter = [&](int st, auto fly_tag, auto issue_tag) {
    constexpr int FLY = decltype(fly_tag)::value;
    constexpr bool ISSUE = decltype(issue_tag)::value;
    constexpr int NF = NTN + NTT;                 // operand reads per k-step
    constexpr int NM = NTN * NTT;                 // MFMAs per k-step
    constexpr int PA = NF < NM ? NF : NM;         // (MFMA, read) pairs
    frags(st, 1, a1, b1);
    mfmas(a0, b0);
#pragma unroll
    for (int q = 0; q < PA; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    if (NM > PA) __builtin_amdgcn_sched_group_barrier(0x008, NM - PA, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep k-step 0's MFMAs above the barrier
    if (FLY >= 0) {
      if (FLY >= 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * LPS) : "memory");
      else if (FLY == 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LPS) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
      if (ISSUE) issue(st + NS);
      frags(st + 1, 0, a0, b0);
      mfmas(a1, b1);
#pragma unroll
      for (int q = 0; q < PA; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);   // 1 LDS read
      }
      if (NM > PA) __builtin_amdgcn_sched_group_barrier(0x008, NM - PA, 1);
    } else {
      mfmas(a1, b1);
    }
  };
  using I2 = std::integral_constant<int, 2>;
  using I1 = std::integral_constant<int, 1>;
  using I0 = std::integral_constant<int, 0>;
  using IN = std::integral_constant<int, -1>;
  using BT_ = std::integral_constant<bool, true>;
  using BF_ = std::integral_constant<bool, false>;
  int st = 0;
  for (; st + NS < nst; ++st) iter(st, I2(), BT_());
  if (st == nst - 4) iter(st++, I2(), BF_());
  if (st == nst - 3) iter(st++, I1(), BF_());
  if (st == nst - 2) iter(st++, I0(), BF_());
  iter(st, IN(), BF_());
  }
  __syncthreads();

  // --- epilogue.  Lane l of tile (i, j): token t = .. + l%32; channels
  // n = .. + 8g + 4(l/32) + e for g, e in 0..3 hold acc[i][j][4g + e].
  // y = fp32(fp32(xs[t] * ws[n]) * fp32(acc)) + bias[n].
  const bool full_tile = (t0 + BT <= T) && (n0 + BN <= N);
  if (OUT == OUT_BF16) {
    // Stage the wave's WTT x WTN bf16 tile in LDS (rows of 2*WTN bytes, padded
    // to EPS), then write it out 16 bytes per lane along the row: each store
    // covers whole rows of the wave's tile instead of 32 rows x 16 bytes.
    int8_t* ep = smem + wave * WTT * EPS;
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int tw = j * 32 + frow;                  // row in the wave's tile
      const float xst = s_xs[wt * WTT + tw];
#pragma unroll
      for (int i = 0; i < NTN; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nw = i * 32 + g * 8 + fhalf * 4;   // column in the wave's tile
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(s_ws + wn * WTN + nw);
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(s_b + wn * WTN + nw);
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sc = xst * w4[e];
            const float v = sc * (float)acc[i][j][4 * g + e];
            o[e] = has_bias ? v + b4[e] : v;
          }
          u32x2 pk;
          pk[0] = pack_bf16x2(o[0], o[1]);
          pk[1] = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<u32x2*>(ep + tw * EPS + nw * 2) = pk;
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave reads only its own tile
    constexpr int CPR = WTN / 8;          // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPR;         // rows per store instruction
    const int rr = lane / CPR, cc = lane % CPR;
#pragma unroll 4
    for (int r0 = 0; r0 < WTT; r0 += RPI) {
      const int tw = r0 + rr;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ep + tw * EPS + cc * 16);
      const int t = t0 + wt * WTT + tw;
      const int n = n0 + wn * WTN + cc * 8;
      uint16_t* dst = reinterpret_cast<uint16_t*>(yout) + (int64_t)t * ldy + n;
      if (full_tile || (t < T && n + 8 <= N)) {
        // non-temporal: the output is not read again here, and it then leaves
        // no dirty lines in the caches to be written back under the next
        // kernels' streams
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
      } else if (t < T) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) dst[e] = (uint16_t)((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      }
    }
    return;
  }
  // fp32 and int32 outputs: straight from the accumulator layout
  const bool full_i32 = full_tile && (OUT != OUT_I32 || (N & 3) == 0);
#pragma unroll
  for (int j = 0; j < NTT; ++j) {
    const int tl = wt * WTT + j * 32 + frow;
    const int t = t0 + tl;
    const float xst = (OUT == OUT_I32) ? 0.0f : s_xs[tl];
#pragma unroll
    for (int i = 0; i < NTN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * WTN + i * 32 + g * 8 + fhalf * 4;
        const int n = n0 + nl;
        if (OUT == OUT_I32) {
          int32_t* dst = reinterpret_cast<int32_t*>(yout) + (int64_t)t * N + n;
          v4i o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (F8) {
              // bit_cast of the vector-element lvalue itself reads element 0
              // of the vector; go through a scalar copy
              const float f = acc[i][j][4 * g + e];
              o[e] = __builtin_bit_cast(int32_t, f);
            }
            else o[e] = acc[i][j][4 * g + e];
          }
          if (full_i32) {
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
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------

template <int BT, int BN, int WGT, int WGN, bool F8>
static void gemm_tile(const int8_t* xq, const float* xs, int T, int K, const int8_t* wq,
                      const float* ws, int N, const float* bias, void* y, int ldy, int out,
                      hipStream_t st) {
  constexpr int SWZ = 2;
  const int ntiles = ((T + BT - 1) / BT) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)ntiles), block(64 * WGT * WGN);
  const int group_t = 4;
  if (out == OUT_BF16)
    hipLaunchKernelGGL((k_gemm_w8a8<BT, BN, WGT, WGN, SWZ, OUT_BF16, F8>), grid, block, 0, st, xq,
                       xs, T, K, wq, ws, N, bias, y, ldy, group_t);
  else if (out == OUT_F32)
    hipLaunchKernelGGL((k_gemm_w8a8<BT, BN, WGT, WGN, SWZ, OUT_F32, F8>), grid, block, 0, st, xq,
                       xs, T, K, wq, ws, N, bias, y, ldy, group_t);
  else
    hipLaunchKernelGGL((k_gemm_w8a8<BT, BN, WGT, WGN, SWZ, OUT_I32, F8>), grid, block, 0, st, xq,
                       xs, T, K, wq, ws, N, bias, y, ldy, group_t);
}

// compute units of the current device (looked up once per device; threads
// that race on the first lookup store the same value)
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <bool F8>
static void gemm_sizes(const int8_t* xq, const float* xs, int64_t T, int64_t K, const int8_t* wq,
                       const float* ws, int64_t N, const float* bias, void* y, int64_t ldy,
                       int out, hipStream_t st) {
  const int it = (int)T, ik = (int)K, in = (int)N, il = (int)ldy;
  // 256 x 256 tiles (8 waves) have the most reuse and win whenever they keep
  // at least 3/4 of the compute units busy; below that 128 x 256 tiles (8
  // waves), then 128 x 128 (4 waves), trade reuse for occupancy (measured on
  // the 2048-token q|k|v, o, down and gate|up shapes).
  const int64_t busy = 3 * (int64_t)cu_count() / 4;
  const int64_t t256 = ((T + 255) / 256) * ((N + 255) / 256);
  const int64_t t128x256 = ((T + 127) / 128) * ((N + 255) / 256);
  if (t256 >= busy)
    gemm_tile<256, 256, 2, 4, F8>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  else if (t128x256 >= busy)
    gemm_tile<128, 256, 2, 4, F8>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
  else
    gemm_tile<128, 128, 2, 2, F8>(xq, xs, it, ik, wq, ws, in, bias, y, il, out, st);
}

void launch_gemm(const int8_t* xq, const float* xs, int64_t T, int64_t K, const int8_t* wq,
                 const float* ws, int64_t N, const float* bias, void* y, int64_t ldy, int out,
                 hipStream_t st) {
  if (T <= 0 || N <= 0) return;
  if (T <= 64) {
    launch_gemm_decode(xq, xs, T, K, wq, ws, N, bias, y, ldy, out, st);
    return;
  }
  gemm_sizes<false>(xq, xs, T, K, wq, ws, N, bias, y, ldy, out, st);
}

// FP8 E4M3 operands; out 2 = the raw fp32 accumulators.  Few tokens run the
// tile kernel too (its rows past T read as zeros).
void launch_gemm_fp8(const uint8_t* xq, const float* xs, int64_t T, int64_t K, const uint8_t* wq,
                     const float* ws, int64_t N, const float* bias, void* y, int64_t ldy, int out,
                     hipStream_t st) {
  if (T <= 0 || N <= 0) return;
  gemm_sizes<true>(reinterpret_cast<const int8_t*>(xq), xs, T, K,
                   reinterpret_cast<const int8_t*>(wq), ws, N, bias, y, ldy, out, st);
}

}  // namespace sqk
