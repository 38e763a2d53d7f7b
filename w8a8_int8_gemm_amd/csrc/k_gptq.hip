// k_gptq.hip -- GPTQ error-compensating rounding of the migrated weight on
// gfx950 ("06 -- SmoothQuant", section 10: SmoothQuant migration first, then
// GPTQ on the migrated weights; the pages name the step, the algorithm is the
// published GPTQ).  Everything runs in fp64, the chip's full-rate vector
// precision for this offline step.
//
//   1. H = X^T X over the calibration tokens' x^ (formed exactly as the
//      activation quantizer forms it), lower 64 x 64 tiles only.
//   2. Dead inputs (H_jj = 0) get H_jj = 1 and a zero weight row; then
//      H += damp * mean(diag H) * I.
//   3. GPTQ needs U, the upper Cholesky factor of H^-1 (H^-1 = U^T U).  With J
//      the index reversal, A = J H J = L L^T (lower Cholesky) gives
//      H = (J L J)(J L J)^T with J L J upper, so H^-1 = (J L^-1 J)^T (J L^-1 J)
//      and U = J L^-1 J: one blocked Cholesky (one-wave diagonal panels,
//      trailing updates in lazy batches of kLazy column blocks) and one
//      recursive triangular inverse (X21 = -X22 L21 X11 on halves, as fp64
//      GEMMs), and U[j][k] is read as X[K-1-j][K-1-k] from X = L^-1.
//   4. Rows of W^ (input channels) in blocks of 64: inside a block each row
//      is rounded with the plain quantizer's per-channel step, its error
//      e = (w - step * q) / U_jj is pushed onto the block's later rows (one
//      wave per 64 output channels, in registers), and the errors of a lazy
//      batch of kLazy blocks then update the later rows (fp64 GEMMs).  Output
//      channels are independent, so workgroups split N.
// The tile products run on the fp64 matrix instruction (Tile64).
#include "sq_common.h"
#include "sq_internal.h"

namespace sqk {

namespace {

constexpr int NB = 64;          // tile / block edge
constexpr int LDP = NB + 1;     // padded LDS row (fp64)
constexpr int kLazy = 4;        // blocks per lazy batch (Cholesky and GPTQ updates)

typedef double v4d __attribute__((ext_vector_type(4)));

// 64 x 64 product tile, acc += As * Bs over 64 k, on the fp64 matrix
// instruction v_mfma_f64_16x16x4f64 (workgroup of 4 waves).  Wave w owns the
// 32 x 32 quarter at rows 32 * (w / 2), columns 32 * (w % 2): 2 x 2 blocks of
// 16 x 16.  Operand lanes: A row lane % 16 and k lane / 16, B column lane % 16
// and k lane / 16; result value v of lane l is row 4v + l / 16, column l % 16
// of its block (layouts read off the instruction by a probe).  Every output
// element sums its 64 products in the same k order, so a tile and its
// transpose give bit-identical sums.
struct Tile64 {
  v4d acc[2][2];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
  }

  __device__ __forceinline__ void mma(const double (*As)[LDP], const double (*Bs)[LDP]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
    const int li = lane & 15, lk = lane >> 4;
#pragma unroll 4
    for (int k = 0; k < NB; k += 4) {
      const double a0 = As[r0 + li][k + lk], a1 = As[r0 + 16 + li][k + lk];
      const double b0 = Bs[k + lk][c0 + li], b1 = Bs[k + lk][c0 + 16 + li];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
  }

  // f(row, column, value) for this lane's 16 elements of the 64 x 64 tile
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (wave >> 1) * 32 + (lane >> 4), c0 = (wave & 1) * 32 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) f(r0 + 16 * i + 4 * v, c0 + 16 * j, acc[i][j][v]);
  }
};

// block (ti, tj), ti >= tj, of a lower-triangular tile grid from a linear index
__device__ __forceinline__ void lower_pair(int64_t idx, int& ti, int& tj) {
  int i = (int)((sqrt(8.0 * (double)idx + 1.0) - 1.0) * 0.5);
  while ((int64_t)(i + 1) * (i + 2) / 2 <= idx) ++i;
  while ((int64_t)i * (i + 1) / 2 > idx) --i;
  ti = i;
  tj = (int)(idx - (int64_t)i * (i + 1) / 2);
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  return s;
}

}  // namespace

// ---------------------------------------------------------------------------
// r_t of each calibration row, in the activation quantizer's own order
// (lane l sums chunks l, l+64, ... with fused squares, then a wave sum), so the
// Hessian sees the quantizer's x^ bit for bit.
// ---------------------------------------------------------------------------
template <class In>
__global__ __launch_bounds__(256) void k_rms_rows(const typename In::elem* __restrict__ x,
                                                  int64_t T, int64_t K, int64_t ld, float eps,
                                                  float* __restrict__ r) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t nchunk = K >> 3;
  double ss = 0.0;
  for (int64_t ch = lane; ch < nchunk; ch += 64) {
    float v[8];
    In::load8(x + t * ld + ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double dv = (double)v[i];
      ss = fma(dv, dv, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) r[t] = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

// ---------------------------------------------------------------------------
// 1. Hessian, lower tiles: H[ti*64 + i][tj*64 + j] = sum_t x^[t][.] x^[t][.]
// x^ = fp32(fp32(x * r_t) * g_k) (norm) or fp32(x * g_k); the fp32 products
// are exact in fp64, so only the order of the sum differs from any other
// evaluation.
// ---------------------------------------------------------------------------
template <class In, bool NORM>
__global__ __launch_bounds__(256) void k_hessian(const typename In::elem* __restrict__ x,
                                                 int64_t T, int64_t K, int64_t ld,
                                                 const float* __restrict__ r,
                                                 const float* __restrict__ g,
                                                 double* __restrict__ H) {
  __shared__ double As[NB][LDP];   // As[i][t] = x^[t0 + t][ti*64 + i]
  __shared__ double Bs[NB][LDP];   // Bs[t][j] = x^[t0 + t][tj*64 + j]
  int ti, tj;
  lower_pair(blockIdx.x, ti, tj);
  Tile64 acc;
  acc.zero();
  // loader: thread -> (row lt = tid / 4, 16 columns at 16 * (tid % 4)) of
  // each 64-token chunk, for the ti panel (half 0) and the tj panel (half 1).
  // The next chunk's raw values are loaded while this chunk's products run.
  const int lt = threadIdx.x >> 2, lc = (threadIdx.x & 3) * 16;
  int64_t col0[2];
  col0[0] = (int64_t)ti * NB + lc;
  col0[1] = (int64_t)tj * NB + lc;
  float gv[2][16];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 16; ++e) gv[h][e] = g ? g[col0[h] + e] : 1.0f;
  typename In::Raw raw[2][2];
  float rt = 1.0f;
  auto load = [&](int64_t t0) {
    const int64_t t = min(t0 + lt, T - 1);   // rows past T: zeroed at the store
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      raw[h][0] = In::raw8(x + t * ld + col0[h]);
      raw[h][1] = In::raw8(x + t * ld + col0[h] + 8);
    }
    if (NORM) rt = r[t];
  };
  load(0);
  for (int64_t t0 = 0; t0 < T; t0 += NB) {
    const bool live = t0 + lt < T;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v[16];
      In::widen(raw[h][0], *reinterpret_cast<float(*)[8]>(&v[0]));
      In::widen(raw[h][1], *reinterpret_cast<float(*)[8]>(&v[8]));
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float u = NORM ? v[e] * rt : v[e];
        const double xh = live ? (double)(u * gv[h][e]) : 0.0;
        if (h == 0) As[lc + e][lt] = xh;
        else Bs[lt][lc + e] = xh;
      }
    }
    __syncthreads();
    if (t0 + NB < T) load(t0 + NB);
    asm volatile("" ::: "memory");   // keep those loads ahead of the products
    acc.mma(As, Bs);
    __syncthreads();
  }
  acc.each([&](int r, int c, double v) { H[((int64_t)ti * NB + r) * K + (int64_t)tj * NB + c] = v; });
}

// ---------------------------------------------------------------------------
// 2. Dead inputs and damping (one workgroup): dg[j] = (H_jj == 0 ? 1 : H_jj)
// + damp * mean_j(that value); dead[j] = 1 where H_jj == 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_hess_diag(const double* __restrict__ H, int64_t K,
                                                   float damp, double* __restrict__ dg,
                                                   unsigned char* __restrict__ dead) {
  __shared__ double red[4];
  double s = 0.0;
  for (int64_t j = threadIdx.x; j < K; j += 256) {
    const double h = H[j * K + j];
    s += (h == 0.0) ? 1.0 : h;
  }
  const double mean = block_sum(s, red) / (double)K;
  const double add = (double)damp * mean;
  for (int64_t j = threadIdx.x; j < K; j += 256) {
    const double h = H[j * K + j];
    dead[j] = (h == 0.0) ? 1 : 0;
    dg[j] = ((h == 0.0) ? 1.0 : h) + add;
  }
}

// A = J H J, lower tiles: A[i][j] = H[K-1-i][K-1-j] = Hlow[K-1-j][K-1-i] for
// i > j, the fixed diagonal on i == j, 0 above it.
__global__ __launch_bounds__(256) void k_hess_reverse(const double* __restrict__ H, int64_t K,
                                                      const double* __restrict__ dg,
                                                      double* __restrict__ A) {
  int ti, tj;
  lower_pair(blockIdx.x, ti, tj);
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int64_t i = (int64_t)ti * NB + e / NB, j = (int64_t)tj * NB + e % NB;
    double v;
    if (i == j) v = dg[K - 1 - i];
    else if (i > j) v = H[(K - 1 - j) * K + (K - 1 - i)];
    else v = 0.0;
    A[i * K + j] = v;
  }
}

// ---------------------------------------------------------------------------
// 3. Blocked Cholesky of A (lower, in place) and the inverse of its factor.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// 1 / sqrt(x): the hardware estimate and two Newton steps
__device__ __forceinline__ double rsqrt_nr(double x) {
  double y = __builtin_amdgcn_rsq(x);
#pragma unroll
  for (int it = 0; it < 2; ++it) y = fma(0.5 * y, fma(-x * y, y, 1.0), y);
  return y;
}

// The update stream of a 64 x 64 triangle in chunks: row jj (0 .. 62) takes
// the groups g = (jj + 1) / 8 .. 7 of its entries 8g .. 8g + 7 (the entries
// past the diagonal, rounded out to whole groups).
struct UChunks {
  int row[NB * 8], grp[NB * 8], n;
};
constexpr UChunks make_uchunks() {
  UChunks L{};
  int n = 0;
  for (int jj = 0; jj + 1 < NB; ++jj)
    for (int g = (jj + 1) / 8; g < NB / 8; ++g) {
      L.row[n] = jj;
      L.grp[n] = g;
      ++n;
    }
  L.n = n;
  return L;
}
constexpr UChunks kUChunks = make_uchunks();
// index in kUChunks of row jj's first chunk
constexpr int first_uchunk(int jj) {
  int n = 0;
  for (int r = 0; r < jj; ++r) n += NB / 8 - (r + 1) / 8;
  return n;
}
constexpr int kRing = 4;   // chunks in flight (4 LDS reads each; lgkmcnt counts to 15)

// An empty asm that takes v[0 .. 7] as read-write VGPR operands, with a
// memory clobber: the products that update them, and the loads issued before
// it, stay before it.  Without such pins the scheduler hoists whole triangles
// of LDS loads, or sinks the row-by-row products to first use, and either way
// holds thousands of values; with them, each chunk's loads are issued kRing
// chunks ahead of its products.
__device__ __forceinline__ void pin8(double* v) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
               "+v"(v[6]), "+v"(v[7])::"memory");
}

// Diagonal block p, one wave: lane i holds row i of the 64 x 64 block in
// VGPRs.  Right-looking Cholesky, column c: the pivot reaches every lane by
// readlane, lane i puts L[i][c] in row c of LT (the factor transposed, in
// LDS), and every lane reads that row at once (a broadcast) for its updates.
// The next column's pivot comes first (its one update takes L[c+1][c] by
// readlane) so that its square root overlaps the rest of column c's updates.
// Then the factor's inverse, right-looking too: lane m holds column m of
// L^-1; step k scales entry k by 1 / L[k][k] and subtracts its multiples of
// L[a][k] (row k of LT) from the entries a > k.  One wave and LDS accesses
// in program order: a wave barrier suffices between a row's writes and its
// reads.  Written to A (lower, zeros above) and Dinv[p].
__global__ __launch_bounds__(64) void k_chol_panel(double* __restrict__ A, int64_t K, int p,
                                                   double* __restrict__ Dinv) {
  __shared__ __align__(16) double LT[NB][NB];   // LT[c][i] = L[i][c]
  __shared__ double Rd[NB];                     // 1 / L[c][c]
  const int i = threadIdx.x;
  const int64_t o = (int64_t)p * NB;
  double r[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) r[j] = A[(o + i) * K + o + j];   // upper part: never read
  double ring[kRing][8];
  double piv = readlane_f64(r[0], 0);
  double y = rsqrt_nr(piv);
  // every index below is a compile-time constant (static_for), so r, x and
  // the ring stay in VGPRs: no private (scratch) memory
  static_for<NB>([&](auto c_) {
    constexpr int c = decltype(c_)::value;
    const double lc = (i == c) ? piv * y : r[c] * y;
    r[c] = lc;
    LT[c][i] = lc;
    if (i == c) Rd[c] = y;
    __builtin_amdgcn_wave_barrier();
    if constexpr (c + 1 < NB) {
      // the next pivot first; the rest of the column's updates run meanwhile,
      // their LT reads kRing chunks ahead within the row
      r[c + 1] = fma(-lc, readlane_f64(lc, c + 1), r[c + 1]);
      piv = readlane_f64(r[c + 1], c + 1);
      y = rsqrt_nr(piv);
      constexpr int g0 = (c + 2) / 8, ng = c + 2 < NB ? NB / 8 - g0 : 0;
      auto fetch = [&](auto u_) {
        constexpr int u = decltype(u_)::value;
#pragma unroll
        for (int t = 0; t < 8; ++t) ring[u % kRing][t] = LT[c][8 * (g0 + u) + t];
      };
      static_for<(kRing < ng ? kRing : ng)>(fetch);
      static_for<ng>([&](auto u_) {
        constexpr int u = decltype(u_)::value;
        constexpr int g = g0 + u;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (8 * g + t >= c + 2) r[8 * g + t] = fma(-lc, ring[u % kRing][t], r[8 * g + t]);
        if constexpr (u + kRing < ng) fetch(std::integral_constant<int, u + kRing>());
        pin8(r + 8 * g);   // this chunk's products here, the next reads after
      });
    }
  });
#pragma unroll
  for (int j = 0; j < NB; ++j) A[(o + i) * K + o + j] = (j <= i) ? r[j] : 0.0;
  __builtin_amdgcn_wave_barrier();
  // column m = i of L^-1 (entries above m stay 0: zero right side); the rows
  // of LT stream through the ring kRing chunks ahead, across rows
  double x[NB];
#pragma unroll
  for (int a = 0; a < NB; ++a) x[a] = (a == i) ? 1.0 : 0.0;
  auto fetch = [&](auto ci_) {
    constexpr int ci = decltype(ci_)::value;
    const double* src = &LT[kUChunks.row[ci]][8 * kUChunks.grp[ci]];
#pragma unroll
    for (int t = 0; t < 8; ++t) ring[ci % kRing][t] = src[t];
  };
  static_for<kRing>(fetch);
  static_for<NB - 1>([&](auto k_) {
    constexpr int k = decltype(k_)::value;
    x[k] = x[k] * Rd[k];
    constexpr int g0 = (k + 1) / 8, ci0 = first_uchunk(k);
    static_for<NB / 8 - g0>([&](auto u_) {
      constexpr int u = decltype(u_)::value;
      constexpr int g = g0 + u, ci = ci0 + u;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (8 * g + t > k) x[8 * g + t] = fma(-ring[ci % kRing][t], x[k], x[8 * g + t]);
      if constexpr (ci + kRing < kUChunks.n) fetch(std::integral_constant<int, ci + kRing>());
      pin8(x + 8 * g);
    });
  });
  x[NB - 1] = x[NB - 1] * Rd[NB - 1];
#pragma unroll
  for (int a = 0; a < NB; ++a) Dinv[(o + a) * NB + i] = x[a];
}

// Column panel below block p: L_ip = A_ip * (L_pp^-1)^T, block i = p + 1 + blockIdx.x.
__global__ __launch_bounds__(256) void k_chol_trsm(double* __restrict__ A, int64_t K, int p,
                                                   const double* __restrict__ Dinv) {
  __shared__ double As[NB][LDP];
  __shared__ double Bs[NB][LDP];
  const int i = p + 1 + blockIdx.x;
  const int64_t ro = (int64_t)i * NB, co = (int64_t)p * NB;
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int a = e / NB, b = e % NB;
    As[a][b] = A[(ro + a) * K + co + b];
    Bs[a][b] = Dinv[((int64_t)p * NB + b) * NB + a];   // Bs[k][c] = Dinv[c][k]
  }
  __syncthreads();
  Tile64 acc;
  acc.zero();
  acc.mma(As, Bs);
  acc.each([&](int r, int c, double v) { A[(ro + r) * K + co + c] = v; });
}

// Trailing update A_ij -= sum over the column blocks c of L_ic L_jc^T, c0 =
// 64 * (first c) and depth = 64 * (number of c), for the tiles
//   tri:  j0 <= j <= i < nt (the index lower_pair(blockIdx.x), offset by j0)
//   else: j = j0 + blockIdx.y, i = j + blockIdx.x < nt.
// The tiles written (j >= j0) never hold the columns read (c < j0).  The next
// 64-deep chunk of both operands is loaded while this one's products run.
__global__ __launch_bounds__(256) void k_chol_syrk(double* __restrict__ A, int64_t K, int64_t c0,
                                                   int depth, int j0, int nt, int tri) {
  __shared__ double As[NB][LDP];
  __shared__ double Bs[NB][LDP];
  int i, j;
  if (tri) {
    lower_pair(blockIdx.x, i, j);
    i += j0;
    j += j0;
  } else {
    j = j0 + (int)blockIdx.y;
    i = j + (int)blockIdx.x;
    if (i >= nt) return;   // whole workgroup
  }
  const int64_t ri = (int64_t)i * NB, rj = (int64_t)j * NB;
  Tile64 acc;
  acc.zero();
  // element e = threadIdx.x + 256 u (u < 16): row e / 64, column e % 64 of the
  // chunk, As[a][b] = L_ic[a][b] and Bs[b][a] = L_jc[a][b]
  double pa[16], pb[16];
  auto load = [&](int c) {
    const int64_t co = c0 + (int64_t)c * NB;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = threadIdx.x + 256 * u, a = e / NB, b = e % NB;
      pa[u] = A[(ri + a) * K + co + b];
      pb[u] = A[(rj + a) * K + co + b];
    }
  };
  load(0);
  for (int c = 0; c < depth / NB; ++c) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = threadIdx.x + 256 * u, a = e / NB, b = e % NB;
      As[a][b] = pa[u];
      Bs[b][a] = pb[u];
    }
    __syncthreads();
    if (c + 1 < depth / NB) load(c + 1);
    asm volatile("" ::: "memory");   // keep those loads ahead of the products
    acc.mma(As, Bs);
    __syncthreads();
  }
  acc.each([&](int r, int c, double v) {
    double* q = A + (ri + r) * K + rj + c;
    *q = *q - v;
  });
}

// C = alpha * A B on 64 x 64 tiles (M, N, Kd multiples of 64), row-major
// with leading dimensions; tile (blockIdx.y, blockIdx.x).  Used for the
// triangular inverse.  tri bit 0: A is block lower triangular (its 64 x 64
// blocks right of the diagonal are zero); bit 1: B is; the products of zero
// blocks are skipped.
constexpr int kTriA = 1, kTriB = 2;
__global__ __launch_bounds__(256) void k_dgemm(int64_t M, int64_t N, int64_t Kd, double alpha,
                                               const double* __restrict__ A, int64_t lda,
                                               const double* __restrict__ B, int64_t ldb,
                                               double* __restrict__ C, int64_t ldc, int tri) {
  __shared__ double As[NB][LDP];
  __shared__ double Bs[NB][LDP];
  const int64_t m0 = (int64_t)blockIdx.y * NB, n0 = (int64_t)blockIdx.x * NB;
  const int64_t k_lo = (tri & kTriB) ? n0 : 0;
  const int64_t k_hi = (tri & kTriA) ? min(Kd, m0 + NB) : Kd;
  Tile64 acc;
  acc.zero();
  // element e = threadIdx.x + 256 i (i < 16) of each 64 x 64 operand chunk;
  // the next chunk is loaded while this one's products run
  double pa[16], pb[16];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = threadIdx.x + 256 * i, a = e / NB, b = e % NB;
      pa[i] = A[(m0 + a) * lda + k0 + b];
      pb[i] = B[(k0 + a) * ldb + n0 + b];
    }
  };
  if (k_lo < k_hi) load(k_lo);
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += NB) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = threadIdx.x + 256 * i, a = e / NB, b = e % NB;
      As[a][b] = pa[i];
      Bs[a][b] = pb[i];
    }
    __syncthreads();
    if (k0 + NB < k_hi) load(k0 + NB);
    asm volatile("" ::: "memory");   // keep those loads ahead of the products
    acc.mma(As, Bs);
    __syncthreads();
  }
  acc.each([&](int r, int c, double x) { C[(m0 + r) * ldc + n0 + c] = alpha * x; });
}

// X = L^-1 before the recursion: X_ii = Dinv[i], every other block 0 (the
// products below read whole square ranges of X, upper blocks included);
// block (blockIdx.y, blockIdx.x)
__global__ __launch_bounds__(256) void k_trinv_init(int64_t K, const double* __restrict__ Dinv,
                                                    double* __restrict__ X) {
  const int64_t ro = (int64_t)blockIdx.y * NB, co = (int64_t)blockIdx.x * NB;
  const bool diag = blockIdx.x == blockIdx.y;
  for (int e = threadIdx.x; e < NB * NB; e += 256)
    X[(ro + e / NB) * K + co + e % NB] = diag ? Dinv[(ro + e / NB) * NB + e % NB] : 0.0;
}

// ---------------------------------------------------------------------------
// 4. The rounding loop.  W64 [K, N] fp64 holds W^ = fp32(W * s) (dead rows 0).
// ---------------------------------------------------------------------------
template <class In>
__global__ __launch_bounds__(256) void k_gptq_init(const typename In::elem* __restrict__ w,
                                                   int64_t K, int64_t N, int64_t ld,
                                                   const float* __restrict__ s,
                                                   const unsigned char* __restrict__ dead,
                                                   double* __restrict__ W64) {
  const int64_t per = (N + 7) >> 3;   // the last chunk of a row may be ragged
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= K * per) return;
  const int64_t j = c / per, n0 = (c - j * per) * 8;
  float v[8];
  In::widen(raw8_upto<In>(w + j * ld + n0, N - n0), v);
  const float sj = s ? s[j] : 1.0f;
  double* dst = W64 + j * N + n0;
  if (n0 + 8 <= N) {   // whole chunks: eight adjacent stores the compiler merges
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = dead[j] ? 0.0 : (double)(v[e] * sj);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (n0 + e < N) dst[e] = dead[j] ? 0.0 : (double)(v[e] * sj);
  }
}

// Block b (rows r0 = b*64 .. +63) of the rounding for the 64 output channels
// n = blockIdx.x*64 + lane, one wave: each lane holds its channel's 64 rows in
// registers and carries the row-by-row updates there; U[r0 + jj][r0 + kk]
// (kk > jj) is read by every lane at the same LDS address (a broadcast).
// U[j][k] = X[K-1-j][K-1-k].  The reads stream through a ring of kRing
// chunks of eight values, issued kRing chunks ahead of their products, and
// row jj + 1's code and error are computed right after the chunk that updates
// it.  E has row stride ldE = N rounded up to 64: the lanes past N write
// zeros there.
//
// The code of w / d is rint(w * (1 / d)), except within 1e-9 of a
// half-integer h, where the sign of w - h d (one fused multiply-add: exact in
// sign) picks the side, and a zero (w / d = h exactly) rounds h to even.  That
// is the rounding of the exact quotient; it can differ from rounding the
// correctly rounded quotient only within half an ulp of h.
__device__ __forceinline__ double gptq_code(double wv, double d, double rd) {
  const double t = wv * rd;
  const double h = floor(t) + 0.5;
  const double side = fma(-h, d, wv);
  const double up = h + 0.5, dn = h - 0.5, even = rint(h);
  double qn = side > 0.0 ? up : even;
  qn = side < 0.0 ? dn : qn;
  asm volatile("" : "+v"(qn));   // computed on every row: a select, not a branch
  const double q = fabs(t - h) < 1e-9 ? qn : rint(t);
  return d > 0.0 ? fmin(fmax(q, -127.0), 127.0) : 0.0;
}

__global__ __launch_bounds__(64) void k_gptq_block(const double* __restrict__ W64, int64_t K,
                                                   int64_t N, int64_t ldE, int b,
                                                   const double* __restrict__ X,
                                                   const float* __restrict__ wscale,
                                                   int8_t* __restrict__ wq,
                                                   double* __restrict__ E) {
  __shared__ __align__(16) double Ub[NB][NB];
  __shared__ double Ur[NB];        // 1 / U_jj
  const int c = threadIdx.x;
  const int64_t n = (int64_t)blockIdx.x * NB + c;
  const bool live = n < N;
  const int64_t nc = live ? n : N - 1;   // past-the-end lanes load a valid column
  const int64_t r0 = (int64_t)b * NB;
  const double* xr = X + (K - 1 - r0) * K + (K - 1 - r0 - c);   // U[r0][r0 + c]
  double w[NB];
#pragma unroll
  for (int jj = 0; jj < NB; ++jj) {
    Ub[jj][c] = xr[-(int64_t)jj * K];
    const double v = W64[(r0 + jj) * N + nc];
    w[jj] = live ? v : 0.0;
  }
  const double d = live ? (double)wscale[nc] : 0.0;
  const double rd = d > 0.0 ? 1.0 / d : 0.0;
  __syncthreads();
  Ur[c] = 1.0 / Ub[c][c];
  __syncthreads();
  double ring[kRing][8];
  auto fetch = [&](auto ci_) {
    constexpr int ci = decltype(ci_)::value;
    const double* src = &Ub[kUChunks.row[ci]][8 * kUChunks.grp[ci]];
#pragma unroll
    for (int t = 0; t < 8; ++t) ring[ci % kRing][t] = src[t];
  };
  static_for<kRing>(fetch);
  uint32_t packed[NB / 4];
#pragma unroll
  for (int i = 0; i < NB / 4; ++i) packed[i] = 0;
  double q = gptq_code(w[0], d, rd);
  double e = (w[0] - d * q) * Ur[0];
  // compile-time indices throughout (static_for): w, packed and the ring
  // stay in VGPRs, no private (scratch) memory
  static_for<NB>([&](auto jj_) {
    constexpr int jj = decltype(jj_)::value;
    packed[jj >> 2] |= ((uint32_t)(int)q & 0xffu) << (8 * (jj & 3));
    E[(int64_t)jj * ldE + n] = e;
    if constexpr (jj + 1 < NB) {
      double qn = 0.0, en = 0.0;
      constexpr int g0 = (jj + 1) / 8, ci0 = first_uchunk(jj);
      static_for<NB / 8 - g0>([&](auto u_) {
        constexpr int u = decltype(u_)::value;
        constexpr int g = g0 + u, ci = ci0 + u;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (8 * g + t > jj) w[8 * g + t] = fma(-ring[ci % kRing][t], e, w[8 * g + t]);
        if constexpr (u == 0) {
          qn = gptq_code(w[jj + 1], d, rd);
          en = (w[jj + 1] - d * qn) * Ur[jj + 1];
        }
        if constexpr (ci + kRing < kUChunks.n) fetch(std::integral_constant<int, ci + kRing>());
        pin8(w + 8 * g);   // this chunk's products here, the next reads after
      });
      q = qn;
      e = en;
    }
  });
  if (live) {
    // codes: output channel n, input channels r0 .. r0+63
    uint4* dst = reinterpret_cast<uint4*>(wq + n * K + r0);
#pragma unroll
    for (int i = 0; i < NB / 16; ++i)
      dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  }
}

// Later rows: W64[i][n] -= sum_jj U[r0 + jj][i] * E[jj][n], jj < depth (a
// multiple of 64: the error rows of one block, or of a whole lazy batch), for
// the rows i = i_first + 64 * blockIdx.y + (0 .. 63), all past r0 + depth;
// columns n0 = 64 * blockIdx.x.  E's row stride ldE covers every slab.
__global__ __launch_bounds__(256) void k_gptq_update(double* __restrict__ W64, int64_t K,
                                                     int64_t N, int64_t ldE, int64_t r0, int depth,
                                                     int64_t i_first,
                                                     const double* __restrict__ X,
                                                     const double* __restrict__ E) {
  __shared__ double As[NB][LDP];   // As[i][jj] = U[r0 + 64c + jj][i0 + i]
  __shared__ double Bs[NB][LDP];   // Bs[jj][col] = E[64c + jj][n0 + col]
  const int64_t i0 = i_first + (int64_t)blockIdx.y * NB;
  const int64_t n0 = (int64_t)blockIdx.x * NB;
  Tile64 acc;
  acc.zero();
  // element e = threadIdx.x + 256 i (i < 16) of each chunk's operands: U[j0 +
  // q][i0 + a] = X[K-1-j0-q][K-1-i0-a] (i0 + a > j0 + q: lower part of X),
  // consecutive threads on consecutive a (one row of X), and E[j0 - r0 + a][n0
  // + q].  The next chunk is loaded while this one's products run.
  double pu[16], pe[16];
  auto load = [&](int c) {
    const int64_t j0 = r0 + (int64_t)c * NB;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = threadIdx.x + 256 * i;
      pu[i] = X[(K - 1 - j0 - e / NB) * K + (K - 1 - i0 - e % NB)];
      pe[i] = E[((int64_t)c * NB + e / NB) * ldE + n0 + e % NB];
    }
  };
  load(0);
  for (int c = 0; c < depth / NB; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = threadIdx.x + 256 * i;
      As[e % NB][e / NB] = pu[i];
      Bs[e / NB][e % NB] = pe[i];
    }
    __syncthreads();
    if (c + 1 < depth / NB) load(c + 1);
    asm volatile("" ::: "memory");   // keep those loads ahead of the products
    acc.mma(As, Bs);
    __syncthreads();
  }
  acc.each([&](int r, int c, double v) {
    const int64_t nn = n0 + c;
    if (nn < N) {
      double* q = W64 + (i0 + r) * N + nn;
      *q = *q - v;
    }
  });
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

size_t gptq_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  auto r256 = [](int64_t b) { return (size_t)((b + 255) & ~int64_t(255)); };
  return r256(K * K * 8) * 2 + r256(K * NB * 8) + r256(K * 8) + r256(K) + r256(T * 4) +
         r256(K * N * 8) + r256((int64_t)kLazy * NB * ((N + NB - 1) / NB * NB) * 8) +
         r256(K * K * 2);
}

// X = L^-1 on the block range [b0, b0 + nb) (diagonal blocks already in X):
// for L = [[L11, 0], [L21, L22]], X21 = -X22 (L21 X11).
static void trinv_rec(const double* L, double* X, double* tmp, int64_t K, int b0, int nb,
                      hipStream_t st) {
  if (nb <= 1) return;
  const int h = nb / 2, h2 = nb - h;
  trinv_rec(L, X, tmp, K, b0, h, st);
  trinv_rec(L, X, tmp, K, b0 + h, h2, st);
  const int64_t o1 = (int64_t)b0 * NB, o2 = (int64_t)(b0 + h) * NB;
  const int64_t s1 = (int64_t)h * NB, s2 = (int64_t)h2 * NB;
  // tmp [s2, s1] = L21 X11
  hipLaunchKernelGGL(k_dgemm, dim3((unsigned)h, (unsigned)h2), dim3(256), 0, st, s2, s1, s1, 1.0,
                     L + o2 * K + o1, K, X + o1 * K + o1, K, tmp, s1, kTriB);
  // X21 = -X22 tmp
  hipLaunchKernelGGL(k_dgemm, dim3((unsigned)h, (unsigned)h2), dim3(256), 0, st, s2, s1, s2, -1.0,
                     X + o2 * K + o2, K, tmp, s1, X + o2 * K + o1, K, kTriA);
}

void launch_gptq(const void* x, bool xbf16, int64_t T, int64_t ldx, bool norm,
                 const float* gamma_f, float eps, const void* w, bool wbf16, int64_t K, int64_t N,
                 int64_t ldw, const float* s, float damp, int8_t* wq, float* wscale,
                 float* rrow_out, void* workspace, hipStream_t st) {
  auto r256 = [](int64_t b) { return (size_t)((b + 255) & ~int64_t(255)); };
  char* p = static_cast<char*>(workspace);
  double* H = reinterpret_cast<double*>(p);            p += r256(K * K * 8);   // then X = L^-1
  double* A = reinterpret_cast<double*>(p);            p += r256(K * K * 8);
  double* Dinv = reinterpret_cast<double*>(p);         p += r256(K * NB * 8);
  double* dg = reinterpret_cast<double*>(p);           p += r256(K * 8);
  unsigned char* dead = reinterpret_cast<unsigned char*>(p); p += r256(K);
  float* rr = rrow_out ? rrow_out : reinterpret_cast<float*>(p);  p += r256(T * 4);
  double* W64 = reinterpret_cast<double*>(p);          p += r256(K * N * 8);
  const int64_t ldE = (N + NB - 1) / NB * NB;
  double* E = reinterpret_cast<double*>(p);             p += r256((int64_t)kLazy * NB * ldE * 8);
  double* tmp = reinterpret_cast<double*>(p);
  const int nt = (int)(K / NB);
  const int64_t tiles = (int64_t)nt * (nt + 1) / 2;

  // the plain quantizer's per-output-channel step of W^ = W * s
  launch_fill_f32(wscale, N, 0.0f, st);
  launch_col_absmax(w, wbf16, K, N, ldw, s, 127.0f, wscale, st);

  // 1. Hessian
  if (norm) {
    const dim3 g((unsigned)((T + 3) / 4));
    if (xbf16) hipLaunchKernelGGL(k_rms_rows<Bf16In>, g, dim3(256), 0, st, (const uint16_t*)x, T, K, ldx, eps, rr);
    else hipLaunchKernelGGL(k_rms_rows<F32In>, g, dim3(256), 0, st, (const float*)x, T, K, ldx, eps, rr);
  }
  const dim3 gt((unsigned)tiles);
  if (xbf16) {
    if (norm) hipLaunchKernelGGL((k_hessian<Bf16In, true>), gt, dim3(256), 0, st, (const uint16_t*)x, T, K, ldx, rr, gamma_f, H);
    else hipLaunchKernelGGL((k_hessian<Bf16In, false>), gt, dim3(256), 0, st, (const uint16_t*)x, T, K, ldx, rr, gamma_f, H);
  } else {
    if (norm) hipLaunchKernelGGL((k_hessian<F32In, true>), gt, dim3(256), 0, st, (const float*)x, T, K, ldx, rr, gamma_f, H);
    else hipLaunchKernelGGL((k_hessian<F32In, false>), gt, dim3(256), 0, st, (const float*)x, T, K, ldx, rr, gamma_f, H);
  }
  // 2. dead inputs, damping, reversal
  hipLaunchKernelGGL(k_hess_diag, dim3(1), dim3(256), 0, st, H, K, damp, dg, dead);
  hipLaunchKernelGGL(k_hess_reverse, gt, dim3(256), 0, st, H, K, dg, A);
  // 3. Cholesky of A, then X = L^-1 into H's storage.  Right-looking in
  // lazy batches of kLazy column blocks: a block column's update reaches the
  // rest of its batch's columns (all rows) at once, and the columns past the
  // batch once per batch with all of its column blocks, so the trailing
  // matrix is read and written K / (64 kLazy) times instead of K / 64.
  for (int s0 = 0; s0 < nt; s0 += kLazy) {
    const int s1 = min(nt, s0 + kLazy);
    for (int q = s0; q < s1; ++q) {
      hipLaunchKernelGGL(k_chol_panel, dim3(1), dim3(64), 0, st, A, K, q, Dinv);
      const int rest = nt - q - 1;
      if (rest > 0) {
        hipLaunchKernelGGL(k_chol_trsm, dim3((unsigned)rest), dim3(256), 0, st, A, K, q, Dinv);
        if (q + 1 < s1)
          hipLaunchKernelGGL(k_chol_syrk, dim3((unsigned)rest, (unsigned)(s1 - q - 1)), dim3(256),
                             0, st, A, K, (int64_t)q * NB, NB, q + 1, nt, 0);
      }
    }
    const int rest = nt - s1;
    if (rest > 0)
      hipLaunchKernelGGL(k_chol_syrk, dim3((unsigned)((int64_t)rest * (rest + 1) / 2)), dim3(256),
                         0, st, A, K, (int64_t)s0 * NB, (s1 - s0) * NB, s1, nt, 1);
  }
  hipLaunchKernelGGL(k_trinv_init, dim3((unsigned)nt, (unsigned)nt), dim3(256), 0, st, K, Dinv, H);
  trinv_rec(A, H, tmp, K, 0, nt, st);
  // 4. rounding
  {
    const int64_t chunks = K * ((N + 7) >> 3);
    const dim3 g((unsigned)((chunks + 255) / 256));
    if (wbf16) hipLaunchKernelGGL(k_gptq_init<Bf16In>, g, dim3(256), 0, st, (const uint16_t*)w, K, N, ldw, s, dead, W64);
    else hipLaunchKernelGGL(k_gptq_init<F32In>, g, dim3(256), 0, st, (const float*)w, K, N, ldw, s, dead, W64);
  }
  // Lazy batches of kLazy blocks: a block's errors update the rest of its
  // batch at once, and the rows past the batch once per batch with all of its
  // error rows, so the fp64 weight below is read and written K / (64 kLazy)
  // times instead of K / 64.  The same terms reach every row; only the order
  // of their sum changes.
  const unsigned nslab = (unsigned)((N + NB - 1) / NB);
  for (int s0 = 0; s0 < nt; s0 += kLazy) {
    const int s1 = min(nt, s0 + kLazy);
    for (int b = s0; b < s1; ++b) {
      double* Eb = E + (int64_t)(b - s0) * NB * ldE;
      hipLaunchKernelGGL(k_gptq_block, dim3(nslab), dim3(64), 0, st, W64, K, N, ldE, b, H, wscale,
                         wq, Eb);
      const int rest_in = s1 - b - 1;
      if (rest_in > 0)
        hipLaunchKernelGGL(k_gptq_update, dim3(nslab, (unsigned)rest_in), dim3(256), 0, st, W64,
                           K, N, ldE, (int64_t)b * NB, NB, (int64_t)(b + 1) * NB, H, Eb);
    }
    const int rest = nt - s1;
    if (rest > 0)
      hipLaunchKernelGGL(k_gptq_update, dim3(nslab, (unsigned)rest), dim3(256), 0, st, W64, K, N,
                         ldE, (int64_t)s0 * NB, (s1 - s0) * NB, (int64_t)s1 * NB, H, E);
  }
}

}  // namespace sqk
