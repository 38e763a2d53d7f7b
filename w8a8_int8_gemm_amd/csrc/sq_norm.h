// sq_norm.h -- device helper for the LayerNorm statistics shared by the
// LayerNorm calibration and the LayerNorm quantizers.
#pragma once
#include "sq_common.h"

namespace sqk {

// LayerNorm statistics of a row of K values v in one pass, from sums shifted
// by c, an element of the row (v - c is formed in fp64: exact unless the two
// are more than 2^29 apart in magnitude, then rounded to 53 bits):
//   s1 = sum(v - c),  s2 = sum((v - c)^2)  (fp64, each square by one fma)
//   mean = c + s1/K,  var = s2/K - (s1/K)^2 = mean of (v - mean)^2.
// Because c is one of the values, (c - mean)^2 <= K var, so
// s2/K <= (K + 1) var and the cancellation in var costs at most a factor
// 3 (K + 1) on the fp64 summation error; with per-lane sums of K/64 terms and
// a 64-lane butterfly, K <= 65536 keeps var within 2.3e-8 relative and r
// within 0.2 fp32 ulp of the exact value.  The mean's error is that of any
// fp64 sum of the row, shifted or not.  m = fp32(mean),
// r = fp32(1 / sqrt(var + eps)); var is clamped at 0 (rounding may leave a
// tiny negative for a constant row, where it is exactly 0).
__device__ __forceinline__ void ln_stats(double c, double s1, double s2, int64_t K, float eps,
                                         float& m, float& r) {
  const double dK = (double)K;
  const double dm = s1 / dK;
  const double var = fmax(s2 / dK - dm * dm, 0.0);
  m = (float)(c + dm);
  r = (float)(1.0 / sqrt(var + (double)eps));
}

}  // namespace sqk
