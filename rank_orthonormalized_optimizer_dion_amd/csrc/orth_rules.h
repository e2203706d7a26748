// How orth() of a factor Q chooses its CholeskyQR passes, shared by the
// blocked factorization (k_chol.hip) and the one-workgroup step of small
// matrices (k_small.hip), so that both take the same decisions.
//
// Pivot ratio d_j / S_jj: the j-th pivot over column j's squared norm, the
// squared sine of the angle between column j and the span of the columns
// before it.  A pivot ratio below kRatioRetry (or a failed pivot) abandons
// the first pass for the shifted retry; below kRatioTwo it asks for a
// second pass.  The finer decision comes from t = trace(C^{-1}), C the
// column-scaled Gram matrix: one pass leaves Q T^{-1} with an orthogonality
// error of about lambda_min(C)^-1 times the Gram matrix's relative error,
// and t lies between 1 / lambda_min(C) and r / lambda_min(C).  t <=
// kTraceTwo r keeps that error at float32's level (the workloads here stay
// below 2 r); t > kTraceRetry r means the first pass's result is too far
// from orthonormal for a second pass to repair.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dion {

constexpr double kRatioTwo = 1e-6;
constexpr double kRatioRetry = 1e-8;
constexpr double kTraceTwo = 1e3;
constexpr double kTraceRetry = 1e7;

// Shift of the retry, relative to each column's squared norm: A = S +
// s diag(S).  The float64 Gram matrix of a float32 factor of `rows` rows is
// exact in its products and rounds its sums, so each entry is within
// rows 2^-53 sqrt(S_ii S_jj), and the column-scaled error matrix within
// r rows 2^-53 in norm; with the Cholesky's own rounding, (r rows + r^2)
// 2^-50 is eight times what makes the shifted factorization succeed for any
// factor with finite, nonzero columns.  It is kept at 2^-30 or more so that
// T^{-1} (norm up to 1 / sqrt(s) in column-scaled units) stays small enough
// for the float64 triangular multiply to leave an exactly dependent column
// dependent to about 2^-53 sqrt(r) / s (see second_tol).  Every pivot ratio
// is then at least about s, and Q1 = Q T^{-1} has a condition number of
// about sqrt(s) kappa.  The retry accepts pivot ratios above s / 2.
__device__ __forceinline__ double retry_shift(int rows, int r) {
  const double s = (static_cast<double>(r) * rows + static_cast<double>(r) * r) * 0x1p-50;
  return s > 0x1p-30 ? s : 0x1p-30;
}

// Smallest pivot ratio the second pass accepts: r 2^-40.  A direction in
// which Q is exactly deficient keeps, in Q1 = fl32(Q T^{-1}), a relative
// size of at most about 2^-24 sqrt(r) from the float32 rounding and
// 2^-53 sqrt(r) / s <= 2^-23 sqrt(r) from the float64 products: a pivot
// ratio of order r 2^-46, which r 2^-40 clears by 2^6.  Genuinely
// ill-conditioned factors give ratios near 1 / (s kappa^2), so factors up
// to kappa of about 1e8 (beyond what float32 resolves) pass.
__device__ __forceinline__ double second_tol(int r) { return r * 0x1p-40; }

// Lane `k` (wavefront-uniform) of a float64 register, without the LDS
// round trip of a shuffle.
__device__ __forceinline__ double read_lane(double v, int k) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u), k);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), k);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// 1 / sqrt(x) for a positive normal x: the hardware estimate refined by two
// Newton-Raphson steps y <- y (3 - x y^2) / 2, each of which doubles the
// number of correct bits (to full float64 precision from an estimate good
// to 2^-14 or better).  Replaces a square root and a division on the
// factorization's serial path.
__device__ __forceinline__ double rsqrt_nr(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x, y * y, 1.5);
  y = y * fma(-0.5 * x, y * y, 1.5);
  return y;
}

}  // namespace dion
