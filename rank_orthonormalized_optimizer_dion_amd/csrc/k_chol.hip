// float64 Cholesky factorization S = T^T T (T upper triangular, positive
// diagonal) of the Gram matrix of a CholeskyQR pass, together with
// Y = T^{-T}, in blocks of 64 (kCholNB).  orth(Q) = Q T^{-1} is then one
// float32 MFMA product (k_trmm).  Y comes out of the same sweep: the row
// operations of the right-looking factorization are applied to an identity
// block column, i.e. forward substitution of T^T Y = I.
//
// Per block step kb (host loop):
//   k_chol_diag   factor the diagonal block, Dinv = T_kk^{-1}, Y_kk = T_kk^{-T}
//   k_chol_panel  T_kj = T_kk^{-T} A_kj (j > kb);  Y_kc = T_kk^{-T} Y_kc (c < kb)
//   k_chol_trail  A_ij -= T_ki^T T_kj (kb < i <= j);  Y_ic -= T_ki^T Y_kc (c <= kb),
//                 with look-ahead: block steps run in pairs (kb, kb + 1); mode 1
//                 updates block row kb + 1 alone with panel kb, so that block
//                 kb + 1 can be factored, and mode 2 then updates block rows
//                 kb + 2 on with both panels at once (128 reduction rows), one
//                 pass over the trailing matrix per two block steps
// k_chol_init sums the Gram partials into A (float64) first and pads the
// rows past r with the identity.
#include <math.h>

#include "device_common.h"
#include "launchers.h"

namespace dion {

namespace {

constexpr int NB = kCholNB;

// A pivot below this fraction of the column's original squared norm means
// the factor's condition number is beyond about 1e3, where the float32
// product Q T^{-1} would no longer have orthonormal columns to float32
// accuracy: the factor is declared numerically rank-deficient.
constexpr double kPivotTol = 1e-6;

__device__ __forceinline__ bool skipped(const Launch& L, const MatDesc& d) {
  return L.status[d.slot] != 0;
}

__device__ __forceinline__ double* dptr(const Launch& L, int64_t off) {
  return reinterpret_cast<double*>(L.ws + off);
}

// C += L^T R for 64 x 64 blocks over 64 reduction rows, C[i][j] +=
// sum_e L[e][i] R[e][j] (L, R row-major with pitches ll, lr), on the
// 16 x 16 x 4 float64 MFMA: 2 x 2 wavefronts of 32 x 32, each lane loading
// its own operands from memory (lane l: row 4 s + l / 16, column l % 16 of
// a 16-wide column strip, 16 consecutive doubles per 16 lanes).  All loads
// of a wavefront are issued before its first MFMA.
__device__ __forceinline__ void block_tn_add(const double* Lp, int64_t ll, const double* Rp,
                                             int64_t lr, f64x4 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int ci = (wave >> 1) * 32 + (lane & 15), cj = (wave & 1) * 32 + (lane & 15);
  gptr<const double> L = to_global(Lp);
  gptr<const double> R = to_global(Rp);
  double a[NB / 4][2], b[NB / 4][2];
#pragma unroll
  for (int s = 0; s < NB / 4; ++s)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      a[s][f] = L[(4 * s + g) * ll + ci + 16 * f];
      b[s][f] = R[(4 * s + g) * lr + cj + 16 * f];
    }
#pragma unroll
  for (int s = 0; s < NB / 4; ++s)
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s][fm], b[s][fn], acc[fm][fn], 0, 0, 0);
}

// C = L^T R (block_tn_add from zero).
__device__ __forceinline__ void block_tn(const double* Lp, int64_t ll, const double* Rp, int64_t lr,
                                         f64x4 (&acc)[2][2]) {
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) acc[fm][fn] = f64x4{0.0, 0.0, 0.0, 0.0};
  block_tn_add(Lp, ll, Rp, lr, acc);
}

// Offset of the element lane holds in register v of output block (fm, fn)
// of block_tn (16 x 16 float64 MFMA output: row l / 16 + 4 v, column l % 16).
__device__ __forceinline__ int64_t block_off(int fm, int fn, int v, int64_t ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = (wave >> 1) * 32 + fm * 16 + (lane >> 4) + 4 * v;
  const int col = (wave & 1) * 32 + fn * 16 + (lane & 15);
  return row * ld + col;
}

__global__ __launch_bounds__(kThreads) void k_chol_init(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int nblk = d.rp / NB;
  int p = local, bi = 0;
  while (p >= nblk - bi) {
    p -= nblk - bi;
    ++bi;
  }
  const int bj = bi + p;
  const double* S = reinterpret_cast<const double*>(L.ws + d.oS);
  double* A = dptr(L, d.oA);
  double* Sd = dptr(L, d.oD) + NB * NB;
  const int64_t rp = d.rp, plane = rp * rp;
  for (int e = threadIdx.x; e < NB * NB; e += kThreads) {
    const int gi = bi * NB + e / NB, gj = bj * NB + e % NB;
    double v;
    if (gi < d.r && gj < d.r) {
      // the Gram kernel writes the upper triangle (gi <= gj) only
      const int64_t e = static_cast<int64_t>(min(gi, gj)) * rp + max(gi, gj);
      v = 0.0;
      for (int s = 0; s < ci.splits; ++s) v += S[s * plane + e];
    } else {
      v = gi == gj ? 1.0 : 0.0;
    }
    A[gi * rp + gj] = v;
    if (gi == gj) Sd[gi] = v;
  }
}

// One 64 x 64 diagonal block: T_kk (upper, positive diagonal) with
// T_kk^T T_kk = A_kk, and Z = T_kk^{-T} from the same row operations on an
// identity block.  Thread (wavefront w, lane c) keeps rows 4 q + w of column
// c of both in registers; step k's scaled pivot row is broadcast through a
// double-buffered LDS row, so one barrier per step suffices (a buffer is
// rewritten two steps later, after every thread has passed the barrier that
// follows its last read).  A failed pivot is flagged in the same buffer, so
// every wavefront leaves the loop at the same step.
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

__global__ __launch_bounds__(kThreads) void k_chol_diag(Launch L) {
  __shared__ double rowA[2][NB];
  __shared__ double rowZ[2][NB];
  __shared__ double sd[NB];
  __shared__ int badf[2];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int kb = L.kb;
  const int64_t rp = d.rp, o = static_cast<int64_t>(kb) * NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  gptr<const double> A = to_global(dptr(L, d.oA) + o * rp + o);
  double a[NB / 4], z[NB / 4];
#pragma unroll
  for (int q = 0; q < NB / 4; ++q) {
    a[q] = A[(4 * q + wave) * rp + lane];
    z[q] = 4 * q + wave == lane ? 1.0 : 0.0;
  }
  if (threadIdx.x < NB) sd[threadIdx.x] = dptr(L, d.oD)[NB * NB + o + threadIdx.x];
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int q = 0; q < NB / 4; ++q) {
#pragma nounroll
    for (int w = 0; w < 4; ++w) {
      const int k = 4 * q + w, buf = k & 1;
      if (wave == w) {   // this wavefront holds row k
        const double dk = read_lane(a[q], k);
        const bool ok = dk > kPivotTol * sd[k] && dk < INFINITY;
        const double inv = rsqrt_nr(dk), t = dk * inv;
        a[q] = lane > k ? a[q] * inv : (lane == k ? t : 0.0);
        z[q] = lane <= k ? z[q] * inv : 0.0;
        rowA[buf][lane] = a[q];
        rowZ[buf][lane] = z[q];
        if (lane == 0) badf[buf] = ok ? 0 : 1;
      }
      __syncthreads();
      // every read of the broadcast row is issued before the first use
      const int flag = badf[buf];
      const double rj = rowA[buf][lane], zj = rowZ[buf][lane];
      double ai[NB / 4];
#pragma unroll
      for (int qq = q; qq < NB / 4; ++qq) ai[qq] = rowA[buf][4 * qq + wave];
      if (flag) {
        bad = true;
        break;
      }
#pragma unroll
      for (int qq = q; qq < NB / 4; ++qq) {
        if (qq == q && wave <= w) continue;   // rows 4 qq + wave <= k
        if (lane > k) a[qq] -= ai[qq] * rj;
        z[qq] -= ai[qq] * zj;
      }
    }
    if (bad) break;
  }
  if (bad) {
    if (threadIdx.x == 0) atomicOr(&L.status[d.slot], L.flag);
    return;
  }
  // Dinv = T_kk^{-1} = Z^T (upper triangular), Y_kk = Z (lower, zeros above).
  gptr<double> Dinv = to_global(dptr(L, d.oD));
  gptr<double> Y = to_global(dptr(L, d.oY) + o * rp + o);
#pragma unroll
  for (int q = 0; q < NB / 4; ++q) {
    const int i = 4 * q + wave;
    Dinv[lane * NB + i] = lane <= i ? z[q] : 0.0;
    Y[i * rp + lane] = z[q];
  }
}

// out = Dinv^T * in for one 64 x 64 block, in place.
__global__ __launch_bounds__(kThreads) void k_chol_panel(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int kb = L.kb, nblk = d.rp / NB;
  const int64_t rp = d.rp, o = static_cast<int64_t>(kb) * NB;
  const int right = nblk - kb - 1;
  double* blk = local < right ? dptr(L, d.oA) + o * rp + (kb + 1 + local) * NB
                              : dptr(L, d.oY) + o * rp + (local - right) * NB;
  f64x4 acc[2][2];
  block_tn(dptr(L, d.oD), NB, blk, rp, acc);
  __syncthreads();   // every wavefront has read the block before any writes it
  gptr<double> out = to_global(blk);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int v = 0; v < 4; ++v) out[block_off(fm, fn, v, rp)] = acc[fm][fn][v];
}

// Trailing update of the factorization and of the identity block columns,
// for the block-step pair (kb, kb + 1).  Rows kb and kb + 1 of T (and of Y)
// are 128 consecutive rows, so the two panels form one 128-row reduction.
//   mode 1: block row kb + 1 with panel kb: A_(kb+1)j for j > kb and
//           Y_(kb+1)c for c <= kb (first write at c = kb).
//   mode 2: block rows i >= kb + 2 with panels kb and kb + 1: A_ij for
//           j >= i, and Y_ic for c <= kb + 1.  Y_kb,(kb+1) lies above Y's
//           diagonal and is never written, so column block kb + 1 takes the
//           second panel only; Y_i,kb and Y_i,(kb+1) are first writes.
// Four blocks per CU (at most 128 registers per lane): more wavefronts to
// cover the operand loads, which each wavefront issues all at once.
__global__ __launch_bounds__(kThreads, 4) void k_chol_trail(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int kb = L.kb, nblk = d.rp / NB;
  const int64_t rp = d.rp, o = static_cast<int64_t>(kb) * NB;
  double* A = dptr(L, d.oA);
  double* Y = dptr(L, d.oY);
  const double* left;   // T rows of the panel(s), column block bi
  const double* rgt;
  double* out;
  bool assign = false, both = false, second_only = false;
  if (L.mode == 1) {
    const int nl = nblk - kb - 1, bi = kb + 1;
    left = A + o * rp + bi * NB;
    if (local < nl) {
      rgt = A + o * rp + (bi + local) * NB;
      out = A + static_cast<int64_t>(bi) * NB * rp + (bi + local) * NB;
    } else {
      const int c = local - nl;
      rgt = Y + o * rp + c * NB;
      out = Y + static_cast<int64_t>(bi) * NB * rp + c * NB;
      assign = c == kb;
    }
  } else {
    const int nl = nblk - kb - 2;
    const int nsym = nl * (nl + 1) / 2;
    both = true;
    if (local < nsym) {
      int p = local, i = 0;
      while (p >= nl - i) {
        p -= nl - i;
        ++i;
      }
      const int bi = kb + 2 + i, bj = bi + p;
      left = A + o * rp + bi * NB;
      rgt = A + o * rp + bj * NB;
      out = A + static_cast<int64_t>(bi) * NB * rp + bj * NB;
    } else {
      const int t = local - nsym;
      const int bi = kb + 2 + t / (kb + 2), c = t % (kb + 2);
      left = A + o * rp + bi * NB;
      rgt = Y + o * rp + c * NB;
      out = Y + static_cast<int64_t>(bi) * NB * rp + c * NB;
      assign = c >= kb;
      second_only = c == kb + 1;
    }
  }
  f64x4 acc[2][2];
  const int64_t next = static_cast<int64_t>(NB) * rp;   // the second panel's rows
  if (second_only) {
    block_tn(left + next, rp, rgt + next, rp, acc);
  } else {
    block_tn(left, rp, rgt, rp, acc);
    if (both) block_tn_add(left + next, rp, rgt + next, rp, acc);
  }
  gptr<double> q = to_global(out);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t e = block_off(fm, fn, v, rp);
        q[e] = assign ? -acc[fm][fn][v] : q[e] - acc[fm][fn][v];
      }
}

template <class K>
hipError_t go(K kernel, const Launch& L, hipStream_t st) {
  if (L.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(L.total), dim3(kThreads), 0, st, L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chol_init(const Launch& L, hipStream_t st) { return go(k_chol_init, L, st); }
hipError_t launch_chol_diag(const Launch& L, hipStream_t st) { return go(k_chol_diag, L, st); }
hipError_t launch_chol_panel(const Launch& L, hipStream_t st) { return go(k_chol_panel, L, st); }
hipError_t launch_chol_trail(const Launch& L, hipStream_t st) { return go(k_chol_trail, L, st); }

}  // namespace dion
