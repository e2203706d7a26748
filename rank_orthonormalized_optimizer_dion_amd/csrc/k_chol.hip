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
//
// The chain above is the first CholeskyQR pass of every factor.  A factor
// whose pivots show it ill-conditioned takes more (the per-matrix status
// bits of dion_types.h steer this on the device, so the host never waits):
//   k_chol_one  the whole factorization of one matrix in one workgroup:
//               the shifted retry of the first pass, and the second pass
//   k_trmm64    Q T^{-1} with float64 products, rounded once to float32
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launchers.h"
#include "orth_rules.h"

namespace dion {

namespace {

constexpr int NB = kCholNB;

__device__ __forceinline__ double* dptr(const Launch& L, int64_t off) {
  return reinterpret_cast<double*>(L.ws + off);
}

// C += L^T R (NEG: C -= L^T R) for 64 x 64 blocks over 64 reduction rows, C[i][j] +=
// sum_e L[e][i] R[e][j] (L, R row-major with pitches ll, lr), on the
// 16 x 16 x 4 float64 MFMA: 2 x 2 wavefronts of 32 x 32, each lane loading
// its own operands from memory (lane l: row 4 s + l / 16, column l % 16 of
// a 16-wide column strip, 16 consecutive doubles per 16 lanes).  All loads
// of a wavefront are issued before its first MFMA.
template <bool NEG = false>
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
      if constexpr (NEG) a[s][f] = -a[s][f];
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

// Dataflow flags of matrix d (one launch for the whole factorization,
// k_chol_flow): nb x nb words after its trace partials; word (i, j), i <= j:
// block (i, j) of T is final (for i = j: Dinv_i and Y_ii are written);
// word (i, c), c < i: block (i, c) of Y is final.
__device__ __forceinline__ int* flow_flags(const Launch& L, const MatDesc& d) {
  const int nb = d.rp / NB;
  return reinterpret_cast<int*>(dptr(L, d.oD) + NB * NB + d.rp + nb * nb);
}

// A = the Gram matrix (the sum of its reduction slices' partials, upper
// triangle, mirrored), rows past r padded with the identity; diag(S) kept
// aside.  Work item: one of PARTS row bands of one 64 x 64 upper block (a
// quarter when the launch has few blocks, so that it still fills the chip);
// each thread issues the loads of eight slices' partials of its elements
// before adding them (in slice order).
template <int PARTS>
__global__ __launch_bounds__(kThreads) void k_chol_init(Launch L) {
  constexpr int kInitParts = PARTS;
  MatDesc d;
  ClassInfo ci;
  int local;
  // A factorization starts with no control bits (no other kernel of this
  // launch reads them), in the matrices' words and in their union
  // and the dataflow factorization's counters
  if (blockIdx.x == 0 && threadIdx.x < 1 + kFlowWords) L.status[L.any_slot + threadIdx.x] = 0;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  if (local == 0 && threadIdx.x == 0) L.status[d.slot] &= kStatusMask;
  const int quarter = local % kInitParts;
  const int nblk = d.rp / NB;
  int p = local / kInitParts, bi = 0;
  while (p >= nblk - bi) {
    p -= nblk - bi;
    ++bi;
  }
  const int bj = bi + p;
  if (quarter == 0 && threadIdx.x == 0) {   // the blocks' dataflow flags
    int* fl = flow_flags(L, d);
    fl[bi * nblk + bj] = 0;
    fl[bj * nblk + bi] = 0;
  }
  gptr<const double> S = to_global(reinterpret_cast<const double*>(L.ws + d.oS));
  double* A = dptr(L, d.oA);
  double* Sd = dptr(L, d.oD) + NB * NB;
  const int64_t rp = d.rp, plane = rp * rp;
  constexpr int ROWS = NB / kInitParts, PER = ROWS * NB / kThreads;
  static_assert(PER * kThreads == ROWS * NB, "whole elements per thread");
  int gi[PER], gj[PER];
  int64_t e[PER];
  bool in[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int el = threadIdx.x + kThreads * u;
    gi[u] = bi * NB + quarter * ROWS + el / NB;
    gj[u] = bj * NB + el % NB;
    in[u] = gi[u] < d.r && gj[u] < d.r;
    // the Gram kernels write the upper triangle (gi <= gj) only
    e[u] = static_cast<int64_t>(min(gi[u], gj[u])) * rp + max(gi[u], gj[u]);
  }
  double acc[PER] = {};
  constexpr int kSlices = PER >= 16 ? 1 : 32 / PER;   // slices' loads in flight per element
  for (int s0 = 0; s0 < ci.splits; s0 += kSlices) {
    double v[kSlices][PER];
#pragma unroll
    for (int q = 0; q < kSlices; ++q)
#pragma unroll
      for (int u = 0; u < PER; ++u)
        v[q][u] = in[u] && s0 + q < ci.splits ? S[(s0 + q) * plane + e[u]] : 0.0;
#pragma unroll
    for (int q = 0; q < kSlices; ++q)
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] += v[q][u];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const double val = in[u] ? acc[u] : (gi[u] == gj[u] ? 1.0 : 0.0);
    A[gi[u] * rp + gj[u]] = val;
    if (gi[u] == gj[u]) Sd[gi[u]] = val;
  }
}

// Sum of one value per thread over the workgroup, in a fixed order (lanes
// by a butterfly, then the four wavefronts in turn), the same in every
// thread.
__device__ __forceinline__ double block_sum(double v) {
  __shared__ double red[kThreads / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// One 64 x 64 diagonal block: T_kk (upper, positive diagonal) with
// T_kk^T T_kk = A_kk, and Z = T_kk^{-T} from the same row operations on an
// identity block, by one wavefront that holds the whole block.  It factors
// the column-scaled block A' = D A_kk D, D = diag(S)^{-1/2} over the
// block's columns (S the Gram matrix before any update): then T' = T_kk D,
// Z = Z' D, every pivot of A' is the pivot ratio the checks compare, at
// most 1, and the in-place row update below (B + (zt - I) B) keeps float64
// accuracy relative to its result whatever the data's scale.  4 x 4 tiles
// of 16 x 16, the ten upper tiles of A (the only part read) and the ten
// lower tiles of Z, each as a 16 x 16 x 4 float64 MFMA accumulator
// (register v of lane 16 g + c: row 4 v + g, column c of the tile).
// Sixteen steps of four columns; step s (rows and columns 4 s .. 4 s + 3:
// register s % 4 of tile row s / 4):
//   1. the step's 4 x 4 diagonal block t^T t, read from its lanes, is
//      factored in every lane with the same float64 operations (pivot
//      checks included) together with zt = t^{-T};
//   2. the step's rows of A and of Z become zt times themselves, one MFMA
//      per tile that adds (zt - I) times them in place (the rows of T, and
//      of Z, are then final);
//   3. the rows below take the rank-4 update A_IJ -= T_sI^T T_sJ and
//      Z_IJ -= T_sI^T Z_sJ, one MFMA per tile, whose operands are the
//      step's rows as they sit in the registers, the next step's diagonal
//      tile first.  The accumulators are only ever updated whole.
// No barrier and no LDS traffic inside the factorization: about 235 MFMAs
// and the per-step 4 x 4 work on one SIMD.  Every pivot is the Schur
// complement's diagonal, as in the column-by-column factorization.
constexpr int kZPitch = NB + 1;   // LDS row pitch (doubles) of the transposed Z

// f(std::integral_constant<int, i>) for i = B .. E - 1, each with i a
// constant (so that register arrays stay indexed by constants)
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ f64x4 mfma64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
// tile (I, J) of the upper (I <= J) and of the lower (J <= I) triangle
__host__ __device__ constexpr int up_tile(int I, int J) { return I * 4 - I * (I - 1) / 2 + (J - I); }
__host__ __device__ constexpr int lo_tile(int I, int J) { return I * (I + 1) / 2 + J; }

// Factors diagonal block kb of matrix d (Dinv and Y_kk written to the
// workspace).  A pivot fails when it is not above tol times the column's
// original squared norm (or is not finite); returns false then, with
// nothing written.  small: some pivot ratio was below kRatioTwo.  Called
// by the whole workgroup; wavefront 0 factors, all threads store Dinv
// (row-major, row pitch ldd, at dinv).
__device__ __forceinline__ bool diag_block(const Launch& L, const MatDesc& d, int kb, double tol,
                                           bool& small, double* part, double* dinv, int64_t ldd) {
  __shared__ double zs[NB][kZPitch];   // Z transposed, for the Dinv stores
  __shared__ double dsc[NB];           // D = diag(S)^{-1/2} of the block's columns
  __shared__ int res[2];
  const int64_t rp = d.rp, o = static_cast<int64_t>(kb) * NB;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
    gptr<const double> A = to_global(dptr(L, d.oA) + o * rp + o);
    const double sdv = dptr(L, d.oD)[NB * NB + o + lane];   // lane l: diag(S) of column l
    dsc[lane] = rsqrt_nr(sdv);   // read back below by the same wavefront (in-order LDS)
    double dr[4][4], dc[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      dc[I] = dsc[16 * I + c];
#pragma unroll
      for (int v = 0; v < 4; ++v) dr[I][v] = dsc[16 * I + 4 * v + g];
    }
    f64x4 ta[10], tz[10];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (I <= J)
            ta[up_tile(I, J)][v] = A[(16 * I + 4 * v + g) * rp + 16 * J + c] * dr[I][v] * dc[J];
          if (J <= I) tz[lo_tile(I, J)][v] = I == J && 4 * v + g == c ? 1.0 : 0.0;
        }
    bool ok = true, sm = false;
    static_for<0, 16>([&](auto step) {
      constexpr int s = decltype(step)::value, S = s / 4, v = s % 4;
      // 1. the 4 x 4 block (element (k, j) in lane 16 k + 4 v + j) and its
      // factor: f holds t above the diagonal, 1 / t_kk on it
      double f[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = k; j < 4; ++j) f[k][j] = read_lane(ta[up_tile(S, S)][v], 16 * k + 4 * v + j);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double dk = f[k][k];   // the pivot ratio
        ok = ok && dk > tol && dk < INFINITY;
        sm = sm || !(dk >= kRatioTwo);
        const double inv = rsqrt_nr(dk);
        f[k][k] = inv;
#pragma unroll
        for (int j = k + 1; j < 4; ++j) f[k][j] *= inv;
#pragma unroll
        for (int i = k + 1; i < 4; ++i)
#pragma unroll
          for (int j = i; j < 4; ++j) f[i][j] -= f[k][i] * f[k][j];
      }
      // (a failed pivot is acted on after the loop: the factorization runs
      // on through NaNs in registers, so that the loop stays one basic
      // block and the scheduler can interleave the MFMAs with the next
      // step's float64 work)
      // zt = t^{-T} (lower triangular), then lane 16 g + c's operand
      // zt[c][g] (zero outside the first four rows and above the diagonal)
      double z[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i][i] = f[i][i];
#pragma unroll
        for (int j = 0; j < i; ++j) {
          double acc = 0.0;
#pragma unroll
          for (int m = j; m < i; ++m) acc += f[m][i] * z[m][j];
          z[i][j] = -f[i][i] * acc;
        }
      }
      // operand of the in-place row update: zt - I in rows 4 v .. 4 v + 3
      // of the 16 x 4 operand (lane 16 g + c: row c, column g), zero
      // elsewhere, so that one MFMA D = C + (zt - I) B leaves every other
      // row of the tile as it is
      double col[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        double x = z[3][j];
#pragma unroll
        for (int i = 2; i >= j; --i) x = c == 4 * v + i ? z[i][j] : x;
        col[j] = x;
      }
      double op = col[3];
#pragma unroll
      for (int j = 2; j >= 0; --j) op = g == j ? col[j] : op;
      const int ci = c - 4 * v;
      op = ci >= 0 && ci < 4 && g <= ci ? op - (g == ci ? 1.0 : 0.0) : 0.0;
      // 2. the step's rows (their entries left of the diagonal in the
      // diagonal tile are not used below and not cleared)
#pragma unroll
      for (int J = S; J < 4; ++J) ta[up_tile(S, J)] = mfma64(op, ta[up_tile(S, J)][v], ta[up_tile(S, J)]);
#pragma unroll
      for (int J = 0; J <= S; ++J) tz[lo_tile(S, J)] = mfma64(op, tz[lo_tile(S, J)][v], tz[lo_tile(S, J)]);
      if constexpr (s == 15) return;
      // 3. rank-4 update; lane l's operand of T_sI is register v of tile
      // (S, I) in lane l: T[4 s + l / 16][16 I + l % 16], cleared in tile
      // row S for columns up to the step's (so that the step's rows and
      // those above take no update, and the entries left of the diagonal
      // are not read)
      double a[4];
#pragma unroll
      for (int I = S; I < 4; ++I) {
        const double x = -ta[up_tile(S, I)][v];
        a[I] = I == S && c < 4 * v + 4 ? 0.0 : x;
      }
      const int Sn = (s + 1) / 4;
      ta[up_tile(Sn, Sn)] = mfma64(a[Sn], ta[up_tile(S, Sn)][v], ta[up_tile(Sn, Sn)]);
#pragma unroll
      for (int I = S; I < 4; ++I)
#pragma unroll
        for (int J = I; J < 4; ++J)
          if (!(I == Sn && J == Sn))
            ta[up_tile(I, J)] = mfma64(a[I], ta[up_tile(S, J)][v], ta[up_tile(I, J)]);
#pragma unroll
      for (int I = S; I < 4; ++I)
#pragma unroll
        for (int J = 0; J <= S; ++J)
          tz[lo_tile(I, J)] = mfma64(a[I], tz[lo_tile(S, J)][v], tz[lo_tile(I, J)]);
    });
    if (lane == 0) {
      res[0] = ok ? 1 : 0;
      res[1] = sm ? 1 : 0;
    }
    if (ok) {
      // Y_kk = Z (lower, zeros above), Z^T staged in LDS for Dinv, and this
      // block's share of trace(C^{-1}): S_cc Y_jc^2 over its columns c < r
      gptr<double> Y = to_global(dptr(L, d.oY) + o * rp + o);
      double tr = 0.0;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        double q = 0.0;
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 16 * I + 4 * v + g, cl = 16 * J + c;
            const double zv = J <= I ? tz[lo_tile(I, J)][v] * dc[J] : 0.0;
            Y[row * rp + cl] = zv;
            zs[cl][row] = zv;
            q += zv * zv;
          }
        const int cl = 16 * J + c;
        const double sd = __shfl(sdv, cl);
        tr += o + cl < d.r ? sd * q : 0.0;
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) tr += __shfl_xor(tr, m);
      if (part && lane == 0) *part = tr;
    }
  }
  __syncthreads();
  const bool ok = res[0] != 0;
  small = res[1] != 0;
  if (ok) {   // Dinv = T_kk^{-1} = Z^T (upper triangular), row-major
    gptr<double> Dinv = to_global(dinv);
#pragma unroll
    for (int e = threadIdx.x; e < NB * NB; e += kThreads) Dinv[(e / NB) * ldd + e % NB] = zs[e / NB][e % NB];
  }
  __syncthreads();   // the shared buffers are free for the next call
  return ok;
}

// Diagonal block step of the first pass (one workgroup per matrix).
// Partial sums of the trace of C^{-1} (C the column-scaled Gram matrix):
// trace = sum over c <= j of S_cc Y_jc^2 (Y = T^{-T}, c < r), kept per
// 64 x 64 block of Y in the workspace after diag(S), block (jb, c) at
// jb * nblk + c.  Each is written once, by the kernel that leaves that
// block of Y final.
__device__ __forceinline__ double* trace_part(const Launch& L, const MatDesc& d, int jb, int c) {
  return dptr(L, d.oD) + NB * NB + d.rp + static_cast<int64_t>(jb) * (d.rp / NB) + c;
}

__global__ __launch_bounds__(kThreads) void k_chol_diag(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  bool small;
  const bool ok = diag_block(L, d, L.kb, L.retry ? kRatioRetry : kRatioTwo, small,
                             trace_part(L, d, L.kb, L.kb), dptr(L, d.oD), NB);
  if (threadIdx.x == 0) {
    const int32_t bits = !ok ? (L.retry ? (kCtlRetry | kCtlTwo) : L.flag)
                             : (small && L.retry ? kCtlTwo : 0);
    if (bits) {
      atomicOr(&L.status[d.slot], bits);
      if (bits & (kCtlRetry | kCtlTwo)) atomicOr(&L.status[L.any_slot], bits);
    }
  }
}

// ---------------------------------------------------------------------------
// The first-pass factorization in one launch.  Work items are the 64 x 64
// blocks of T (upper triangle, in A's storage) and of Y = T^{-T} (strictly
// lower triangle), one workgroup each, in block-row order over all
// matrices: row i of a matrix is its diagonal block, then the blocks (i, j)
// of T, j > i, then the blocks (i, c) of Y, c < i.  Every block reads only
// blocks of earlier rows and the diagonal block of its own row, and sums
// its whole update before it is written (left-looking):
//   diagonal (i, i):  A_ii - sum_{k<i} T_ki^T T_ki, then diag_block
//                     (Dinv_i stored in place of A_ii, Y_ii, the trace
//                     partial, the pivot decisions);
//   T (i, j):         T_ij = Dinv_i^T (A_ij - sum_{k<i} T_ki^T T_kj);
//   Y (i, c):         Y_ic = -Dinv_i^T sum_{k=c}^{i-1} T_ki^T Y_kc (Y_cc is
//                     the diagonal block c's).
// This is the arithmetic of k_chol_diag / k_chol_panel / k_chol_trail in
// another order of the same sums.  A workgroup takes its item from a
// ticket counter when it starts, so every item it waits on is held by a
// workgroup that started before it: the waits end however many workgroups
// are resident.  A block's flag is set with an agent-scope release after
// its stores; a reader polls it with an agent-scope acquire (the L2 caches
// of the XCDs are not coherent) before it loads the block.  A wait gives up
// after kFlowWait ticks of the 100 MHz wall clock (0.2 s, far beyond any
// factorization here) or kFlowSpin polls, whichever comes first: it flags
// its matrix broken down and sets the abort
// word, after which every wait of the launch returns at once; the launch
// then still ends, its results are not used, and the step reports the
// breakdown.  The last workgroup to finish resets the counters for the
// next launch.
constexpr int64_t kFlowWait = 20000000;   // wall-clock ticks
constexpr int kFlowSpin = 1 << 24;        // polls of at least 64 cycles each

__device__ __forceinline__ void flow_wait(const Launch& L, const MatDesc& d, const int* f) {
  if (threadIdx.x == 0) {
    int32_t* abort_w = L.status + L.any_slot + 3;
    const int64_t t0 = static_cast<int64_t>(wall_clock64());
    for (int n = 0; __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0; ++n) {
      if (n >= kFlowSpin || static_cast<int64_t>(wall_clock64()) - t0 > kFlowWait ||
          __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        __hip_atomic_store(abort_w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomicOr(&L.status[d.slot], L.flag);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void flow_signal(int* f) {
  __syncthreads();   // every wavefront's stores are issued
  if (threadIdx.x == 0) {
    __threadfence();
    __hip_atomic_store(f, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void load_block(const double* p, int64_t ld, f64x4 (&acc)[2][2]) {
  gptr<const double> q = to_global(p);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[fm][fn][v] = q[block_off(fm, fn, v, ld)];
}

__device__ __forceinline__ void store_block(double* p, int64_t ld, const f64x4 (&acc)[2][2],
                                            double sign = 1.0) {
  gptr<double> q = to_global(p);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int v = 0; v < 4; ++v) q[block_off(fm, fn, v, ld)] = sign * acc[fm][fn][v];
}

__global__ __launch_bounds__(kThreads) void k_chol_flow(Launch L) {
  __shared__ int ticket;
  int32_t* words = L.status + L.any_slot;   // [1] ticket, [2] finished items, [3] abort
  if (threadIdx.x == 0) ticket = atomicAdd(&words[1], 1);
  __syncthreads();
  // the item: block row i of its matrix, position pos in that row; each
  // row of a matrix with nb blocks a side has nb items
  int t = ticket, i = 0, pos = 0, mi = -1, nb = 0;
  for (;;) {
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) {
      if (mi >= 0 || c >= L.nclass) continue;
      const int nbc = L.cls[c].tx;
      if (nbc <= i) continue;
      const int seg = L.cls[c].count * nbc;
      if (t < seg) {
        mi = L.cls[c].first + t / nbc;
        nb = nbc;
        pos = t % nbc;
      } else {
        t -= seg;
      }
    }
    if (mi >= 0 || i >= 63) break;
    ++i;
  }
  if (mi >= 0) {
    const MatDesc d = L.table ? L.table[mi] : L.inl;
    const int64_t rp = d.rp;
    double* A = dptr(L, d.oA);
    double* Y = dptr(L, d.oY);
    int* fl = flow_flags(L, d);
    auto blk = [&](double* base, int r, int c) { return base + static_cast<int64_t>(r) * NB * rp + c * NB; };
    f64x4 acc[2][2], out[2][2];
    if (pos < nb - i) {   // block (i, j) of T
      const int j = i + pos;
      load_block(blk(A, i, j), rp, acc);
      for (int k = 0; k < i; ++k) {
        flow_wait(L, d, &fl[k * nb + i]);
        if (j != i) flow_wait(L, d, &fl[k * nb + j]);
        block_tn_add<true>(blk(A, k, i), rp, blk(A, k, j), rp, acc);
      }
      store_block(blk(A, i, j), rp, acc);
      if (j == i) {
        __syncthreads();   // the block is in memory for diag_block
        bool small;
        const bool ok = diag_block(L, d, i, L.retry ? kRatioRetry : kRatioTwo, small,
                                   trace_part(L, d, i, i), blk(A, i, i), rp);
        if (threadIdx.x == 0) {
          const int32_t bits = !ok ? (L.retry ? (kCtlRetry | kCtlTwo) : L.flag)
                                   : (small && L.retry ? kCtlTwo : 0);
          if (bits) {
            atomicOr(&L.status[d.slot], bits);
            if (bits & (kCtlRetry | kCtlTwo)) atomicOr(&L.status[L.any_slot], bits);
          }
        }
      } else {
        flow_wait(L, d, &fl[i * nb + i]);   // (its barrier also orders the stores above)
        block_tn(blk(A, i, i), rp, blk(A, i, j), rp, out);
        __syncthreads();   // every wavefront has read the block before any writes it
        store_block(blk(A, i, j), rp, out);
      }
      flow_signal(&fl[i * nb + j]);
    } else {   // block (i, c) of Y
      const int c = pos - (nb - i);
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) acc[fm][fn] = f64x4{0.0, 0.0, 0.0, 0.0};
      for (int k = c; k < i; ++k) {
        flow_wait(L, d, &fl[k * nb + i]);
        flow_wait(L, d, &fl[k * nb + c]);   // Y_kc (the diagonal block c for k = c)
        block_tn_add(blk(A, k, i), rp, blk(Y, k, c), rp, acc);
      }
      store_block(blk(Y, i, c), rp, acc);
      flow_wait(L, d, &fl[i * nb + i]);
      block_tn(blk(A, i, i), rp, blk(Y, i, c), rp, out);
      __syncthreads();   // every wavefront has read the block before any writes it
      store_block(blk(Y, i, c), rp, out, -1.0);
      // block (i, c) of Y is final: its share of trace(C^{-1})
      const double* sd = dptr(L, d.oD) + NB * NB + c * NB;
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      double tq = 0.0;
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const int col = (wave & 1) * 32 + fn * 16 + (lane & 15);
        double q = 0.0;
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int v = 0; v < 4; ++v) q += out[fm][fn][v] * out[fm][fn][v];
        tq += c * NB + col < d.r ? sd[col] * q : 0.0;
      }
      tq = block_sum(tq);
      if (threadIdx.x == 0) *trace_part(L, d, i, c) = tq;
      flow_signal(&fl[i * nb + c]);
    }
  }
  if (threadIdx.x == 0 && atomicAdd(&words[2], 1) == static_cast<int>(gridDim.x) - 1) {
    words[1] = 0;   // every item has finished: counters for the next launch
    words[2] = 0;
    words[3] = 0;
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
  if (local >= right) {
    // block (kb, c) of Y is final: its share of trace(C^{-1})
    const int c = local - right;
    const double* sd = dptr(L, d.oD) + NB * NB + c * NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double t = 0.0;
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
      const int col = (wave & 1) * 32 + fn * 16 + (lane & 15);
      double q = 0.0;
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int v = 0; v < 4; ++v) q += acc[fm][fn][v] * acc[fm][fn][v];
      t += c * NB + col < d.r ? sd[col] * q : 0.0;
    }
    t = block_sum(t);
    if (threadIdx.x == 0) *trace_part(L, d, kb, c) = t;
  }
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

// Whether orth() of each matrix needs more than its first CholeskyQR pass
// (orth_rules.h), decided once the first pass's factorization is complete
// (one workgroup per matrix, after the chain, for plans whose first pass
// may be followed by more).  The chain left trace(C^{-1}) in per-block
// partial sums; they are added in a fixed order (a strided sum per thread,
// then block_sum), so the decision does not depend on timing.  Sets
// kCtlTwo, or kCtlTwo | kCtlRetry, in the status word; the diagonal steps
// may have set them already (small or failed pivots).
__global__ __launch_bounds__(kThreads) void k_orth_decide(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int nblk = d.rp / NB;
  const double* part = dptr(L, d.oD) + NB * NB + d.rp;
  double t = 0.0;
  for (int e = threadIdx.x; e < nblk * nblk; e += kThreads) {
    const int jb = e / nblk, c = e - jb * nblk;
    if (c <= jb) t += part[e];
  }
  t = block_sum(t);
  if (threadIdx.x == 0) {
    int32_t more = 0;
    if (!(t <= kTraceRetry * d.r)) more = kCtlTwo | kCtlRetry;
    else if (!(t <= kTraceTwo * d.r)) more = kCtlTwo;
    if (more) {
      atomicOr(&L.status[d.slot], more);
      atomicOr(&L.status[L.any_slot], more);
    }
  }
}

// The whole factorization of one matrix in one workgroup (the shifted
// retry of the first pass, gate kGateRetry, and the second pass, gate
// kGateTwo with pass 2): A from the Gram partials (plus s diag(S) for the
// retry), then every block step in turn: the diagonal block, the panel
// row, and the trailing update of A and of Y, with the same arithmetic as
// the chain's kernels.  A failed pivot is a breakdown.  Work items: one per matrix,
// taken in a loop so that a launch with few workgroups covers any list.
__global__ __launch_bounds__(kThreads) void k_chol_one(Launch L) {
  for_items(L, [&](const MatDesc& d, const ClassInfo& ci, int) {
    const int rows = L.which == 0 ? d.m : d.n;
    const int nblk = d.rp / NB;
    const int64_t rp = d.rp, plane = rp * rp;
    const bool shifted = L.gate == kGateRetry;
    const double shift = shifted ? retry_shift(rows, d.r) : 0.0;
    const double* S = reinterpret_cast<const double*>(L.ws + d.oS);
    double* A = dptr(L, d.oA);
    double* Y = dptr(L, d.oY);
    double* Sd = dptr(L, d.oD) + NB * NB;
    for (int bi = 0; bi < nblk; ++bi)
      for (int bj = bi; bj < nblk; ++bj)
        for (int e = threadIdx.x; e < NB * NB; e += kThreads) {
          const int gi = bi * NB + e / NB, gj = bj * NB + e % NB;
          double v;
          if (gi < d.r && gj < d.r) {
            const int64_t x = static_cast<int64_t>(min(gi, gj)) * rp + max(gi, gj);
            v = 0.0;
            for (int sp = 0; sp < ci.splits; ++sp) v += S[sp * plane + x];
          } else {
            v = gi == gj ? 1.0 : 0.0;
          }
          if (gi == gj) {
            Sd[gi] = v;
            if (gi < d.r) v += shift * v;
          }
          A[gi * rp + gj] = v;
        }
    __syncthreads();
    const double tol = shifted ? 0.5 * shift : second_tol(d.r);
    bool failed = false;
    for (int kb = 0; kb < nblk; ++kb) {
      bool small;
      if (!diag_block(L, d, kb, tol, small, nullptr, dptr(L, d.oD), NB)) {
        failed = true;
        break;
      }
      __syncthreads();
      const int64_t o = static_cast<int64_t>(kb) * NB;
      const int right = nblk - kb - 1;
      // panel: T_kj = Dinv^T A_kj (j > kb), Y_kc = Dinv^T Y_kc (c < kb)
      for (int b = 0; b < right + kb; ++b) {
        double* blk = b < right ? A + o * rp + (kb + 1 + b) * NB : Y + o * rp + (b - right) * NB;
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
      __syncthreads();
      // trailing: A_ij -= T_ki^T T_kj (kb < i <= j); Y_ic -= T_ki^T Y_kc
      // (c <= kb, a first write at c = kb)
      for (int i = kb + 1; i < nblk; ++i) {
        const double* left = A + o * rp + i * NB;
        for (int j = 0; j < nblk - i + kb + 1; ++j) {
          const bool on_a = j < nblk - i;
          const int c = j - (nblk - i);
          const double* rgt = on_a ? A + o * rp + (i + j) * NB : Y + o * rp + c * NB;
          double* outp = on_a ? A + static_cast<int64_t>(i) * NB * rp + (i + j) * NB
                              : Y + static_cast<int64_t>(i) * NB * rp + c * NB;
          const bool assign = !on_a && c == kb;
          f64x4 acc[2][2];
          block_tn(left, rp, rgt, rp, acc);
          gptr<double> q = to_global(outp);
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
      }
      __syncthreads();
    }
    if (failed && threadIdx.x == 0) atomicOr(&L.status[d.slot], L.flag);
    __syncthreads();   // the next work item reuses the shared buffers
  });
}

// Q1 = Q T^{-1} with float64 products and sums, rounded once to float32:
// both triangular multiplies of a two-pass orth (gate kGateTwo).  T^{-1} is
// upper triangular with a positive diagonal, so Q1 has exactly the Q factor
// of Q; computed this way Q1 differs from the exact product only by one
// float32 rounding per entry, and the Q factor the second pass extracts is
// accurate to about that rounding times Q1's (small) condition number,
// however ill-conditioned Q was.  64 x 64 output tiles, 2 x 2 wavefronts of 32 x 32
// on the 16 x 16 x 4 float64 MFMA; each lane loads its own operands
// (lane l: row l % 16 of the A fragment and column l % 16 of the B
// fragment at reduction step l / 16), bounds-checked.  T^{-1}[k][j] =
// Y[j][k] for k <= j (Y = T^{-T} lower triangular; its upper part is not
// read).  Work items as for_items hands them out.
__global__ __launch_bounds__(kThreads) void k_trmm64(Launch L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  for_items(L, [&](const MatDesc& d, const ClassInfo& ci, int local) {
    const int rows = L.which == 0 ? d.m : d.n;
    const int tm = local / ci.ty, tn = local - (local / ci.ty) * ci.ty;
    gptr<const float> Q = to_global(orth_src(L, d));
    gptr<float> dst = to_global(orth_dst(L, d));
    gptr<const double> Yp = to_global(static_cast<const double*>(dptr(L, d.oY)));
    const int r = d.r;
    const int64_t rp = d.rp;
    const int row0 = tm * NB + (wave >> 1) * 32, col0 = tn * NB + (wave & 1) * 32;
    f64x4 acc[2][2];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) acc[fm][fn] = f64x4{0.0, 0.0, 0.0, 0.0};
    const int kend = min(r, (tn + 1) * NB);
    for (int k0 = 0; k0 < kend; k0 += 4) {
      const int k = k0 + g;
      double a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int row = row0 + 16 * f + c16, col = col0 + 16 * f + c16;
        a[f] = row < rows && k < r ? static_cast<double>(Q[static_cast<int64_t>(row) * r + k]) : 0.0;
        b[f] = col < r && k <= col ? Yp[col * rp + k] : 0.0;
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = row0 + 16 * fm + g + 4 * v, col = col0 + 16 * fn + c16;
          if (row < rows && col < r) dst[static_cast<int64_t>(row) * r + col] = static_cast<float>(acc[fm][fn][v]);
        }
  });
}

template <class K>
hipError_t go(K kernel, const Launch& L, hipStream_t st) {
  if (L.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(L.total), dim3(kThreads), 0, st, L);
  return hipGetLastError();
}

// Kernels that take their work items in a loop: at most kGatedGrid
// workgroups, so that a launch in which every matrix is skipped costs little.
template <class K>
hipError_t go_capped(K kernel, const Launch& L, hipStream_t st) {
  if (L.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(gated_grid(L.total)), dim3(kThreads), 0, st, L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chol_init(const Launch& L, int parts, hipStream_t st) {
  return parts == kCholInitParts ? go(k_chol_init<kCholInitParts>, L, st) : go(k_chol_init<1>, L, st);
}
hipError_t launch_chol_diag(const Launch& L, hipStream_t st) { return go(k_chol_diag, L, st); }
hipError_t launch_chol_panel(const Launch& L, hipStream_t st) { return go(k_chol_panel, L, st); }
hipError_t launch_chol_trail(const Launch& L, hipStream_t st) { return go(k_chol_trail, L, st); }
hipError_t launch_chol_flow(const Launch& L, hipStream_t st) { return go(k_chol_flow, L, st); }
hipError_t launch_chol_one(const Launch& L, hipStream_t st) { return go_capped(k_chol_one, L, st); }
hipError_t launch_orth_decide(const Launch& L, hipStream_t st) { return go(k_orth_decide, L, st); }
hipError_t launch_trmm64(const Launch& L, hipStream_t st) { return go_capped(k_trmm64, L, st); }

}  // namespace dion
