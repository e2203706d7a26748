// The whole step of one small matrix in one workgroup (Orth-Dion page,
// equation block; Dion's rule from its closing remark): for matrices whose
// step is far too small to fill the GPU, one launch does what the grouped
// schedule spreads over about 60 dependent launches, each of which would
// idle almost every compute unit.
//
//   P = (G + R) V          float32 FMAs, columns of M staged through LDS
//   U = orth(P)            float64 Gram matrix, Cholesky with T^{-1} on one
//                          wavefront, U = fl32(P T^{-1}) from float64
//                          products; a second pass or the shifted retry by
//                          the rules of orth_rules.h
//   W = (G + R)^T U        float32 FMAs
//   Vbar = orth(W) | colnorm(W)
//   X -= eta U Vbar^T, R = beta (G + R - U W^T), V <- Vbar
//
// The factors stay in LDS with their columns padded to RB (8 or 16 >= r)
// and zeros in the padding: (m + n + n32) RB float32 values, n32 = n rounded
// up to 32 (the host admits only shapes that fit).  P, U and W are also
// written to the workspace (oP, oB, oW, pitch r), where dion_plan_buffer
// finds them.  The status word is written once, at the end: the breakdown
// flag of the factorization that failed (X, R and V are then left as they
// were), and the control bits of the last factorization.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "dion.h"
#include "launchers.h"
#include "orth_rules.h"

namespace dion {

namespace {

constexpr int kSmallRank = kSmallMaxRank;      // largest r
constexpr int kSmallFloats = kSmallFactorFloats;
constexpr int kChunk = 16;                     // columns of M per staged chunk of M V

// LDS of orth() and of Dion's column norms (r <= kSmallRank).
struct OrthLds {
  double s[kSmallRank][kSmallRank + 1];          // Gram matrix (both triangles)
  double tinv[kSmallRank][kSmallRank + 1];       // T^{-1} (upper triangle)
  float inv[kSmallRank];                         // Dion: inverse column norms
  double trace;
  int bad, small;
};

// Streaming form: M read from global memory in each of its three passes.
struct alignas(16) SmallLds {
  float f[kSmallFloats];                         // P / U, W, V then Vbar
  float ms[kThreads][kChunk + 1];                // chunk of M (M V), partial sums (M^T U)
  OrthLds o;
};

// Resident form: M = G + R read once into LDS (row pitch n + 1), after the
// factors U (m x RB) and V, then W, then Vbar (n32 x RB).
constexpr int kResFloats = kSmallResidentFloats;
struct alignas(16) ResLds {
  float f[kResFloats];
  OrthLds o;
};
static_assert(sizeof(ResLds) <= 160 * 1024, "one workgroup's LDS");

template <typename GT>
__device__ __forceinline__ float widen(GT g) {
  if constexpr (sizeof(GT) == 2) return bf16_to_f32(g);
  else return g;
}

// P = M V for rows [rs, rs + kThreads) at a time: thread t owns row rs + t;
// M is staged kChunk columns at a time (each 32-lane half loads 128
// consecutive bytes of one row), the next chunk's loads in flight while the
// current one is used.  V (Vs, n32 x RB, zero padded) is read by broadcast.
template <typename GT, int RB>
__device__ __forceinline__ void small_mv(const MatDesc& d, SmallLds& sh, float* Qs, const float* Vs, float* Pw) {
  const int t = threadIdx.x, m = d.m, n = d.n, r = d.r;
  gptr<const GT> G = to_global(static_cast<const GT*>(d.G));
  gptr<const float> R = to_global(static_cast<const float*>(d.R));
  const int nch = (n + kChunk - 1) / kChunk;
  static_assert(kThreads % kChunk == 0, "whole rows per load round");
  constexpr int RSTEP = kThreads / kChunk;       // rows covered by one load round
  constexpr int NQ = kThreads / RSTEP;           // load rounds per chunk of kThreads rows
  for (int rs = 0; rs < m; rs += kThreads) {
    float acc[RB];
#pragma unroll
    for (int c = 0; c < RB; ++c) acc[c] = 0.0f;
    GT gv[NQ];
    float rv[NQ];
    auto fetch = [&](int j0) {
      const int col = j0 + (t % kChunk);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int row = rs + q * RSTEP + t / kChunk;
        if (row < m && col < n) {
          const int64_t o = static_cast<int64_t>(row) * n + col;
          gv[q] = G[o];
          rv[q] = R[o];
        } else {
          gv[q] = GT(0);
          rv[q] = 0.0f;
        }
      }
    };
    fetch(0);
    for (int ch = 0; ch < nch; ++ch) {
      __syncthreads();   // every thread is done with the previous chunk
#pragma unroll
      for (int q = 0; q < NQ; ++q) sh.ms[q * RSTEP + t / kChunk][t % kChunk] = widen(gv[q]) + rv[q];
      __syncthreads();
      if (ch + 1 < nch) fetch((ch + 1) * kChunk);
      const float* vrow = Vs + ch * kChunk * RB;
#pragma unroll 4
      for (int jj = 0; jj < kChunk; ++jj) {
        const float mv = sh.ms[t][jj];
        const f32x4* v4 = reinterpret_cast<const f32x4*>(vrow + jj * RB);
#pragma unroll
        for (int c4 = 0; c4 < RB / 4; ++c4) {
          const f32x4 v = v4[c4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * c4 + e] = fmaf(mv, v[e], acc[4 * c4 + e]);
        }
      }
    }
    const int i = rs + t;
    if (i < m) {
#pragma unroll
      for (int c = 0; c < RB; ++c) Qs[i * RB + c] = acc[c];
      gptr<float> pw = to_global(Pw);
#pragma unroll
      for (int c = 0; c < RB; ++c)
        if (c < r) pw[static_cast<int64_t>(i) * r + c] = acc[c];
    }
  }
  __syncthreads();
}

// Thread layout of the passes over M by columns (M^T U and the update):
// tc = min(n, kThreads) threads per row, rpar = kThreads / tc row groups;
// thread t takes column cs + t % tc of every rpar-th row starting at t / tc.
struct ColMap {
  int tc, rpar, g, jj;
  bool act;
  __device__ explicit ColMap(int n) {
    tc = n < kThreads ? n : kThreads;
    rpar = kThreads / tc;
    g = threadIdx.x / tc;
    jj = threadIdx.x % tc;
    act = g < rpar;
  }
};

// W = M^T U: each thread sums its rows in order, 8 rows' loads at a time;
// the row groups' partial sums are added in group order.
template <typename GT, int RB>
__device__ __forceinline__ void small_mtu(const MatDesc& d, SmallLds& sh, const float* Us, float* Ws, float* Ww) {
  const int m = d.m, n = d.n, r = d.r;
  gptr<const GT> G = to_global(static_cast<const GT*>(d.G));
  gptr<const float> R = to_global(static_cast<const float*>(d.R));
  const ColMap cm(n);
  float* part = &sh.ms[0][0];   // rpar x tc x RB partial sums (<= kThreads RB floats)
  for (int cs = 0; cs < n; cs += cm.tc) {
    const int j = cs + cm.jj;
    const bool on = cm.act && j < n;
    float acc[RB];
#pragma unroll
    for (int c = 0; c < RB; ++c) acc[c] = 0.0f;
    if (on) {
      constexpr int U8 = 8;
      int i = cm.g;
      for (; i + (U8 - 1) * cm.rpar < m; i += U8 * cm.rpar) {
        GT gv[U8];
        float rv[U8];
#pragma unroll
        for (int u = 0; u < U8; ++u) {
          const int64_t o = static_cast<int64_t>(i + u * cm.rpar) * n + j;
          gv[u] = G[o];
          rv[u] = R[o];
        }
#pragma unroll
        for (int u = 0; u < U8; ++u) {
          const float mv = widen(gv[u]) + rv[u];
          const f32x4* u4 = reinterpret_cast<const f32x4*>(Us + (i + u * cm.rpar) * RB);
#pragma unroll
          for (int c4 = 0; c4 < RB / 4; ++c4) {
            const f32x4 uv = u4[c4];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * c4 + e] = fmaf(mv, uv[e], acc[4 * c4 + e]);
          }
        }
      }
      for (; i < m; i += cm.rpar) {
        const int64_t o = static_cast<int64_t>(i) * n + j;
        const float mv = widen(G[o]) + R[o];
        const f32x4* u4 = reinterpret_cast<const f32x4*>(Us + i * RB);
#pragma unroll
        for (int c4 = 0; c4 < RB / 4; ++c4) {
          const f32x4 uv = u4[c4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * c4 + e] = fmaf(mv, uv[e], acc[4 * c4 + e]);
        }
      }
    }
    if (cm.rpar > 1) {   // one column set (n < kThreads): add the row groups in order
      if (on)
#pragma unroll
        for (int c = 0; c < RB; ++c) part[(cm.g * cm.tc + cm.jj) * RB + c] = acc[c];
      __syncthreads();
      if (on && cm.g == 0)
#pragma unroll
        for (int c = 0; c < RB; ++c) {
          float s = part[cm.jj * RB + c];
          for (int gg = 1; gg < cm.rpar; ++gg) s += part[(gg * cm.tc + cm.jj) * RB + c];
          acc[c] = s;
        }
    }
    if (on && cm.g == 0) {
#pragma unroll
      for (int c = 0; c < RB; ++c) Ws[j * RB + c] = acc[c];
      gptr<float> ww = to_global(Ww);
#pragma unroll
      for (int c = 0; c < RB; ++c)
        if (c < r) ww[static_cast<int64_t>(j) * r + c] = acc[c];
    }
  }
  __syncthreads();
}

// S = Q^T Q in float64 (products of float32 values are exact), 16 x 16
// with both triangles (rows and columns past r are zero), on wavefront 0
// with the float64 16 x 16 x 4 MFMA: lane l supplies Q[i0 + l / 16][l % 16]
// as both operands, and S[l / 16 + 4 v][l % 16] comes out in register v.
// Four row groups' loads are issued before their MFMAs.
template <int RB, int QP>
__device__ __forceinline__ void small_gram(OrthLds& sh, const float* Q, int rows, int r) {
  static_assert(RB <= 16, "one 16 x 16 block");
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, kr = lane >> 4, c = lane & 15;
    // four accumulators (row groups 4 u .. 4 u + 3 of every 16 rows), added
    // in a fixed order at the end
    f64x4 acc[4] = {};
    int i0 = 0;
    for (; i0 + 16 <= rows; i0 += 16) {
      double a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = c < RB ? static_cast<double>(Q[(i0 + 4 * u + kr) * QP + c]) : 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[u], a[u], acc[u], 0, 0, 0);
    }
    for (int u = 0; i0 < rows; i0 += 4, ++u) {
      const int i = i0 + kr;
      const double a = i < rows && c < RB ? static_cast<double>(Q[i * QP + c]) : 0.0;
      acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, a, acc[u], 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) sh.s[kr + 4 * v][c] = (acc[0][v] + acc[1][v]) + (acc[2][v] + acc[3][v]);
  }
  __syncthreads();
}

// f(std::integral_constant<int, i>) for i = B .. E - 1, each with i a
// constant (so that register values stay indexed by constants)
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

// T^{-1} (into tinv), the trace of C^{-1} (C the column-scaled Gram matrix)
// and the pivot decisions for A = S + shift diag(S) (rows and columns past
// r: the identity), on wavefront 0.  A pivot fails (bad) when its ratio
// d_k / S_kk is not above tol or is not finite; small: some ratio is below
// kRatioTwo.  A is scaled to A' = D A D, D = diag(S)^{-1/2}, so that its
// pivots are those ratios; A' and Z' = T'^{-T} (T' = T D, Z = Z' D) are
// one 16 x 16 float64 MFMA accumulator each (register v of lane 16 g + c:
// row 4 v + g, column c), factored in steps of four columns: the step's
// 4 x 4 block, read from its lanes, is factored alike in every lane
// together with zt = t^{-T}; one MFMA adds (zt - I) times the step's rows
// to them in place (rows of T' and of Z' final); one more per tile makes
// the rank-4 update of the rows below (the operand cleared up to the
// step's columns, so that those rows take none).
template <int RB>
__device__ __forceinline__ void small_chol(OrthLds& sh, int r, double shift, double tol) {
  __syncthreads();   // every thread has read the previous factorization's results
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
    const double sc = c < r ? rsqrt_nr(sh.s[c][c]) : 1.0;   // D of the lane's column
    f64x4 ta, tz;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 4 * v + g;
      double a = row == c ? 1.0 : 0.0;
      if (row < r && c < r) {
        const double sr = rsqrt_nr(sh.s[row][row]);
        a = (sh.s[row][c] + (row == c ? shift * sh.s[row][row] : 0.0)) * sr * sc;
      }
      ta[v] = a;
      tz[v] = row == c ? 1.0 : 0.0;
    }
    bool ok = true, sm = false;
    static_for<0, RB / 4>([&](auto step) {
      constexpr int v = decltype(step)::value;
      double f[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = k; j < 4; ++j) f[k][j] = read_lane(ta[v], 16 * k + 4 * v + j);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double dk = f[k][k];   // the pivot ratio
        if (4 * v + k < r) {
          ok = ok && dk > tol && dk < INFINITY;
          sm = sm || !(dk >= kRatioTwo);
        }
        const double inv = rsqrt_nr(dk);
        f[k][k] = inv;
#pragma unroll
        for (int j = k + 1; j < 4; ++j) f[k][j] *= inv;
#pragma unroll
        for (int i = k + 1; i < 4; ++i)
#pragma unroll
          for (int j = i; j < 4; ++j) f[i][j] -= f[k][i] * f[k][j];
      }
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
      // lane 16 g + c's operand: zt[c - 4 v][g] - [c - 4 v == g] in rows
      // 4 v .. 4 v + 3 of the 16 x 4 operand, zero elsewhere
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
      ta = mfma64(op, ta[v], ta);
      tz = mfma64(op, tz[v], tz);
      if constexpr (v + 1 < RB / 4) {
        const double a = c < 4 * v + 4 ? 0.0 : -ta[v];
        ta = mfma64(a, ta[v], ta);
        tz = mfma64(a, tz[v], tz);
      }
    });
    // T^{-1} = Z^T = (Z' D)^T, and sum over columns c < r of S_cc |Z e_c|^2
    double q = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const double zv = tz[v] * sc;
      sh.tinv[c][4 * v + g] = zv;
      q += zv * zv;
    }
    double tr = c < r ? sh.s[c][c] * q : 0.0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tr += __shfl_xor(tr, o);
    if (lane == 0) {
      sh.bad = ok ? 0 : 1;
      sh.small = sm ? 1 : 0;
      sh.trace = tr;
    }
  }
  __syncthreads();
}

// Out = fl32(Q T^{-1}) with float64 products and sums, 16 rows per float64
// 16 x 16 x 4 MFMA block, blocks dealt to the wavefronts in turn: C[i][j] =
// sum_k A[k][i] B[k][j] with A[k][i] = Q[i0 + i][k] and B = T^{-1} (from
// tinv; identity past r, where Q's columns are zero, so padded columns of
// Out come out zero).  A wavefront reads its block before writing it, so
// Out may be Q.
template <int NT, int RB, int QP>
__device__ __forceinline__ void small_trmm(OrthLds& sh, const float* Q, float* Out, int rows, int r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, kr = lane >> 4, c = lane & 15;
  double b[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const int k = 4 * s4 + kr;
    b[s4] = k < RB && c < RB ? sh.tinv[k][c] : 0.0;
  }
  for (int i0 = 16 * wave; i0 < rows; i0 += 16 * (NT / 64)) {
    double a[4];
    const int ia = i0 + c;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int k = 4 * s4 + kr;
      a[s4] = ia < rows && k < RB ? static_cast<double>(Q[ia * QP + k]) : 0.0;
    }
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s4], b[s4], acc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + kr + 4 * v;
      if (i < rows && c < RB) Out[i * QP + c] = static_cast<float>(acc[v]);
    }
  }
  __syncthreads();
}

// orth(Q) into Out (Out may be Q) with the passes orth_rules.h chooses;
// ctl gets the control bits of this factorization.  False on a breakdown.
template <int NT, int RB, int QP>
__device__ __forceinline__ bool small_orth(OrthLds& sh, const float* Q, float* Out, int rows, int r, int& ctl) {
  small_gram<RB, QP>(sh, Q, rows, r);
  small_chol<RB>(sh, r, 0.0, kRatioRetry);
  ctl = 0;
  if (sh.bad || !(sh.trace <= kTraceRetry * r)) ctl = kCtlTwo | kCtlRetry;
  else if (sh.small || !(sh.trace <= kTraceTwo * r)) ctl = kCtlTwo;
  if (ctl & kCtlRetry) {   // the first pass again, on S + s diag(S)
    const double s = retry_shift(rows, r);
    small_chol<RB>(sh, r, s, 0.5 * s);
    if (sh.bad) return false;
  }
  small_trmm<NT, RB, QP>(sh, Q, Out, rows, r);
  if (ctl & kCtlTwo) {     // the second pass, on the first pass's result
    small_gram<RB, QP>(sh, Out, rows, r);
    small_chol<RB>(sh, r, 0.0, second_tol(r));
    if (sh.bad) return false;
    small_trmm<NT, RB, QP>(sh, Out, Out, rows, r);
  }
  return true;
}

// Dion: Vbar = W diag(1 / |W_:c|), column sums of squares in float64 over
// 16 row groups added in order; a zero or non-finite norm is a breakdown.
// Vb may be Ws.
template <int NT, int RB, int QP>
__device__ __forceinline__ bool small_colnorm(OrthLds& sh, const float* Ws, float* Vb, int n, int r) {
  const int t = threadIdx.x, c = t % kSmallRank, g = t / kSmallRank;
  constexpr int NG = kSmallRank;   // row groups: the Gram area holds their sums
  static_assert(NT >= NG * kSmallRank, "a thread per group and column");
  if (t < NG * kSmallRank) {
    double s = 0.0;
    if (c < r)
      for (int i = g; i < n; i += NG) {
        const double w = Ws[i * QP + c];
        s = fma(w, w, s);
      }
    sh.s[g][c] = s;
  }
  if (t == 0) sh.bad = 0;
  __syncthreads();
  if (t < r) {
    double tot = sh.s[0][t];
    for (int gg = 1; gg < NG; ++gg) tot += sh.s[gg][t];
    if (!(tot > 0.0) || !(tot < INFINITY)) sh.bad = 1;
    else sh.inv[t] = static_cast<float>(1.0 / sqrt(tot));
  }
  __syncthreads();
  if (sh.bad) return false;
  for (int e = t; e < n * QP; e += NT) {
    const int cc = e % QP;
    Vb[e] = cc < r ? Ws[e] * sh.inv[cc] : 0.0f;
  }
  __syncthreads();
  return true;
}

// X -= eta U Vbar^T, R = beta ((G + R) - U W^T): each thread keeps its
// column's rows of Vbar and W in registers and takes 4 rows' loads at a time.
template <typename GT, int RB>
__device__ __forceinline__ void small_update(const Launch& L, const MatDesc& d, const float* Us, const float* Ws,
                             const float* Vb) {
  const int m = d.m, n = d.n;
  gptr<const GT> G = to_global(static_cast<const GT*>(d.G));
  gptr<float> X = to_global(d.X);
  gptr<float> R = to_global(d.R);
  const float eta = L.eta, beta = L.beta;
  const ColMap cm(n);
  if (!cm.act) return;
  for (int cs = 0; cs < n; cs += cm.tc) {
    const int j = cs + cm.jj;
    if (j >= n) continue;
    float vb[RB], w[RB];
#pragma unroll
    for (int c = 0; c < RB; ++c) {
      vb[c] = Vb[j * RB + c];
      w[c] = Ws[j * RB + c];
    }
    auto row = [&](int i, GT g, float rv, float xv, int64_t o) {
      const f32x4* u4 = reinterpret_cast<const f32x4*>(Us + i * RB);
      float dx = 0.0f, dr = 0.0f;
#pragma unroll
      for (int c4 = 0; c4 < RB / 4; ++c4) {
        const f32x4 u = u4[c4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dx = fmaf(u[e], vb[4 * c4 + e], dx);
          dr = fmaf(u[e], w[4 * c4 + e], dr);
        }
      }
      X[o] = xv - eta * dx;
      R[o] = beta * ((widen(g) + rv) - dr);
    };
    constexpr int U4 = 4;
    int i = cm.g;
    for (; i + (U4 - 1) * cm.rpar < m; i += U4 * cm.rpar) {
      GT gv[U4];
      float rv[U4], xv[U4];
      int64_t o[U4];
#pragma unroll
      for (int u = 0; u < U4; ++u) {
        o[u] = static_cast<int64_t>(i + u * cm.rpar) * n + j;
        gv[u] = G[o[u]];
        rv[u] = R[o[u]];
        xv[u] = X[o[u]];
      }
#pragma unroll
      for (int u = 0; u < U4; ++u) row(i + u * cm.rpar, gv[u], rv[u], xv[u], o[u]);
    }
    for (; i < m; i += cm.rpar) {
      const int64_t o = static_cast<int64_t>(i) * n + j;
      row(i, G[o], R[o], X[o], o);
    }
  }
}

// V (n x r, global) into Vb (n32 x RB, zero padded).
template <int NT, int QP>
__device__ __forceinline__ void load_v(const MatDesc& d, float* Vb) {
  const int n = d.n, r = d.r, n32 = (n + 31) / 32 * 32;
  gptr<const float> V0 = to_global(static_cast<const float*>(d.V));
  for (int e = threadIdx.x; e < n32 * QP; e += NT) {
    const int j = e / QP, c = e % QP;
    Vb[e] = j < n && c < r ? V0[static_cast<int64_t>(j) * r + c] : 0.0f;
  }
}

// A factor from LDS (rows x QP) into the workspace (rows x r).
template <int NT, int QP>
__device__ __forceinline__ void store_factor(const float* F, float* out_, int rows, int r) {
  gptr<float> out = to_global(out_);
  for (int e = threadIdx.x; e < rows * r; e += NT) out[e] = F[(e / r) * QP + e % r];
}

// Streaming form.  L.mode: the rule (1 Orth-Dion, 0 Dion).  One workgroup
// per matrix.
template <typename GT, int RB>
__global__ __launch_bounds__(kThreads) void k_small(Launch L) {
  __shared__ SmallLds sh;
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, blockIdx.x, d, ci, local);
  const int t = threadIdx.x, m = d.m, n = d.n, r = d.r;
  float* Us = sh.f;            // P, then U (m x RB)
  float* Ws = Us + m * RB;     // W (n x RB)
  float* Vb = Ws + n * RB;     // V (n32 x RB, zero padded), then Vbar
  load_v<kThreads, RB>(d, Vb);
  __syncthreads();
  small_mv<GT, RB>(d, sh, Us, Vb, reinterpret_cast<float*>(L.ws + d.oP));
  int ctl = 0, flags = 0;
  if (!small_orth<kThreads, RB, RB>(sh.o, Us, Us, m, r, ctl)) {
    flags = DION_STATUS_ORTH_P;
  } else {
    store_factor<kThreads, RB>(Us, reinterpret_cast<float*>(L.ws + d.oB), m, r);
    small_mtu<GT, RB>(d, sh, Us, Ws, reinterpret_cast<float*>(L.ws + d.oW));
    bool ok;
    if (L.mode == 1) {
      ok = small_orth<kThreads, RB, RB>(sh.o, Ws, Vb, n, r, ctl);
      if (!ok) flags = DION_STATUS_ORTH_W;
    } else {
      ok = small_colnorm<kThreads, RB, RB>(sh.o, Ws, Vb, n, r);
      if (!ok) flags = DION_STATUS_COLNORM;
    }
    if (ok) {
      small_update<GT, RB>(L, d, Us, Ws, Vb);
      store_factor<kThreads, RB>(Vb, d.V, n, r);
    }
  }
  if (t == 0) L.status[d.slot] = flags | ctl;
}

// ---------------------------------------------------------------------------
// Resident form: M = G + R is read from global memory once, into LDS, by a
// workgroup of kResThreads (two wavefronts per SIMD, so that one's LDS and
// memory waits overlap the other's arithmetic).
constexpr int kResThreads = 512;

__device__ __forceinline__ bool aligned_to(const void* p, int bytes) {
  return (reinterpret_cast<uintptr_t>(p) & static_cast<uintptr_t>(bytes - 1)) == 0;
}

// Four consecutive elements of G as float32 (one 16-byte or 8-byte load).
__device__ __forceinline__ f32x4 load4(gptr<const float> G, int64_t e) {
  return *reinterpret_cast<gptr<const f32x4>>(G + e);
}
__device__ __forceinline__ f32x4 load4(gptr<const uint16_t> G, int64_t e) {
  const u32x2 w = *reinterpret_cast<gptr<const u32x2>>(G + e);
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}

// Whether the rows of X, G and R can be read and written in aligned groups
// of four elements.
template <typename GT>
__device__ __forceinline__ bool quads_ok(const MatDesc& d) {
  return d.n % 4 == 0 && aligned_to(d.G, 4 * sizeof(GT)) && aligned_to(d.R, 16) &&
         aligned_to(d.X, 16);
}

// M into Ms (row pitch n + 1, so that a column of M read by consecutive
// rows' threads falls in distinct banks).  Each thread has up to kBatch
// loads of four elements (or of one, when rows are not in aligned groups of
// four) in flight before it stores any.
template <typename GT>
__device__ __forceinline__ void res_load_m(const MatDesc& d, float* Ms) {
  constexpr int NT = kResThreads, kBatch = 16;
  const int m = d.m, n = d.n, pitch = n + 1, t = threadIdx.x;
  gptr<const GT> G = to_global(static_cast<const GT*>(d.G));
  gptr<const float> R = to_global(static_cast<const float*>(d.R));
  if (quads_ok<GT>(d)) {
    const int nq = m * n / 4;   // groups of four never cross a row (n % 4 == 0)
    for (int q0 = 0; q0 < nq; q0 += NT * kBatch) {
      f32x4 gv[kBatch], rv[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int q = q0 + b * NT + t;
        if (q < nq) {
          gv[b] = load4(G, 4 * static_cast<int64_t>(q));
          rv[b] = *reinterpret_cast<gptr<const f32x4>>(R + 4 * static_cast<int64_t>(q));
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int q = q0 + b * NT + t;
        if (q < nq) {
          const int e = 4 * q, i = e / n, j = e - i * n;
#pragma unroll
          for (int k = 0; k < 4; ++k) Ms[i * pitch + j + k] = gv[b][k] + rv[b][k];
        }
      }
    }
    return;
  }
  const int mn = m * n;
  for (int e0 = 0; e0 < mn; e0 += NT * kBatch) {
    GT gv[kBatch];
    float rv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * NT + t;
      if (e < mn) {
        gv[b] = G[e];
        rv[b] = R[e];
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * NT + t;
      if (e < mn) {
        const int i = e / n, j = e - i * n;
        Ms[i * pitch + j] = widen(gv[b]) + rv[b];
      }
    }
  }
}

// The resident form's products on the float32 16 x 16 x 4 MFMA: D = A B
// with lane l supplying A[l % 16][l / 16] and B[l / 16][l % 16], and
// holding D[4 (l / 16) + v][l % 16] in register v.  Each wavefront takes
// whole 16 x 16 output blocks in turn; out-of-range rows, columns and
// reduction indices contribute zeros.
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// P = M V (m x RB): blocks of 16 rows; the reduction over M's columns in
// steps of 4, kK steps' reads issued before their MFMAs, alternating
// between two accumulators.
template <int RB>
__device__ __forceinline__ void res_mv(const MatDesc& d, const float* Ms, const float* Vb,
                                       float* Us, float* Pw_) {
  constexpr int NW = kResThreads / 64, kK = 8;
  const int m = d.m, n = d.n, r = d.r, pitch = n + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lk = lane >> 4;
  gptr<float> Pw = to_global(Pw_);
  for (int blk = wave; blk * 16 < m; blk += NW) {
    const int i0 = blk * 16, ia = i0 + li;
    f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    for (int j0 = 0; j0 < n; j0 += 4 * kK) {
      float a[kK], b[kK];
#pragma unroll
      for (int u = 0; u < kK; ++u) {
        const int j = j0 + 4 * u + lk;
        a[u] = ia < m && j < n ? Ms[ia * pitch + j] : 0.0f;
        b[u] = li < RB && j < n ? Vb[j * (RB + 1) + li] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kK; ++u) acc[u & 1] = mfma16(a[u], b[u], acc[u & 1]);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + 4 * lk + v;
      if (i < m && li < RB) {
        const float p = acc[0][v] + acc[1][v];
        Us[i * (RB + 1) + li] = p;
        if (li < r) Pw[static_cast<int64_t>(i) * r + li] = p;
      }
    }
  }
  __syncthreads();
}

// W = M^T U (n x RB) into Wb (V's place): blocks of 16 columns of M; the
// reduction over M's rows as in res_mv.
template <int RB>
__device__ __forceinline__ void res_mtu(const MatDesc& d, const float* Ms, const float* Us,
                                        float* Wb, float* Ww_) {
  constexpr int NW = kResThreads / 64, kK = 8;
  const int m = d.m, n = d.n, r = d.r, pitch = n + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lk = lane >> 4;
  gptr<float> Ww = to_global(Ww_);
  for (int blk = wave; blk * 16 < n; blk += NW) {
    const int j0 = blk * 16, ja = j0 + li;
    f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    for (int i0 = 0; i0 < m; i0 += 4 * kK) {
      float a[kK], b[kK];
#pragma unroll
      for (int u = 0; u < kK; ++u) {
        const int i = i0 + 4 * u + lk;
        a[u] = ja < n && i < m ? Ms[i * pitch + ja] : 0.0f;
        b[u] = li < RB && i < m ? Us[i * (RB + 1) + li] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kK; ++u) acc[u & 1] = mfma16(a[u], b[u], acc[u & 1]);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + 4 * lk + v;
      if (j < n && li < RB) {
        const float w = acc[0][v] + acc[1][v];
        Wb[j * (RB + 1) + li] = w;
        if (li < r) Ww[static_cast<int64_t>(j) * r + li] = w;
      }
    }
  }
  __syncthreads();
}

// Operands of the 16 x 16 block (i0, j0) of U F^T (F: W or Vbar, n x RB in
// LDS): RB / 4 reduction steps of 4.
template <int RB>
struct BlockOps {
  float a[RB / 4], b[RB / 4];
  __device__ void load(const float* Us, const float* F, int i0, int j0, int m, int n) {
    const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
#pragma unroll
    for (int s4 = 0; s4 < RB / 4; ++s4) {
      const int k = 4 * s4 + lk;
      a[s4] = i0 + li < m ? Us[(i0 + li) * (RB + 1) + k] : 0.0f;
      b[s4] = j0 + li < n ? F[(j0 + li) * (RB + 1) + k] : 0.0f;
    }
  }
  __device__ f32x4 product() const {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s4 = 0; s4 < RB / 4; ++s4) acc = mfma16(a[s4], b[s4], acc);
    return acc;
  }
};

// R_new = beta (M - U W^T) into Ms, in place (M is not read after this), by
// batches of kT blocks per wavefront: every LDS read of a batch (operands
// and M) is issued before its MFMAs and its writes.
template <int RB>
__device__ __forceinline__ void res_residual(const Launch& L, const MatDesc& d, float* Ms,
                                             const float* Us, const float* Wb) {
  constexpr int NW = kResThreads / 64, kT = 4;
  const int m = d.m, n = d.n, pitch = n + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lk = lane >> 4;
  const int nb = (n + 15) / 16, nt = (m + 15) / 16 * nb;
  const float beta = L.beta;
  for (int t0 = wave; t0 < nt; t0 += NW * kT) {
    BlockOps<RB> op[kT];
    float mv[kT][4];
#pragma unroll
    for (int b = 0; b < kT; ++b) {
      const int tile = t0 + b * NW;
      const int i0 = tile / nb * 16, j0 = tile % nb * 16, j = j0 + li;
      op[b].load(Us, Wb, i0, j0, tile < nt ? m : 0, n);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + 4 * lk + v;
        mv[b][v] = tile < nt && i < m && j < n ? Ms[i * pitch + j] : 0.0f;
      }
    }
    f32x4 acc[kT];
#pragma unroll
    for (int b = 0; b < kT; ++b) acc[b] = op[b].product();
#pragma unroll
    for (int b = 0; b < kT; ++b) {
      const int tile = t0 + b * NW;
      const int i0 = tile / nb * 16, j = tile % nb * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + 4 * lk + v;
        if (tile < nt && i < m && j < n) Ms[i * pitch + j] = beta * (mv[b][v] - acc[b][v]);
      }
    }
  }
  __syncthreads();
}

// X -= eta U Vbar^T and R = R_new from LDS: a wavefront issues the X loads
// of kT of its blocks, then takes the blocks one by one (operands and
// R_new from LDS, MFMAs, X and R stores).
template <int RB>
__device__ __forceinline__ void res_update(const Launch& L, const MatDesc& d, const float* Ms,
                                           const float* Us, const float* Vb) {
  constexpr int NW = kResThreads / 64, kT = 16;
  const int m = d.m, n = d.n, pitch = n + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lk = lane >> 4;
  const int nb = (n + 15) / 16, nt = (m + 15) / 16 * nb;
  gptr<float> X = to_global(d.X);
  gptr<float> R = to_global(d.R);
  const float eta = L.eta;
  for (int t0 = wave; t0 < nt; t0 += NW * kT) {
    float xv[kT][4];
#pragma unroll
    for (int b = 0; b < kT; ++b) {
      const int tile = t0 + b * NW;
      const int i0 = tile / nb * 16, j = tile % nb * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + 4 * lk + v;
        xv[b][v] = tile < nt && i < m && j < n ? X[static_cast<int64_t>(i) * n + j] : 0.0f;
      }
    }
#pragma unroll
    for (int b = 0; b < kT; ++b) {
      const int tile = t0 + b * NW;
      if (tile >= nt) break;
      const int i0 = tile / nb * 16, j0 = tile % nb * 16, j = j0 + li;
      BlockOps<RB> op;
      op.load(Us, Vb, i0, j0, m, n);
      float rv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + 4 * lk + v;
        rv[v] = i < m && j < n ? Ms[i * pitch + j] : 0.0f;
      }
      const f32x4 acc = op.product();
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + 4 * lk + v;
        if (i < m && j < n) {
          const int64_t o = static_cast<int64_t>(i) * n + j;
          X[o] = xv[b][v] - eta * acc[v];
          R[o] = rv[v];
        }
      }
    }
  }
}

// Resident form of the whole step.  X, R and V are written only once both
// factorizations have succeeded.
template <typename GT, int RB>
__global__ __launch_bounds__(kResThreads) void k_small_res(Launch L) {
  constexpr int NT = kResThreads, QP = RB + 1;   // odd factor pitch: conflict-free MFMA reads
  __shared__ ResLds sh;
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, blockIdx.x, d, ci, local);
  const int t = threadIdx.x, m = d.m, n = d.n, r = d.r;
  const int n32 = (n + 31) / 32 * 32;
  float* Us = sh.f;                 // P, then U (m x QP)
  float* Vb = Us + m * QP;          // V, then W, then Vbar (n32 x QP)
  float* Ms = Vb + n32 * QP;        // M, then R_new (m x (n + 1))
  load_v<NT, QP>(d, Vb);
  res_load_m<GT>(d, Ms);
  __syncthreads();
  res_mv<RB>(d, Ms, Vb, Us, reinterpret_cast<float*>(L.ws + d.oP));
  int ctl = 0, flags = 0;
  if (!small_orth<NT, RB, QP>(sh.o, Us, Us, m, r, ctl)) {
    flags = DION_STATUS_ORTH_P;
  } else {
    store_factor<NT, QP>(Us, reinterpret_cast<float*>(L.ws + d.oB), m, r);
    res_mtu<RB>(d, Ms, Us, Vb, reinterpret_cast<float*>(L.ws + d.oW));
    res_residual<RB>(L, d, Ms, Us, Vb);
    bool ok;
    if (L.mode == 1) {
      ok = small_orth<NT, RB, QP>(sh.o, Vb, Vb, n, r, ctl);
      if (!ok) flags = DION_STATUS_ORTH_W;
    } else {
      ok = small_colnorm<NT, RB, QP>(sh.o, Vb, Vb, n, r);
      if (!ok) flags = DION_STATUS_COLNORM;
    }
    if (ok) {
      res_update<RB>(L, d, Ms, Us, Vb);
      store_factor<NT, QP>(Vb, d.V, n, r);
    }
  }
  if (t == 0) L.status[d.slot] = flags | ctl;
}

template <typename GT, bool RES>
hipError_t go_small(const Launch& L, int rb, hipStream_t st) {
  if (L.total <= 0) return hipSuccess;
  const dim3 grid(L.total), block(kThreads);
  static_assert(kSmallRank == 16, "rank blocks 8 and 16");
  if constexpr (RES) {
    const dim3 rblock(kResThreads);
    if (rb == 8) hipLaunchKernelGGL((k_small_res<GT, 8>), grid, rblock, 0, st, L);
    else hipLaunchKernelGGL((k_small_res<GT, 16>), grid, rblock, 0, st, L);
  } else {
    if (rb == 8) hipLaunchKernelGGL((k_small<GT, 8>), grid, block, 0, st, L);
    else hipLaunchKernelGGL((k_small<GT, 16>), grid, block, 0, st, L);
  }
  return hipGetLastError();
}

}  // namespace

int small_rank_block(int r) { return r <= 8 ? 8 : r <= kSmallRank ? 16 : 0; }

hipError_t launch_small(const Launch& L, int gdtype, int rb, bool resident, hipStream_t st) {
  if (resident)
    return gdtype == 0 ? go_small<float, true>(L, rb, st) : go_small<uint16_t, true>(L, rb, st);
  return gdtype == 0 ? go_small<float, false>(L, rb, st) : go_small<uint16_t, false>(L, rb, st);
}

}  // namespace dion
