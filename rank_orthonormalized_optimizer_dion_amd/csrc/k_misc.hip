// Small bandwidth kernels of the step:
//   k_reduce    sum of split-K partial products, in a fixed order
//   k_colnorm   Dion's rule, part 1: sums of squares of W's columns, per row slice
//   k_colnorm_fin  inverse Euclidean norms from the slices
//   k_colscale  Dion's rule, part 2: Vbar = W diag(1/||w_j||) written into V
//   k_split_t   split-bfloat16 planes of V^T for M V, of U^T for M^T U
//   k_split_n   split-bfloat16 planes of U, W and Vbar for the fused update
// (right-factor rule of the Orth-Dion page's closing remark; column scaling
// as the Orth-Dion abstract describes it).
#include <math.h>

#include "device_common.h"
#include "launchers.h"

namespace dion {

namespace {

constexpr int kElemsPerTile = 4 * kThreads;

// which = 0: P (m x r) from the M V partials; 1: W (n x r) from the M^T U
// partials.
__global__ __launch_bounds__(kThreads) void k_reduce(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int64_t elems = static_cast<int64_t>(L.which == 0 ? d.m : d.n) * d.r;
  const float* part = reinterpret_cast<const float*>(L.ws + d.oK);
  float* out = reinterpret_cast<float*>(L.ws + (L.which == 0 ? d.oP : d.oW));
  const int64_t base = static_cast<int64_t>(local) * kElemsPerTile + threadIdx.x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t i = base + e * kThreads;
    if (i >= elems) break;
    float s = 0.0f;
    for (int p = 0; p < ci.splits; ++p) s += part[p * elems + i];
    out[i] = s;
  }
}

// Column sums of squares of W in float64, split over rows so that one
// matrix of few columns still fills the GPU: work item (slice sp, column
// group cg) covers rows [sp klen, (sp + 1) klen) of 64 columns, 4 row
// groups accumulate and combine in a fixed order, and the slice's sums go
// to row sp of a (splits x r) float64 array in the Gram area (free by
// now: the factorization of P has consumed it).
__global__ __launch_bounds__(kThreads) void k_colnorm(Launch L) {
  __shared__ double red[4][64];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int groups = (d.r + 63) / 64;
  const int sp = local / groups, cg = local - sp * groups;
  const float* W = reinterpret_cast<const float*>(L.ws + d.oW);
  double* part = reinterpret_cast<double*>(L.ws + d.oS);
  const int col = cg * 64 + (threadIdx.x & 63);
  const int rg = threadIdx.x >> 6;
  const int i0 = sp * ci.klen, i1 = min(d.n, i0 + ci.klen);
  double acc = 0.0;
  if (col < d.r)
    for (int i = i0 + rg; i < i1; i += 4) {
      const double w = W[static_cast<int64_t>(i) * d.r + col];
      acc += w * w;
    }
  red[rg][threadIdx.x & 63] = acc;
  __syncthreads();
  if (rg == 0 && col < d.r)
    part[static_cast<int64_t>(sp) * d.r + col] =
        ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x];
}

// Inverse column norms from the slices' sums, added in slice order; a zero
// or non-finite norm is a breakdown.
__global__ __launch_bounds__(kThreads) void k_colnorm_fin(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int col = local * kThreads + threadIdx.x;
  if (col >= d.r) return;
  const double* part = reinterpret_cast<const double*>(L.ws + d.oS);
  double s = 0.0;
  for (int sp = 0; sp < ci.splits; ++sp) s += part[static_cast<int64_t>(sp) * d.r + col];
  if (!(s > 0.0) || !(s < INFINITY)) {
    atomicOr(&L.status[d.slot], L.flag);
  } else {
    reinterpret_cast<float*>(L.ws + d.oN)[col] = static_cast<float>(1.0 / sqrt(s));
  }
}

__global__ __launch_bounds__(kThreads) void k_colscale(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const float* W = reinterpret_cast<const float*>(L.ws + d.oW);
  const float* inv = reinterpret_cast<const float*>(L.ws + d.oN);
  const int64_t elems = static_cast<int64_t>(d.n) * d.r;
  const int64_t base = static_cast<int64_t>(local) * kElemsPerTile + threadIdx.x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t i = base + e * kThreads;
    if (i >= elems) break;
    d.V[i] = W[i] * inv[i % d.r];
  }
}

// Q^T (r x rows, from Q: rows x r float32; Q = V for which = 0, U for
// which = 1) as hi / lo bfloat16 planes of plane_pitch(rows) columns (zero
// past column rows) in plane_cell_r order, split as BfShape describes: a
// cell holds 8 consecutive rows of one column of Q, and the cells of one
// group of 8 rows are contiguous over the r columns, so that M V and
// M^T U copy their rank-r operand straight into LDS.  One workgroup per 64 x 64 tile of Q: coalesced float4 row
// reads into LDS, then each thread splits two cells (8 rows of one column).
__global__ __launch_bounds__(kThreads) void k_split_t(Launch L) {
  constexpr int T = kSplitTile;
  __shared__ float tile[T][T + 1];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  // The V split opens the step, before M V clears the status words: a
  // breakdown flagged by the previous step must not skip it.
  if (L.which == 1 && skipped(L, d)) return;
  const int ti = local / ci.ty, tj = local % ci.ty;
  const int i0 = ti * T, j0 = tj * T;
  const int rows = L.which == 0 ? d.n : d.m, kp = plane_pitch(rows);
  gptr<const float> Q = to_global(L.which == 0 ? d.V : reinterpret_cast<const float*>(L.ws + d.oB));
  const bool vec = (d.r & 3) == 0;
#pragma unroll
  for (int s = 0; s < T * T / 4 / kThreads; ++s) {
    const int e = threadIdx.x + kThreads * s;
    const int i = e / (T / 4), j = 4 * (e % (T / 4));
    const int gi = i0 + i, gj = j0 + j;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (gi < rows) {
      const int64_t o = static_cast<int64_t>(gi) * d.r + gj;
      if (vec && gj + 3 < d.r) {
        v = *(gptr<const f32x4>)(Q + o);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = gj + c < d.r ? Q[o + c] : 0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) tile[i][j + c] = v[c];
  }
  __syncthreads();
  uint16_t* hi = reinterpret_cast<uint16_t*>(L.ws + d.oH);
  const int64_t plane = static_cast<int64_t>(d.r) * kp;
#pragma unroll
  for (int s = 0; s < T * T / 8 / kThreads; ++s) {
    const int c = threadIdx.x + kThreads * s;
    const int j = c % T, i = 8 * (c / T);   // consecutive threads: consecutive columns j
    if (j0 + j >= d.r || i0 + i >= kp) continue;
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = tile[i + e][j];
      b[e] = tile[i + 4 + e][j];
    }
    u32x2 ha, la, hb, lb;
    bf_split4(a, ha, la);
    bf_split4(b, hb, lb);
    const int64_t o = plane_cell_r(d.r, j0 + j, (i0 + i) / 8);
    gptr<u32x4> ph = (gptr<u32x4>)to_global(hi);
    ph[o] = u32x4{ha.x, ha.y, hb.x, hb.y};
    ph[plane / 8 + o] = u32x4{la.x, la.y, lb.x, lb.y};
  }
}

// U (m x r), W and Vbar (n x r) as hi / lo bfloat16 planes in plane_cell_r
// order (cell (x, k8): elements 8 k8 .. 8 k8 + 7 of row x), zero in columns
// r .. plane_pitch(r), split as BfShape describes.  One workgroup per 64 x 64
// tile of a factor: coalesced float4 row reads into LDS, then each thread
// splits two cells; consecutive threads write consecutive rows of one k8.
__global__ __launch_bounds__(kThreads) void k_split_n(Launch L) {
  constexpr int T = kSplitTile;
  __shared__ float tile[T][T + 1];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int cr = (d.r + T - 1) / T;
  const int tu = (d.m + T - 1) / T * cr, tv = (d.n + T - 1) / T * cr;
  const int rq = plane_pitch(d.r);
  const int64_t cu = static_cast<int64_t>(d.m) * (rq / 8), cn = static_cast<int64_t>(d.n) * (rq / 8);
  u32x4* out = reinterpret_cast<u32x4*>(L.ws + d.oE);
  const float* src;
  int rows, t = local;
  int64_t plane;
  if (t < tu) {
    src = reinterpret_cast<const float*>(L.ws + d.oB);
    rows = d.m;
    plane = cu;
  } else if ((t -= tu) < tv) {
    src = reinterpret_cast<const float*>(L.ws + d.oW);
    rows = d.n;
    plane = cn;
    out += 2 * cu;
  } else {
    t -= tv;
    src = d.V;
    rows = d.n;
    plane = cn;
    out += 2 * cu + 2 * cn;
  }
  const int i0 = (t / cr) * T, j0 = (t % cr) * T;
  gptr<const float> Q = to_global(src);
  const bool vec = (d.r & 3) == 0;
#pragma unroll
  for (int s = 0; s < T * T / 4 / kThreads; ++s) {
    const int e = threadIdx.x + kThreads * s;
    const int i = e / (T / 4), j = 4 * (e % (T / 4));
    const int gi = i0 + i, gj = j0 + j;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (gi < rows) {
      const int64_t o = static_cast<int64_t>(gi) * d.r + gj;
      if (vec && gj + 3 < d.r) {
        v = *(gptr<const f32x4>)(Q + o);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = gj + c < d.r ? Q[o + c] : 0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) tile[i][j + c] = v[c];
  }
  __syncthreads();
  gptr<u32x4> po = to_global(out);
#pragma unroll
  for (int s = 0; s < T * T / 8 / kThreads; ++s) {
    const int c = threadIdx.x + kThreads * s;
    const int x = c % T, k8 = c / T;
    if (i0 + x >= rows || j0 + 8 * k8 >= rq) continue;
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = tile[x][8 * k8 + e];
      b[e] = tile[x][8 * k8 + 4 + e];
    }
    u32x2 ha, la, hb, lb;
    bf_split4(a, ha, la);
    bf_split4(b, hb, lb);
    const int64_t o = plane_cell_r(rows, i0 + x, j0 / 8 + k8);
    po[o] = u32x4{ha.x, ha.y, hb.x, hb.y};
    po[plane + o] = u32x4{la.x, la.y, lb.x, lb.y};
  }
}

template <class K>
hipError_t go(K kernel, const Launch& L, hipStream_t st) {
  if (L.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(L.total), dim3(kThreads), 0, st, L);
  return hipGetLastError();
}

}  // namespace

int elems_per_tile() { return kElemsPerTile; }
hipError_t launch_reduce(const Launch& L, hipStream_t st) { return go(k_reduce, L, st); }
hipError_t launch_colnorm(const Launch& L, hipStream_t st) { return go(k_colnorm, L, st); }
hipError_t launch_colnorm_fin(const Launch& L, hipStream_t st) { return go(k_colnorm_fin, L, st); }
hipError_t launch_colscale(const Launch& L, hipStream_t st) { return go(k_colscale, L, st); }
hipError_t launch_split_t(const Launch& L, hipStream_t st) { return go(k_split_t, L, st); }
hipError_t launch_split_n(const Launch& L, hipStream_t st) { return go(k_split_n, L, st); }

}  // namespace dion
