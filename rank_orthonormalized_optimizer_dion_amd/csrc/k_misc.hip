// Small bandwidth kernels of the step:
//   k_reduce    sum of split-K partial products, in a fixed order
//   k_colnorm   Dion's rule, part 1: inverse Euclidean norms of W's columns
//   k_colscale  Dion's rule, part 2: Vbar = W diag(1/||w_j||) written into V
// (right-factor rule of the Orth-Dion page's closing remark; column scaling
// as the Orth-Dion abstract describes it).
#include <math.h>

#include "device_common.h"
#include "launchers.h"

namespace dion {

namespace {

constexpr int kElemsPerTile = 4 * kThreads;

__device__ __forceinline__ bool skipped(const Launch& L, const MatDesc& d) {
  return L.status[d.slot] != 0;
}

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

// One workgroup per 64 columns: 4 row groups accumulate squares in float64,
// then combine in a fixed order.
__global__ __launch_bounds__(kThreads) void k_colnorm(Launch L) {
  __shared__ double red[4][64];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const float* W = reinterpret_cast<const float*>(L.ws + d.oW);
  float* inv = reinterpret_cast<float*>(L.ws + d.oN);
  const int col = local * 64 + (threadIdx.x & 63);
  const int rg = threadIdx.x >> 6;
  double acc = 0.0;
  if (col < d.r)
    for (int i = rg; i < d.n; i += 4) {
      const double w = W[static_cast<int64_t>(i) * d.r + col];
      acc += w * w;
    }
  red[rg][threadIdx.x & 63] = acc;
  __syncthreads();
  if (rg == 0 && col < d.r) {
    const double s = ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) +
                     red[3][threadIdx.x];
    if (!(s > 0.0) || !(s < INFINITY)) {
      atomicOr(&L.status[d.slot], L.flag);
    } else {
      inv[col] = static_cast<float>(1.0 / sqrt(s));
    }
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
hipError_t launch_colscale(const Launch& L, hipStream_t st) { return go(k_colscale, L, st); }

}  // namespace dion
