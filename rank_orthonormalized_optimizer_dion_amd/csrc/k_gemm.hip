// The dense contractions of one Dion / Orth-Dion step, as grouped float32
// MFMA kernels for gfx950 (Orth-Dion page, equation block):
//   k_mv    P = M V            (M = G + R formed while loading)
//   k_mtu   W = M^T U          (equation 3)
//   k_gram  S = Q^T Q          (Gram matrix of a CholeskyQR pass)
//   k_trmm  Q' = Q T^{-1}      (T^{-1} upper triangular, read from T^{-T});
//           k_trmm6 the same with float32 accuracy on bfloat16 matrix cores
//   k_epi   X -= eta U Vbar^T and R = beta (M - U W^T)   (equations 5, 6)
#include "device_common.h"
#include "launchers.h"

namespace dion {

namespace {

constexpr int BM = 128;

template <int TBM, int TBN>
__device__ __forceinline__ void store_tile(float* out_, int64_t ld, int r0, int c0,
                                           int rmax, int cmax,
                                           const f32x16 (&acc)[Warps<TBM, TBN>::FM][Warps<TBM, TBN>::FN]) {
  using W = Warps<TBM, TBN>;
  gptr<float> out = to_global(out_);
#pragma unroll
  for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn) {
      const int col = c0 + acc_col<TBM, TBN>(fn);
      if (col >= cmax) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = r0 + acc_row<TBM, TBN>(fm, v);
        if (row < rmax) out[static_cast<int64_t>(row) * ld + col] = acc[fm][fn][v];
      }
    }
}

// The fused update's epilogue for a tile at (r0, c0) whose accumulators
// hold U Vbar^T (ax) and U W^T (ar) in the 32 x 32 MFMA layout of wavefront
// grid W: X -= eta ax, R = beta ((G + R) - ar).
//
// Interior tiles: the 16 values of one accumulator block sit in 4 groups of
// 8 rows; within a group the lane's 4 rows are at fixed offsets from the
// group's first element.  That element's address is wavefront-uniform (a
// scalar base), so every load and store is a scalar base plus one of 4
// per-lane 32-bit byte offsets (the group spans 8 rows: 8 n < 2^28 when
// m >= 256 and m n < 2^31).  E elements per lane are loaded before the
// first store of a batch (X, G and R may alias as far as the compiler
// knows, so loads interleaved with stores would wait one element at a time).
//
// Edge tiles check every element, 8 at a time.  m n < 2^31 (checked at the
// boundary): element offsets are 32-bit.
template <class T>
__device__ __forceinline__ gptr<T> uniform_ptr(gptr<T> p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr<T>>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <class T>
__device__ __forceinline__ gptr<T> byte_off(gptr<T> base, uint32_t bytes) {
  return reinterpret_cast<gptr<T>>(reinterpret_cast<gptr<char>>(const_cast<gptr<char>>(
                                       reinterpret_cast<gptr<const char>>(base))) + bytes);
}

template <class W, typename GT, int E>
__device__ __forceinline__ void update_epilogue_full(const Launch& L, const MatDesc& d, int r0,
                                                     int c0, const f32x16 (&ax)[W::FM][W::FN],
                                                     const f32x16 (&ar)[W::FM][W::FN]) {
  static_assert(E % 4 == 0, "whole groups of 4 rows");
  constexpr int GPB = E / 4, NGRP = W::FM * W::FN * 4;
  static_assert(NGRP % GPB == 0, "batch must divide the groups");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wave / W::GN, wn = wave % W::GN;
  const uint32_t n = static_cast<uint32_t>(d.n);
  uint32_t o4[4], o2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t e = (4u * static_cast<uint32_t>(lane >> 5) + j) * n + static_cast<uint32_t>(lane & 31);
    o4[j] = 4u * e;
    o2[j] = static_cast<uint32_t>(sizeof(GT)) * e;
  }
  const float eta = L.eta, beta = L.beta;
  // X, G and R are streamed once: nontemporal accesses keep them from
  // displacing the rank-r panels that the tiles still running read
#pragma unroll
  for (int g0 = 0; g0 < NGRP; g0 += GPB) {
    float gv[E], rv[E], xv[E];
#pragma unroll
    for (int b = 0; b < GPB; ++b) {
      const int g = g0 + b, fm = g / (4 * W::FN), fn = (g / 4) % W::FN, q = g % 4;
      const int64_t e0 = static_cast<int64_t>(r0 + wm * W::TM + fm * 32 + 8 * q) * d.n +
                         (c0 + wn * W::TN + fn * 32);
      const gptr<const GT> gp = uniform_ptr(to_global(static_cast<const GT*>(d.G)) + e0);
      const gptr<const float> xp = uniform_ptr(to_global(static_cast<const float*>(d.X)) + e0);
      const gptr<const float> rp = uniform_ptr(to_global(static_cast<const float*>(d.R)) + e0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(GT) == 2) gv[4 * b + j] = bf16_to_f32(__builtin_nontemporal_load(byte_off(gp, o2[j])));
        else gv[4 * b + j] = __builtin_nontemporal_load(byte_off(gp, o2[j]));
        rv[4 * b + j] = __builtin_nontemporal_load(byte_off(rp, o4[j]));
        xv[4 * b + j] = __builtin_nontemporal_load(byte_off(xp, o4[j]));
      }
    }
#pragma unroll
    for (int b = 0; b < GPB; ++b) {
      const int g = g0 + b, fm = g / (4 * W::FN), fn = (g / 4) % W::FN, q = g % 4;
      const int64_t e0 = static_cast<int64_t>(r0 + wm * W::TM + fm * 32 + 8 * q) * d.n +
                         (c0 + wn * W::TN + fn * 32);
      const gptr<float> xp = uniform_ptr(to_global(d.X) + e0);
      const gptr<float> rp = uniform_ptr(to_global(d.R) + e0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_nontemporal_store(xv[4 * b + j] - eta * ax[fm][fn][4 * q + j], byte_off(xp, o4[j]));
        __builtin_nontemporal_store(beta * ((gv[4 * b + j] + rv[4 * b + j]) - ar[fm][fn][4 * q + j]), byte_off(rp, o4[j]));
      }
    }
  }
}

template <class W, typename GT, bool FULL, int E = 8>
__device__ __forceinline__ void update_epilogue(const Launch& L, const MatDesc& d, int r0, int c0,
                                                const f32x16 (&ax)[W::FM][W::FN],
                                                const f32x16 (&ar)[W::FM][W::FN]) {
  if constexpr (FULL) {
    update_epilogue_full<W, GT, E>(L, d, r0, c0, ax, ar);
    return;
  }
  gptr<const GT> G = to_global(static_cast<const GT*>(d.G));
  gptr<float> X = to_global(d.X);
  gptr<float> R = to_global(d.R);
  const float eta = L.eta, beta = L.beta;
#pragma unroll
  for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn)
#pragma unroll
      for (int h = 0; h < 16; h += 8) {
        const int col = c0 + W::col(fn);
        float gv[8], rv[8], xv[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int row = r0 + W::row(fm, h + v);
          if (row < d.m && col < d.n) {
            const unsigned o = static_cast<unsigned>(row * d.n + col);
            if constexpr (sizeof(GT) == 2) gv[v] = bf16_to_f32(G[o]); else gv[v] = G[o];
            rv[v] = R[o];
            xv[v] = X[o];
          }
        }
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int row = r0 + W::row(fm, h + v);
          if (row < d.m && col < d.n) {
            const unsigned o = static_cast<unsigned>(row * d.n + col);
            X[o] = xv[v] - eta * ax[fm][fn][h + v];
            R[o] = beta * ((gv[v] + rv[v]) - ar[fm][fn][h + v]);
          }
        }
      }
}


// P = (G + R) V over the reduction slice [kbeg, kend) of n.
template <typename GT, int BN, bool VEC, bool FULL>
__device__ __forceinline__ void mv_body(const Launch& L, const MatDesc& d, const ClassInfo& ci,
                                        int s, int tm, int tn, int kbeg, int kend, f32x4* smem) {
  constexpr int BK = 32;
  const SrcM<GT> sm(static_cast<const GT*>(d.G), d.R);
  LoadKC<BM, BK, VEC, false, SrcM<GT>> la0(sm, d.n, tm * BM, d.m, kend), la1 = la0;
  LoadXC<BN, BK, VEC, SrcF32> lb0(SrcF32{d.V}, d.r, tn * BN, d.r, kend), lb1 = lb0;
  f32x16 acc[Warps<BM, BN>::FM][Warps<BM, BN>::FN];
  zero_acc(acc);
  pipeline2<BM, BN, BK, FULL>(la0, la1, lb0, lb1, kbeg, (kend - kbeg + BK - 1) / BK, smem,
                              [&](const f32x4* a, const f32x4* b) { mma_tile<BM, BN, BK>(a, b, acc); });
  float* out = ci.splits == 1
                   ? reinterpret_cast<float*>(L.ws + d.oP)
                   : reinterpret_cast<float*>(L.ws + d.oK) + static_cast<int64_t>(s) * d.m * d.r;
  store_tile<BM, BN>(out, d.r, tm * BM, tn * BN, d.m, d.r, acc);
}

template <typename GT, int BN, bool VEC>
__global__ __launch_bounds__(kThreads) void k_mv(Launch L) {
  constexpr int BK = 32;
  __shared__ f32x4 smem[mainloop_cells<BM, BN, BK>()];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  // The first kernel of a step clears the matrix's status word.
  if (local == 0 && threadIdx.x == 0) L.status[d.slot] = 0;
  const int per = ci.tx * ci.ty;
  const int s = local / per;
  int tm, tn;
  tile_order(local - s * per, ci.tx, ci.ty, tm, tn);
  const int kbeg = s * ci.klen;
  const int kend = min(d.n, kbeg + ci.klen);
  const bool full = VEC && (tm + 1) * BM <= d.m && (tn + 1) * BN <= d.r && (kend - kbeg) % BK == 0;
  if (full) mv_body<GT, BN, VEC, true>(L, d, ci, s, tm, tn, kbeg, kend, smem);
  else mv_body<GT, BN, VEC, false>(L, d, ci, s, tm, tn, kbeg, kend, smem);
}

// W = (G + R)^T U over the reduction slice [kbeg, kend) of m.
template <typename GT, int BN, bool VEC, bool FULL>
__device__ __forceinline__ void mtu_body(const Launch& L, const MatDesc& d, const ClassInfo& ci,
                                         int s, int tm, int tn, int kbeg, int kend, f32x4* smem) {
  constexpr int BK = 32;
  const SrcM<GT> sm(static_cast<const GT*>(d.G), d.R);
  LoadXC<BM, BK, VEC, SrcM<GT>> la0(sm, d.n, tm * BM, d.n, kend), la1 = la0;
  const float* U = reinterpret_cast<const float*>(L.ws + d.oB);
  LoadXC<BN, BK, VEC, SrcF32> lb0(SrcF32{U}, d.r, tn * BN, d.r, kend), lb1 = lb0;
  f32x16 acc[Warps<BM, BN>::FM][Warps<BM, BN>::FN];
  zero_acc(acc);
  pipeline2<BM, BN, BK, FULL>(la0, la1, lb0, lb1, kbeg, (kend - kbeg + BK - 1) / BK, smem,
                              [&](const f32x4* a, const f32x4* b) { mma_tile<BM, BN, BK>(a, b, acc); });
  float* out = ci.splits == 1
                   ? reinterpret_cast<float*>(L.ws + d.oW)
                   : reinterpret_cast<float*>(L.ws + d.oK) + static_cast<int64_t>(s) * d.n * d.r;
  store_tile<BM, BN>(out, d.r, tm * BM, tn * BN, d.n, d.r, acc);
}

template <typename GT, int BN, bool VEC>
__global__ __launch_bounds__(kThreads) void k_mtu(Launch L) {
  constexpr int BK = 32;
  __shared__ f32x4 smem[mainloop_cells<BM, BN, BK>()];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int per = ci.tx * ci.ty;
  const int s = local / per;
  int tm, tn;
  tile_order(local - s * per, ci.tx, ci.ty, tm, tn);
  const int kbeg = s * ci.klen;
  const int kend = min(d.m, kbeg + ci.klen);
  const bool full = VEC && (tm + 1) * BM <= d.n && (tn + 1) * BN <= d.r && (kend - kbeg) % BK == 0;
  if (full) mtu_body<GT, BN, VEC, true>(L, d, ci, s, tm, tn, kbeg, kend, smem);
  else mtu_body<GT, BN, VEC, false>(L, d, ci, s, tm, tn, kbeg, kend, smem);
}

// Partial Gram matrix S_s = Q[kbeg:kend]^T Q[kbeg:kend] on the upper
// triangle of BG x BG tiles, in float64: float32 products are exact in
// float64 and the sums are float64, so S is accurate enough for a single
// CholeskyQR pass.
template <int BG, bool VEC, bool FULL>
__device__ __forceinline__ void gram_body(const Launch& L, const MatDesc& d, const float* Q, int s,
                                          int ti, int tj, int kbeg, int kend, f32x4* smem) {
  constexpr int BK = 32, FB = BG / 32;
  LoadXC<BG, BK, VEC, SrcF32> la(SrcF32{Q}, d.r, ti * BG, d.r, kend);
  LoadXC<BG, BK, VEC, SrcF32> lb(SrcF32{Q}, d.r, tj * BG, d.r, kend);
  f64x4 acc[FB][FB];
#pragma unroll
  for (int fm = 0; fm < FB; ++fm)
#pragma unroll
    for (int fn = 0; fn < FB; ++fn) acc[fm][fn] = f64x4{0.0, 0.0, 0.0, 0.0};
  // On a diagonal tile the wavefront of rows BG/2.. and columns ..BG/2 lies
  // wholly below the diagonal: it loads its share of the tile for the
  // others but computes and stores nothing (the factorization reads the
  // upper triangle only).
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool below = ti == tj && wm > wn;
  pipeline<BG, BG, BK, FULL>(la, lb, kbeg, (kend - kbeg + BK - 1) / BK, smem,
                             [&](const f32x4* a, const f32x4* b) {
                               if (!below) mma_tile_f64<BG, BK>(a, b, acc);
                             });
  if (below) return;
  gptr<double> out = to_global(reinterpret_cast<double*>(L.ws + d.oS) +
                               static_cast<int64_t>(s) * d.rp * d.rp);
#pragma unroll
  for (int fm = 0; fm < FB; ++fm)
#pragma unroll
    for (int fn = 0; fn < FB; ++fn) {
      const int col = tj * BG + wn * (BG / 2) + fn * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // 16 x 16 float64 MFMA output: lane l, register v holds row
        // l / 16 + 4 v, column l % 16.
        const int row = ti * BG + wm * (BG / 2) + fm * 16 + (lane >> 4) + 4 * v;
        if (FULL || (row < d.r && col < d.r)) out[static_cast<int64_t>(row) * d.rp + col] = acc[fm][fn][v];
      }
    }
}

// Four blocks per CU (at most 128 registers per lane): the float64 MFMAs
// are long, and the extra wavefronts cover the tile loads and barriers.
// Work item `local` of a Gram launch: tile (ti, tj) of the upper triangle
// and reduction slice s.
template <int BG, bool VEC>
__device__ __forceinline__ void gram_item(const Launch& L, const MatDesc& d, const float* Q,
                                          const ClassInfo& ci, int local, f32x4* smem) {
  constexpr int BK = 32;
  const int rows = L.which == 0 ? d.m : d.n;
  const int nt = ci.tx;
  const int pairs = nt * (nt + 1) / 2;
  const int s = local / pairs;
  int p = local - s * pairs;
  int ti = 0;
  while (p >= nt - ti) {
    p -= nt - ti;
    ++ti;
  }
  const int tj = ti + p;
  const int kbeg = s * ci.klen;
  const int kend = min(rows, kbeg + ci.klen);
  const bool full = VEC && (tj + 1) * BG <= d.r && (kend - kbeg) % BK == 0;
  if (full) gram_body<BG, VEC, true>(L, d, Q, s, ti, tj, kbeg, kend, smem);
  else gram_body<BG, VEC, false>(L, d, Q, s, ti, tj, kbeg, kend, smem);
}

// Four blocks per CU (at most 128 registers per lane): the float64 MFMAs
// are long, and the extra wavefronts cover the tile loads and barriers.
template <int BG, bool VEC>
__global__ __launch_bounds__(kThreads, 4) void k_gram(Launch L) {
  constexpr int BK = 32;
  __shared__ f32x4 smem[mainloop_cells<BG, BG, BK>()];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  gram_item<BG, VEC>(L, d, first_src(L, d), ci, local, smem);
}

// The same for the gated launches of orth's extra passes (see
// dion_types.h): fewer workgroups than items, each taking a chunk
// (for_items).
template <int BG, bool VEC>
__global__ __launch_bounds__(kThreads) void k_gram_gated(Launch L) {
  constexpr int BK = 32;
  __shared__ f32x4 smem[mainloop_cells<BG, BG, BK>()];
  for_items(L, [&](const MatDesc& d, const ClassInfo& ci, int local) {
    gram_item<BG, VEC>(L, d, orth_src(L, d), ci, local, smem);
    __syncthreads();   // the next item reuses the LDS stages
  });
}

// Q' = Q T^{-1}.  T^{-1} is upper triangular, so output column block tn
// only needs reduction steps k < (tn + 1) BN.  T^{-1}[k][j] = Y[j][k] with
// Y = T^{-T} (lower triangular, float64; its strictly upper part is never
// written and is masked on load).
template <int BN, bool VEC, bool FULL>
__device__ __forceinline__ void trmm_body(const Launch& L, const MatDesc& d, int rows, int tm,
                                          int tn, int kend, f32x4* smem) {
  constexpr int BK = 32;
  const float* Q = first_src(L, d);
  float* dst = final_dst(L, d);
  const double* Y = reinterpret_cast<const double*>(L.ws + d.oY);
  LoadKC<BM, BK, VEC, false, SrcF32> la(SrcF32{Q}, d.r, tm * BM, rows, kend);
  LoadKC<BN, BK, true, true, SrcF64> lb(SrcF64{Y}, d.rp, tn * BN, d.r, kend);
  f32x16 acc[Warps<BM, BN>::FM][Warps<BM, BN>::FN];
  zero_acc(acc);
  gemm_mainloop<BM, BN, BK, FULL>(la, lb, 0, (kend + BK - 1) / BK, smem, acc);
  store_tile<BM, BN>(dst, d.r, tm * BM, tn * BN, rows, d.r, acc);
}

template <int BN, bool VEC>
__global__ __launch_bounds__(kThreads) void k_trmm(Launch L) {
  constexpr int BK = 32;
  __shared__ f32x4 smem[mainloop_cells<BM, BN, BK>()];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int rows = L.which == 0 ? d.m : d.n;
  int tm, tn;
  tile_order(local, ci.tx, ci.ty, tm, tn);
  const int kend = min(d.r, (tn + 1) * BN);
  const bool full = VEC && (tm + 1) * BM <= rows && (tn + 1) * BN <= d.r && kend % BK == 0;
  if (full) trmm_body<BN, VEC, true>(L, d, rows, tm, tn, kend, smem);
  else trmm_body<BN, VEC, false>(L, d, rows, tm, tn, kend, smem);
}

// Q T^{-1} with float32 accuracy on the bfloat16 matrix cores (split-
// bfloat16 plans): both operands split three ways (bf_split4x3), six
// bfloat16 products per float32 product, float32 accumulation.  BK = 16 so
// that two stages of three planes per operand leave room for three blocks
// per CU.
template <int BN, bool VEC, bool FULL>
__device__ __forceinline__ void trmm6_body(const Launch& L, const MatDesc& d, int rows, int tm,
                                           int tn, int kend, u32x4* smem) {
  constexpr int BK = 16;
  constexpr int CA = BfShape<BM, BK>::CELLS, CB = BfShape<BN, BK>::CELLS;
  constexpr int STAGE = 3 * (CA + CB);
  const float* Q = first_src(L, d);
  float* dst = final_dst(L, d);
  const double* Y = reinterpret_cast<const double*>(L.ws + d.oY);
  LoadKC<BM, BK, VEC, false, SrcF32> la(SrcF32{Q}, d.r, tm * BM, rows, kend);
  LoadKC<BN, BK, true, true, SrcF64> lb(SrcF64{Y}, d.rp, tn * BN, d.r, kend);
  f32x16 acc[Warps<BM, BN>::FM][Warps<BM, BN>::FN];
  zero_acc(acc);
  auto store = [&](int st) {
    u32x2* b = reinterpret_cast<u32x2*>(smem + st * STAGE);
    la.store_bf3(b, b + 2 * CA, b + 4 * CA);
    lb.store_bf3(b + 6 * CA, b + 6 * CA + 2 * CB, b + 6 * CA + 4 * CB);
  };
  const int nk = (kend + BK - 1) / BK;
  la.template load<FULL>(0);
  lb.template load<FULL>(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      la.template load<FULL>((kt + 1) * BK);
      lb.template load<FULL>((kt + 1) * BK);
    }
    const u32x4* b = smem + (kt & 1) * STAGE;
    mma_tile_bf6<BM, BN, BK>(b, b + 3 * CA, acc);
    if (more) store((kt + 1) & 1);
    __syncthreads();
  }
  store_tile<BM, BN>(dst, d.r, tm * BM, tn * BN, rows, d.r, acc);
}

// Three blocks per CU (at most 168 registers per lane).
template <int BN, bool VEC>
__global__ __launch_bounds__(kThreads, 3) void k_trmm6(Launch L) {
  constexpr int BK = 16;
  __shared__ u32x4 smem[2 * 3 * (BfShape<BM, BK>::CELLS + BfShape<BN, BK>::CELLS)];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int rows = L.which == 0 ? d.m : d.n;
  int tm, tn;
  tile_order(local, ci.tx, ci.ty, tm, tn);
  const int kend = min(d.r, (tn + 1) * BN);
  const bool full = VEC && (tm + 1) * BM <= rows && (tn + 1) * BN <= d.r && kend % BK == 0;
  if (full) trmm6_body<BN, VEC, true>(L, d, rows, tm, tn, kend, smem);
  else trmm6_body<BN, VEC, false>(L, d, rows, tm, tn, kend, smem);
}

// Fused weight and residual update over one BM x BN tile of X and R:
//   X <- X - eta U Vbar^T,   R <- beta ((G + R) - U W^T)
// Both products share the left operand U; K = r.
template <typename GT, int BN, bool VEC, bool FULL>
__device__ __forceinline__ void epi_body(const Launch& L, const MatDesc& d, int tm, int tn,
                                         f32x4* smem) {
  constexpr int BK = 16;
  constexpr int CA = TileShape<BM, BK>::CELLS, CB = TileShape<BN, BK>::CELLS;
  constexpr int STAGE = CA + 2 * CB;
  using Wp = Warps<BM, BN>;
  const float* U = reinterpret_cast<const float*>(L.ws + d.oB);
  const float* Wf = reinterpret_cast<const float*>(L.ws + d.oW);
  LoadKC<BM, BK, VEC, false, SrcF32> la(SrcF32{U}, d.r, tm * BM, d.m, d.r);
  LoadKC<BN, BK, VEC, false, SrcF32> lv(SrcF32{d.V}, d.r, tn * BN, d.n, d.r);
  LoadKC<BN, BK, VEC, false, SrcF32> lw(SrcF32{Wf}, d.r, tn * BN, d.n, d.r);
  f32x16 ax[Wp::FM][Wp::FN], ar[Wp::FM][Wp::FN];
  zero_acc(ax);
  zero_acc(ar);
  const int nk = (d.r + BK - 1) / BK;
  la.template load<FULL>(0);
  lv.template load<FULL>(0);
  lw.template load<FULL>(0);
  la.store(smem);
  lv.store(smem + CA);
  lw.store(smem + CA + CB);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    f32x4* cur = smem + (kt & 1) * STAGE;
    f32x4* nxt = smem + (STAGE - (kt & 1) * STAGE);
    const bool more = kt + 1 < nk;
    if (more) {
      la.template load<FULL>((kt + 1) * BK);
      lv.template load<FULL>((kt + 1) * BK);
      lw.template load<FULL>((kt + 1) * BK);
    }
    mma_tile<BM, BN, BK>(cur, cur + CA, ax);
    mma_tile<BM, BN, BK>(cur, cur + CA + CB, ar);
    if (more) {
      la.store(nxt);
      lv.store(nxt + CA);
      lw.store(nxt + CA + CB);
    }
    __syncthreads();
  }
  // Element by element: one batch's loads would add registers and cost this
  // float32-MFMA-bound kernel its third wavefront per SIMD.
  gptr<const GT> G = to_global(static_cast<const GT*>(d.G));
  gptr<float> X = to_global(d.X);
  gptr<float> R = to_global(d.R);
  const float eta = L.eta, beta = L.beta;
#pragma unroll
  for (int fm = 0; fm < Wp::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Wp::FN; ++fn) {
      const int col = tn * BN + acc_col<BM, BN>(fn);
      if (!FULL && col >= d.n) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = tm * BM + acc_row<BM, BN>(fm, v);
        if (!FULL && row >= d.m) continue;
        const int64_t o = static_cast<int64_t>(row) * d.n + col;
        float g;
        if constexpr (sizeof(GT) == 2) g = bf16_to_f32(G[o]); else g = G[o];
        const float mv = g + R[o];
        X[o] = X[o] - eta * ax[fm][fn][v];
        R[o] = beta * (mv - ar[fm][fn][v]);
      }
    }
}

template <typename GT, int BN, bool VEC>
__global__ __launch_bounds__(kThreads) void k_epi(Launch L) {
  constexpr int BK = 16;
  constexpr int STAGE = TileShape<BM, BK>::CELLS + 2 * TileShape<BN, BK>::CELLS;
  __shared__ f32x4 smem[2 * STAGE];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  int tm, tn;
  tile_order(local, ci.tx, ci.ty, tm, tn);
  const bool full = VEC && (tm + 1) * BM <= d.m && (tn + 1) * BN <= d.n && d.r % BK == 0;
  if (full) epi_body<GT, BN, VEC, true>(L, d, tm, tn, smem);
  else epi_body<GT, BN, VEC, false>(L, d, tm, tn, smem);
}

// ---------------------------------------------------------------------------
// Split-bfloat16 variants of k_mv, k_mtu and k_epi: the same tiles and
// loaders, with float32 products taken as three bfloat16 MFMA products (see
// BfShape).  Relative product error <= 2^-16 instead of float32's 2^-24.
template <typename GT, int BN, bool VEC, bool FULL>
__device__ __forceinline__ void mv3_body(const Launch& L, const MatDesc& d, const ClassInfo& ci,
                                         int s, int tm, int tn, int kbeg, int kend, u32x4* smem) {
  constexpr int BK = 32;
  const SrcM<GT> sm(static_cast<const GT*>(d.G), d.R);
  LoadKC<BM, BK, VEC, false, SrcM<GT>> la0(sm, d.n, tm * BM, d.m, kend), la1 = la0;
  // V^T planes (r rows of plane_pitch(n), zero past column n): cells of 8
  // consecutive rows of V
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(L.ws + d.oH);
  LoadPl<BN, BK> lb0(vt, vt + static_cast<int64_t>(d.r) * plane_pitch(d.n), d.r, tn * BN, d.r),
      lb1 = lb0;
  f32x16 acc[Warps<BM, BN>::FM][Warps<BM, BN>::FN];
  zero_acc(acc);
  pipeline2_bf<BM, BN, BK, FULL>(
      la0, la1, lb0, lb1, kbeg, (kend - kbeg + BK - 1) / BK, smem,
      [&](const u32x4* ah, const u32x4* al, const u32x4* bh, const u32x4* bl) {
        mma_tile_bf3<BM, BN, BK>(ah, al, bh, bl, acc);
      });
  float* out = ci.splits == 1
                   ? reinterpret_cast<float*>(L.ws + d.oP)
                   : reinterpret_cast<float*>(L.ws + d.oK) + static_cast<int64_t>(s) * d.m * d.r;
  store_tile<BM, BN>(out, d.r, tm * BM, tn * BN, d.m, d.r, acc);
}

template <typename GT, int BN, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void k_mv3(Launch L) {
  constexpr int BK = 32;
  __shared__ u32x4 smem[2 * bf_stage_cells<BM, BN, BK>()];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (local == 0 && threadIdx.x == 0) L.status[d.slot] = 0;
  const int per = ci.tx * ci.ty;
  const int s = local / per;
  int tm, tn;
  tile_order(local - s * per, ci.tx, ci.ty, tm, tn);
  const int kbeg = s * ci.klen;
  const int kend = min(d.n, kbeg + ci.klen);
  const bool full = VEC && (tm + 1) * BM <= d.m && (tn + 1) * BN <= d.r && (kend - kbeg) % BK == 0;
  if (full) mv3_body<GT, BN, VEC, true>(L, d, ci, s, tm, tn, kbeg, kend, smem);
  else mv3_body<GT, BN, VEC, false>(L, d, ci, s, tm, tn, kbeg, kend, smem);
}

// M V on 256 x 256 tiles: 8 wavefronts (2 x 4) of 128 x 64, two per SIMD.
// Against 128 x 128 tiles: a third less LDS traffic and half the
// split-bfloat16 conversion work per MFMA.
using WB = WGrid<256, 256, 2, 4>;
constexpr int kBigThreads = WB::NT;
// The same products on 256 x 192 tiles (8 wavefronts, 4 x 2, of 64 x 96)
// for ranks 129 .. 192: one column tile, so each element of M is loaded
// and split into bfloat16 planes once per product, where 128 x 64 tiles
// take it three times at r = 192 (M V on the 3B stack at r = 1/16: 4.7 ms
// against 6.4).
using WS = WGrid<256, 192, 4, 2>;

template <class W>
__device__ __forceinline__ void store_tile_w(float* out_, int64_t ld, int r0, int c0, int rmax,
                                             int cmax, const f32x16 (&acc)[W::FM][W::FN]) {
  gptr<float> out = to_global(out_);
#pragma unroll
  for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn) {
      const int col = c0 + W::col(fn);
      if (col >= cmax) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = r0 + W::row(fm, v);
        if (row < rmax) out[static_cast<int64_t>(row) * ld + col] = acc[fm][fn][v];
      }
    }
}

// Column maxima of |acc| over the tile's rows below rmax, as float bits (a
// non-finite entry gives at least the bits of +inf), into part[c0 + c] for
// the columns below cmax: lanes, then lane halves, then the wavefront rows
// through LDS.  Called by the whole block after the main loop's last
// barrier, when LDS is free.
template <class W>
__device__ __forceinline__ void store_colmax(uint32_t* part_, int r0, int c0, int rmax, int cmax,
                                             const f32x16 (&acc)[W::FM][W::FN], u32x4* smem) {
  uint32_t* red = reinterpret_cast<uint32_t*>(smem);   // [GM][BN]
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int fn = 0; fn < W::FN; ++fn) {
    uint32_t mx = 0;
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (r0 + W::row(fm, v) < rmax) mx = max(mx, __float_as_uint(acc[fm][fn][v]) & 0x7fffffffu);
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), 32)));
    if (lane < 32) red[W::wm() * W::BN + W::col(fn)] = mx;
  }
  __syncthreads();
  gptr<uint32_t> part = to_global(part_);
  for (int c = threadIdx.x; c < W::BN; c += W::NT) {
    uint32_t mx = 0;
#pragma unroll
    for (int g = 0; g < W::GM; ++g) mx = max(mx, red[g * W::BN + c]);
    if (c0 + c < cmax) part[c0 + c] = mx;
  }
}

// The sliced Gram's maxima slot of row tile tm (see q_fused_max).
__device__ __forceinline__ uint32_t* colmax_slot(const Launch& L, const MatDesc& d, int tm) {
  return reinterpret_cast<uint32_t*>(L.ws + d.oQ + q_max_off(max(d.m, d.n), d.r)) + tm * q_cols(d.r);
}

template <class W, typename GT, bool VEC, bool FULL>
__device__ __forceinline__ void mv3b_body(const Launch& L, const MatDesc& d, const ClassInfo& ci,
                                          int s, int tm, int tn, int kbeg, int kend, u32x4* smem) {
  constexpr int BK = 32;
  const SrcM<GT> sm(static_cast<const GT*>(d.G), d.R);
  LoadKC<W::BM, BK, VEC, false, SrcM<GT>, W::NT> la(sm, d.n, tm * W::BM, d.m, kend);
  const u32x4* vt = reinterpret_cast<const u32x4*>(L.ws + d.oH);
  const LoadDma<W::BN, BK, W::NT> lb{vt, vt + static_cast<int64_t>(d.r) * plane_pitch(d.n) / 8, d.r,
                                      tn * W::BN, d.r};
  f32x16 acc[W::FM][W::FN];
  zero_acc(acc);
  pipeline_bf_dma<W::BM, W::BN, BK, FULL>(
      la, lb, kbeg, (kend - kbeg + BK - 1) / BK, smem,
      [&](const u32x4* ah, const u32x4* al, const u32x4* bh, const u32x4* bl) {
        mma_tile_bf3w<W, BK>(ah, al, bh, bl, acc);
      });
  float* out = ci.splits == 1
                   ? reinterpret_cast<float*>(L.ws + d.oP)
                   : reinterpret_cast<float*>(L.ws + d.oK) + static_cast<int64_t>(s) * d.m * d.r;
  store_tile_w<W>(out, d.r, tm * W::BM, tn * W::BN, d.m, d.r, acc);
  if (q_fused_max(d.oQ, ci.splits, ci.tx))
    store_colmax<W>(colmax_slot(L, d, tm), tm * W::BM, tn * W::BN, d.m, d.r, acc, smem);
}

template <class W, typename GT, bool VEC>
__device__ __forceinline__ void mv3b_kernel(const Launch& L, u32x4* smem) {
  constexpr int BK = 32;
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (local == 0 && threadIdx.x == 0) L.status[d.slot] = 0;
  const int per = ci.tx * ci.ty;
  const int s = local / per;
  int tm, tn;
  tile_order(local - s * per, ci.tx, ci.ty, tm, tn);
  const int kbeg = s * ci.klen;
  const int kend = min(d.n, kbeg + ci.klen);
  const bool full = VEC && (tm + 1) * W::BM <= d.m && (tn + 1) * W::BN <= d.r &&
                    (kend - kbeg) % BK == 0;
  if (full) mv3b_body<W, GT, VEC, true>(L, d, ci, s, tm, tn, kbeg, kend, smem);
  else mv3b_body<W, GT, VEC, false>(L, d, ci, s, tm, tn, kbeg, kend, smem);
}

template <typename GT, bool VEC>
__global__ __launch_bounds__(kBigThreads) void k_mv3b(Launch L) {
  __shared__ u32x4 smem[2 * bf_stage_cells<WB::BM, WB::BN, 32>()];
  mv3b_kernel<WB, GT, VEC>(L, smem);
}

template <typename GT, bool VEC>
__global__ __launch_bounds__(WS::NT) void k_mv3s(Launch L) {
  __shared__ u32x4 smem[2 * bf_stage_cells<WS::BM, WS::BN, 32>()];
  mv3b_kernel<WS, GT, VEC>(L, smem);
}

// M^T U on the same tiles (output rows: n, columns: r).
template <class W, typename GT, bool VEC, bool FULL>
__device__ __forceinline__ void mtu3b_body(const Launch& L, const MatDesc& d, const ClassInfo& ci,
                                           int s, int tm, int tn, int kbeg, int kend, u32x4* smem) {
  constexpr int BK = 32;
  const SrcM<GT> sm(static_cast<const GT*>(d.G), d.R);
  LoadXC<W::BM, BK, VEC, SrcM<GT>, W::NT> la(sm, d.n, tm * W::BM, d.n, kend);
  const u32x4* ut = reinterpret_cast<const u32x4*>(L.ws + d.oH);
  const LoadDma<W::BN, BK, W::NT> lb{ut, ut + static_cast<int64_t>(d.r) * plane_pitch(d.m) / 8, d.r,
                                      tn * W::BN, d.r};
  f32x16 acc[W::FM][W::FN];
  zero_acc(acc);
  pipeline_bf_dma<W::BM, W::BN, BK, FULL>(
      la, lb, kbeg, (kend - kbeg + BK - 1) / BK, smem,
      [&](const u32x4* ah, const u32x4* al, const u32x4* bh, const u32x4* bl) {
        mma_tile_bf3w<W, BK>(ah, al, bh, bl, acc);
      });
  float* out = ci.splits == 1
                   ? reinterpret_cast<float*>(L.ws + d.oW)
                   : reinterpret_cast<float*>(L.ws + d.oK) + static_cast<int64_t>(s) * d.n * d.r;
  store_tile_w<W>(out, d.r, tm * W::BM, tn * W::BN, d.n, d.r, acc);
  if (q_fused_max(d.oQ, ci.splits, ci.tx))
    store_colmax<W>(colmax_slot(L, d, tm), tm * W::BM, tn * W::BN, d.n, d.r, acc, smem);
}

template <class W, typename GT, bool VEC>
__device__ __forceinline__ void mtu3b_kernel(const Launch& L, u32x4* smem) {
  constexpr int BK = 32;
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int per = ci.tx * ci.ty;
  const int s = local / per;
  int tm, tn;
  tile_order(local - s * per, ci.tx, ci.ty, tm, tn);
  const int kbeg = s * ci.klen;
  const int kend = min(d.m, kbeg + ci.klen);
  const bool full = VEC && (tm + 1) * W::BM <= d.n && (tn + 1) * W::BN <= d.r &&
                    (kend - kbeg) % BK == 0;
  if (full) mtu3b_body<W, GT, VEC, true>(L, d, ci, s, tm, tn, kbeg, kend, smem);
  else mtu3b_body<W, GT, VEC, false>(L, d, ci, s, tm, tn, kbeg, kend, smem);
}

template <typename GT, bool VEC>
__global__ __launch_bounds__(kBigThreads) void k_mtu3b(Launch L) {
  __shared__ u32x4 smem[2 * bf_stage_cells<WB::BM, WB::BN, 32>()];
  mtu3b_kernel<WB, GT, VEC>(L, smem);
}

template <typename GT, bool VEC>
__global__ __launch_bounds__(WS::NT) void k_mtu3s(Launch L) {
  __shared__ u32x4 smem[2 * bf_stage_cells<WS::BM, WS::BN, 32>()];
  mtu3b_kernel<WS, GT, VEC>(L, smem);
}

template <typename GT, int BN, bool VEC, bool FULL>
__device__ __forceinline__ void mtu3_body(const Launch& L, const MatDesc& d, const ClassInfo& ci,
                                          int s, int tm, int tn, int kbeg, int kend, u32x4* smem) {
  constexpr int BK = 32;
  const SrcM<GT> sm(static_cast<const GT*>(d.G), d.R);
  LoadXC<BM, BK, VEC, SrcM<GT>> la0(sm, d.n, tm * BM, d.n, kend), la1 = la0;
  // U^T planes (r rows of plane_pitch(m), zero past column m): cells of 8
  // consecutive rows of U
  const uint16_t* ut = reinterpret_cast<const uint16_t*>(L.ws + d.oH);
  LoadPl<BN, BK> lb0(ut, ut + static_cast<int64_t>(d.r) * plane_pitch(d.m), d.r, tn * BN, d.r),
      lb1 = lb0;
  f32x16 acc[Warps<BM, BN>::FM][Warps<BM, BN>::FN];
  zero_acc(acc);
  pipeline2_bf<BM, BN, BK, FULL>(
      la0, la1, lb0, lb1, kbeg, (kend - kbeg + BK - 1) / BK, smem,
      [&](const u32x4* ah, const u32x4* al, const u32x4* bh, const u32x4* bl) {
        mma_tile_bf3<BM, BN, BK>(ah, al, bh, bl, acc);
      });
  float* out = ci.splits == 1
                   ? reinterpret_cast<float*>(L.ws + d.oW)
                   : reinterpret_cast<float*>(L.ws + d.oK) + static_cast<int64_t>(s) * d.n * d.r;
  store_tile<BM, BN>(out, d.r, tm * BM, tn * BN, d.n, d.r, acc);
}

template <typename GT, int BN, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void k_mtu3(Launch L) {
  constexpr int BK = 32;
  __shared__ u32x4 smem[2 * bf_stage_cells<BM, BN, BK>()];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int per = ci.tx * ci.ty;
  const int s = local / per;
  int tm, tn;
  tile_order(local - s * per, ci.tx, ci.ty, tm, tn);
  const int kbeg = s * ci.klen;
  const int kend = min(d.m, kbeg + ci.klen);
  const bool full = VEC && (tm + 1) * BM <= d.n && (tn + 1) * BN <= d.r && (kend - kbeg) % BK == 0;
  if (full) mtu3_body<GT, BN, VEC, true>(L, d, ci, s, tm, tn, kbeg, kend, smem);
  else mtu3_body<GT, BN, VEC, false>(L, d, ci, s, tm, tn, kbeg, kend, smem);
}

// Fused X / R update on 256 x 128 tiles: 8 wavefronts (4 x 2) of 64 x 64,
// two per SIMD, each holding both products (U Vbar^T, U W^T).  The rank-r
// factors come as split-bfloat16 planes written by k_split_n and are copied
// straight into LDS.
constexpr int kEpiBatch = 32;   // epilogue elements per lane loaded before a batch's stores
using WE = WGrid<256, 128, 4, 2>;

template <typename GT, bool VEC, bool FULL>
__device__ __forceinline__ void epi3b_body(const Launch& L, const MatDesc& d, int tm, int tn,
                                           u32x4* smem) {
  constexpr int BK = 32;
  static_assert(kPlaneK % BK == 0, "planes hold whole reduction tiles");
  constexpr int CA = BfShape<WE::BM, BK>::CELLS, CB = BfShape<WE::BN, BK>::CELLS;
  constexpr int STAGE = 2 * (CA + 2 * CB);
  // split-bfloat16 planes of U (m rows), W and Vbar (n rows), plane_cell_r
  // order, zero past column r
  const int rq = plane_pitch(d.r);
  const u32x4* pu = reinterpret_cast<const u32x4*>(L.ws + d.oE);
  const int64_t cu = static_cast<int64_t>(d.m) * (rq / 8), cn = static_cast<int64_t>(d.n) * (rq / 8);
  const u32x4* pw = pu + 2 * cu;
  const u32x4* pv = pw + 2 * cn;
  const LoadDma<WE::BM, BK, WE::NT> la{pu, pu + cu, d.m, tm * WE::BM, d.m};
  const LoadDma<WE::BN, BK, WE::NT> lv{pv, pv + cn, d.n, tn * WE::BN, d.n};
  const LoadDma<WE::BN, BK, WE::NT> lw{pw, pw + cn, d.n, tn * WE::BN, d.n};
  f32x16 ax[WE::FM][WE::FN], ar[WE::FM][WE::FN];
  zero_acc(ax);
  zero_acc(ar);
  // stage layout: A hi, A lo, V hi, V lo, W hi, W lo; double-buffered: the
  // next tile's copies run during this tile's MFMAs and are waited for at
  // the barrier that ends it
  auto issue = [&](int k0, u32x4* b) {
    la.issue(k0, b, b + CA);
    lv.issue(k0, b + 2 * CA, b + 2 * CA + CB);
    lw.issue(k0, b + 2 * CA + 2 * CB, b + 2 * CA + 3 * CB);
  };
  const int nk = rq / BK;
  issue(0, smem);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) issue((kt + 1) * BK, smem + ((kt + 1) & 1) * STAGE);
    const u32x4* b = smem + (kt & 1) * STAGE;
    mma_tile_bf3w2<WE, BK>(b, b + CA, b + 2 * CA, b + 2 * CA + CB, b + 2 * CA + 2 * CB,
                           b + 2 * CA + 3 * CB, ax, ar);
    __syncthreads();
  }
  update_epilogue<WE, GT, FULL, kEpiBatch>(L, d, tm * WE::BM, tn * WE::BN, ax, ar);
}

template <typename GT, bool VEC>
__global__ __launch_bounds__(kBigThreads) void k_epi3b(Launch L) {
  constexpr int BK = 32;
  constexpr int STAGE = 2 * (BfShape<WE::BM, BK>::CELLS + 2 * BfShape<WE::BN, BK>::CELLS);
  __shared__ u32x4 smem[2 * STAGE];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  int tm, tn;
  tile_order(local, ci.tx, ci.ty, tm, tn);
  const bool full = (tm + 1) * WE::BM <= d.m && (tn + 1) * WE::BN <= d.n;
  if (full) epi3b_body<GT, VEC, true>(L, d, tm, tn, smem);
  else epi3b_body<GT, VEC, false>(L, d, tm, tn, smem);
}

template <typename GT, int BN, bool VEC, bool FULL>
__device__ __forceinline__ void epi3_body(const Launch& L, const MatDesc& d, int tm, int tn,
                                          u32x4* smem) {
  constexpr int BK = 32;
  constexpr int CA = BfShape<BM, BK>::CELLS, CB = BfShape<BN, BK>::CELLS;
  constexpr int STAGE = 2 * (CA + 2 * CB);
  using Wp = Warps<BM, BN>;
  const float* U = reinterpret_cast<const float*>(L.ws + d.oB);
  const float* Wf = reinterpret_cast<const float*>(L.ws + d.oW);
  LoadKC<BM, BK, VEC, false, SrcF32> la0(SrcF32{U}, d.r, tm * BM, d.m, d.r), la1 = la0;
  LoadKC<BN, BK, VEC, false, SrcF32> lv0(SrcF32{d.V}, d.r, tn * BN, d.n, d.r), lv1 = lv0;
  LoadKC<BN, BK, VEC, false, SrcF32> lw0(SrcF32{Wf}, d.r, tn * BN, d.n, d.r), lw1 = lw0;
  f32x16 ax[Wp::FM][Wp::FN], ar[Wp::FM][Wp::FN];
  zero_acc(ax);
  zero_acc(ar);
  // stage layout: A hi, A lo, V hi, V lo, W hi, W lo.  Three-stage pipeline:
  // LDS holds tile kt, one register set tile kt+1, the other has tile
  // kt+2's loads in flight (the operands are read from L2, and one tile of
  // split-bfloat16 MFMAs is too short to hide that latency).
  auto store = [&](auto& la, auto& lv, auto& lw, int st) {
    u32x4* b = smem + st * STAGE;
    la.store_bf(reinterpret_cast<u32x2*>(b), reinterpret_cast<u32x2*>(b + CA));
    lv.store_bf(reinterpret_cast<u32x2*>(b + 2 * CA), reinterpret_cast<u32x2*>(b + 2 * CA + CB));
    lw.store_bf(reinterpret_cast<u32x2*>(b + 2 * CA + 2 * CB),
                reinterpret_cast<u32x2*>(b + 2 * CA + 3 * CB));
  };
  auto load = [&](auto& la, auto& lv, auto& lw, int k0) {
    la.template load<FULL>(k0);
    lv.template load<FULL>(k0);
    lw.template load<FULL>(k0);
  };
  auto compute = [&](int st) {
    u32x4* b = smem + st * STAGE;
    mma_tile_bf3<BM, BN, BK>(b, b + CA, b + 2 * CA, b + 2 * CA + CB, ax);
    mma_tile_bf3<BM, BN, BK>(b, b + CA, b + 2 * CA + 2 * CB, b + 2 * CA + 3 * CB, ar);
  };
  const int nk = (d.r + BK - 1) / BK;
  load(la0, lv0, lw0, 0);
  if (nk > 1) load(la1, lv1, lw1, BK);
  store(la0, lv0, lw0, 0);
  __syncthreads();
  const int pairs = nk >> 1;
  for (int p = 0; p < pairs; ++p) {
    const int kt = 2 * p;
    const bool more0 = kt + 2 < nk;
    if (more0) load(la0, lv0, lw0, (kt + 2) * BK);
    compute(0);
    store(la1, lv1, lw1, 1);
    __syncthreads();
    if (kt + 3 < nk) load(la1, lv1, lw1, (kt + 3) * BK);
    compute(1);
    if (more0) store(la0, lv0, lw0, 0);
    __syncthreads();
  }
  if (nk & 1) compute(0);
  update_epilogue<WGrid<BM, BN, 2, 2>, GT, FULL>(L, d, tm * BM, tn * BN, ax, ar);
}

template <typename GT, int BN, bool VEC>
__global__ __launch_bounds__(kThreads) void k_epi3(Launch L) {
  constexpr int BK = 32;
  constexpr int STAGE = 2 * (BfShape<BM, BK>::CELLS + 2 * BfShape<BN, BK>::CELLS);
  __shared__ u32x4 smem[2 * STAGE];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  int tm, tn;
  tile_order(local, ci.tx, ci.ty, tm, tn);
  const bool full = VEC && (tm + 1) * BM <= d.m && (tn + 1) * BN <= d.n && d.r % BK == 0;
  if (full) epi3_body<GT, BN, VEC, true>(L, d, tm, tn, smem);
  else epi3_body<GT, BN, VEC, false>(L, d, tm, tn, smem);
}

template <class K>
hipError_t go(K kernel, const Launch& L, hipStream_t st, int threads = kThreads, int grid = 0) {
  if (L.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(grid > 0 ? grid : L.total), dim3(threads), 0, st, L);
  return hipGetLastError();
}

}  // namespace

#define DION_PICK(K, GT, BNV, VECV) \
  (math ? go(K##3<GT, BNV, VECV>, L, st) : go(K<GT, BNV, VECV>, L, st))

#define DION_DISPATCH(K)                                                         \
  if (gdtype == 0) {                                                             \
    if (bn == 128) return vec ? DION_PICK(K, float, 128, true) : DION_PICK(K, float, 128, false); \
    return vec ? DION_PICK(K, float, 64, true) : DION_PICK(K, float, 64, false);  \
  }                                                                              \
  if (bn == 128) return vec ? DION_PICK(K, uint16_t, 128, true) : DION_PICK(K, uint16_t, 128, false); \
  return vec ? DION_PICK(K, uint16_t, 64, true) : DION_PICK(K, uint16_t, 64, false);

hipError_t launch_mv(const Launch& L, int gdtype, int bn, bool vec, int math, hipStream_t st) {
  if (bn == 192) {   // split-bfloat16 only
    constexpr int T = WS::NT;
    if (gdtype == 0)
      return vec ? go(k_mv3s<float, true>, L, st, T) : go(k_mv3s<float, false>, L, st, T);
    return vec ? go(k_mv3s<uint16_t, true>, L, st, T) : go(k_mv3s<uint16_t, false>, L, st, T);
  }
  if (bn == 256) {   // split-bfloat16 only
    constexpr int T = kBigThreads;
    if (gdtype == 0)
      return vec ? go(k_mv3b<float, true>, L, st, T) : go(k_mv3b<float, false>, L, st, T);
    return vec ? go(k_mv3b<uint16_t, true>, L, st, T) : go(k_mv3b<uint16_t, false>, L, st, T);
  }
  DION_DISPATCH(k_mv)
}

hipError_t launch_mtu(const Launch& L, int gdtype, int bn, bool vec, int math, hipStream_t st) {
  if (bn == 192) {   // split-bfloat16 only
    constexpr int T = WS::NT;
    if (gdtype == 0)
      return vec ? go(k_mtu3s<float, true>, L, st, T) : go(k_mtu3s<float, false>, L, st, T);
    return vec ? go(k_mtu3s<uint16_t, true>, L, st, T) : go(k_mtu3s<uint16_t, false>, L, st, T);
  }
  if (bn == 256) {   // split-bfloat16 only
    constexpr int T = kBigThreads;
    if (gdtype == 0)
      return vec ? go(k_mtu3b<float, true>, L, st, T) : go(k_mtu3b<float, false>, L, st, T);
    return vec ? go(k_mtu3b<uint16_t, true>, L, st, T) : go(k_mtu3b<uint16_t, false>, L, st, T);
  }
  DION_DISPATCH(k_mtu)
}

hipError_t launch_gram(const Launch& L, int bg, bool vec, hipStream_t st) {
  if (L.gate >= kGateRetry) {   // gated (only some matrices need it): a capped grid
    const int g = gated_grid(L.total);
    return vec ? go(k_gram_gated<64, true>, L, st, kThreads, g)
               : go(k_gram_gated<64, false>, L, st, kThreads, g);
  }
  if (bg == 128) return vec ? go(k_gram<128, true>, L, st) : go(k_gram<128, false>, L, st);
  return vec ? go(k_gram<64, true>, L, st) : go(k_gram<64, false>, L, st);
}

hipError_t launch_trmm(const Launch& L, int bn, bool vec, int math, hipStream_t st) {
  if (math) {
    if (bn == 128) return vec ? go(k_trmm6<128, true>, L, st) : go(k_trmm6<128, false>, L, st);
    return vec ? go(k_trmm6<64, true>, L, st) : go(k_trmm6<64, false>, L, st);
  }
  if (bn == 128) return vec ? go(k_trmm<128, true>, L, st) : go(k_trmm<128, false>, L, st);
  return vec ? go(k_trmm<64, true>, L, st) : go(k_trmm<64, false>, L, st);
}

hipError_t launch_epi(const Launch& L, int gdtype, int bn, bool vec, int math, hipStream_t st) {
  if (bn == 256) {   // split-bfloat16 only: 256 x 128 tiles
    constexpr int T = kBigThreads;
    if (gdtype == 0)
      return vec ? go(k_epi3b<float, true>, L, st, T) : go(k_epi3b<float, false>, L, st, T);
    return vec ? go(k_epi3b<uint16_t, true>, L, st, T) : go(k_epi3b<uint16_t, false>, L, st, T);
  }
  DION_DISPATCH(k_epi)
}

}  // namespace dion
