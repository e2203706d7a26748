// Gram matrix S = Q^T Q of a CholeskyQR pass (orth() of the Orth-Dion
// page's equations 2 and 4) on the int8 matrix cores.
//
// A float32 column q_j scaled by 2^-e_j (the power of two just above
// max |q_j|) is a sum of kQDigits signed base-2^7 digits plus a remainder
// below 2^-35:  q_j = 2^e_j sum_t d_jt 2^-(7 t + 6).  Then
//   S_ij = 2^(e_i + e_j) sum_l 2^-(7 l + 12) sum_{a + b = l} D_ia . D_jb
// and every digit product sum D_ia . D_jb is an integer, summed exactly by
// the int32 accumulation of v_mfma_i32_32x32x32_i8.  Keeping the levels
// l <= kQDigits - 1 (15 digit products) forms each product q_ik q_jk to
// within 2^-30 max|q_i| max|q_j|: the terms d_a 2^-(7 a + 6) with a >= 1 are
// at most 2^-7a in size, so the dropped products (a + b >= kQDigits) and the remainders
// of the two columns add up to about 6 2^-35 in units of 2^(e_i + e_j) <=
// 4 max|q_i| max|q_j|.  Those errors come from rounding each entry to
// digits and add like independent roundings over the rows.  The levels
// are combined exactly in int64 and rounded once to float64; each level's
// int32 sum is moved out (added into the output) every kQFlushSteps steps,
// before it could overflow.
//
//   k_qmax    max |q_j| over row slices, as float bits (a non-finite entry
//             gives a maximum at or above the bits of +inf)
//   k_qslice  column exponents and the digit planes
//   k_gram8   upper-triangle 64 x 64 tiles of S from the digit planes
#include <math.h>

#include "device_common.h"
#include "launchers.h"

namespace dion {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// 2048 steps of 32 rows: a level adds at most kQDigits products of digits
// of magnitude <= 64 per row, 65536 * 5 * 4096 < 2^31.
constexpr int kQFlushSteps = 2048;

__device__ __forceinline__ int rows_max(const MatDesc& d) { return d.m > d.n ? d.m : d.n; }

// Work item (slice sp, 256-column group cg): the largest |q| bit pattern
// of each column over rows [sp klen, (sp + 1) klen).  Wavefront w takes
// rows w, w + 4, ..., lane l columns 256 cg + l + 64 j (j < 4), 8 rows per
// round with all 32 loads issued together (indices clamped into the matrix:
// a repeated row or column does not change a maximum, and columns past r
// are not stored); the 4 wavefronts combine through LDS.
__global__ __launch_bounds__(kThreads) void k_qmax(Launch L) {
  __shared__ uint32_t red[4][256];
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int rows = L.which == 0 ? d.m : d.n;
  const int groups = (d.r + 255) / 256;
  const int sp = local / groups, cg = local - sp * groups;
  gptr<const uint32_t> Q = to_global(reinterpret_cast<const uint32_t*>(first_src(L, d)));
  const int lane = threadIdx.x & 63, rg = threadIdx.x >> 6;
  int cc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cc[j] = min(cg * 256 + lane + 64 * j, d.r - 1);
  const int i0 = sp * ci.klen, i1 = min(rows, i0 + ci.klen);
  uint32_t mx[4] = {0, 0, 0, 0};
  for (int i = i0 + rg; i < i1; i += 32) {
    uint32_t v[8][4];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = static_cast<int64_t>(min(i + 4 * k, i1 - 1)) * d.r;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[k][j] = Q[row + cc[j]];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx[j] = max(mx[j], v[k][j] & 0x7fffffffu);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[rg][lane + 64 * j] = mx[j];
  __syncthreads();
  const int c = threadIdx.x, col = cg * 256 + c;
  if (col < d.r) {
    uint32_t* part = reinterpret_cast<uint32_t*>(L.ws + d.oQ + q_max_off(rows_max(d), d.r));
    part[static_cast<int64_t>(sp) * q_cols(d.r) + col] = max(max(red[0][c], red[1][c]), max(red[2][c], red[3][c]));
  }
}

// Work item (32-row block kb, group cg of 4 column blocks); wavefront w
// writes fragment (4 cg + w, kb) of every digit plane.  Lane c + 32 h takes
// rows 16 h .. 16 h + 15 of column 32 (4 cg + w) + c.  Consecutive work
// items read consecutive 512-byte spans of the same 32 rows.
__global__ __launch_bounds__(kThreads) void k_qslice(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
  const int rows = L.which == 0 ? d.m : d.n;
  const int ncb = static_cast<int>(q_cols(d.r) / 32), nkb = static_cast<int>(q_rows(rows) / 32);
  const int ncg = (ncb + 3) / 4;
  const int kb = local / ncg;
  const int cb = (local - kb * ncg) * 4 + (threadIdx.x >> 6);
  if (cb >= ncb) return;
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const int col = cb * 32 + c;
  const int rmax = rows_max(d);
  const char* region = L.ws + d.oQ;
  // Loads below use in-range indices (clamped) and discard what lies
  // outside, so that each group of them is issued at once.
  const int colc = min(col, d.r - 1);
  uint32_t mx = 0;
  {
    gptr<const uint32_t> part = to_global(reinterpret_cast<const uint32_t*>(region + q_max_off(rmax, d.r)));
    for (int sp = 0; sp < ci.splits; sp += 8) {
      uint32_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = part[static_cast<int64_t>(min(sp + j, ci.splits - 1)) * q_cols(d.r) + colc];
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = max(mx, v[j]);
    }
    if (col >= d.r) mx = 0;
  }
  const bool bad = mx >= 0x7f800000u;
  int e = 0;
  if (!bad && mx != 0) frexpf(__uint_as_float(mx), &e);   // max |q| < 2^e
  if (kb == 0 && h == 0)
    reinterpret_cast<int*>(L.ws + d.oQ + q_exp_off(rmax, d.r))[col] = bad ? kQBadExp : e;
  gptr<const float> Q = to_global(first_src(L, d));
  uint32_t w[kQDigits][4];
#pragma unroll
  for (int t = 0; t < kQDigits; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) w[t][j] = 0;
  const bool live = col < d.r && !bad;
  float qv[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) qv[b] = Q[static_cast<int64_t>(min(kb * 32 + 16 * h + b, rows - 1)) * d.r + colc];
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const int row = kb * 32 + 16 * h + b;
    const float q = live && row < rows ? qv[b] : 0.0f;
    // |y| < 1; every step below is exact in float32 (y keeps at most the
    // 24 significant bits of q; a y below 2^-126 loses only bits far
    // under the digits' reach)
    float y = ldexpf(q, -e);
#pragma unroll
    for (int t = 0; t < kQDigits; ++t) {
      const float up = ldexpf(1.0f, 7 * t + 6), down = ldexpf(1.0f, -(7 * t + 6));
      const float x = rintf(y * up);   // |x| <= 64
      y -= x * down;
      w[t][b >> 2] |= (static_cast<uint32_t>(static_cast<int>(x)) & 0xffu) << (8 * (b & 3));
    }
  }
  gptr<u32x4> planes = to_global(reinterpret_cast<u32x4*>(L.ws + d.oQ));
  const int64_t frag = (static_cast<int64_t>(cb) * nkb + kb) * 64 + lane;
  const int64_t tstride = static_cast<int64_t>(ncb) * nkb * 64;
#pragma unroll
  for (int t = 0; t < kQDigits; ++t) planes[t * tstride + frag] = u32x4{w[t][0], w[t][1], w[t][2], w[t][3]};
}

__device__ __forceinline__ void load_frags(gptr<const i32x4> pa, gptr<const i32x4> pb, int64_t tstride,
                                           int kb, i32x4 (&a)[kQDigits], i32x4 (&b)[kQDigits]) {
#pragma unroll
  for (int t = 0; t < kQDigits; ++t) {
    a[t] = pa[t * tstride + kb * 64];
    b[t] = pb[t * tstride + kb * 64];
  }
}

// acc[l] += sum over digit pairs a + b = l of D_a^T D_b (15 MFMAs).
__device__ __forceinline__ void digit_products(const i32x4 (&a)[kQDigits], const i32x4 (&b)[kQDigits],
                                               i32x16 (&acc)[kQDigits]) {
#pragma unroll
  for (int l = 0; l < kQDigits; ++l)
#pragma unroll
    for (int ta = 0; ta <= l; ++ta)
      acc[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ta], b[l - ta], acc[l], 0, 0, 0);
}
// The levels of one result entry, sum_l acc[l] 2^-(7 l + 12), combined
// exactly in int64 (|acc[l]| < 2^31, so the sum stays below 2^62) and
// rounded once to float64.
__device__ __forceinline__ double level_sum(const i32x16 (&acc)[kQDigits], int v) {
  int64_t x = 0;
#pragma unroll
  for (int l = 0; l < kQDigits; ++l) x += static_cast<int64_t>(acc[l][v]) << (7 * (kQDigits - 1 - l));
  return ldexp(static_cast<double>(x), -(7 * (kQDigits - 1) + 12));
}

// Partial Gram matrix S_s = Q[kbeg:kend]^T Q[kbeg:kend] on 64 x 64 upper-
// triangle tiles: four wavefronts of 32 x 32, each loading its own digit
// fragments straight into registers two steps ahead (no LDS).  On a diagonal
// tile the wavefront of rows 32.. and columns ..32 lies below the diagonal
// and does nothing (the factorization reads the upper triangle only).
// Two blocks per CU (at most 256 registers per lane).
__global__ __launch_bounds__(kThreads, 2) void k_gram8(Launch L) {
  MatDesc d;
  ClassInfo ci;
  int local;
  locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
  if (skipped(L, d)) return;
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (ti == tj && wm > wn) return;
  const int ncb = static_cast<int>(q_cols(d.r) / 32), nkb = static_cast<int>(q_rows(rows) / 32);
  const int cba = ti * 2 + wm, cbb = tj * 2 + wn;   // cba <= cbb
  if (cbb >= ncb) return;
  const int kbeg = s * ci.klen;
  const int kend = min(rows, kbeg + ci.klen);
  if (kend <= kbeg) return;
  const int kb0 = kbeg / 32, kb1 = (kend + 31) / 32;
  const int64_t tstride = static_cast<int64_t>(ncb) * nkb * 64;
  gptr<const i32x4> planes = to_global(reinterpret_cast<const i32x4*>(L.ws + d.oQ));
  gptr<const i32x4> pa = planes + static_cast<int64_t>(cba) * nkb * 64 + lane;
  gptr<const i32x4> pb = planes + static_cast<int64_t>(cbb) * nkb * 64 + lane;
  const int* qexp = reinterpret_cast<const int*>(L.ws + d.oQ + q_exp_off(rows_max(d), d.r));
  gptr<double> out = to_global(reinterpret_cast<double*>(L.ws + d.oS) + static_cast<int64_t>(s) * d.rp * d.rp);
  const int col = cbb * 32 + (lane & 31);
  const int ej = qexp[min(col, d.r - 1)];
  i32x4 a[kQDigits], b[kQDigits], a1[kQDigits], b1[kQDigits];
  load_frags(pa, pb, tstride, kb0, a, b);
  load_frags(pa, pb, tstride, min(kb0 + 1, kb1 - 1), a1, b1);
  for (int c0 = kb0; c0 < kb1; c0 += kQFlushSteps) {
    const int c1 = min(kb1, c0 + kQFlushSteps);
    i32x16 acc[kQDigits];
#pragma unroll
    for (int l = 0; l < kQDigits; ++l)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[l][v] = 0;
    for (int kb = c0; kb < c1; ++kb) {
      i32x4 an[kQDigits], bn[kQDigits];
      load_frags(pa, pb, tstride, min(kb + 2, kb1 - 1), an, bn);   // the last steps reload the last
      digit_products(a, b, acc);
#pragma unroll
      for (int t = 0; t < kQDigits; ++t) {
        a[t] = a1[t];
        b[t] = b1[t];
        a1[t] = an[t];
        b1[t] = bn[t];
      }
    }
    // this interval's share of S, into the tile's own entries of S_s
    // (written by the first interval, added to by later ones)
    if (col < d.r) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // 32 x 32 MFMA result: lane l, register v holds row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
        const int row = cba * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < d.r) {
          const int ei = qexp[row];
          double x = level_sum(acc, v);
          x = ei == kQBadExp || ej == kQBadExp ? __builtin_nan("") : ldexp(x, ei + ej);
          const int64_t o = static_cast<int64_t>(row) * d.rp + col;
          out[o] = c0 == kb0 ? x : out[o] + x;
        }
      }
    }
  }
}

template <class K>
hipError_t go(K kernel, const Launch& L, hipStream_t st) {
  if (L.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(L.total), dim3(kThreads), 0, st, L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qmax(const Launch& L, hipStream_t st) { return go(k_qmax, L, st); }
hipError_t launch_qslice(const Launch& L, hipStream_t st) { return go(k_qslice, L, st); }
hipError_t launch_gram8(const Launch& L, hipStream_t st) { return go(k_gram8, L, st); }

}  // namespace dion
