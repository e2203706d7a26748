// Types shared by the host scheduler and the gfx950 kernels of libdion.
#pragma once
#include <stdint.h>

namespace dion {

// Block size of the float64 Cholesky / triangular-inverse kernels.
constexpr int kCholNB = 64;
// Split-bfloat16 planes of a factor are padded to a multiple of this many
// columns (the reduction tile of the kernels that read them).
constexpr int kPlaneK = 32;
inline __host__ __device__ int plane_pitch(int rows) { return (rows + kPlaneK - 1) / kPlaneK * kPlaneK; }
// The one-workgroup step of a small matrix (k_small): r <= kSmallMaxRank,
// and the factors P / U, W and V / Vbar, columns padded to rb (8 or 16) and
// V's rows to a multiple of 32, in kSmallFactorFloats float32 values of
// LDS: (m + n + n32) rb <= kSmallFactorFloats.
constexpr int kSmallMaxRank = 16;
constexpr int kSmallFactorFloats = 16384;
// Its resident form keeps M = G + R in LDS as well, read from global memory
// once, and pads the factors' rows to rb + 1: m (n + 1) + (m + n32) (rb + 1)
// <= kSmallResidentFloats.
constexpr int kSmallResidentFloats = 39680;
// Grouped launches carry at most this many shape classes.
constexpr int kMaxClasses = 8;
// Status words after the per-matrix ones and their union: the dataflow
// factorization's ticket counter, its count of finished tasks, and its
// abort word (a wait that ran out).
constexpr int kFlowWords = 3;

// Sliced Gram matrix.  Each column of the factor Q is scaled by a power of
// two 2^-e into (-1, 1) and written as kQDigits signed base-2^7 digits
// (int8 values in [-64, 64]): q = 2^e sum_t d_t 2^-(7 t + 6), with a
// remainder below 2^(e - 35).  The digits sit in fragment planes: plane t,
// 32-column block cb, 32-row block kb is one 1 KB fragment whose lane
// c + 32 h (16 bytes) holds rows 16 h .. 16 h + 15 of column c, the operand
// order of the 32 x 32 x 32 int8 MFMA.  Rows and columns past the factor
// are zero digits.  After the planes: per-slice column maxima (kQMaxSplits
// x qcols uint32, the bits of max |q|) and the column exponents (qcols
// int32), qcols = r rounded up to 32.
constexpr int kQDigits = 5;
constexpr int kQMaxSplits = 64;
constexpr int kQMaxRows = 256;       // fewest rows per column-maximum slice
constexpr int kQBadExp = 1 << 30;    // exponent of a column with a non-finite entry
inline __host__ __device__ int64_t q_cols(int r) { return (r + 31) / 32 * 32; }
inline __host__ __device__ int64_t q_rows(int rows) { return (static_cast<int64_t>(rows) + 31) / 32 * 32; }
// byte offsets inside the region, for factors of at most `rows_max` rows
inline __host__ __device__ int64_t q_max_off(int rows_max, int r) {
  return kQDigits * q_cols(r) * q_rows(rows_max);
}
inline __host__ __device__ int64_t q_exp_off(int rows_max, int r) {
  return q_max_off(rows_max, r) + kQMaxSplits * q_cols(r) * 4;
}
inline __host__ __device__ int64_t q_bytes(int rows_max, int r) { return q_exp_off(rows_max, r) + q_cols(r) * 4; }
// The split-bfloat16 256 x 256 kernels that produce P (M V) and W (M^T U)
// write the column maxima of each 256-row tile into slice `row tile` of the
// maxima themselves when the region exists, the reduction is not split and
// there are at most kQMaxSplits row tiles.
inline __host__ __device__ bool q_fused_max(int64_t oQ, int splits, int row_tiles) {
  return oQ != 0 && splits == 1 && row_tiles <= kQMaxSplits;
}

// One matrix as the kernels see it.  Workspace offsets are bytes from the
// workspace base.  rp = r rounded up to kCholNB.
struct MatDesc {
  float* X;
  const void* G;
  float* R;
  float* V;
  int32_t m, n, r, rp;
  int32_t slot;      // index in the caller's list = status word index
  int32_t pad0;
  int64_t oP;        // m x r      float32: P = M V
  int64_t oB;        // m x r      float32: U = orth(P)
  int64_t oC;        // max(m,n) x r float32: the first pass's output when
                     // orth takes a second CholeskyQR pass
  int64_t oW;        // n x r      float32: W = M^T U
  int64_t oS;        // splits x rp x rp float32: Gram partial sums
  int64_t oA;        // rp x rp    float64: Cholesky work matrix (upper blocks)
  int64_t oY;        // rp x rp    float64: T^{-T} (lower blocks)
  int64_t oD;        // kCholNB^2 + rp float64: diagonal-block inverse, diag(S)
  int64_t oN;        // r          float32: inverse column norms (Dion)
  int64_t oK;        // split-K partial products (float32)
  int64_t oE;        // split-bfloat16 planes (hi, then lo) of U (m rows), W
                     // and Vbar (n rows) for the fused update, row-major
                     // cells (plane_cell_r), pitch plane_pitch(r); 0 if unused
  int64_t oH;        // split-bfloat16 planes (hi, then lo) of V^T during
                     // M V, of U^T during M^T U: r x plane_pitch(rows)
                     // bfloat16 each in plane_cell_r order (cell = 8
                     // consecutive rows of V or U), zero past the last row;
                     // 0 without them
  int64_t oQ;        // sliced Gram: digit planes, column maxima and
                     // exponents of the factor being orthogonalized
                     // (layout above, rows_max = max(m, n)); 0 if unused
};

// Status word of a matrix (one int32 per matrix slot).  Bits 0-7 are the
// breakdown flags dion_status reports (DION_STATUS_*); any of them makes
// every later kernel of the step skip the matrix.  Bits 8-9 steer the
// factorization in progress (orth of P, then of W) and are cleared at its
// start:
//   kCtlTwo    the first CholeskyQR pass found a pivot ratio below
//              kRatioTwo: its triangular multiply runs in float64 into oC,
//              and a second pass (float64 Gram, float64 triangular
//              multiply) writes the result
//   kCtlRetry  the first pass found a pivot ratio below kRatioRetry or a
//              failed pivot: its factorization is abandoned and a shifted
//              one on a float64 Gram replaces it (kCtlTwo is set as well)
constexpr int32_t kStatusMask = 0xff;
constexpr int32_t kCtlTwo = 1 << 8;
constexpr int32_t kCtlRetry = 1 << 9;

// Which matrices a kernel of an orth() factorization works on (Launch.gate):
//   kGateAll    every matrix that has not broken down
//   kGateFirst  the first pass's Cholesky steps: not the matrices whose
//               factorization was abandoned (kCtlRetry)
//   kGateOne    the first pass's float32 triangular multiply: only the
//               matrices that take a single pass (no kCtlTwo)
//   kGateRetry  the shifted factorization: only kCtlRetry
//   kGateTwo    the float64 triangular multiply of the first pass and the
//               whole second pass: only kCtlTwo
enum Gate : int32_t { kGateAll = 0, kGateFirst = 1, kGateOne = 2, kGateRetry = 3, kGateTwo = 4 };

// Matrices with the same (m, n, r) form a class; inside one launch every
// matrix of a class owns `tiles` consecutive work items starting at `base`.
struct ClassInfo {
  int32_t first;   // first matrix (index into the grouped table)
  int32_t count;   // matrices in the class
  int32_t tiles;   // work items per matrix in this launch
  int32_t base;    // first work item of the class in this launch
  int32_t tx, ty;  // tile grid of one matrix (x: rows, y: cols)
  int32_t splits;  // split of the reduction dimension
  int32_t klen;    // reduction length per split (multiple of the K tile)
};

// Kernel argument block of one grouped launch (passed by value).
struct Launch {
  const MatDesc* table;   // device table, or nullptr to use `inl`
  MatDesc inl;            // the single matrix of a dion_step call
  char* ws;               // workspace base
  int32_t* status;        // status words (one per matrix slot)
  int32_t nclass;
  int32_t total;          // work items in the launch
  ClassInfo cls[kMaxClasses];
  float eta, beta;
  int32_t kb;             // Cholesky block step
  int32_t which;          // 0: factor P (m rows), 1: factor W (n rows)
  int32_t pass;           // CholeskyQR pass 1 or 2 (the factor it reads and writes)
  int32_t flag;           // status bit of this factorization
  int32_t mode;           // Cholesky trailing update: 1 look-ahead block row, 2 the rest
  int32_t gate;           // Gate: which matrices the launch works on
  int32_t retry;          // first pass: 1 = small pivots lead to a second pass or
                          // the shifted retry, 0 = they are breakdowns
  int32_t any_slot;       // status[any_slot]: the control bits of every matrix of
                          // the factorization in progress, OR-ed together (so
                          // that a gated launch no matrix needs ends at once)
};

}  // namespace dion
