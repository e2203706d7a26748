/*
 * libdion — one Dion / Orth-Dion optimizer step on an AMD MI355X (gfx950).
 *
 * The step is the one written out on the "Orth-Dion" documentation page
 * (junaidaliop.github.io, zij/math/orthdion): its equation block and the
 * symbol list below it.  For a weight matrix X (m x n) with gradient G,
 * error-feedback residual R (both m x n) and warm start V (n x r):
 *
 *   M    = G + R                       buffer
 *   U    = orth(M V)                   one warm-started power-iteration step
 *   W    = M^T U                       right factor
 *   Vbar = orth(W)                     Orth-Dion
 *        = W diag(1 / ||w_j||_2)       Dion (the page's closing remark: column
 *                                      normalization in place of orth)
 *   X   <- X - eta U Vbar^T
 *   R   <- beta (M - U W^T)            (U^T M = W^T, so W is reused)
 *   V   <- Vbar                        warm start of the next step
 *
 * orth(A) is the Q factor of the thin QR factorization A = Q T whose upper
 * triangular T has a positive diagonal (the symbol list defines orth as the
 * QR orthonormalization of the column space; the positive diagonal makes Q
 * unique for a full-rank A).  The library computes it by CholeskyQR: a
 * float64 Gram matrix (assembled from exact int8 digit products on the
 * matrix cores by default, see DION_GRAM_F64), a blocked float64 Cholesky
 * factorization S = T^T T that also yields T^{-T}, and the product
 * A T^{-1} on the matrix cores.  The pivots tell how well-conditioned A is
 * (pivot j over S_jj is about 1 / kappa^2 at worst):
 *   - kappa below about 1e3 (every pivot ratio >= 1e-6): that one pass;
 *   - up to about 1e4: a second pass on the result (CholeskyQR2) with a
 *     float64 Gram matrix and float64 products;
 *   - beyond that, or a failed pivot: the first pass is redone with a
 *     diagonal shift on a float64 Gram matrix (shifted CholeskyQR), then
 *     the second pass follows.
 * The choice is made per matrix on the device.  A factor that is rank-
 * deficient to float32 accuracy (the second pass finds a pivot ratio below
 * 2 r 2^-48) is a breakdown (see below).
 *
 * Conventions for every entry point:
 *   - All functions are extern "C"; no C++ exception crosses the boundary.
 *   - Matrices are dense row-major (C order) with no padding: element (i, j)
 *     of an a x b matrix is at p[i * b + j].  X, R, V are float32; G is
 *     float32 or bfloat16 (raw 16-bit patterns), chosen by g_dtype.
 *   - All pointers passed as matrices or workspace are DEVICE pointers on the
 *     current HIP device.  The caller owns them.  X, R and V are updated in
 *     place; G is only read.  X, G, R, V and the workspace must not overlap.
 *     They need natural alignment (4 bytes; 2 for bfloat16 G); 16-byte
 *     aligned pointers with a column count divisible by 4 take the vector
 *     load path.
 *   - stream is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued: the calls return before the GPU finishes and never
 *     synchronize the host, except dion_status, dion_plan_destroy and
 *     dion_plan_timing_enable / _read, which wait for work they must read
 *     or free.  Buffers must stay valid until the enqueued work completes.
 *   - Argument errors are reported synchronously, before any HIP call is
 *     made, and leave every buffer untouched.
 *   - A numerical breakdown (orth of a factor that is rank-deficient to
 *     float32 accuracy or not finite; a zero or non-finite column norm for
 *     Dion) can only be seen on the device.  It is recorded in a status
 *     word inside the workspace, and every later kernel of that matrix skips
 *     its writes, so X, R and V of that matrix keep their previous contents
 *     bit for bit.  Read it with dion_status.
 */
#ifndef LIBDION_DION_H_
#define LIBDION_DION_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define DION_OK               0
#define DION_ERR_INVALID_ARG (-1)  /* null pointer, bad size, rank, variant, dtype, non-finite eta/beta */
#define DION_ERR_WORKSPACE   (-2)  /* workspace missing or smaller than required */
#define DION_ERR_HIP         (-3)  /* a HIP runtime call or kernel launch failed */
#define DION_ERR_BREAKDOWN   (-4)  /* (dion_status only) numerical breakdown on the device */

/* Right-factor rule: equation 4 of the Orth-Dion page, or Dion's column
 * normalization. */
#define DION_VARIANT_DION 0
#define DION_VARIANT_ORTH 1
#define DION_VARIANT_MASK 0xff

/* Arithmetic of the three m x n x r products (P = M V, W = M^T U and the
 * X / R update), OR-ed into the `variant` argument of every entry point.
 * DION_MATH_F32 (default): float32 MFMA products, float32 accumulation.
 * DION_MATH_BF16X3: each float32 operand x is split into bfloat16
 *   hi = bf16(x) and lo = bf16(x - hi), and a product is taken as
 *   hi*hi + hi*lo + lo*hi on the bfloat16 matrix cores with float32
 *   accumulation: relative product error up to 2^-16 instead of 2^-24, at
 *   about five times the float32 matrix rate.  orth() (the Gram matrix
 *   below, the triangular product in float32) is unaffected. */
#define DION_MATH_F32     0x000
#define DION_MATH_BF16X3  0x100
#define DION_MATH_MASK    0x100

/* Gram matrix S = Q^T Q of orth()'s CholeskyQR pass (orth() of equations 2
 * and 4 of the Orth-Dion page), OR-ed into `variant` like the math mode.
 * Default: each float32 column q_j of Q is scaled by a power of two into
 *   (-1, 1) and written as five signed base-128 digits (int8); S is
 *   assembled in float64 from the 15 leading digit products, each summed
 *   exactly in int32 on the int8 matrix cores.  Each product q_ik q_jk
 *   enters S with an error below 2^-30 max|q_i| max|q_j| (the digits'
 *   remainder and the dropped digit products); over many rows these errors
 *   add like independent roundings (measured: Gram entries within 2e-10 of
 *   sqrt(S_ii S_jj) of the float64 Gram).  A non-finite entry of Q makes
 *   its row and column of S NaN, a breakdown of the factorization.
 * DION_GRAM_F64: float32 products summed in float64 on the float64 matrix
 *   cores (products exact, float64 rounding only). */
#define DION_GRAM_F64     0x400

/* Schedule of small matrices.  By default a matrix with r <= 16 whose
 * step is small (factors P, W and V within 64 KB once their columns are
 * padded to 8 or 16, and m n r <= 2^21) takes the whole step in one
 * workgroup of one launch: float32 products, float64 Gram matrix and
 * Cholesky, float64 triangular products (the math mode does not apply to
 * it).  DION_SCHED_GROUPED, OR-ed into `variant`, sends every matrix
 * through the grouped multi-launch schedule instead.  Sharded plans always
 * use the grouped schedule. */
#define DION_SCHED_GROUPED 0x800

/* Row-sharded step (FSDP layout; the sharded setting the Dion and
 * Orth-Dion abstracts motivate).  OR DION_SHARDED into the variant of
 * dion_plan_create for a plan whose matrices are the local row shards of
 * the global matrices: matrix i is rows [a_i, a_i + m_i) of some global
 * X, G, R (m_i x n), and every shard of one global matrix holds its own
 * copy of the same V (n x r).  dion_plan_shard_stage then runs the step in
 * three stages; between them the caller sums one exchange buffer over all
 * shards of each global matrix (an all-reduce across GPUs; with a single
 * shard there is nothing to do) and writes the sum back into every shard's
 * buffer:
 *   stage 0: P_i = M_i V and the local Gram partial P_i^T P_i
 *            -> exchange DION_SHARD_GRAM: float64, rp x rp row-major
 *               (rp = r rounded up to 64); stage 1 reads only the upper
 *               triangle of its leading r x r block
 *   stage 1: T from the summed Gram matrix, U_i = P_i T^{-1},
 *            W_i = M_i^T U_i (one CholeskyQR pass: a further pass would
 *            need another exchange, so a pivot ratio below 1e-6 is a
 *            breakdown here; orth(W) in stage 2 takes every pass it needs)
 *            -> exchange DION_SHARD_W: float32, n x r row-major
 *   stage 2: Vbar from the summed W (computed identically on every shard),
 *            X_i and R_i updated, Vbar written into the shard's V.
 * Summed this way the shards' results equal one step on the global
 * matrices.  dion_plan_shard_buffer gives the byte offset (from the
 * workspace base) and size of exchange buffer `which` (DION_SHARD_*) of
 * matrix `index` (position in the plan's list).  Stage calls follow the
 * order 0, 1, 2 on one workspace and stream; the buffers are valid from
 * the end of the stage that writes them to the start of the next stage.
 * dion_plan_step also runs a sharded plan: all three stages without
 * exchange, i.e. each shard as a matrix of its own.  dion_step and
 * dion_step_batched reject DION_SHARDED (DION_ERR_INVALID_ARG).  Errors:
 * DION_ERR_INVALID_ARG for a null plan, a plan created without
 * DION_SHARDED, a stage outside 0..2, which outside DION_SHARD_*, an index
 * outside the list or a null output pointer; otherwise as dion_plan_step.
 * A shard may have fewer rows than r (only r <= n is required of it); the
 * global matrix needs at least r rows for its Gram matrix to be definite. */
#define DION_SHARDED      0x200
#define DION_SHARD_GRAM   0
#define DION_SHARD_W      1

/* Element type of G. */
#define DION_DTYPE_F32  0
#define DION_DTYPE_BF16 1

/* Per-matrix breakdown flags reported by dion_status (0 = step applied). */
#define DION_STATUS_ORTH_P   1   /* orth(M V) failed */
#define DION_STATUS_ORTH_W   2   /* orth(W) failed (Orth-Dion) */
#define DION_STATUS_COLNORM  4   /* zero or non-finite column norm (Dion) */

/* Upper bounds accepted by the library. */
#define DION_MAX_DIM   (1 << 20)      /* m, n */
#define DION_MAX_RANK  4096           /* r */

/* One matrix of a grouped step.  Device pointers, row-major, see above. */
typedef struct dion_matrix {
    float*       X;   /* m x n, updated in place */
    const void*  G;   /* m x n, float32 or bfloat16 per g_dtype, read only */
    float*       R;   /* m x n, updated in place */
    float*       V;   /* n x r, warm start in, Vbar out */
    int64_t      m, n, r;
} dion_matrix;

/* Opaque handle for a grouped step over a fixed list of matrices. */
typedef struct dion_plan dion_plan;

/* Library version as major * 10000 + minor * 100 + patch. */
int dion_version(void);

/* Static string for a return code (never NULL). */
const char* dion_error_string(int code);

/* Workspace bytes one dion_step call on an m x n matrix of rank r needs.
 * Returns 0 when the arguments are invalid. */
size_t dion_workspace_size(int64_t m, int64_t n, int64_t r, int variant, int g_dtype);

/* One step on one matrix (the equations at the top of this header).
 *   X, G, R, V: device pointers (see conventions); m, n >= 1; 1 <= r <= min(m, n).
 *   eta: learning rate, beta: error-feedback coefficient (finite floats).
 *   variant: DION_VARIANT_*; g_dtype: DION_DTYPE_*.
 *   workspace: device buffer of at least dion_workspace_size(...) bytes,
 *   16-byte aligned, owned by the caller; its contents need not be preserved
 *   between calls except for the status word read by dion_status.
 * Returns DION_OK once the work is enqueued, or an error code (nothing
 * enqueued for argument errors). */
int dion_step(float* X, const void* G, float* R, float* V,
              int64_t m, int64_t n, int64_t r, float eta, float beta,
              int variant, int g_dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/* dion_step for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid allocation): the
 * same step with the same kernels, its workspace taken from a scratch array
 * that the library holds on each GPU (32 MiB, kept until the process ends)
 * instead of a caller buffer.  No device memory is allocated or freed.
 * Shapes whose workspace (dion_workspace_size) exceeds 32 MiB are rejected
 * with DION_ERR_WORKSPACE before any HIP call (for example 1024 x 1024 at
 * rank 256, or 768 x 3072 at rank 192, fit; 2048 x 2048 at rank 512 does
 * not).  All calls on one GPU share its scratch, so calls that overlap on
 * one GPU (other streams, other threads) race; calls in stream order do
 * not.  status_out (optional, a device pointer to one int) receives the
 * matrix's status word when the step ends: its bits 0-7 are the
 * DION_STATUS_* flags (0: the step was applied); higher bits are internal.
 * Other arguments and errors as dion_step. */
int dion_step_noalloc(float* X, const void* G, float* R, float* V,
                      int64_t m, int64_t n, int64_t r, float eta, float beta,
                      int variant, int g_dtype, int* status_out, void* stream);

/* Grouped step: the same update applied to each matrix of a list (for
 * example all weight matrices of a model) with a handful of kernel launches
 * for the whole list.  The pages apply the step to every weight matrix
 * independently (Orth-Dion page, equation block, per matrix X); the nearest
 * thing they describe to running many of them together is the Dion3
 * abstract's megabatching.  Matrices may have different shapes.  Equivalent
 * to a dion_step call per matrix.  The matrix list is copied; the call
 * keeps an internal cache of plans keyed by the list, so repeating the same
 * list costs no host-side setup (a plan evicted from the cache is freed
 * once its last copy has completed, without waiting for it). */
size_t dion_workspace_size_batched(const dion_matrix* mats, int count,
                                   int variant, int g_dtype);
int dion_step_batched(const dion_matrix* mats, int count, float eta, float beta,
                      int variant, int g_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Explicit plan for a grouped step (what dion_step_batched caches).
 * dion_plan_create validates the list and builds the schedule on the host;
 * it allocates pinned host memory for the matrix table (no device memory).
 * dion_plan_step enqueues one grouped step: an asynchronous copy of the
 * table into the workspace, then the kernels.  dion_plan_destroy waits for
 * the last table copy of this plan to finish, then frees it. */
int    dion_plan_create(const dion_matrix* mats, int count, int variant,
                        int g_dtype, dion_plan** plan_out);
size_t dion_plan_workspace_size(const dion_plan* plan);
int    dion_plan_count(const dion_plan* plan);
int    dion_plan_step(dion_plan* plan, float eta, float beta,
                      void* workspace, size_t workspace_bytes, void* stream);
void   dion_plan_destroy(dion_plan* plan);

int dion_plan_shard_stage(dion_plan* plan, int stage, float eta, float beta,
                          void* workspace, size_t workspace_bytes, void* stream);
int dion_plan_shard_buffer(const dion_plan* plan, int which, int index,
                           size_t* offset, size_t* bytes);

/* Inspection of a plan's intermediate factors.  After a step of `plan` has
 * completed on the stream, the workspace holds, for matrix `index` (its
 * position in the plan's list) unless it broke down:
 *   DION_BUF_P  P = M V                 float32, m x r row-major
 *   DION_BUF_U  U = orth(P)             float32, m x r row-major
 *   DION_BUF_W  W = M^T U               float32, n x r row-major
 * dion_plan_buffer gives the byte offset from the workspace base and the
 * size of one of them.  They stay valid until the next step on that
 * workspace.  Errors: DION_ERR_INVALID_ARG for a null plan or output
 * pointer, `which` outside DION_BUF_* or `index` outside the list. */
#define DION_BUF_W    1   /* the same value as DION_SHARD_W */
#define DION_BUF_P    2
#define DION_BUF_U    3
int dion_plan_buffer(const dion_plan* plan, int which, int index,
                     size_t* offset, size_t* bytes);

/* Phase timing, for measurement.  A step runs five phases, in order:
 *   0  P = M V            1  U = orth(P)          2  W = M^T U
 *   3  Vbar (orth(W) or column normalization; with split-bfloat16 products
 *      also the bfloat16 planes of U, W and Vbar the update reads)
 *   4  X and R update (the update kernel alone)
 * dion_plan_timing_enable(plan, max_steps) makes the next max_steps calls of
 * dion_plan_step record a HIP event at every phase boundary on the step's
 * stream (creating the events now; 0 disables and frees them).
 * dion_plan_timing_read waits for the last recorded event, writes the
 * summed milliseconds of each phase over the recorded steps into
 * ms_per_phase[DION_PHASES] and the step count into *steps, and starts a
 * new recording window. */
#define DION_PHASES 5
int dion_plan_timing_enable(dion_plan* plan, int max_steps);
int dion_plan_timing_read(dion_plan* plan, double* ms_per_phase, int* steps);

/* Breakdown check: waits for `stream`, then reads the status words of the
 * last step enqueued on `workspace` (count = 1 for dion_step, the list
 * length for a grouped step).  per_matrix (optional, count ints) receives
 * each matrix's DION_STATUS_* flags, in the caller's list order.
 * Returns DION_OK, DION_ERR_BREAKDOWN if any matrix broke down, or an
 * argument / HIP error.  The workspace does not record how many matrices
 * the last step had, so the caller passes `count`; a grouped step can
 * break down in some matrices only, so the flags come per matrix rather
 * than as one code. */
int dion_status(const void* workspace, int count, void* stream, int* per_matrix);

#ifdef __cplusplus
}
#endif

#endif /* LIBDION_DION_H_ */
