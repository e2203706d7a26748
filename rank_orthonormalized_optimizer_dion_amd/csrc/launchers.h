// Host-side launchers of libdion's kernels (one grouped launch each).
#pragma once
#include <hip/hip_runtime.h>

#include "dion_types.h"

namespace dion {

// gdtype: 0 = float32 G, 1 = bfloat16 G.  bn: output tile width (64 or 128;
// 256 selects the split-bfloat16 large tiles: 256 x 256 for launch_mv and
// launch_mtu, 256 x 128 for launch_epi; 192 the split-bfloat16 256 x 192
// tiles of launch_mv and launch_mtu).
// vec: every operand of the launch admits 16-byte vector loads.
// math: 0 = float32 MFMA products, 1 = split-bfloat16 (three bf16 MFMAs).
hipError_t launch_mv(const Launch& L, int gdtype, int bn, bool vec, int math, hipStream_t st);
hipError_t launch_mtu(const Launch& L, int gdtype, int bn, bool vec, int math, hipStream_t st);
hipError_t launch_gram(const Launch& L, int bg, bool vec, hipStream_t st);
// Sliced Gram matrix: column maxima, digit planes, int8 MFMA products.
hipError_t launch_qmax(const Launch& L, hipStream_t st);
hipError_t launch_qslice(const Launch& L, hipStream_t st);
hipError_t launch_gram8(const Launch& L, hipStream_t st);
// math = 1: three-way split bfloat16 products of float32 accuracy (k_trmm6)
hipError_t launch_trmm(const Launch& L, int bn, bool vec, int math, hipStream_t st);
hipError_t launch_epi(const Launch& L, int gdtype, int bn, bool vec, int math, hipStream_t st);

// work items per 64 x 64 upper block of k_chol_init: kCholInitParts row
// bands when the launch has at most kCholInitSplit blocks, else one
constexpr int kCholInitParts = 4;
constexpr int kCholInitSplit = 1024;
hipError_t launch_chol_init(const Launch& L, int parts, hipStream_t st);
hipError_t launch_chol_diag(const Launch& L, hipStream_t st);
hipError_t launch_chol_panel(const Launch& L, hipStream_t st);
hipError_t launch_chol_trail(const Launch& L, hipStream_t st);
// the whole first-pass factorization (what k_chol_diag, k_chol_panel and
// k_chol_trail do over all block steps) in one launch: one workgroup per
// 64 x 64 block of T and of Y (ClassInfo: tx = blocks per side, tiles =
// tx * tx), ordered by block row, each waiting on the blocks it reads
hipError_t launch_chol_flow(const Launch& L, hipStream_t st);
// the most work items (blocks of T and of Y over the launch) for which the
// factorization takes k_chol_flow: those of one workgroup per CU
constexpr int kFlowItems = 256;
// the whole factorization of each matrix in one workgroup (shifted retry,
// second pass) and the float64 triangular multiply that follows it
hipError_t launch_chol_one(const Launch& L, hipStream_t st);
// sets the per-matrix decision whether orth takes more passes (one
// workgroup per matrix, after the first pass's factorization)
hipError_t launch_orth_decide(const Launch& L, hipStream_t st);
hipError_t launch_trmm64(const Launch& L, hipStream_t st);

// The whole step of each matrix of the launch in one workgroup (small
// matrices; L.mode = 1 for Orth-Dion, 0 for Dion).  rb: the rank block
// small_rank_block(r) of every matrix of the launch; resident: M is held in
// LDS (every matrix of the launch fits kSmallResidentFloats).
int small_rank_block(int r);   // 8, 16, or 0 when r > kSmallMaxRank
hipError_t launch_small(const Launch& L, int gdtype, int rb, bool resident, hipStream_t st);

hipError_t launch_reduce(const Launch& L, hipStream_t st);
hipError_t launch_colnorm(const Launch& L, hipStream_t st);
hipError_t launch_colnorm_fin(const Launch& L, hipStream_t st);
hipError_t launch_colscale(const Launch& L, hipStream_t st);
// V^T (which = 0) or U^T (which = 1) split-bfloat16 planes, in
// kSplitTile x kSplitTile tiles of V or U
constexpr int kSplitTile = 64;
hipError_t launch_split_t(const Launch& L, hipStream_t st);
// U, W and Vbar split-bfloat16 planes for the large-tile fused update, in
// kSplitTile x kSplitTile tiles of each factor
hipError_t launch_split_n(const Launch& L, hipStream_t st);
int elems_per_tile();

}  // namespace dion
