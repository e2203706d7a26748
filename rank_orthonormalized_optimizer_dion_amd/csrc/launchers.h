// Host-side launchers of libdion's kernels (one grouped launch each).
#pragma once
#include <hip/hip_runtime.h>

#include "dion_types.h"

namespace dion {

// gdtype: 0 = float32 G, 1 = bfloat16 G.  bn: output tile width (64 or 128;
// 256 selects the split-bfloat16 large tiles: 256 x 256 for launch_mv and
// launch_mtu, 256 x 128 for launch_epi).
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

hipError_t launch_chol_init(const Launch& L, hipStream_t st);
hipError_t launch_chol_diag(const Launch& L, hipStream_t st);
hipError_t launch_chol_panel(const Launch& L, hipStream_t st);
hipError_t launch_chol_trail(const Launch& L, hipStream_t st);

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
