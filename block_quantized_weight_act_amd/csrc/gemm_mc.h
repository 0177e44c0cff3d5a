// Launchers of the integer matrix-core kernels for many activation vectors that have no other
// header of their own.
#pragma once

#include "qgemv_internal.h"

namespace qgemv {

// Q6_K x 9..kMaxBatch vectors (gemm_q6k_mc.hip): grid row_tiles x groups x splits work items,
// each 32 RW rows x 32 VW vectors (vw = VW = 1, 2 or 4, RW = 4 / VW) over sb_per_split blocks
// of 32 columns (a multiple of 4); a.nb = cols / 32. out is [splits][nvec][rows]; the debug
// form writes P [nvec][rows][cols/16] and S [nvec][cols/32] instead.
hipError_t launch_gemm_q6k_mc(const GemmArgs &a, int vw, bool debug, hipStream_t stream);

}  // namespace qgemv
