// Launchers of the integer matrix-core kernels for 9..kMaxBatch activation vectors of the
// formats with one product per block (Q8_0, Q4_0: gemm_q32.hip) or per sub-block (Q6_K:
// gemm_q6k_mc.hip).
#pragma once

#include "qgemv_internal.h"

namespace qgemv {

// Workgroup shapes, by the vector tiles of 32 a workgroup covers (vt = 1, 2 or 4): 128 rows x
// 32 vectors, 128 x 64, 64 x 128. The grid is row_tiles (of mc32_rows_per_wg rows) x groups (of
// 32 vt vectors) x splits work items, each over sb_per_split blocks of 32 columns (a multiple
// of 8: the kernels' steps); a.nb = cols / 32. out is [splits][nvec][rows]; the debug form writes P [nvec][rows]
// [cols/32] (Q6_K: [cols/16]) and S [nvec][cols/32] instead.
constexpr int mc32_rows_per_wg(int vt) { return vt == 4 ? 64 : 128; }

// Blocks of 32 columns per step of those kernels, by format and shape: 8 (whole 128-byte lines
// of every codes plane per row, one LDS buffer) or 4 (half lines, two LDS buffers, so loads and
// products of consecutive steps overlap more). Measured on MI355X (262144 x 1536 and
// 16384 x 2048, 16 / 64 / 256 vectors): 8 was as fast or faster everywhere (Q8_0 x 16: 112 us
// against 129; Q6_K x 16: 108 against 127) except Q4_0 with 33..64 vectors (262144 x 1536 x 64:
// 174 against 156 us), whose weight tile is half as wide.
constexpr int mc32_step_blocks(int wtype, int vt) { return wtype == kTypeQ40 && vt == 2 ? 4 : 8; }

hipError_t launch_gemm_q32_mc(int wtype, const GemmArgs &a, int vt, bool debug,
                              hipStream_t stream);

// Q8_0, Q4_0, Q6_K and Q4_K with 1..kQ32I8MaxVec vectors on the integer matrix cores
// (gemm_q32_i8.hip; Q6_K and Q4_K rows of whole super-blocks): a
// workgroup of up to kQ32I8MaxWaves waves takes 16 rows at a time over a column split of
// kQ32I8BlocksPerWave blocks of 32 columns per wave (GemmArgs::sb_per_split ==
// kQ32I8BlocksPerWave * waves, a.nb = cols / 32, row_tiles = ceil(rows / 16)); out is
// [splits][nvec][rows]; the debug form writes P [nvec][rows][cols/32] and S [nvec][cols/32]
// instead.
constexpr int kQ32I8BlocksPerWave = 16;
constexpr int kQ32I8MaxWaves = 4;
constexpr int kQ32I8MaxVec = 16;
hipError_t launch_gemm_q32_i8(int wtype, const GemmArgs &a, int waves, bool debug,
                              hipStream_t stream);
hipError_t launch_gemm_q6k_mc(const GemmArgs &a, int vt, bool debug, hipStream_t stream);

}  // namespace qgemv
