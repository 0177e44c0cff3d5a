// Internal declarations shared by the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qgemv {

constexpr int kQK = 256;           // weights per super-block
constexpr int kQ4KBytes = 144;     // Q4_K super-block
constexpr int kQ6KBody = 208;      // Q6_K super-block body (fp16 d in a separate plane)
constexpr int kChunksPerBlock = 8; // 16-byte code chunks (32 columns each) per super-block
constexpr int kMaxVec = 8;

// Row groups whose loads a wave issues together before computing any of them. A group costs
// 8 * chunks_per_lane VGPRs of loaded data; up to ~32 VGPRs of loads per step are in flight
// without cutting occupancy much, so lanes with fewer chunks load more groups at once.
constexpr int groups_per_step(int chunks_per_lane) {
    return chunks_per_lane == 1 ? 4 : (chunks_per_lane == 2 ? 2 : 1);
}

// Largest workgroup of the one-matrix GEMV, in waves: 8 for a wide activation slice (a lane
// group reading nvec * lanes_per_row * chunks_per_lane >= 128 blocks of 32 columns), whose
// quantization in the fused form the workgroup's lanes share; 4 otherwise, which keeps the
// register budget of the narrow-slice kernels at that of 256-thread workgroups.
constexpr int kWideSliceBlocks = 128;
constexpr int gemv_max_waves(int nvec, int lanes_per_row, int chunks_per_lane) {
    return nvec * lanes_per_row * chunks_per_lane >= kWideSliceBlocks ? 8 : 4;
}

// LDS a launch that splits the columns inside the workgroup may take (the fused form's slice of
// every chunk plus the chunks' row sums); wider fused splits take the workspace instead.
constexpr size_t kMaxSplitLds = 64 * 1024;

// One GEMV launch: the kernels read everything they need from here.
struct GemvArgs {
    const uint8_t *w;      // weight tensor (Q4_K blocks, or Q6_K bodies followed by the d plane)
    const int8_t *xq;      // [nvec][cols]
    const float *xd;       // [nvec][cols/32]
    float *out;            // [splits][nvec][rows] (y itself when splits == 1)
    int32_t *P;            // debug partials or nullptr
    int32_t *S;            // debug activation block sums or nullptr
    const float *x;        // float32 activations [nvec][cols] to quantize in the kernel, or nullptr
    int8_t *xq_out;        // where the fused kernel also stores the codes (may be nullptr)
    float *xd_out;         // ... and the scales (nullptr exactly when xq_out is)
    int32_t rows;
    int32_t nb;            // weight blocks per row (256-weight super-blocks for Q4_K / Q6_K,
                           // 32-weight blocks for Q4_0 / Q8_0)
    int32_t nchunks;       // 16-byte chunks per row = 8 * nb
    int32_t threads;       // threads per workgroup of the launch, set by the launcher (the
                           // kernels use it instead of blockDim, which the compiler may read
                           // with a vector load and a wait at the kernel's start)
    int32_t wg_splits;     // column chunks split inside the workgroup (gemv_split_kernel)
};

// Kernel forms, a template parameter so that each has its own name in kernel traces:
// kModePlain reads the activation codes made by qgemv_quantize_act; kModeDebug does the same
// and writes the integer partials instead of y; kModeFused quantizes the float32 activation
// itself (GemvArgs::x).
enum KernelMode : int { kModePlain = 0, kModeDebug = 1, kModeFused = 2 };

// Several matrices sharing one activation in one launch (gemv_multi.hip).
constexpr int kMaxMats = 8;
constexpr int kTypeQ4K = 1;        // the ABI's QGEMV_Q4K
constexpr int kTypeQ6K = 2;        // the ABI's QGEMV_Q6K
constexpr int kTypeQ40 = 3;        // the ABI's QGEMV_Q4_0
constexpr int kTypeQ80 = 4;        // the ABI's QGEMV_Q8_0
struct MatDesc {
    const uint8_t *w;      // planar tensor of rows x cols
    float *out;            // y of this matrix, [nvec][rows]
    int32_t rows;
    int32_t nb;            // weight blocks per row (256-weight super-blocks for Q4_K / Q6_K,
                           // 32-weight blocks for Q4_0 / Q8_0)
    int32_t wtype;         // kTypeQ4K, kTypeQ6K, kTypeQ40 or kTypeQ80
    int32_t step0;         // the matrix's first step in the launch's step numbering
};
// The matrices of one format in a launch: their steps are consecutive in the launch's
// numbering, and a range of the grid's workgroups walks them (and only them).
constexpr int kMaxFmtGroups = 4;
struct FmtGroup {
    int32_t wtype;
    int32_t step0;         // the group's first step
    int32_t steps;
    int32_t block0;        // the group's first workgroup
    int32_t blocks;
};
struct MultiArgs {
    GemvArgs act;          // the activation fields (xq, xd or x, xq_out, xd_out, nchunks)
    int32_t nmats;
    int32_t steps;         // steps of all matrices together
    MatDesc m[kMaxMats];   // ordered by format, so each format's steps are consecutive
    int32_t ngroups;
    FmtGroup g[kMaxFmtGroups];
};

struct LaunchShape {
    int lanes;             // lanes per row (T)
    int chunks;            // chunks per lane (NC)
    int waves;             // waves per workgroup
    int blocks;            // workgroups per column chunk
    int splits;            // column chunks
};

// Kernel launchers; each returns the HIP status of its launch.
hipError_t launch_quantize_act(const float *x, int8_t *xq, float *xd, int64_t nblocks32,
                               hipStream_t stream);
hipError_t launch_gemv_q4k(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream);
hipError_t launch_gemv_q6k(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream);
hipError_t launch_gemv_q40(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream);
hipError_t launch_gemv_q80(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream);
// Several matrices: any mix of formats (gemv_multi.hip), or all of one format (the per-format
// files, with the one-matrix walk)
hipError_t launch_gemv_multi(const MultiArgs &a, const LaunchShape &s, int nvec,
                             hipStream_t stream);
hipError_t launch_gemv_multi_q4k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
hipError_t launch_gemv_multi_q6k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
hipError_t launch_gemv_multi_q40(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
hipError_t launch_gemv_multi_q80(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
// The unfused product of a plan with column splits, the splits inside the workgroup
// (gemv_split_kernel in gemv_walk.h): s.splits chunks, s.waves a multiple of it
hipError_t launch_gemv_split_q4k(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
hipError_t launch_gemv_split_q6k(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
hipError_t launch_gemv_split_q40(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
hipError_t launch_gemv_split_q80(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream);
// Several matrices of one format with rows wider than one pass, the split inside the
// workgroup as above (plain or fused)
hipError_t launch_gemv_multi_split_q4k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream);
hipError_t launch_gemv_multi_split_q6k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream);
hipError_t launch_gemv_multi_split_q40(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream);
hipError_t launch_gemv_multi_split_q80(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream);
// ... and a mix of formats (gemv_multi.hip)
hipError_t launch_gemv_multi_split(const MultiArgs &a, const LaunchShape &s, int nvec,
                                   hipStream_t stream);
// LDS bytes of a launch that splits the columns inside the workgroup: in the fused form the
// quantized slice of every chunk (32 code bytes and a float32 scale per activation block),
// then the chunks' row sums, float32 [splits][nvec][rows of the workgroup's step].
constexpr size_t gemv_split_lds_bytes(int nvec, int lanes, int chunks, bool fused, int splits,
                                      int waves) {
    return (fused ? size_t{36} * nvec * lanes * chunks * splits : 0) +
           sizeof(float) * static_cast<size_t>(nvec) * waves * groups_per_step(chunks) *
               (64 / lanes);
}
hipError_t launch_splitk_reduce(const float *part, float *y, int64_t n, int splits,
                                hipStream_t stream);
// Rows [row0, row0 + nrows) of a rows x cols matrix (w points at row row0) into their places
// in the whole tensor `out`.
hipError_t launch_quantize_q4k(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream);
hipError_t launch_quantize_q6k(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream);
hipError_t launch_quantize_q40(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream);
hipError_t launch_quantize_q80(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream);

hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, int blocks,
                             hipStream_t stream);

// Whether a (lanes, chunks, nvec) combination has a compiled kernel.
bool gemv_variant_exists(int lanes, int chunks, int nvec);

// Many vectors on the matrix cores (gemm_mfma.hip): a workgroup of 4 waves takes 128 rows
// (32 per wave) and a group of 32 * nt vectors over the super-blocks of one column split.
constexpr int kMaxBatch = 256;     // vectors per product on the matrix-core path
constexpr int kMcRows = 128;       // rows per workgroup
struct GemmArgs {
    const uint8_t *w;      // Q4_K tensor
    const int8_t *xq;      // [nvec][cols]
    const float *xd;       // [nvec][cols/32]
    float *out;            // [splits][nvec][rows] (y itself when splits == 1)
    int32_t *P;            // debug: [nvec][rows][cols/32] integer partials, or nullptr
    int32_t *S;            // debug: [nvec][cols/32] activation block sums, or nullptr
    uint8_t *tiles;        // workspace: the staged fp16 activation tiles (pre-pass output)
    const float *x;        // integer-core path only: float32 activations [nvec][cols] that
                           // the kernel quantizes itself, or nullptr (then xq, xd are read)
    int8_t *xq_out;        // ... where it also stores the codes and scales (or nullptr)
    float *xd_out;
    int32_t rows;
    int32_t nb;            // super-blocks per row
    int32_t nvec;
    int32_t sb_per_split;  // super-blocks per column split
    int32_t row_tiles;     // work items: row tiles x vector groups x splits
    int32_t groups;
    int32_t splits;
};
// Two launches: the staging pre-pass (grid super-blocks x groups) writes the tiles, then the
// product (grid row tiles x groups x splits); nt = 1..3 tiles of 32 vectors per group.
constexpr int64_t mc_tile_bytes(int nt) { return int64_t{nt} * (32 * 512 + 8 * 32 * 8); }
hipError_t launch_gemm_q4k_mfma(const GemmArgs &a, int nt, int row_tiles, int groups, int splits,
                                bool debug, hipStream_t stream);

// 1..16 vectors on the integer matrix cores (gemm_i8.hip): a workgroup of up to kI8MaxWaves
// waves takes 16 rows at a time over a column split of kI8SbPerWave super-blocks per wave
// (GemmArgs::sb_per_split == kI8SbPerWave * waves; row_tiles = ceil(rows / 16); splits
// column splits writing out [splits][nvec][rows]; tiles unused). One launch; with x set, the
// kernel quantizes the activation itself (the codes of qgemv_quantize_act, bit for bit).
constexpr int kI8SbPerWave = 2;
constexpr int kI8MaxWaves = 4;
constexpr int kI8MaxVec = 16;      // vectors per launch (two groups of 8)
hipError_t launch_gemm_q4k_i8(const GemmArgs &a, int waves, bool debug, hipStream_t stream);

// The static device scratch buffer (scratch.hip): its size, and its device address on the
// current device (looked up once per device; QGEMV_OK, or the failure status).
constexpr size_t kScratchBytes = size_t{32} << 20;
int scratch_address(void **ptr);


// Host: record a HIP error (or a message) as this thread's last error text and return the
// status the C ABI reports (QGEMV_EHIP, or `status`).
int hip_fail(hipError_t e);
int fail_with(int status, const char *text);

}  // namespace qgemv
