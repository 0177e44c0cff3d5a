// Several matrices that multiply the same activation, in one launch (any mix of Q4_K, Q6_K,
// Q4_0 and Q8_0, up to kMaxMats of them, all with the same column count).
//
// genie-ai-runtime (jared-hpc.com), "v1.2.0": the attention projections of a decode step share
// one quantized activation, which is made once and read by all of them instead of once per
// product. Here they also share one launch: the matrices' row steps are numbered one after
// the other (grouped by format) and waves walk the numbering with a grid-wide stride, each step
// taking the tile (tile.h) of the matrix it falls in. A wave's activation slice is loaded (or,
// in the fused form, quantized by its workgroup) once and serves every matrix, since lane t's
// columns are the same in all of them. A row wider than one pass of the shared lane geometry
// is split into column chunks inside the workgroup, as for one matrix (gemv_split_walk in
// gemv_walk.h). This file holds the kernels for a mix of formats, whose workgroups are split
// between the formats in proportion to their steps, each range walking its own format's
// steps; matrices all of one format take the one-matrix walks over the same step numbering
// (gemv_multi_fmt_kernel and gemv_multi_split_fmt_kernel in gemv_walk.h).
#include "gemv_walk.h"

namespace qgemv {

template <int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(256) gemv_multi_kernel(MultiArgs a) {
    static_assert(Q4kTile<V, T, NC>::G == Q6kTile<V, T, NC>::G &&
                      Q4kTile<V, T, NC>::G == Q40Tile<V, T, NC>::G &&
                      Q4kTile<V, T, NC>::G == Q80Tile<V, T, NC>::G &&
                      Q4kTile<V, T, NC>::RPW == Q6kTile<V, T, NC>::RPW,
                  "one step geometry for every format");
    // The workgroup's format group (wave-uniform), then that format's whole walk: each branch
    // issues its first step's weights ahead of the activation slice and waits for exactly the
    // loads of its own format, as the one-format walk does.
    int gi = 0;
#pragma unroll
    for (int i = 1; i < kMaxFmtGroups; i++)
        if (i < a.ngroups && static_cast<int>(blockIdx.x) >= a.g[i].block0) gi = i;
    const FmtGroup &g = a.g[gi];
    const GroupSteps src{a, g.step0, g.steps};
    const int blk = static_cast<int>(blockIdx.x) - g.block0;
    if (g.wtype == kTypeQ4K)
        gemv_walk<Q4kTile<V, T, NC>, V, T, NC, MODE>(a.act, src, g.steps, blk, g.blocks);
    else if (g.wtype == kTypeQ6K)
        gemv_walk<Q6kTile<V, T, NC>, V, T, NC, MODE>(a.act, src, g.steps, blk, g.blocks);
    else if (g.wtype == kTypeQ40)
        gemv_walk<Q40Tile<V, T, NC>, V, T, NC, MODE>(a.act, src, g.steps, blk, g.blocks);
    else
        gemv_walk<Q80Tile<V, T, NC>, V, T, NC, MODE>(a.act, src, g.steps, blk, g.blocks);
}

// The same with each row split into column chunks inside the workgroup.
template <int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(64 * gemv_max_waves(V, T, NC)) gemv_multi_split_kernel(MultiArgs a) {
    constexpr bool FUSED = MODE == kModeFused;
    int gi = 0;
#pragma unroll
    for (int i = 1; i < kMaxFmtGroups; i++)
        if (i < a.ngroups && static_cast<int>(blockIdx.x) >= a.g[i].block0) gi = i;
    const FmtGroup &g = a.g[gi];
    const GroupSteps src{a, g.step0, g.steps};
    const int blk = static_cast<int>(blockIdx.x) - g.block0;
    if (g.wtype == kTypeQ4K)
        gemv_split_walk<Q4kTile<V, T, NC>, V, T, NC, FUSED>(a.act, src, g.steps, blk, g.blocks);
    else if (g.wtype == kTypeQ6K)
        gemv_split_walk<Q6kTile<V, T, NC>, V, T, NC, FUSED>(a.act, src, g.steps, blk, g.blocks);
    else if (g.wtype == kTypeQ40)
        gemv_split_walk<Q40Tile<V, T, NC>, V, T, NC, FUSED>(a.act, src, g.steps, blk, g.blocks);
    else
        gemv_split_walk<Q80Tile<V, T, NC>, V, T, NC, FUSED>(a.act, src, g.steps, blk, g.blocks);
}

namespace {

using MultiLauncher = hipError_t (*)(const MultiArgs &, const LaunchShape &, hipStream_t);

template <int V, int T, int NC>
hipError_t launch_multi_variant(const MultiArgs &a, const LaunchShape &s, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(s.blocks));
    const dim3 block(static_cast<unsigned>(64 * s.waves));
    const size_t lds = act_slice_lds_bytes<V, T, NC>();
    MultiArgs b = a;
    b.act.threads = 64 * s.waves;
    if (a.act.x != nullptr)
        hipLaunchKernelGGL((gemv_multi_kernel<V, T, NC, kModeFused>), grid, block, lds, stream, b);
    else
        hipLaunchKernelGGL((gemv_multi_kernel<V, T, NC, kModePlain>), grid, block, 0, stream, b);
    return hipGetLastError();
}

template <int V, int T, int NC>
hipError_t launch_multi_split_variant(const MultiArgs &a, const LaunchShape &s,
                                      hipStream_t stream) {
    if (s.splits < 2 || s.waves % s.splits != 0 || s.waves > gemv_max_waves(V, T, NC))
        return hipErrorInvalidValue;
    const bool fused = a.act.x != nullptr;
    const size_t lds = gemv_split_lds_bytes(V, T, NC, fused, s.splits, s.waves);
    if (lds > kMaxSplitLds) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(s.blocks));
    const dim3 block(static_cast<unsigned>(64 * s.waves));
    MultiArgs b = a;
    b.act.threads = 64 * s.waves;
    b.act.wg_splits = s.splits;
    if (fused)
        hipLaunchKernelGGL((gemv_multi_split_kernel<V, T, NC, kModeFused>), grid, block, lds,
                           stream, b);
    else
        hipLaunchKernelGGL((gemv_multi_split_kernel<V, T, NC, kModePlain>), grid, block, lds,
                           stream, b);
    return hipGetLastError();
}

template <int V, int T, int NC, bool SPLIT>
constexpr MultiLauncher pick() {
    if constexpr (V * NC > 8)
        return nullptr;
    else if constexpr (SPLIT)
        return &launch_multi_split_variant<V, T, NC>;
    else
        return &launch_multi_variant<V, T, NC>;
}

#define QGEMV_NC_ROW(V, T, S) \
    {pick<V, T, 1, S>(), pick<V, T, 2, S>(), pick<V, T, 3, S>(), pick<V, T, 4, S>()}
#define QGEMV_T_ROW(V, S) \
    {QGEMV_NC_ROW(V, 8, S), QGEMV_NC_ROW(V, 16, S), QGEMV_NC_ROW(V, 32, S), QGEMV_NC_ROW(V, 64, S)}
#define QGEMV_TABLE(S)                                                                       \
    {QGEMV_T_ROW(1, S), QGEMV_T_ROW(2, S), QGEMV_T_ROW(3, S), QGEMV_T_ROW(4, S),            \
     QGEMV_T_ROW(5, S), QGEMV_T_ROW(6, S), QGEMV_T_ROW(7, S), QGEMV_T_ROW(8, S)}
const MultiLauncher kMultiTable[8][4][4] = QGEMV_TABLE(false);
const MultiLauncher kMultiSplitTable[8][4][4] = QGEMV_TABLE(true);
#undef QGEMV_TABLE
#undef QGEMV_T_ROW
#undef QGEMV_NC_ROW

hipError_t launch_from(const MultiLauncher (&table)[8][4][4], const MultiArgs &a,
                       const LaunchShape &s, int nvec, hipStream_t stream) {
    int ti = -1;
    switch (s.lanes) {
        case 8: ti = 0; break;
        case 16: ti = 1; break;
        case 32: ti = 2; break;
        case 64: ti = 3; break;
        default: return hipErrorInvalidValue;
    }
    if (nvec < 1 || nvec > 8 || s.chunks < 1 || s.chunks > 4) return hipErrorInvalidValue;
    const MultiLauncher fn = table[nvec - 1][ti][s.chunks - 1];
    if (!fn) return hipErrorInvalidValue;
    return fn(a, s, stream);
}

}  // namespace

hipError_t launch_gemv_multi(const MultiArgs &a, const LaunchShape &s, int nvec,
                             hipStream_t stream) {
    if (s.splits != 1) return hipErrorInvalidValue;
    return launch_from(kMultiTable, a, s, nvec, stream);
}

hipError_t launch_gemv_multi_split(const MultiArgs &a, const LaunchShape &s, int nvec,
                                   hipStream_t stream) {
    return launch_from(kMultiSplitTable, a, s, nvec, stream);
}

}  // namespace qgemv
