// Q6_K weight x int8 activation GEMV for gfx950.
//
// genie-ai-runtime (jared-hpc.com), "The decode arc": int8 4-way dot-product mat-vec for
// Q6_K; "v1.3.0": split the reduction dimension when rows alone cannot fill the GPU.
//
// The same wave walk as the Q4_K kernel over the planar Q6_K tensor (each field in its own
// plane, so every load is naturally aligned and the low- and high-bit runs are streamed);
// the per-lane step is Q6kTile in tile.h.
#include "act_slice.h"
#include "device_common.h"
#include "qgemv_internal.h"
#include "tile.h"

namespace qgemv {

template <int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(256) gemv_q6k_kernel(GemvArgs a) {
    constexpr bool DBG = MODE == kModeDebug;
    constexpr bool FUSED = MODE == kModeFused;
    using Tile = Q6kTile<V, T, NC>;
    const LaneGeom<T, NC> L(a.nchunks);
    // the wave index is the same in all 64 lanes: keep it (and the step numbers) in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int wpb = blockDim.x >> 6;
    const int groups = (a.rows + Tile::RPW - 1) / Tile::RPW;
    const int steps = (groups + Tile::G - 1) / Tile::G;
    const int stride = gridDim.x * wpb;
    const int st0 = blockIdx.x * wpb + wave;

    typename Tile::Regs regs;
    uint32_t xw[V][NC][8];
    float xs[V][NC];
    int xlo[V][NC], xhi[V][NC];             // activation code sums of the two 16-column halves
    ActPending<V, T, NC, FUSED> pend;
    act_slice_issue<V, T, NC, FUSED>(a, L.g, L.cv, xw, xs, pend);
    __builtin_amdgcn_sched_barrier(0);
    Tile::issue(regs, a.w, a.rows, a.nb, st0, L);   // rows (>= 1) clamped: valid even when st0 >= steps
    __builtin_amdgcn_sched_barrier(0);
    act_slice_finish<V, T, NC, FUSED>(a, L.cv, L.t, xw, xs, pend);
    q6k_act_sums<V, NC>(xw, xlo, xhi);
    if (DBG && blockIdx.x == 0 && wave == 0 && L.rsub == 0) {
#pragma unroll
        for (int v = 0; v < V; v++)
#pragma unroll
            for (int k = 0; k < NC; k++)
                if (L.cv[k]) a.S[static_cast<int64_t>(v) * a.nchunks + L.g[k]] = xlo[v][k] + xhi[v][k];
    }

    for (int st = st0; st < steps; st += stride) {
        __builtin_amdgcn_sched_barrier(0);
        Tile::template compute<DBG>(regs, xw, xs, xlo, xhi, a.out, a.rows, st, L, a.P, a.nchunks);
        __builtin_amdgcn_sched_barrier(0);
        if (st + stride < steps) Tile::issue(regs, a.w, a.rows, a.nb, st + stride, L);
    }
}

namespace {

using Launcher = hipError_t (*)(const GemvArgs &, const LaunchShape &, bool, hipStream_t);

template <int V, int T, int NC>
hipError_t launch_variant(const GemvArgs &a, const LaunchShape &s, bool debug,
                          hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(s.blocks), static_cast<unsigned>(s.splits));
    const dim3 block(static_cast<unsigned>(64 * s.waves));
    const size_t lds = act_slice_lds_bytes<V, T, NC>();
    if (debug)
        hipLaunchKernelGGL((gemv_q6k_kernel<V, T, NC, kModeDebug>), grid, block, 0, stream, a);
    else if (a.x != nullptr)
        hipLaunchKernelGGL((gemv_q6k_kernel<V, T, NC, kModeFused>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((gemv_q6k_kernel<V, T, NC, kModePlain>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int V, int T, int NC>
constexpr Launcher pick() {
    if constexpr (V * NC <= 8)
        return &launch_variant<V, T, NC>;
    else
        return nullptr;
}

#define QGEMV_NC_ROW(V, T) {pick<V, T, 1>(), pick<V, T, 2>(), pick<V, T, 3>(), pick<V, T, 4>()}
#define QGEMV_T_ROW(V) \
    {QGEMV_NC_ROW(V, 8), QGEMV_NC_ROW(V, 16), QGEMV_NC_ROW(V, 32), QGEMV_NC_ROW(V, 64)}
const Launcher kTable[8][4][4] = {QGEMV_T_ROW(1), QGEMV_T_ROW(2), QGEMV_T_ROW(3), QGEMV_T_ROW(4),
                                  QGEMV_T_ROW(5), QGEMV_T_ROW(6), QGEMV_T_ROW(7), QGEMV_T_ROW(8)};
#undef QGEMV_T_ROW
#undef QGEMV_NC_ROW

int lanes_index(int lanes) {
    switch (lanes) {
        case 8: return 0;
        case 16: return 1;
        case 32: return 2;
        case 64: return 3;
        default: return -1;
    }
}

}  // namespace

hipError_t launch_gemv_q6k(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream) {
    const int ti = lanes_index(s.lanes);
    if (nvec < 1 || nvec > 8 || ti < 0 || s.chunks < 1 || s.chunks > 4) return hipErrorInvalidValue;
    const Launcher fn = kTable[nvec - 1][ti][s.chunks - 1];
    if (!fn) return hipErrorInvalidValue;
    return fn(a, s, debug, stream);
}

}  // namespace qgemv
