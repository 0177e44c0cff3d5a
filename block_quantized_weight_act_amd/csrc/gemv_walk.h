// The one-matrix GEMV kernel for gfx950: the walk of the waves over the matrix, shared by the
// four weight formats (the per-lane pieces are the tiles in tile.h).
//
// genie-ai-runtime (jared-hpc.com), "The decode arc": the quantized matrix-vector product is
// done with int8 4-way dot products instead of dequantizing to floating point, the codes are
// handled as whole 32-bit words, and a row is shared by the lanes of one warp. "v1.3.0": when
// rows alone cannot fill the GPU, split the reduction dimension and sum the pieces in a
// separate pass. Here:
//
//  * Waves walk steps of G row groups with a grid-wide stride; blockIdx.y selects a column
//    chunk (split-K) whose partial sums go to a workspace that a second kernel adds in order.
//  * A wave's loads go out in this order: its activation slice, its first step's weights, then
//    (while the weights are in flight) the slice is finished; each later step's loads go out
//    at the end of the previous step's arithmetic. Loads complete in issue order, so waiting
//    for the slice never waits for the weights.
//  * Workgroups have up to 4 waves, or up to 8 where the lanes of a row read a wide activation
//    slice: the fused form quantizes the slice once per workgroup, so more waves share it.
//  * Kernel forms (kModePlain / kModeFused / kModeDebug) are a template parameter, so each has
//    its own name in kernel traces.
//
// The library is built with -ffp-contract=off: every fused multiply-add is an explicit fmaf.
#pragma once

#include "act_slice.h"
#include "device_common.h"
#include "qgemv_internal.h"
#include "tile.h"

namespace qgemv {

// Weight-format tags: the tile each format uses.
struct Q4K {
    template <int V, int T, int NC>
    using Tile = Q4kTile<V, T, NC>;
};
struct Q6K {
    template <int V, int T, int NC>
    using Tile = Q6kTile<V, T, NC>;
};
struct Q40 {
    template <int V, int T, int NC>
    using Tile = Q40Tile<V, T, NC>;
};
struct Q80 {
    template <int V, int T, int NC>
    using Tile = Q80Tile<V, T, NC>;
};

template <class F, int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(64 * gemv_max_waves(V, T, NC)) gemv_kernel(GemvArgs a) {
    constexpr bool DBG = MODE == kModeDebug;
    constexpr bool FUSED = MODE == kModeFused;
    using Tile = typename F::template Tile<V, T, NC>;
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
    ActTerms<V, NC> at;
    ActPending<V, T, NC, FUSED> pend;
    act_slice_issue<V, T, NC, FUSED>(a, L.g, L.cv, xw, xs, pend);
    __builtin_amdgcn_sched_barrier(0);
    Tile::issue(regs, a.w, a.rows, a.nb, st0, L);   // rows (>= 1) clamped: valid for any st0
    __builtin_amdgcn_sched_barrier(0);
    act_slice_finish<V, T, NC, FUSED>(a, L.cv, L.t, xw, xs, pend);
    act_terms<V, NC>(xw, at);
    if (DBG && blockIdx.x == 0 && wave == 0 && L.rsub == 0) {
#pragma unroll
        for (int v = 0; v < V; v++)
#pragma unroll
            for (int k = 0; k < NC; k++)
                if (L.cv[k]) a.S[static_cast<int64_t>(v) * a.nchunks + L.g[k]] = at.sum[v][k];
    }

    for (int st = st0; st < steps; st += stride) {
        // Keep every load of the step ahead of the arithmetic: without this fence the
        // scheduler interleaves them to save registers and waits for each load in turn.
        __builtin_amdgcn_sched_barrier(0);
        Tile::template compute<DBG>(regs, xw, xs, at, a.out, a.rows, st, L, a.P, a.nchunks);
        // The next step's loads go out as soon as this step's arithmetic is done, so the
        // values of one step are never live across the loop's back edge with the next ones.
        __builtin_amdgcn_sched_barrier(0);
        if (st + stride < steps) Tile::issue(regs, a.w, a.rows, a.nb, st + stride, L);
    }
}

// The launch of one format: a table over (vectors, lanes per row, chunks per lane) of the
// compiled instances (nvec * chunks <= 8, so the activation slice fits in VGPRs).
template <class F>
struct GemvLaunch {
    using Launcher = hipError_t (*)(const GemvArgs &, const LaunchShape &, bool, hipStream_t);

    template <int V, int T, int NC>
    static hipError_t variant(const GemvArgs &a, const LaunchShape &s, bool debug,
                              hipStream_t stream) {
        if (s.waves < 1 || s.waves > gemv_max_waves(V, T, NC)) return hipErrorInvalidValue;
        const dim3 grid(static_cast<unsigned>(s.blocks), static_cast<unsigned>(s.splits));
        const dim3 block(static_cast<unsigned>(64 * s.waves));
        const size_t lds = act_slice_lds_bytes<V, T, NC>();
        if (debug)
            hipLaunchKernelGGL((gemv_kernel<F, V, T, NC, kModeDebug>), grid, block, 0, stream, a);
        else if (a.x != nullptr)
            hipLaunchKernelGGL((gemv_kernel<F, V, T, NC, kModeFused>), grid, block, lds, stream, a);
        else
            hipLaunchKernelGGL((gemv_kernel<F, V, T, NC, kModePlain>), grid, block, 0, stream, a);
        return hipGetLastError();
    }

    template <int V, int T, int NC>
    static constexpr Launcher pick() {
        if constexpr (V * NC <= 8)
            return &variant<V, T, NC>;
        else
            return nullptr;
    }

    template <int V, int T>
    static constexpr void row(Launcher (&out)[4]) {
        out[0] = pick<V, T, 1>();
        out[1] = pick<V, T, 2>();
        out[2] = pick<V, T, 3>();
        out[3] = pick<V, T, 4>();
    }

    template <int V>
    static constexpr void fill(Launcher (&out)[4][4]) {
        row<V, 8>(out[0]);
        row<V, 16>(out[1]);
        row<V, 32>(out[2]);
        row<V, 64>(out[3]);
    }

    static hipError_t launch(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                             hipStream_t stream) {
        static Launcher table[8][4][4] = {};
        static const bool filled = [] {
            fill<1>(table[0]);
            fill<2>(table[1]);
            fill<3>(table[2]);
            fill<4>(table[3]);
            fill<5>(table[4]);
            fill<6>(table[5]);
            fill<7>(table[6]);
            fill<8>(table[7]);
            return true;
        }();
        (void)filled;
        int ti = -1;
        switch (s.lanes) {
            case 8: ti = 0; break;
            case 16: ti = 1; break;
            case 32: ti = 2; break;
            case 64: ti = 3; break;
            default: return hipErrorInvalidValue;
        }
        if (nvec < 1 || nvec > 8 || s.chunks < 1 || s.chunks > 4) return hipErrorInvalidValue;
        const Launcher fn = table[nvec - 1][ti][s.chunks - 1];
        if (!fn) return hipErrorInvalidValue;
        return fn(a, s, debug, stream);
    }
};

}  // namespace qgemv
