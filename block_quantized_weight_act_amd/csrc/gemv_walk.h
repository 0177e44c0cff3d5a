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

// Where the weights and the outputs of one step are: the matrix's planes, its y, its rows and
// blocks per row, and the step's number within the matrix (local).
struct StepMat {
    const uint8_t *w;
    float *out;
    int rows, nb, wtype, local;
};

// One matrix: step st is its own step st.
struct OneMatrix {
    const GemvArgs &a;
    __device__ __forceinline__ StepMat at(int st) const {
        return StepMat{a.w, a.out, a.rows, a.nb, 0, st};
    }
};

// Several matrices sharing the activation (MultiArgs): their steps are numbered one after the
// other, and step st falls in the last matrix whose first step is not after it. Only the first
// steps are scanned; the chosen descriptor is then read with a wave-uniform index, so it comes
// from the argument block by scalar loads. A step past the end falls in the last matrix (its
// rows are clamped like any row past the end).
struct MatrixList {
    const MultiArgs &a;
    __device__ __forceinline__ StepMat at(int st) const {
        int mi = 0;
#pragma unroll
        for (int i = 1; i < kMaxMats; i++)
            if (i < a.nmats && st >= a.m[i].step0) mi = i;
        const MatDesc &d = a.m[mi];
        return StepMat{d.w, d.out, d.rows, d.nb, d.wtype, st - d.step0};
    }
};

// The steps of one format group of a mixed launch, in the group's own numbering. A step past
// the group's end reads its last step's rows, so it stays within matrices of the group's format.
struct GroupSteps {
    const MultiArgs &a;
    int step0, steps;
    __device__ __forceinline__ StepMat at(int st) const {
        return MatrixList{a}.at(step0 + (st < steps ? st : steps - 1));
    }
};

// The walk of a wave over its steps for one tile type: workgroup blk of the nblk that share
// the `steps` steps takes steps st0, st0 + stride, ...; `src` says where each step's weights
// and outputs are.
template <class Tile, int V, int T, int NC, int MODE, class Steps>
__device__ __forceinline__ void gemv_walk(const GemvArgs &a, const Steps &src, int steps, int blk,
                                          int nblk) {
    constexpr bool DBG = MODE == kModeDebug;
    constexpr bool FUSED = MODE == kModeFused;
    const LaneGeom<T, NC> L(a.nchunks);
    // the wave index is the same in all 64 lanes: keep it (and the step numbers) in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int wpb = a.threads >> 6;
    const int stride = nblk * wpb;
    const int st0 = blk * wpb + wave;

    typename Tile::Regs regs;
    uint32_t xw[V][NC][8];
    float xs[V][NC];
    ActTerms<V, NC> at;
    ActPending<V, T, NC, FUSED> pend;
    const ChunkSpan sp{static_cast<int>(blockIdx.y), 1, 0};
    act_slice_issue<V, T, NC, FUSED>(a, sp, L.g, L.cv, xw, xs, pend);
    __builtin_amdgcn_sched_barrier(0);
    {
        const StepMat m = src.at(st0);   // rows (>= 1) clamped: valid for any st0
        Tile::issue(regs, m.w, m.rows, m.nb, m.local, L);
    }
    __builtin_amdgcn_sched_barrier(0);
    act_slice_finish<V, T, NC, FUSED>(a, sp, L.cv, L.t, xw, xs, pend);
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
        const StepMat m = src.at(st);
        Tile::template compute<DBG>(regs, xw, xs, at, m.out, m.rows, m.local, L, a.P, a.nchunks);
        // The next step's loads go out as soon as this step's arithmetic is done, so the
        // values of one step are never live across the loop's back edge with the next ones.
        __builtin_amdgcn_sched_barrier(0);
        if (st + stride < steps) {
            const StepMat n = src.at(st + stride);
            Tile::issue(regs, n.w, n.rows, n.nb, n.local, L);
        }
    }
}

template <class F, int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(64 * gemv_max_waves(V, T, NC)) gemv_kernel(GemvArgs a) {
    using Tile = typename F::template Tile<V, T, NC>;
    const int groups = (a.rows + Tile::RPW - 1) / Tile::RPW;
    const int steps = (groups + Tile::G - 1) / Tile::G;
    gemv_walk<Tile, V, T, NC, MODE>(a, OneMatrix{a}, steps, blockIdx.x, gridDim.x);
}

// Several matrices of this one format sharing the activation (qgemv_multi with a single
// format): the same walk over their combined step numbering, so the first step's weights go
// out before the activation slice is finished, as for one matrix.
template <class F, int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(256) gemv_multi_fmt_kernel(MultiArgs a) {
    gemv_walk<typename F::template Tile<V, T, NC>, V, T, NC, MODE>(a.act, MatrixList{a}, a.steps,
                                                                   blockIdx.x, gridDim.x);
}

// The column split inside the workgroup (a plan with splits > 1): the workgroup's waves come in
// sets of `ws` = the plan's column chunks, wave w taking chunk w % ws of row step `slot` =
// w / ws of each workgroup step. After a step the row sums of the chunks (stored by the tiles
// as for the split-K workspace, here into LDS) are added in chunk order, the order of the
// split-K reduce, and written to the matrix each row step falls in, so y is bit-identical to
// the two-launch split in one launch. In the fused form the workgroup first quantizes every
// chunk of the row into LDS (its waves read all of them) and each wave takes its own chunk's
// slice from there. Every wave of a workgroup runs the same number of workgroup steps (the
// barriers), and the next step's loads go out before the sums over the chunks. `src` numbers
// the row steps (one matrix, several matrices, or one format's matrices of a mixed launch).
template <int V, int T, int NC, bool FUSED>
__host__ __device__ constexpr int split_slice_lds_bytes(int ws) {
    return FUSED ? act_slice_lds_bytes<V, T, NC>() * ws : 0;
}

template <class Tile, int V, int T, int NC, bool FUSED, class Steps>
__device__ __forceinline__ void gemv_split_walk(const GemvArgs &a, const Steps &src, int steps,
                                                int blk, int nblk) {
    constexpr int kStepRows = Tile::G * Tile::RPW;
    extern __shared__ float lds_split[];
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int ws = a.wg_splits;
    const int slots = (a.threads >> 6) / ws;
    const int split = wave % ws, slot = wave / ws;
    const LaneGeom<T, NC> L(a.nchunks, split);
    const int wg_steps = (steps + slots - 1) / slots;
    const int rows_local = slots * kStepRows;
    float *part = lds_split + split_slice_lds_bytes<V, T, NC, FUSED>(ws) / 4;   // [ws][V][rows_local]

    typename Tile::Regs regs;
    uint32_t xw[V][NC][8];
    float xs[V][NC];
    ActTerms<V, NC> at;
    ActPending<V, T, NC, FUSED> pend;
    const ChunkSpan sp{0, ws, split};
    act_slice_issue<V, T, NC, FUSED>(a, sp, L.g, L.cv, xw, xs, pend);
    int wst = blk;
    __builtin_amdgcn_sched_barrier(0);
    {
        const StepMat m = src.at(wst * slots + slot);   // rows clamped: valid for any step
        Tile::issue(regs, m.w, m.rows, m.nb, m.local, L);
    }
    __builtin_amdgcn_sched_barrier(0);
    act_slice_finish<V, T, NC, FUSED>(a, sp, L.cv, L.t, xw, xs, pend);
    act_terms<V, NC>(xw, at);
    for (; wst < wg_steps; wst += nblk) {
        __builtin_amdgcn_sched_barrier(0);
        // the workgroup-local rows: every local row is stored (rows past a matrix are dropped
        // below)
        Tile::template compute<false>(regs, xw, xs, at, part, rows_local, slot, L, nullptr,
                                      a.nchunks);
        __builtin_amdgcn_sched_barrier(0);
        if (wst + nblk < wg_steps) {
            const StepMat n = src.at((wst + nblk) * slots + slot);
            Tile::issue(regs, n.w, n.rows, n.nb, n.local, L);
        }
        __syncthreads();
        for (int i = static_cast<int>(threadIdx.x); i < V * rows_local; i += a.threads) {
            const int v = i / rows_local, rl = i - v * rows_local;
            const int st = wst * slots + rl / kStepRows;
            if (st < steps) {
                const StepMat m = src.at(st);
                const int row = m.local * kStepRows + (rl % kStepRows);
                float acc = part[v * rows_local + rl];
                for (int s = 1; s < ws; s++) acc += part[(s * V + v) * rows_local + rl];
                if (row < m.rows) m.out[static_cast<int64_t>(v) * m.rows + row] = acc;
            }
        }
        __syncthreads();
    }
}

template <class F, int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(64 * gemv_max_waves(V, T, NC)) gemv_split_kernel(GemvArgs a) {
    using Tile = typename F::template Tile<V, T, NC>;
    const int groups = (a.rows + Tile::RPW - 1) / Tile::RPW;
    const int steps = (groups + Tile::G - 1) / Tile::G;
    gemv_split_walk<Tile, V, T, NC, MODE == kModeFused>(a, OneMatrix{a}, steps, blockIdx.x,
                                                        gridDim.x);
}

// Several matrices of one format whose rows are wider than one pass: the same split walk over
// their combined step numbering.
template <class F, int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(64 * gemv_max_waves(V, T, NC))
    gemv_multi_split_fmt_kernel(MultiArgs a) {
    gemv_split_walk<typename F::template Tile<V, T, NC>, V, T, NC, MODE == kModeFused>(
        a.act, MatrixList{a}, a.steps, blockIdx.x, gridDim.x);
}

// The LDS layout above, as the host computes it.
static_assert(gemv_split_lds_bytes(3, 32, 2, true, 4, 8) ==
                  4 * act_slice_lds_bytes<3, 32, 2>() +
                      sizeof(float) * 3 * 8 * Q4kTile<3, 32, 2>::G * Q4kTile<3, 32, 2>::RPW,
              "split LDS layout");

// The launches of one format: tables over (vectors, lanes per row, chunks per lane) of the
// compiled instances (nvec * chunks <= 8, so the activation slice fits in VGPRs), one for the
// one-matrix kernel and one for several matrices of this format.
template <class F>
struct GemvLaunch {
    struct One {
        using Args = GemvArgs;
        template <int V, int T, int NC>
        static hipError_t run(const GemvArgs &a, const LaunchShape &s, bool debug,
                              hipStream_t stream) {
            if (s.waves < 1 || s.waves > gemv_max_waves(V, T, NC)) return hipErrorInvalidValue;
            const dim3 grid(static_cast<unsigned>(s.blocks), static_cast<unsigned>(s.splits));
            const dim3 block(static_cast<unsigned>(64 * s.waves));
            const size_t lds = act_slice_lds_bytes<V, T, NC>();
            GemvArgs b = a;
            b.threads = 64 * s.waves;
            if (debug)
                hipLaunchKernelGGL((gemv_kernel<F, V, T, NC, kModeDebug>), grid, block, 0, stream,
                                   b);
            else if (a.x != nullptr)
                hipLaunchKernelGGL((gemv_kernel<F, V, T, NC, kModeFused>), grid, block, lds,
                                   stream, b);
            else
                hipLaunchKernelGGL((gemv_kernel<F, V, T, NC, kModePlain>), grid, block, 0, stream,
                                   b);
            return hipGetLastError();
        }
    };

    struct Multi {
        using Args = MultiArgs;
        template <int V, int T, int NC>
        static hipError_t run(const MultiArgs &a, const LaunchShape &s, bool debug,
                              hipStream_t stream) {
            if (debug || s.waves < 1 || s.waves > 4 || s.splits != 1) return hipErrorInvalidValue;
            const dim3 grid(static_cast<unsigned>(s.blocks));
            const dim3 block(static_cast<unsigned>(64 * s.waves));
            const size_t lds = act_slice_lds_bytes<V, T, NC>();
            MultiArgs b = a;
            b.act.threads = 64 * s.waves;
            if (a.act.x != nullptr)
                hipLaunchKernelGGL((gemv_multi_fmt_kernel<F, V, T, NC, kModeFused>), grid, block,
                                   lds, stream, b);
            else
                hipLaunchKernelGGL((gemv_multi_fmt_kernel<F, V, T, NC, kModePlain>), grid, block,
                                   0, stream, b);
            return hipGetLastError();
        }
    };

    struct Split {
        using Args = GemvArgs;
        template <int V, int T, int NC>
        static hipError_t run(const GemvArgs &a, const LaunchShape &s, bool debug,
                              hipStream_t stream) {
            if (debug || s.splits < 2 || s.waves % s.splits != 0 ||
                s.waves > gemv_max_waves(V, T, NC))
                return hipErrorInvalidValue;
            const bool fused = a.x != nullptr;
            const size_t lds = gemv_split_lds_bytes(V, T, NC, fused, s.splits, s.waves);
            if (lds > kMaxSplitLds) return hipErrorInvalidValue;
            GemvArgs b = a;
            b.threads = 64 * s.waves;
            b.wg_splits = s.splits;
            const dim3 grid(static_cast<unsigned>(s.blocks)), block(static_cast<unsigned>(64 * s.waves));
            if (fused)
                hipLaunchKernelGGL((gemv_split_kernel<F, V, T, NC, kModeFused>), grid, block, lds,
                                   stream, b);
            else
                hipLaunchKernelGGL((gemv_split_kernel<F, V, T, NC, kModePlain>), grid, block, lds,
                                   stream, b);
            return hipGetLastError();
        }
    };

    struct MultiSplit {
        using Args = MultiArgs;
        template <int V, int T, int NC>
        static hipError_t run(const MultiArgs &a, const LaunchShape &s, bool debug,
                              hipStream_t stream) {
            if (debug || s.splits < 2 || s.waves % s.splits != 0 ||
                s.waves > gemv_max_waves(V, T, NC))
                return hipErrorInvalidValue;
            const bool fused = a.act.x != nullptr;
            const size_t lds = gemv_split_lds_bytes(V, T, NC, fused, s.splits, s.waves);
            if (lds > kMaxSplitLds) return hipErrorInvalidValue;
            MultiArgs b = a;
            b.act.threads = 64 * s.waves;
            b.act.wg_splits = s.splits;
            const dim3 grid(static_cast<unsigned>(s.blocks)), block(static_cast<unsigned>(64 * s.waves));
            if (fused)
                hipLaunchKernelGGL((gemv_multi_split_fmt_kernel<F, V, T, NC, kModeFused>), grid, block,
                                   lds, stream, b);
            else
                hipLaunchKernelGGL((gemv_multi_split_fmt_kernel<F, V, T, NC, kModePlain>), grid, block,
                                   lds, stream, b);
            return hipGetLastError();
        }
    };

    template <class K>
    struct Table {
        using Fn = hipError_t (*)(const typename K::Args &, const LaunchShape &, bool,
                                  hipStream_t);
        Fn fn[8][4][4] = {};
        template <int V, int T, int NC>
        constexpr void put(int ti) {
            if constexpr (V * NC <= 8) fn[V - 1][ti][NC - 1] = &K::template run<V, T, NC>;
        }
        template <int V, int T>
        constexpr void row(int ti) {
            put<V, T, 1>(ti);
            put<V, T, 2>(ti);
            put<V, T, 3>(ti);
            put<V, T, 4>(ti);
        }
        template <int V>
        constexpr void vec() {
            row<V, 8>(0);
            row<V, 16>(1);
            row<V, 32>(2);
            row<V, 64>(3);
        }
        constexpr Table() {
            vec<1>();
            vec<2>();
            vec<3>();
            vec<4>();
            vec<5>();
            vec<6>();
            vec<7>();
            vec<8>();
        }
    };

    template <class K>
    static hipError_t dispatch(const typename K::Args &a, const LaunchShape &s, int nvec,
                               bool debug, hipStream_t stream) {
        static const Table<K> table;
        int ti = -1;
        switch (s.lanes) {
            case 8: ti = 0; break;
            case 16: ti = 1; break;
            case 32: ti = 2; break;
            case 64: ti = 3; break;
            default: return hipErrorInvalidValue;
        }
        if (nvec < 1 || nvec > 8 || s.chunks < 1 || s.chunks > 4) return hipErrorInvalidValue;
        const auto fn = table.fn[nvec - 1][ti][s.chunks - 1];
        if (!fn) return hipErrorInvalidValue;
        return fn(a, s, debug, stream);
    }

    static hipError_t launch(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                             hipStream_t stream) {
        return dispatch<One>(a, s, nvec, debug, stream);
    }
    static hipError_t launch_multi(const MultiArgs &a, const LaunchShape &s, int nvec,
                                   hipStream_t stream) {
        return dispatch<Multi>(a, s, nvec, false, stream);
    }
    // s.splits = column chunks (the waves' sets), s.waves a multiple of it, s.blocks workgroups
    static hipError_t launch_split(const GemvArgs &a, const LaunchShape &s, int nvec,
                                   hipStream_t stream) {
        return dispatch<Split>(a, s, nvec, false, stream);
    }
    static hipError_t launch_multi_split(const MultiArgs &a, const LaunchShape &s, int nvec,
                                         hipStream_t stream) {
        return dispatch<MultiSplit>(a, s, nvec, false, stream);
    }
};

}  // namespace qgemv
