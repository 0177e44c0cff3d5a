// Several matrices that multiply the same activation, in one launch (any mix of Q4_K, Q6_K,
// Q4_0 and Q8_0, up to kMaxMats of them, all with the same column count).
//
// genie-ai-runtime (jared-hpc.com), "v1.2.0": the attention projections of a decode step share
// one quantized activation, which is made once and read by all of them instead of once per
// product. Here they also share one launch: the matrices' row steps are numbered one after
// the other and waves walk the combined numbering with a grid-wide stride, each step taking the
// tile (tile.h) of the matrix it falls in. A wave's activation slice is loaded (or,
// in the fused form, quantized by its workgroup) once and serves every matrix, since lane t's
// columns are the same in all of them. No column split: the shared lane geometry covers a
// whole row (at most 256 chunks, 8192 columns). This file holds the kernel for a mix of
// formats; matrices all of one format take the one-matrix walk over the same step numbering
// (gemv_multi_fmt_kernel in gemv_walk.h).
#include "gemv_walk.h"

namespace qgemv {

template <int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(256) gemv_multi_kernel(MultiArgs a) {
    constexpr bool FUSED = MODE == kModeFused;
    using T4 = Q4kTile<V, T, NC>;
    using T6 = Q6kTile<V, T, NC>;
    using T40 = Q40Tile<V, T, NC>;
    using T80 = Q80Tile<V, T, NC>;
    static_assert(T4::G == T6::G && T4::G == T40::G && T4::G == T80::G && T4::RPW == T6::RPW,
                  "one step geometry for every format");
    const LaneGeom<T, NC> L(a.act.nchunks);
    // the wave index is the same in all 64 lanes: keep it (and the step numbers) in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int wpb = a.act.threads >> 6;
    const int stride = gridDim.x * wpb;
    const int st0 = blockIdx.x * wpb + wave;
    typename T4::Regs regs;                  // one register set for every format
    auto issue = [&](int st) {
        const StepMat m = MatrixList{a}.at(st);
        if (m.wtype == kTypeQ4K)
            T4::issue(regs, m.w, m.rows, m.nb, m.local, L);
        else if (m.wtype == kTypeQ6K)
            T6::issue(regs, m.w, m.rows, m.nb, m.local, L);
        else if (m.wtype == kTypeQ40)
            T40::issue(regs, m.w, m.rows, m.nb, m.local, L);
        else
            T80::issue(regs, m.w, m.rows, m.nb, m.local, L);
    };

    // Unlike the one-format walk, the first step's weights are not loaded ahead of the slice:
    // with the load sequence chosen by a branch on the format, the compiler's wait for the
    // slice at the branches' join waits for every load issued in them, so loading the weights
    // first only moved their latency in front of the slice's (measured slower); the walk keeps
    // the plain order, loads then arithmetic.
    uint32_t xw[V][NC][8];
    float xs[V][NC];
    ActTerms<V, NC> at;
    ActPending<V, T, NC, FUSED> pend;
    act_slice_issue<V, T, NC, FUSED>(a.act, L.g, L.cv, xw, xs, pend);
    act_slice_finish<V, T, NC, FUSED>(a.act, L.cv, L.t, xw, xs, pend);
    act_terms<V, NC>(xw, at);

    for (int st = st0; st < a.steps; st += stride) {
        issue(st);
        __builtin_amdgcn_sched_barrier(0);
        const StepMat m = MatrixList{a}.at(st);
        const int nsub = a.act.nchunks;
        if (m.wtype == kTypeQ4K)
            T4::template compute<false>(regs, xw, xs, at, m.out, m.rows, m.local, L, nullptr, nsub);
        else if (m.wtype == kTypeQ6K)
            T6::template compute<false>(regs, xw, xs, at, m.out, m.rows, m.local, L, nullptr, nsub);
        else if (m.wtype == kTypeQ40)
            T40::template compute<false>(regs, xw, xs, at, m.out, m.rows, m.local, L, nullptr,
                                         nsub);
        else
            T80::template compute<false>(regs, xw, xs, at, m.out, m.rows, m.local, L, nullptr,
                                         nsub);
        __builtin_amdgcn_sched_barrier(0);
    }
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
constexpr MultiLauncher pick() {
    if constexpr (V * NC <= 8)
        return &launch_multi_variant<V, T, NC>;
    else
        return nullptr;
}

#define QGEMV_NC_ROW(V, T) {pick<V, T, 1>(), pick<V, T, 2>(), pick<V, T, 3>(), pick<V, T, 4>()}
#define QGEMV_T_ROW(V) \
    {QGEMV_NC_ROW(V, 8), QGEMV_NC_ROW(V, 16), QGEMV_NC_ROW(V, 32), QGEMV_NC_ROW(V, 64)}
const MultiLauncher kMultiTable[8][4][4] = {QGEMV_T_ROW(1), QGEMV_T_ROW(2), QGEMV_T_ROW(3),
                                            QGEMV_T_ROW(4), QGEMV_T_ROW(5), QGEMV_T_ROW(6),
                                            QGEMV_T_ROW(7), QGEMV_T_ROW(8)};
#undef QGEMV_T_ROW
#undef QGEMV_NC_ROW

}  // namespace

hipError_t launch_gemv_multi(const MultiArgs &a, const LaunchShape &s, int nvec,
                             hipStream_t stream) {
    int ti = -1;
    switch (s.lanes) {
        case 8: ti = 0; break;
        case 16: ti = 1; break;
        case 32: ti = 2; break;
        case 64: ti = 3; break;
        default: return hipErrorInvalidValue;
    }
    if (nvec < 1 || nvec > 8 || s.chunks < 1 || s.chunks > 4 || s.splits != 1)
        return hipErrorInvalidValue;
    const MultiLauncher fn = kMultiTable[nvec - 1][ti][s.chunks - 1];
    if (!fn) return hipErrorInvalidValue;
    return fn(a, s, stream);
}

}  // namespace qgemv
