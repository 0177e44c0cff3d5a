// Q4_K weight x int8 activation GEMV for gfx950.
//
// genie-ai-runtime (jared-hpc.com), "The decode arc": the Q4_K matrix-vector product is done
// with int8 4-way dot products instead of dequantizing to floating point, the 4-bit codes are
// handled as whole 32-bit words, and a row is shared by the lanes of one warp. "v1.3.0": when
// rows alone cannot fill the GPU, split the reduction dimension and sum the pieces in a
// separate pass. Here, for a 64-lane gfx950 wavefront:
//
//  * A row is cut into 16-byte chunks of codes. In the Q4_K layout one chunk is exactly one
//    32-column sub-block j, so a lane owns whole sub-blocks: its integer partial
//    P = sum q * xq is exact inside the lane, its low nibbles meet activation bytes 0..15
//    and its high nibbles bytes 16..31 of the same activation block (4 codes per
//    v_dot4_i32_i8 after one AND / shift of a 32-bit word).
//  * T consecutive lanes share a row; lane t takes chunks t, t + T, ... (NC of them), so its
//    columns are the same for every row it visits: the activation codes, scales and block
//    sums it needs stay in VGPRs for the whole kernel and are read from memory once.
//  * The tensor keeps codes and headers in separate planes. 8 consecutive lanes read the 128
//    code bytes of one super-block with one 16-byte load each (a contiguous 128-byte run that
//    no other load touches, so it is read with a nontemporal load and streamed past the
//    caches); the 16-byte header (d, dmin, packed 6-bit scales) is one ordinary 16-byte load
//    from the header plane, the same address for those 8 lanes, and stays cached for the
//    neighbouring blocks whose headers share its cache line.
//  * After the chunks of a row, the T lanes' float sums are combined with a log2(T)-step
//    butterfly; lane t < nvec writes vector t's output.
//  * Waves walk row groups with a grid-wide stride. blockIdx.y selects a column chunk
//    (split-K) whose partial sums go to a workspace that a second kernel adds in order.
//
// The float32 work per sub-block is xd * (d * (sc * P) - dmin * (m * S)): sc * P and m * S
// are exact integers below 2^24. The two products can nearly cancel (a dequantized weight
// d sc q - dmin m close to 0), so the difference is formed with the exact rounding error of
// the min product (a TwoProduct through fmaf) and carries a relative error of about two
// float32 roundings of the sub-block's own value; a sub-block whose dequantized weights
// times activations are all zero contributes exactly zero. The library is built with
// -ffp-contract=off: every fused multiply-add is an explicit fmaf.
#include "act_slice.h"
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

template <int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(256) gemv_q4k_kernel(GemvArgs a) {
    constexpr bool DBG = MODE == kModeDebug;
    constexpr int RPW = 64 / T;              // rows per wave step
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wpb = blockDim.x >> 6;
    const int t = lane & (T - 1);
    const int rsub = lane / T;
    const int split = blockIdx.y;
    const int j = t & 7;                     // sub-block inside the super-block
    const int nsub = a.nchunks;              // 32-column blocks per row
    const int64_t cols = static_cast<int64_t>(nsub) * 32;

    int g[NC];
    bool cv[NC];
    uint32_t hoff[NC], qoff[NC];             // byte offsets of this lane's header / codes in a row
#pragma unroll
    for (int k = 0; k < NC; k++) {
        g[k] = split * T * NC + t + T * k;
        cv[k] = g[k] < nsub;
        // A chunk past the end of the row reads the row's first block instead (always valid
        // memory) and meets an all-zero activation slice below, so it adds exactly zero.
        const uint32_t b = cv[k] ? static_cast<uint32_t>(g[k] >> 3) : 0u;
        hoff[k] = b * 16;
        qoff[k] = b * 128 + 16 * j;
    }

    // Steps of G consecutive row groups: this wave takes steps wave_id, wave_id + stride, ...
    // All loads of a step are issued first and are unconditional: a row past the end of the
    // matrix is clamped to the last row (its result is not stored), so there are no divergent
    // branches around the loads.
    constexpr int G = groups_per_step(NC);
    const int groups = (a.rows + RPW - 1) / RPW;
    const int steps = (groups + G - 1) / G;
    const int stride = gridDim.x * wpb;
    const uint8_t *hplane = a.w + static_cast<int64_t>(a.rows) * a.nb * 128;
    uint4 hdr_s[G][NC], qs_s[G][NC];
    auto issue_step = [&](int st) {
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + rsub;
            const int64_t brow = static_cast<int64_t>(row < a.rows ? row : a.rows - 1) * a.nb;
            const uint8_t *qrow = a.w + brow * 128;
            const uint8_t *hrow = hplane + brow * 16;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                hdr_s[gg][k] = load16(hrow + hoff[k]);
                qs_s[gg][k] = load16_stream(qrow + qoff[k]);
            }
        }
    };

    // This lane's activation slice: 32 codes, the block scale and the block code sum per chunk.
    // Its loads go out first, then the first step's weight loads, then the slice is finished
    // while the weights are in flight.
    constexpr bool FUSED = MODE == kModeFused;
    uint32_t xw[V][NC][8];
    float xs[V][NC];
    float xsumf[V][NC];                      // code sums as float (exact: |S| <= 4064)
    ActPending<V, T, NC, FUSED> pend;
    act_slice_issue<V, T, NC, FUSED>(a, g, cv, xw, xs, pend);
    const int st0 = blockIdx.x * wpb + wave;
    __builtin_amdgcn_sched_barrier(0);
    issue_step(st0);                         // rows (>= 1) clamped: valid even when st0 >= steps
    __builtin_amdgcn_sched_barrier(0);
    act_slice_finish<V, T, NC, FUSED>(a, cv, t, xw, xs, pend);
#pragma unroll
    for (int v = 0; v < V; v++) {
#pragma unroll
        for (int k = 0; k < NC; k++) {
            int sum = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) sum = byte_sum(xw[v][k][i], sum);
            xsumf[v][k] = static_cast<float>(sum);
            if (DBG && cv[k] && blockIdx.x == 0 && wave == 0 && rsub == 0)
                a.S[static_cast<int64_t>(v) * nsub + g[k]] = sum;
        }
    }

    for (int st = st0; st < steps; st += stride) {
        // Keep every load of the step ahead of the arithmetic: without this fence the
        // scheduler interleaves them to save registers and waits for each load in turn.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + rsub;
            const bool rv = row < a.rows;
            const uint4 *hdr = hdr_s[gg];
            const uint4 *qs = qs_s[gg];
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; v++) acc[v] = 0.0f;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const float d = half_to_float(hdr[k].x & 0xFFFFu);
                const float dmin = half_to_float(hdr[k].x >> 16);
                const int sc = static_cast<int>(((hdr[k].y >> (4 * j)) & 15u) |
                                                (((hdr[k].w >> (2 * j)) & 3u) << 4));
                const int m = static_cast<int>(((hdr[k].z >> (4 * j)) & 15u) |
                                               (((hdr[k].w >> (16 + 2 * j)) & 3u) << 4));
                // d * sc and dmin * m are exact in float32 (11-bit fp16 significand times a
                // 6-bit integer) and shared by every vector.
                const float dsc = d * static_cast<float>(sc);
                const float dm = dmin * static_cast<float>(m);
                const uint32_t q[4] = {qs[k].x, qs[k].y, qs[k].z, qs[k].w};
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    lo[i] = q[i] & 0x0F0F0F0Fu;
                    hi[i] = (q[i] >> 4) & 0x0F0F0F0Fu;
                }
#pragma unroll
                for (int v = 0; v < V; v++) {
                    int P = 0;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        P = dot4(lo[i], xw[v][k][i], P);
                        P = dot4(hi[i], xw[v][k][4 + i], P);
                    }
                    // (d sc) P - (dmin m) S rounded once: pb is the rounded min product and
                    // eb its exact rounding error, so fmaf(d sc, P, -pb) - eb is the exact
                    // difference up to two roundings of quantities no larger than the result
                    // (plus eps^2 |pb|); a sub-block whose terms cancel keeps its relative
                    // accuracy.
                    const float pb = dm * xsumf[v][k];
                    const float eb = fmaf(dm, xsumf[v][k], -pb);
                    const float diff = fmaf(dsc, static_cast<float>(P), -pb) - eb;
                    acc[v] = fmaf(xs[v][k], diff, acc[v]);
                    if (DBG && rv && cv[k])
                        a.P[(static_cast<int64_t>(v) * a.rows + row) * nsub + g[k]] = P;
                }
            }
            if constexpr (T == 64 && V >= 3) {
                // one row per wave: scatter the vectors' sums over groups of 8 lanes
                const float o = wave_reduce_scatter8(acc);
                const int vi = scatter_index(lane);
                if (!DBG && rv && (lane & 7) == 0 && vi < V)
                    a.out[(static_cast<int64_t>(split) * V + vi) * a.rows + row] = o;
            } else {
#pragma unroll
                for (int v = 0; v < V; v++) acc[v] = group_sum<T>(acc[v]);
                if (!DBG && rv && t < V) {   // the debug variant writes P and S only
                    float o = acc[0];
#pragma unroll
                    for (int v = 1; v < V; v++)
                        if (t == v) o = acc[v];
                    a.out[(static_cast<int64_t>(split) * V + t) * a.rows + row] = o;
                }
            }
        }
        // The next step's loads go out as soon as this step's arithmetic is done, so the
        // values of one step are never live across the loop's back edge with the next ones.
        __builtin_amdgcn_sched_barrier(0);
        if (st + stride < steps) issue_step(st + stride);
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
        hipLaunchKernelGGL((gemv_q4k_kernel<V, T, NC, kModeDebug>), grid, block, 0, stream, a);
    else if (a.x != nullptr)
        hipLaunchKernelGGL((gemv_q4k_kernel<V, T, NC, kModeFused>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((gemv_q4k_kernel<V, T, NC, kModePlain>), grid, block, 0, stream, a);
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

hipError_t launch_gemv_q4k(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream) {
    const int ti = lanes_index(s.lanes);
    if (nvec < 1 || nvec > 8 || ti < 0 || s.chunks < 1 || s.chunks > 4) return hipErrorInvalidValue;
    const Launcher fn = kTable[nvec - 1][ti][s.chunks - 1];
    if (!fn) return hipErrorInvalidValue;
    return fn(a, s, debug, stream);
}

}  // namespace qgemv
