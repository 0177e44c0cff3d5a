// Q6_K weight x int8 activation GEMV for gfx950.
//
// genie-ai-runtime (jared-hpc.com), "The decode arc": int8 4-way dot-product mat-vec for
// Q6_K; "v1.3.0": split the reduction dimension when rows alone cannot fill the GPU.
//
// Same lane geometry as the Q4_K kernel: a 16-byte chunk of the low-bit plane holds the low
// 4 bits of one 32-column activation block (sub-blocks 2k and 2k+1 of the super-block, in
// the low and high nibbles), the 8 matching bytes of the high-bit plane hold their high 2
// bits arranged so that one shift and mask of a 32-bit word lines them up under the 4 codes
// of the matching low-bit word. A lane rebuilds 4 codes q in [0, 63] per word with
// AND / shift / OR, takes v_dot4_i32_i8 against the activation codes and removes the offset
// of 32 afterwards: sum (q - 32) * x = sum q * x - 32 * sum x, with the activation sums of
// each 16-column half kept in VGPRs. All integer work is exact: |sc * P| < 2^23 per
// sub-block and the sum over the two sub-blocks of a chunk stays below 2^24, so its
// float32 conversion is exact as well.
//
// The tensor keeps each field in its own plane (low bits, high bits, scales, super-scales),
// so every load is naturally aligned, and the low- and high-bit runs that 8 consecutive lanes
// read (128 and 64 contiguous bytes) are touched by no other load: they are read with
// nontemporal loads and streamed past the caches, while the small scale and super-scale
// loads stay cached for the neighbouring blocks that share their lines.
#include "act_slice.h"
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

template <int V, int T, int NC, int MODE>
__global__ void __launch_bounds__(256) gemv_q6k_kernel(GemvArgs a) {
    constexpr bool DBG = MODE == kModeDebug;
    constexpr int RPW = 64 / T;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wpb = blockDim.x >> 6;
    const int t = lane & (T - 1);
    const int rsub = lane / T;
    const int split = blockIdx.y;
    const int kk = t & 7;                    // chunk inside the super-block
    const int nsub = a.nchunks;              // 32-column blocks per row
    const int64_t cols = static_cast<int64_t>(nsub) * 32;
    const int64_t nblocks = static_cast<int64_t>(a.rows) * a.nb;
    const uint8_t *hplane = a.w + nblocks * 128;      // high bits, 64 bytes per block
    const uint8_t *splane = a.w + nblocks * 192;      // sub-scales, 16 bytes per block
    const uint16_t *dplane = reinterpret_cast<const uint16_t *>(a.w + nblocks * 208);

    int g[NC];
    bool cv[NC];
    uint32_t boff[NC];                       // index of this lane's block within a row
#pragma unroll
    for (int k = 0; k < NC; k++) {
        g[k] = split * T * NC + t + T * k;
        cv[k] = g[k] < nsub;
        // A chunk past the end of the row reads the row's first block instead (always valid
        // memory) and meets an all-zero activation slice below, so it adds exactly zero.
        boff[k] = cv[k] ? static_cast<uint32_t>(g[k] >> 3) : 0u;
    }

    // Steps of G row groups as in the Q4_K kernel: unconditional loads, rows clamped to the
    // last one, every load of a step issued before its arithmetic.
    constexpr int G = groups_per_step(NC);
    const int groups = (a.rows + RPW - 1) / RPW;
    const int steps = (groups + G - 1) / G;
    const int stride = gridDim.x * wpb;
    uint4 ql_s[G][NC];
    uint2 qh_s[G][NC];
    uint32_t scw_s[G][NC], dbits_s[G][NC];
    auto issue_step = [&](int st) {
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + rsub;
            const int64_t brow = static_cast<int64_t>(row < a.rows ? row : a.rows - 1) * a.nb;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const int64_t b = brow + boff[k];
                ql_s[gg][k] = load16_stream(a.w + b * 128 + 16 * kk);
                qh_s[gg][k] = load8_stream(hplane + b * 64 + 8 * kk);
                scw_s[gg][k] = *reinterpret_cast<const uint32_t *>(splane + b * 16 + 4 * (kk >> 1));
                dbits_s[gg][k] = dplane[b];
            }
        }
    };

    // The activation slice's loads, then the first step's weight loads, then the slice is
    // finished while the weights are in flight.
    constexpr bool FUSED = MODE == kModeFused;
    uint32_t xw[V][NC][8];
    float xs[V][NC];
    int xlo[V][NC], xhi[V][NC];             // activation code sums of the two 16-column halves
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
            int s0 = 0, s1 = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                s0 = byte_sum(xw[v][k][i], s0);
                s1 = byte_sum(xw[v][k][4 + i], s1);
            }
            xlo[v][k] = s0;
            xhi[v][k] = s1;
            if (DBG && cv[k] && blockIdx.x == 0 && wave == 0 && rsub == 0)
                a.S[static_cast<int64_t>(v) * nsub + g[k]] = s0 + s1;
        }
    }

    for (int st = st0; st < steps; st += stride) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + rsub;
            const bool rv = row < a.rows;
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; v++) acc[v] = 0.0f;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const float d = half_to_float(dbits_s[gg][k]);
                const int sh = 16 * (kk & 1);
                const int sc_lo = static_cast<int>(static_cast<int8_t>(scw_s[gg][k] >> sh));
                const int sc_hi = static_cast<int>(static_cast<int8_t>(scw_s[gg][k] >> (sh + 8)));
                const uint4 l4 = ql_s[gg][k];
                const uint2 h2 = qh_s[gg][k];
                const uint32_t w4[4] = {l4.x, l4.y, l4.z, l4.w};
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    lo[s] = (w4[s] & 0x0F0F0F0Fu) | (((h2.x >> (2 * s)) & 0x03030303u) << 4);
                    hi[s] = ((w4[s] >> 4) & 0x0F0F0F0Fu) | (((h2.y >> (2 * s)) & 0x03030303u) << 4);
                }
#pragma unroll
                for (int v = 0; v < V; v++) {
                    int plo = 0, phi = 0;
#pragma unroll
                    for (int s = 0; s < 4; s++) {
                        plo = dot4(lo[s], xw[v][k][s], plo);
                        phi = dot4(hi[s], xw[v][k][4 + s], phi);
                    }
                    plo -= 32 * xlo[v][k];
                    phi -= 32 * xhi[v][k];
                    const int scp = sc_lo * plo + sc_hi * phi;
                    acc[v] = fmaf(xs[v][k] * d, static_cast<float>(scp), acc[v]);
                    if (DBG && rv && cv[k]) {
                        int32_t *pp = a.P + (static_cast<int64_t>(v) * a.rows + row) * (2 * nsub);
                        pp[2 * g[k]] = plo;
                        pp[2 * g[k] + 1] = phi;
                    }
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
