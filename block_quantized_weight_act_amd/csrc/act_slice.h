// The per-lane activation slice of the GEMV kernels: for each of a lane's NC chunks and each
// vector, the 32 int8 codes (8 words) and the float32 scale of that 32-column activation
// block. Either read from memory (codes and scales made by qgemv_quantize_act) or, in the
// fused form, quantized by the workgroup itself into LDS with the same arithmetic
// (quantize_act_oct), so one launch does both steps of the product.
//
// Getting the slice is split in two so that a kernel can put its first weight loads between
// the halves: act_slice_issue starts the slice's global loads, act_slice_finish consumes
// them. Loads complete in issue order, so the slice is waited for without waiting for the
// weight loads issued after it, and the weights' HBM latency overlaps the slice's work.
//
// In the fused form a workgroup quantizes a span of column chunks: `nch` consecutive chunks
// from chunk `ch0` (one chunk, blockIdx.y, for a workgroup that works on one column chunk; all
// of the row's chunks for a workgroup that splits the columns among its waves), and each wave
// then reads its own chunk `rel` of the span.
#pragma once

#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

// Shape of the fused form's work: the workgroup's column chunk holds kBlocks activation
// blocks (all vectors), kOcts groups of 8 elements, a block per 4 lanes (a DPP quad); each lane
// takes up to kSlots octs per round (oct base + i * a.threads + threadIdx.x of round base).
// kSlots is sized so that one round of a 256-thread workgroup covers the chunk (at most 2
// octs per lane; smaller workgroups and larger chunks take more rounds).
template <int V, int T, int NC>
struct FusedAct {
    static constexpr int kBlocks = V * T * NC;
    static constexpr int kOcts = kBlocks * 4;
    static constexpr int kSlots = kOcts >= 2 * 256 ? 2 : (kOcts + 255) / 256;
};

// LDS bytes the fused form needs: 32 code bytes and one float32 scale per block of the slice
// (of one column chunk; a span of nch chunks takes nch times as much).
template <int V, int T, int NC>
constexpr int act_slice_lds_bytes() {
    return FusedAct<V, T, NC>::kBlocks * (32 + 4);
}

// The column chunks a workgroup's fused form quantizes, and this wave's chunk among them.
struct ChunkSpan {
    int ch0, nch, rel;
};

// What act_slice_issue leaves in flight for act_slice_finish: the fused form's first round of
// float32 octs (the plain form loads straight into the slice registers).
template <int V, int T, int NC, bool FUSED>
struct ActPending {
    float4 xv[FUSED ? FusedAct<V, T, NC>::kSlots : 1][2];
};

namespace fused_detail {

// Oct od of the span: block blk = od / 4 is vector blk / (nch T NC) and column block
// ch0 T NC + blk % (nch T NC); elem is the offset of its 8 floats in x (and of its codes in
// xq_out). True when the oct exists (the same for the 4 octs of a block).
template <int V, int T, int NC>
__device__ __forceinline__ bool oct_at(const GemvArgs &a, const ChunkSpan &sp, int od,
                                       int64_t &elem, int &v, int &gc) {
    const int blk = od >> 2;
    const int span = sp.nch * T * NC;
    v = blk / span;
    gc = sp.ch0 * T * NC + (blk - v * span);
    elem = v * (static_cast<int64_t>(a.nchunks) * 32) + 32 * static_cast<int64_t>(gc) +
           8 * (od & 3);
    return od < FusedAct<V, T, NC>::kOcts * sp.nch && gc < a.nchunks;
}

template <int V, int T, int NC>
__device__ __forceinline__ void load_round(const GemvArgs &a, const ChunkSpan &sp, int base,
                                           float4 (&xv)[FusedAct<V, T, NC>::kSlots][2]) {
#pragma unroll
    for (int i = 0; i < FusedAct<V, T, NC>::kSlots; i++) {
        int64_t elem;
        int v, gc;
        const bool ok = oct_at<V, T, NC>(
            a, sp, base + i * a.threads + static_cast<int>(threadIdx.x), elem, v, gc);
        const float4 *p = reinterpret_cast<const float4 *>(a.x + elem);
        xv[i][0] = ok ? p[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        xv[i][1] = ok ? p[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Quantize one round into LDS (codes words 2 od, 2 od + 1, then the scale of block od / 4
// after all the span's codes); the first workgroup of the span also stores them to xq_out /
// xd_out (4-byte stores: xq_out need only be 4-byte aligned).
template <int V, int T, int NC>
__device__ __forceinline__ void store_round(const GemvArgs &a, const ChunkSpan &sp, int base,
                                            const float4 (&xv)[FusedAct<V, T, NC>::kSlots][2]) {
    using F = FusedAct<V, T, NC>;
    extern __shared__ uint4 lds[];
    const int octs = F::kOcts * sp.nch;
    uint2 *s_codes = reinterpret_cast<uint2 *>(lds);
    float *s_scale = reinterpret_cast<float *>(lds + 2 * F::kBlocks * sp.nch);
#pragma unroll
    for (int i = 0; i < F::kSlots; i++) {
        const int first = base + i * a.threads;   // the same for the workgroup
        if (first >= octs) break;
        const int od = first + static_cast<int>(threadIdx.x);
        int64_t elem;
        int v, gc;
        const bool ok = oct_at<V, T, NC>(a, sp, od, elem, v, gc);
        const ActOct q = quantize_act_oct(xv[i][0], xv[i][1]);   // every lane: DPP over 4
        if (od < octs) {
            s_codes[od] = make_uint2(q.lo, q.hi);
            if ((od & 3) == 0) s_scale[od >> 2] = q.scale;
        }
        if (ok && blockIdx.x == 0 && a.xq_out != nullptr) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.xq_out + elem);
            dst[0] = q.lo;
            dst[1] = q.hi;
            if ((od & 3) == 0) a.xd_out[static_cast<int64_t>(v) * a.nchunks + gc] = q.scale;
        }
    }
}

}  // namespace fused_detail

template <int V, int T, int NC, bool FUSED>
__device__ __forceinline__ void act_slice_issue(const GemvArgs &a, const ChunkSpan &sp,
                                                const int (&g)[NC], const bool (&cv)[NC],
                                                uint32_t (&xw)[V][NC][8], float (&xs)[V][NC],
                                                ActPending<V, T, NC, FUSED> &pend) {
    if constexpr (FUSED) {
        (void)g; (void)cv; (void)xw; (void)xs;
        fused_detail::load_round<V, T, NC>(a, sp, 0, pend.xv);
    } else {
        (void)pend; (void)sp;
        const int nsub = a.nchunks;
        const int64_t cols = static_cast<int64_t>(nsub) * 32;
#pragma unroll
        for (int v = 0; v < V; v++) {
#pragma unroll
            for (int k = 0; k < NC; k++) {
                uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
                float s = 0.0f;
                if (cv[k]) {
                    const int8_t *p = a.xq + v * cols + 32 * static_cast<int64_t>(g[k]);
                    lo = load16(p);
                    hi = load16(p + 16);
                    s = a.xd[static_cast<int64_t>(v) * nsub + g[k]];
                }
                xw[v][k][0] = lo.x; xw[v][k][1] = lo.y; xw[v][k][2] = lo.z; xw[v][k][3] = lo.w;
                xw[v][k][4] = hi.x; xw[v][k][5] = hi.y; xw[v][k][6] = hi.z; xw[v][k][7] = hi.w;
                xs[v][k] = s;
            }
        }
    }
}

template <int V, int T, int NC, bool FUSED>
__device__ __forceinline__ void act_slice_finish(const GemvArgs &a, const ChunkSpan &sp,
                                                 const bool (&cv)[NC], int t,
                                                 uint32_t (&xw)[V][NC][8], float (&xs)[V][NC],
                                                 ActPending<V, T, NC, FUSED> &pend) {
    if constexpr (FUSED) {
        using F = FusedAct<V, T, NC>;
        const int round = F::kSlots * a.threads;
        const int octs = F::kOcts * sp.nch;
        fused_detail::store_round<V, T, NC>(a, sp, 0, pend.xv);
        for (int base = round; base < octs; base += round) {
            fused_detail::load_round<V, T, NC>(a, sp, base, pend.xv);
            fused_detail::store_round<V, T, NC>(a, sp, base, pend.xv);
        }
        __syncthreads();
        extern __shared__ uint4 lds[];
        const float *s_scale = reinterpret_cast<const float *>(lds + 2 * F::kBlocks * sp.nch);
#pragma unroll
        for (int v = 0; v < V; v++) {
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const int blk = (v * sp.nch + sp.rel) * T * NC + t + T * k;
                const uint4 lo = cv[k] ? lds[2 * blk] : make_uint4(0, 0, 0, 0);
                const uint4 hi = cv[k] ? lds[2 * blk + 1] : make_uint4(0, 0, 0, 0);
                xw[v][k][0] = lo.x; xw[v][k][1] = lo.y; xw[v][k][2] = lo.z; xw[v][k][3] = lo.w;
                xw[v][k][4] = hi.x; xw[v][k][5] = hi.y; xw[v][k][6] = hi.z; xw[v][k][7] = hi.w;
                xs[v][k] = cv[k] ? s_scale[blk] : 0.0f;
            }
        }
    } else {
        (void)a; (void)sp; (void)cv; (void)t; (void)xw; (void)xs; (void)pend;
    }
}

}  // namespace qgemv
