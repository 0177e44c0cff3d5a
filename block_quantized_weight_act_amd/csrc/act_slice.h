// The per-lane activation slice of the GEMV kernels: for each of a lane's NC chunks and each
// vector, the 32 int8 codes (8 words) and the float32 scale of that 32-column activation
// block. Either read from memory (codes and scales made by qgemv_quantize_act) or, when the
// kernel is given the float32 activation, quantized by the workgroup itself into LDS with the
// same arithmetic (quantize_act_quad), so one launch does both steps of the product.
#pragma once

#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

// LDS bytes the fused form needs: 32 code bytes and one float32 scale per block of the slice.
template <int V, int T, int NC>
constexpr int act_slice_lds_bytes() {
    return V * T * NC * (32 + 4);
}

template <int V, int T, int NC>
__device__ __forceinline__ void load_act_slice(const GemvArgs &a, const int (&g)[NC],
                                               const bool (&cv)[NC], int t,
                                               uint32_t (&xw)[V][NC][8], float (&xs)[V][NC]) {
    const int nsub = a.nchunks;
    const int64_t cols = static_cast<int64_t>(nsub) * 32;
    if (a.x != nullptr) {
        // The workgroup quantizes the blocks of its column chunk (all vectors) once: quad qd
        // (4 elements) of block blk = qd / 8; block blk is vector blk / (T NC), local block
        // blk % (T NC) = column block chunk0 + local. Blocks past the end of the row are zero.
        constexpr int kBlocks = V * T * NC;
        extern __shared__ uint4 lds[];
        uint32_t *s_codes = reinterpret_cast<uint32_t *>(lds);
        float *s_scale = reinterpret_cast<float *>(lds + 2 * kBlocks);
        const int chunk0 = static_cast<int>(blockIdx.y) * T * NC;
        for (int base = 0; base < kBlocks * 8; base += blockDim.x) {
            const int qd = base + static_cast<int>(threadIdx.x);
            const int blk = qd >> 3;
            const int v = blk / (T * NC), lb = blk % (T * NC);
            const int gc = chunk0 + lb;
            const bool in_slice = qd < kBlocks * 8;
            const bool ok = in_slice && gc < nsub;
            const int64_t elem = v * cols + 32 * static_cast<int64_t>(gc) + 4 * (qd & 7);
            const float4 xv = ok ? *reinterpret_cast<const float4 *>(a.x + elem)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
            const ActQuad q = quantize_act_quad(xv);
            if (in_slice) {
                s_codes[qd] = q.codes;
                if ((qd & 7) == 0) s_scale[blk] = q.scale;
            }
            if (ok && blockIdx.x == 0 && a.xq_out != nullptr) {
                *reinterpret_cast<uint32_t *>(a.xq_out + elem) = q.codes;
                if ((qd & 7) == 0) a.xd_out[static_cast<int64_t>(v) * nsub + gc] = q.scale;
            }
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < V; v++) {
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const int blk = v * T * NC + t + T * k;
                const uint4 lo = cv[k] ? lds[2 * blk] : make_uint4(0, 0, 0, 0);
                const uint4 hi = cv[k] ? lds[2 * blk + 1] : make_uint4(0, 0, 0, 0);
                xw[v][k][0] = lo.x; xw[v][k][1] = lo.y; xw[v][k][2] = lo.z; xw[v][k][3] = lo.w;
                xw[v][k][4] = hi.x; xw[v][k][5] = hi.y; xw[v][k][6] = hi.z; xw[v][k][7] = hi.w;
                xs[v][k] = cv[k] ? s_scale[blk] : 0.0f;
            }
        }
        return;
    }
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

}  // namespace qgemv
