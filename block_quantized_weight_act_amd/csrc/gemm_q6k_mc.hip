// Q6_K weights x 9..256 int8 activation vectors on the integer matrix cores
// (v_mfma_i32_32x32x16_i8).
//
// Many vectors (several tokens verified or prefilled at once) make the vector kernel's int8
// 4-way dot products the bottleneck, and groups of 8 vectors re-read every weight once per
// group (oxinfer README, "Speculative decoding": the multi-token int8 variants are
// instruction-bound at Q4). Q6_K's sub-block is 16 weights with its own int8 scale, and one
// 32 x 32 x 16 product is exactly one sub-block of 32 rows against 32 vectors, so its int32
// result is the sub-block's exact integer partial P = sum (q - 32) * xq for every (row,
// vector) with no zero-masked operand halves:
//
//  * The weight operand is q - 32 as int8 (q the 6-bit code, -32..31). The workgroup forms it
//    once per loaded weight while staging (low nibble from the low-bit plane, two bits from
//    the high-bit plane, then the offset), so every wave reads ready operands from LDS.
//  * Per (row, vector, 32-column block) the two sub-blocks' partials are combined in integer,
//    T = sc0 * P0 + sc1 * P1 (exact: |T| < 2^24), converted once and accumulated with one fma
//    with the activation block's scale xd; the super-block scale d multiplies the step's sum
//    once.
//  * Transposed product: the activation is the row operand (32 vectors), the weights the
//    column operand (32 weight rows), so a lane owns one weight row (its sub-scales and d are
//    per-lane values) and 16 vectors of its wave's tile.
//
// Work split, staging and double buffering as for the 32-weight formats (gemm_q32.hip): a
// workgroup of 4 waves computes 32 RG TR weight rows x 32 VW vectors (RG * VW = 4; each wave TR
// tiles of 32 rows x 32 vectors, so the activation operand and the 16 activation scales a
// lane reads from LDS per block serve TR products) over one column split, in steps of KS
// activation blocks: a whole super-block (8 blocks, 16 sub-blocks: whole 128-byte runs of the
// low-bit plane, one LDS buffer) or half of one (two LDS buffers); the next step's loads are in
// registers while the current step's products read LDS. Rows past the matrix read its last row and are not stored;
// vectors past nvec read zero codes and are not stored. Q6_K rows are whole super-blocks, so
// every step is whole.
//
// Lane layout of the 32 x 32 x 16 int8 product: operand lane l holds row (or column) l % 32
// and K slots 8 (l / 32) .. + 7; result element i is row 8 (i / 4) + 4 (l / 32) + i % 4,
// column l % 32 (the layout of the other 32 x 32 products, with half the K slots per lane).
#include "device_common.h"
#include "gemm_mc.h"

namespace qgemv {

namespace {

typedef int v16i_t __attribute__((ext_vector_type(16)));

// LDS row pitch of the weight operands and of the activation codes: 32 bytes per block plus 8,
// so the 8-byte operand reads of consecutive lanes (consecutive rows) fall in distinct banks
template <int KS>
__host__ __device__ constexpr int pitch6() { return 32 * KS + 8; }

// LDS of one step's buffer: weight operands [32 RW rows][pitch], sub-block scales
// [32 RW][2 KS] int8, super-block scales [32 RW] float, activation codes [32 VW vectors][pitch],
// activation scales [KS blocks][32 VW] float. Every part starts 16-byte aligned.
template <int RW, int VW, int KS>
__host__ __device__ constexpr int q6k_buf_bytes() {
    return 32 * RW * (pitch6<KS>() + 2 * KS + 4) + 32 * VW * (pitch6<KS>() + 4 * KS);
}

// q - 32 of four 6-bit codes given as bytes 0..63: bit 5 flipped, then copied into bits 6, 7
__device__ __forceinline__ uint32_t centre6(uint32_t q) {
    const uint32_t x = q ^ 0x20202020u;
    const uint32_t m = x & 0x20202020u;
    return x | (m << 1) | (m << 2);
}

template <int RG, int VW, int TR, int KS, bool DBG>
__global__ void __launch_bounds__(256) gemm_q6k_mc_kernel(GemmArgs a) {
    static_assert(RG * VW == 4, "four waves");
    static_assert(KS == 4 || KS == 8, "steps of half a super-block (two buffers) or one");
    constexpr int kStep = KS;
    constexpr int kPitch = pitch6<KS>();
    constexpr int RW = RG * TR;                       // row tiles of the workgroup
    constexpr int BUF = q6k_buf_bytes<RW, VW, KS>();
    constexpr int kWItems = 32 * RW * kStep;          // (row, block) pieces of a step
    constexpr int kWLoads = (kWItems + 255) / 256;
    constexpr int kRLoads = (32 * RW + 255) / 256;    // rows (sub-scales and d)
    constexpr int kXChunks = 32 * VW * kStep * 2;     // 16-byte activation chunks
    constexpr int kXLoads = kXChunks / 256;
    constexpr int kSLoads = (32 * VW * kStep + 255) / 256;
    static_assert(kXChunks % 256 == 0, "every lane stores activation chunks");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_q6k[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave / VW, vw = wave % VW;
    const int rows = a.rows, nb = a.nb, nvec = a.nvec;
    const int nsb = nb / 8;                           // super-blocks per row
    const int64_t cols = static_cast<int64_t>(nb) * 32;
    const int item = blockIdx.x;
    const int rt = item % a.row_tiles;
    const int grp = (item / a.row_tiles) % a.groups;
    const int sp = item / (a.row_tiles * a.groups);
    const int row0 = rt * 32 * RW;
    const int v0 = grp * 32 * VW;
    const int b_lo = sp * a.sb_per_split;
    const int b_hi = min(nb, b_lo + a.sb_per_split);
    const int steps = (b_hi - b_lo) / kStep;
    const int64_t nsbt = static_cast<int64_t>(rows) * nsb;   // super-blocks in the tensor
    const uint8_t *lo_plane = a.w;
    const uint8_t *hi_plane = a.w + nsbt * 128;
    const uint8_t *sc_plane = a.w + nsbt * 192;
    const uint16_t *d_plane = reinterpret_cast<const uint16_t *>(a.w + nsbt * 208);

    // ---- one step's global loads (registers), then their LDS stores ----
    uint4 lreg[kWLoads], sreg_w[kRLoads];
    uint2 hreg[kWLoads];
    float dreg[kRLoads];
    uint4 xreg[kXLoads];
    float sreg[kSLoads];
    auto issue = [&](int step) {
        const int b0 = b_lo + step * kStep;           // a multiple of KS
        const int sb = b0 / 8, kb = b0 % 8;           // its super-block, first block there
#pragma unroll
        for (int j = 0; j < kWLoads; j++) {
            const int c = j * 256 + tid;              // (row, block), row-major
            const int row = min(row0 + c / kStep, rows - 1);
            const int64_t i = static_cast<int64_t>(row) * nsb + sb;
            const int kk = kb + c % kStep;            // the block within the super-block
            if (c < kWItems) {
                lreg[j] = load16(lo_plane + i * 128 + 16 * kk);
                hreg[j] = *reinterpret_cast<const uint2 *>(hi_plane + i * 64 + 8 * kk);
            } else {
                lreg[j] = make_uint4(0u, 0u, 0u, 0u);
                hreg[j] = make_uint2(0u, 0u);
            }
        }
#pragma unroll
        for (int j = 0; j < kRLoads; j++) {
            const int c = j * 256 + tid;              // row of the tile
            const int row = min(row0 + c, rows - 1);
            const int64_t i = static_cast<int64_t>(row) * nsb + sb;
            if (c < 32 * RW) {
                if constexpr (KS == 8) {
                    sreg_w[j] = load16(sc_plane + i * 16);
                } else {
                    const uint2 q = *reinterpret_cast<const uint2 *>(sc_plane + i * 16 + 2 * kb);
                    sreg_w[j] = make_uint4(q.x, q.y, 0u, 0u);
                }
                dreg[j] = half_to_float(d_plane[i]);
            } else {
                sreg_w[j] = make_uint4(0u, 0u, 0u, 0u);
                dreg[j] = 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < kXLoads; j++) {
            const int c = j * 256 + tid;              // (vector, block, half), vector-major
            const int v = v0 + c / (2 * kStep);
            const int blk = b0 + (c % (2 * kStep)) / 2;
            xreg[j] = v < nvec ? load16(a.xq + v * cols + static_cast<int64_t>(blk) * 32 + 16 * (c & 1))
                               : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < kSLoads; j++) {
            const int c = j * 256 + tid;              // (vector, block), vector-major
            const int v = v0 + c / kStep;
            const int blk = b0 + c % kStep;
            sreg[j] = c < 32 * VW * kStep && v < nvec ? a.xd[static_cast<int64_t>(v) * nb + blk]
                                                      : 0.0f;
        }
    };
    auto store = [&](int buf, int step) {
        uint8_t *base = lds_q6k + buf * BUF;
        uint8_t *wq = base;
        uint8_t *wsc = base + 32 * RW * kPitch;
        float *wd = reinterpret_cast<float *>(wsc + 32 * RW * 2 * KS);
        uint8_t *xq = reinterpret_cast<uint8_t *>(wd + 32 * RW);
        float *xs = reinterpret_cast<float *>(xq + 32 * VW * kPitch);
#pragma unroll
        for (int j = 0; j < kWLoads; j++) {
            const int c = j * 256 + tid;
            if (c < kWItems) {
                // block k of row r: sub-block g = 0, 1 (weights 16 g + t); weight t's low bits
                // are nibble g of low byte t, its high bits bits 2 (t / 4) of high byte
                // 4 g + t % 4
                const uint32_t L[4] = {lreg[j].x, lreg[j].y, lreg[j].z, lreg[j].w};
                const uint32_t H[2] = {hreg[j].x, hreg[j].y};
                uint32_t o[8];
#pragma unroll
                for (int g = 0; g < 2; g++)
#pragma unroll
                    for (int s = 0; s < 4; s++) {
                        const uint32_t lo = (L[s] >> (4 * g)) & 0x0F0F0F0Fu;
                        const uint32_t hi = ((H[g] >> (2 * s)) & 0x03030303u) << 4;
                        o[4 * g + s] = centre6(lo | hi);
                    }
                uint8_t *dst = wq + (c / kStep) * kPitch + (c % kStep) * 32;
#pragma unroll
                for (int q = 0; q < 4; q++)
                    *reinterpret_cast<uint2 *>(dst + 8 * q) = make_uint2(o[2 * q], o[2 * q + 1]);
            }
        }
#pragma unroll
        for (int j = 0; j < kRLoads; j++) {
            const int c = j * 256 + tid;
            if (c < 32 * RW) {
                if constexpr (KS == 8)
                    *reinterpret_cast<uint4 *>(wsc + 16 * c) = sreg_w[j];
                else
                    *reinterpret_cast<uint2 *>(wsc + 8 * c) = make_uint2(sreg_w[j].x, sreg_w[j].y);
                wd[c] = dreg[j];
            }
        }
#pragma unroll
        for (int j = 0; j < kXLoads; j++) {
            const int c = j * 256 + tid;
            const uint4 q = xreg[j];
            uint8_t *dst = xq + (c / (2 * kStep)) * kPitch + ((c % (2 * kStep)) / 2) * 32 + 16 * (c & 1);
            *reinterpret_cast<uint2 *>(dst) = make_uint2(q.x, q.y);
            *reinterpret_cast<uint2 *>(dst + 8) = make_uint2(q.z, q.w);
            if constexpr (DBG) {
                // the block's code sum over its two halves (lanes tid, tid ^ 1): exact
                const int hs = byte_sum(q.x, byte_sum(q.y, byte_sum(q.z, byte_sum(q.w, 0))));
                const int s = hs + __builtin_amdgcn_update_dpp(0, hs, kDppXor1, 0xF, 0xF, false);
                const int v = v0 + c / (2 * kStep), gb = b_lo + step * kStep + (c % (2 * kStep)) / 2;
                if ((c & 1) == 0 && rt == 0 && v < nvec) a.S[static_cast<int64_t>(v) * nb + gb] = s;
            }
        }
#pragma unroll
        for (int j = 0; j < kSLoads; j++) {
            const int c = j * 256 + tid;
            if (c < 32 * VW * kStep) xs[(c % kStep) * 32 * VW + c / kStep] = sreg[j];
        }
    };

    // ---- this lane's place in its wave's tiles: one weight row of each, 16 vectors ----
    const int l32 = lane & 31, h = lane >> 5;
    float y[TR][16];
#pragma unroll
    for (int t = 0; t < TR; t++)
#pragma unroll
        for (int i = 0; i < 16; i++) y[t][i] = 0.0f;

    issue(0);
    for (int step = 0; step < steps; step++) {
        // two buffers: the step's buffer was last read two steps ago, before the barrier of
        // the last step; one buffer: wait until every wave is done with the last step
        const int buf = KS == 4 ? (step & 1) : 0;
        if (KS == 8 && step > 0) __syncthreads();
        store(buf, step);
        __syncthreads();
        if (step + 1 < steps) issue(step + 1);
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t *base = lds_q6k + buf * BUF;
        const uint8_t *wsc = base + 32 * RW * kPitch;
        const float *wd = reinterpret_cast<const float *>(wsc + 32 * RW * 2 * KS);
        const uint8_t *xq = reinterpret_cast<const uint8_t *>(wd + 32 * RW);
        const float *xs = reinterpret_cast<const float *>(xq + 32 * VW * kPitch);
        const uint8_t *xrow = xq + (vw * 32 + l32) * kPitch + 8 * h;
        uint4 scw[TR];
        float dv[TR];
#pragma unroll
        for (int t = 0; t < TR; t++) {
            const int rl = (rg * TR + t) * 32 + l32;  // the lane's row in the workgroup's tile
            if constexpr (KS == 8) {
                scw[t] = *reinterpret_cast<const uint4 *>(wsc + 16 * rl);
            } else {
                const uint2 q = *reinterpret_cast<const uint2 *>(wsc + 8 * rl);
                scw[t] = make_uint4(q.x, q.y, 0u, 0u);
            }
            dv[t] = wd[rl];
        }
        float acc[TR][16];
#pragma unroll
        for (int k = 0; k < kStep; k++) {
            long A[2];
#pragma unroll
            for (int g = 0; g < 2; g++) A[g] = *reinterpret_cast<const long *>(xrow + k * 32 + 16 * g);
            float xdv[16];
#pragma unroll
            for (int qq = 0; qq < 4; qq++) {
                const float4 f = *reinterpret_cast<const float4 *>(
                    xs + k * 32 * VW + vw * 32 + 8 * qq + 4 * h);
                xdv[4 * qq] = f.x;
                xdv[4 * qq + 1] = f.y;
                xdv[4 * qq + 2] = f.z;
                xdv[4 * qq + 3] = f.w;
            }
#pragma unroll
            for (int t = 0; t < TR; t++) {
                const uint8_t *wrow = base + ((rg * TR + t) * 32 + l32) * kPitch + 8 * h;
                v16i_t P[2];
#pragma unroll
                for (int g = 0; g < 2; g++) {
                    const long B = *reinterpret_cast<const long *>(wrow + k * 32 + 16 * g);
                    const v16i_t zero = {};
                    P[g] = __builtin_amdgcn_mfma_i32_32x32x16_i8(A[g], B, zero, 0, 0, 0);
                }
                // the row's scales of sub-blocks 2 k and 2 k + 1 (bytes of the step's 2 KS)
                const uint32_t scd = k < 2 ? scw[t].x : k < 4 ? scw[t].y : k < 6 ? scw[t].z : scw[t].w;
                const int sc0 = static_cast<int>(static_cast<int8_t>(scd >> (16 * (k & 1))));
                const int sc1 = static_cast<int>(static_cast<int8_t>(scd >> (16 * (k & 1) + 8)));
                const int my_row = row0 + (rg * TR + t) * 32 + l32;
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    if constexpr (DBG) {
                        const int v = v0 + vw * 32 + 8 * (i / 4) + 4 * h + i % 4;
                        const int sub = 2 * (b_lo + step * kStep + k);
                        if (my_row < rows && v < nvec) {
                            int32_t *p = a.P + (static_cast<int64_t>(v) * rows + my_row) * (2 * nb) + sub;
                            p[0] = P[0][i];
                            p[1] = P[1][i];
                        }
                    } else {
                        const int tt = __mul24(sc0, P[0][i]) + __mul24(sc1, P[1][i]);
                        acc[t][i] = k == 0 ? xdv[i] * static_cast<float>(tt)
                                           : fmaf(xdv[i], static_cast<float>(tt), acc[t][i]);
                    }
                }
            }
        }
        if constexpr (!DBG) {
#pragma unroll
            for (int t = 0; t < TR; t++)
#pragma unroll
                for (int i = 0; i < 16; i++) y[t][i] = fmaf(dv[t], acc[t][i], y[t][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (!DBG) {
#pragma unroll
        for (int t = 0; t < TR; t++) {
            const int my_row = row0 + (rg * TR + t) * 32 + l32;
            if (my_row < rows) {
                float *out = a.out + static_cast<int64_t>(sp) * nvec * rows + my_row;
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int v = v0 + vw * 32 + 8 * (i / 4) + 4 * h + i % 4;
                    if (v < nvec) out[static_cast<int64_t>(v) * rows] = y[t][i];
                }
            }
        }
    }
}

template <int RG, int VW, int TR, int KS>
hipError_t launch_rv(const GemmArgs &a, bool debug, hipStream_t stream) {
    const size_t lds = static_cast<size_t>(q6k_buf_bytes<RG * TR, VW, KS>()) * (KS == 4 ? 2 : 1);
    const int64_t items = static_cast<int64_t>(a.row_tiles) * a.groups * a.splits;
    if (items < 1 || items > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(items));
    if (debug)
        hipLaunchKernelGGL((gemm_q6k_mc_kernel<RG, VW, TR, KS, true>), grid, dim3(256), lds, stream, a);
    else
        hipLaunchKernelGGL((gemm_q6k_mc_kernel<RG, VW, TR, KS, false>), grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

// The workgroup shapes of mc32_rows_per_wg: 128 rows x 32 vectors, 128 x 64, 64 x 128.
hipError_t launch_gemm_q6k_mc(const GemmArgs &a, int vt, bool debug, hipStream_t stream) {
    if (a.nb < 8 || a.nb % 8 != 0 || a.sb_per_split < 1 || a.sb_per_split % 8 != 0 ||
        a.row_tiles < 1 || a.groups < 1 || a.splits < 1 || a.nvec < 1 || a.nvec > kMaxBatch)
        return hipErrorInvalidValue;
    switch (vt) {
        case 1: return launch_rv<4, 1, 1, mc32_step_blocks(kTypeQ6K, 1)>(a, debug, stream);
        case 2: return launch_rv<2, 2, 2, mc32_step_blocks(kTypeQ6K, 2)>(a, debug, stream);
        case 4: return launch_rv<1, 4, 2, mc32_step_blocks(kTypeQ6K, 4)>(a, debug, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
