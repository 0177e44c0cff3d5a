// Q8_0 and Q4_0 weights x 9..256 int8 activation vectors on the integer matrix cores
// (v_mfma_i32_32x32x32_i8).
//
// With many vectors (several tokens verified or prefilled at once) the vector kernel's int8
// 4-way dot products dominate and the weights are re-read once per group of 8 vectors
// (oxinfer README, "Speculative decoding": the multi-token int8 variants are instruction-bound
// at Q4). One 32 x 32 x 32 product is exactly one 32-weight block of 32 rows against 32
// vectors, so its int32 result is the block's exact integer partial P for every (row, vector):
//
//  * Q8_0: the weight operand is the stored int8 codes; P = sum q * xq.
//  * Q4_0: the weight operand is 16 (q - 8) as int8: each code's nibble moved to the high half
//    of its byte with the top bit flipped (one xor, one shift and one mask per 4 codes), so the
//    product is 16 P exactly, P = sum (q - 8) xq, and a block of zero weights adds exactly 0.
//    The factor 16 rides through the float sum and is taken out once per output at the end:
//    scaling by a power of two commutes with float32 rounding, so y is the same as from P
//    itself wherever the sums stay normal and finite (|y| below 2^123).
//  * Float work per (row, vector, block): the conversion of P and one fma with d * xd (d the
//    weight block's scale, xd the activation block's scale): y = sum over blocks of
//    (d * xd) * P in float32.
//
// Work split: a workgroup of 4 waves computes 32 RW rows x 32 VG TV vectors (RW * VG = 4; each
// wave 32 rows x TV tiles of 32 vectors, so the weight operand and the 16 row scales a lane
// reads from LDS per block serve TV products: those scale reads are most of the LDS traffic)
// over one column split, in steps of KS blocks. Each step's weights (codes and scales of the
// workgroup's rows) and activation (codes and scales of its vectors) are loaded with
// coalesced 16-byte loads into LDS tiles padded against bank conflicts; the next step's loads
// go out into registers before the current step's products, which read only LDS. KS = 8: 8
// lanes per 128-byte line of each codes plane, one LDS buffer (two or three workgroups per CU);
// KS = 4: half lines, two LDS buffers (mc32_step_blocks picks by format and shape). A ragged
// last step reads valid blocks against zero activation codes, so the extra blocks add exactly
// 0; rows past the matrix read its last row and are not stored.
//
// Lane layout of the 32 x 32 x 32 product (checked on gfx950): operand lane l holds row (or
// column) l % 32 and K slots 16 (l / 32) .. + 15; result element i is row 8 (i / 4) +
// 4 (l / 32) + i % 4, column l % 32. Here the weights are the row operand (32 weight rows),
// the activation the column operand (32 vectors): lane l of a wave owns vector l % 32 and
// 16 rows of its tile.
#include "device_common.h"
#include "gemm_mc.h"

namespace qgemv {

namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));

// LDS row pitches for steps of KS blocks, padded by 16 bytes so that the 32 rows a read
// touches fall in distinct banks (16-lane groups)
template <int FMT, int KS>
__host__ __device__ constexpr int wpitch() { return (FMT == kTypeQ80 ? 32 : 16) * KS + 16; }
template <int KS>
__host__ __device__ constexpr int xpitch() { return 32 * KS + 16; }

// LDS of one step's buffer: weight codes [32 RW rows][pitch], weight scales [KS blocks][32 RW]
// float, activation codes [32 VW vectors][pitch], activation scales [KS][32 VW] (VW = VG TV
// vector tiles).
template <int FMT, int RW, int VW, int KS>
__host__ __device__ constexpr int q32_buf_bytes() {
    return 32 * RW * wpitch<FMT, KS>() + KS * 32 * RW * 4 + 32 * VW * xpitch<KS>() +
           KS * 32 * VW * 4;
}

template <int FMT, int RW, int VG, int TV, int KS, bool DBG>
__global__ void __launch_bounds__(256) gemm_q32_mc_kernel(GemmArgs a) {
    static_assert(RW * VG == 4, "four waves");
    static_assert(KS == 4 || KS == 8, "steps of 4 blocks (two buffers) or 8 (one buffer)");
    constexpr int kStep = KS;
    constexpr int VW = VG * TV;                       // vector tiles of the workgroup
    constexpr int WP = wpitch<FMT, KS>();
    constexpr int kXPitch = xpitch<KS>();
    constexpr int BUF = q32_buf_bytes<FMT, RW, VW, KS>();
    // codes chunks (16 bytes) of the weight tile and of the activation tile per step
    constexpr int kWChunks = 32 * RW * kStep * (FMT == kTypeQ80 ? 2 : 1);
    constexpr int kXChunks = 32 * VW * kStep * 2;
    constexpr int kWLoads = (kWChunks + 255) / 256;
    constexpr int kXLoads = (kXChunks + 255) / 256;
    constexpr int kDLoads = (32 * RW * kStep + 255) / 256;
    constexpr int kSLoads = (32 * VW * kStep + 255) / 256;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_q32[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rw = wave / VG, vg = wave % VG;
    const int rows = a.rows, nb = a.nb, nvec = a.nvec;
    const int64_t cols = static_cast<int64_t>(nb) * 32;
    // work item: (row tile, vector group, column split)
    const int item = blockIdx.x;
    const int rt = item % a.row_tiles;
    const int grp = (item / a.row_tiles) % a.groups;
    const int sp = item / (a.row_tiles * a.groups);
    const int row0 = rt * 32 * RW;
    const int v0 = grp * 32 * VW;
    const int b_lo = sp * a.sb_per_split;
    const int b_hi = min(nb, b_lo + a.sb_per_split);
    const int steps = (b_hi - b_lo + kStep - 1) / kStep;
    const int64_t nblocks = static_cast<int64_t>(rows) * nb;
    const uint8_t *codes0 = a.w;
    const uint8_t *codes1 = a.w + nblocks * 16;      // Q8_0: codes 16..31 of every block
    const uint8_t *dplane = a.w + nblocks * (FMT == kTypeQ80 ? 32 : 16);

    // ---- one step's global loads (registers), then their LDS stores ----
    uint4 wreg[kWLoads], xreg[kXLoads];
    float dreg[kDLoads], sreg[kSLoads];
    auto issue = [&](int step) {
        const int b0 = b_lo + step * kStep;
#pragma unroll
        for (int j = 0; j < kWLoads; j++) {
            const int c = j * 256 + tid;
            const int per_plane = 32 * RW * kStep;
            const int p = FMT == kTypeQ80 ? c / per_plane : 0;
            const int cc = c - p * per_plane;
            const int row = min(row0 + cc / kStep, rows - 1);
            const int blk = min(b0 + cc % kStep, nb - 1);
            const uint8_t *src = (p ? codes1 : codes0) + (static_cast<int64_t>(row) * nb + blk) * 16;
            wreg[j] = c < kWChunks ? load16(src) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < kDLoads; j++) {
            const int c = j * 256 + tid;                 // (row, block) of the tile, row-major
            const int row = min(row0 + c / kStep, rows - 1);
            const int blk = min(b0 + c % kStep, nb - 1);
            const int64_t bi = static_cast<int64_t>(row) * nb + blk;
            float d = 0.0f;
            if (c < 32 * RW * kStep) {
                if constexpr (FMT == kTypeQ80)
                    d = reinterpret_cast<const float *>(dplane)[bi];
                else
                    d = half_to_float(reinterpret_cast<const uint16_t *>(dplane)[bi]);
            }
            dreg[j] = d;
        }
#pragma unroll
        for (int j = 0; j < kXLoads; j++) {
            const int c = j * 256 + tid;                 // (vector, block, half), vector-major
            const int v = v0 + c / (2 * kStep);
            const int blk = b0 + (c % (2 * kStep)) / 2;
            const bool live = c < kXChunks && v < nvec && blk < b_hi;
            xreg[j] = live ? load16(a.xq + v * cols + static_cast<int64_t>(blk) * 32 + 16 * (c & 1))
                           : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < kSLoads; j++) {
            const int c = j * 256 + tid;                 // (vector, block), vector-major
            const int v = v0 + c / kStep;
            const int blk = b0 + c % kStep;
            const bool live = c < 32 * VW * kStep && v < nvec && blk < b_hi;
            sreg[j] = live ? a.xd[static_cast<int64_t>(v) * nb + blk] : 0.0f;
        }
    };
    auto store = [&](int buf, int step) {
        uint8_t *base = lds_q32 + buf * BUF;
        uint8_t *wq = base;
        float *wd = reinterpret_cast<float *>(base + 32 * RW * WP);
        uint8_t *xq = base + 32 * RW * WP + kStep * 32 * RW * 4;
        float *xs = reinterpret_cast<float *>(xq + 32 * VW * kXPitch);
#pragma unroll
        for (int j = 0; j < kWLoads; j++) {
            const int c = j * 256 + tid;
            if (c < kWChunks) {
                const int per_plane = 32 * RW * kStep;
                const int p = FMT == kTypeQ80 ? c / per_plane : 0;
                const int cc = c - p * per_plane;
                *reinterpret_cast<uint4 *>(wq + (cc / kStep) * WP +
                                           (cc % kStep) * (FMT == kTypeQ80 ? 32 : 16) + 16 * p) = wreg[j];
            }
        }
#pragma unroll
        for (int j = 0; j < kDLoads; j++) {
            const int c = j * 256 + tid;
            if (c < 32 * RW * kStep) wd[(c % kStep) * 32 * RW + c / kStep] = dreg[j];
        }
        static_assert(kXChunks % 256 == 0, "every lane stores activation chunks");
#pragma unroll
        for (int j = 0; j < kXLoads; j++) {
            const int c = j * 256 + tid;
            *reinterpret_cast<uint4 *>(xq + (c / (2 * kStep)) * kXPitch +
                                       ((c % (2 * kStep)) / 2) * 32 + 16 * (c & 1)) = xreg[j];
            if constexpr (DBG) {
                // the block's code sum over its two halves (lanes tid, tid ^ 1): exact
                const uint4 q = xreg[j];
                const int half = byte_sum(q.x, byte_sum(q.y, byte_sum(q.z, byte_sum(q.w, 0))));
                const int s = half + __builtin_amdgcn_update_dpp(0, half, kDppXor1, 0xF, 0xF, false);
                if ((c & 1) == 0 && rt == 0) {
                    const int v = v0 + c / (2 * kStep), gb = b_lo + step * kStep + (c % (2 * kStep)) / 2;
                    if (v < nvec && gb < b_hi) a.S[static_cast<int64_t>(v) * nb + gb] = s;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kSLoads; j++) {
            const int c = j * 256 + tid;
            if (c < 32 * VW * kStep) xs[(c % kStep) * 32 * VW + c / kStep] = sreg[j];
        }
    };

    // ---- this lane's place in its wave's tiles: vector l % 32 of each, 16 rows ----
    const int l32 = lane & 31, h = lane >> 5;
    float acc[TV][16];
#pragma unroll
    for (int t = 0; t < TV; t++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[t][i] = 0.0f;

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
        const uint8_t *base = lds_q32 + buf * BUF;
        const uint8_t *wq = base + (rw * 32 + l32) * WP;
        const float *wd = reinterpret_cast<const float *>(base + 32 * RW * WP);
        const uint8_t *xq = base + 32 * RW * WP + kStep * 32 * RW * 4;
        const float *xs = reinterpret_cast<const float *>(xq + 32 * VW * kXPitch);
        const int nblk = min(kStep, b_hi - (b_lo + step * kStep));
#pragma unroll
        for (int k = 0; k < kStep; k++) {
            if (k < nblk) {                           // the same in every lane of the workgroup
                v4i_t A;
                if constexpr (FMT == kTypeQ80) {
                    A = *reinterpret_cast<const v4i_t *>(wq + k * 32 + 16 * h);
                } else {
                    // weights 16 h .. 16 h + 15 of the block: nibble h of its 16 code bytes,
                    // as 16 (q - 8): bit 3 of the nibble flipped, the nibble in the high half
                    const uint4 raw = *reinterpret_cast<const uint4 *>(wq + k * 16);
                    const int sh = 4 - 4 * h;
                    A = v4i_t{static_cast<int>(((raw.x ^ 0x88888888u) << sh) & 0xF0F0F0F0u),
                              static_cast<int>(((raw.y ^ 0x88888888u) << sh) & 0xF0F0F0F0u),
                              static_cast<int>(((raw.z ^ 0x88888888u) << sh) & 0xF0F0F0F0u),
                              static_cast<int>(((raw.w ^ 0x88888888u) << sh) & 0xF0F0F0F0u)};
                }
                v16i_t P[TV];
#pragma unroll
                for (int t = 0; t < TV; t++) {
                    const uint8_t *xrow = xq + ((vg * TV + t) * 32 + l32) * kXPitch;
                    const v4i_t B = *reinterpret_cast<const v4i_t *>(xrow + k * 32 + 16 * h);
                    const v16i_t zero = {};
                    P[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, zero, 0, 0, 0);
                }
                float dv[16];
#pragma unroll
                for (int qq = 0; qq < 4; qq++) {
                    const float4 f = *reinterpret_cast<const float4 *>(
                        wd + k * 32 * RW + rw * 32 + 8 * qq + 4 * h);
                    dv[4 * qq] = f.x;
                    dv[4 * qq + 1] = f.y;
                    dv[4 * qq + 2] = f.z;
                    dv[4 * qq + 3] = f.w;
                }
#pragma unroll
                for (int t = 0; t < TV; t++) {
                    const int vl = (vg * TV + t) * 32 + l32;
                    const float xdv = xs[k * 32 * VW + vl];
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const int p = P[t][i];    // exact: P (Q8_0), 16 P (Q4_0)
                        if constexpr (DBG) {
                            const int row = row0 + rw * 32 + 8 * (i / 4) + 4 * h + i % 4;
                            const int gb = b_lo + step * kStep + k;
                            const int v = v0 + vl;
                            if (row < rows && v < nvec)
                                a.P[(static_cast<int64_t>(v) * rows + row) * nb + gb] =
                                    FMT == kTypeQ40 ? p >> 4 : p;
                        } else {
                            acc[t][i] = fmaf(dv[i] * xdv, static_cast<float>(p), acc[t][i]);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (!DBG) {
#pragma unroll
        for (int t = 0; t < TV; t++) {
            const int v = v0 + (vg * TV + t) * 32 + l32;
            if (v < nvec) {
                float *yv = a.out + (static_cast<int64_t>(sp) * nvec + v) * rows;
#pragma unroll
                for (int qq = 0; qq < 4; qq++) {
                    const int row = row0 + rw * 32 + 8 * qq + 4 * h;
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (row + i < rows)
                            yv[row + i] = FMT == kTypeQ40 ? acc[t][4 * qq + i] * 0.0625f
                                                          : acc[t][4 * qq + i];
                }
            }
        }
    }
}

template <int FMT, int RW, int VG, int TV, int KS>
hipError_t launch_rv(const GemmArgs &a, bool debug, hipStream_t stream) {
    const size_t lds = static_cast<size_t>(q32_buf_bytes<FMT, RW, VG * TV, KS>()) * (KS == 4 ? 2 : 1);
    const int64_t items = static_cast<int64_t>(a.row_tiles) * a.groups * a.splits;
    if (items < 1 || items > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(items));
    if (debug)
        hipLaunchKernelGGL((gemm_q32_mc_kernel<FMT, RW, VG, TV, KS, true>), grid, dim3(256), lds, stream, a);
    else
        hipLaunchKernelGGL((gemm_q32_mc_kernel<FMT, RW, VG, TV, KS, false>), grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

// The workgroup shapes (mc32_rows_per_wg): 128 rows x 32 vectors, 128 x 64, 64 x 128.
template <int FMT>
hipError_t launch_fmt(const GemmArgs &a, int vt, bool debug, hipStream_t stream) {
    switch (vt) {
        case 1: return launch_rv<FMT, 4, 1, 1, mc32_step_blocks(FMT, 1)>(a, debug, stream);
        case 2: return launch_rv<FMT, 4, 1, 2, mc32_step_blocks(FMT, 2)>(a, debug, stream);
        case 4: return launch_rv<FMT, 2, 2, 2, mc32_step_blocks(FMT, 4)>(a, debug, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm_q32_mc(int wtype, const GemmArgs &a, int vt, bool debug,
                              hipStream_t stream) {
    if (a.sb_per_split < 1 || a.sb_per_split % 8 != 0 || a.row_tiles < 1 || a.groups < 1 ||
        a.splits < 1 || a.nvec < 1 || a.nvec > kMaxBatch)
        return hipErrorInvalidValue;
    if (wtype == kTypeQ80) return launch_fmt<kTypeQ80>(a, vt, debug, stream);
    if (wtype == kTypeQ40) return launch_fmt<kTypeQ40>(a, vt, debug, stream);
    return hipErrorInvalidValue;
}

}  // namespace qgemv
