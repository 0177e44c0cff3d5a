// Q4_K weights x many int8 activation vectors on the matrix cores (v_mfma_f32_32x32x16_f16).
//
// With more than a handful of vectors the product stops being a stream of weights and becomes a
// skinny dense contraction (oxinfer README, "Speculative decoding": the many-token int8 decode
// variants are instruction-bound at Q4; genie-ai-runtime, "The prefill kernel cycle": the
// same integer products on tensor cores). The integer sub-block products are formed on the
// matrix cores, still exactly:
//
//  * Every operand is a small integer: the activation code xq (|xq| <= 127) and the weight code
//    times its 6-bit sub-scale, sc * q <= 63 * 15 = 945. An fp16 holds both exactly; sc * q is
//    stored as the raw fp16 bit pattern, i.e. the subnormal (sc * q) * 2^-24, which the matrix
//    cores multiply without flushing. Every product and every partial sum of a 32-column block
//    is then an integer times 2^-24 below 2^24 in magnitude (945 * 127 * 32 < 2^22), so the
//    float32 result is exactly 2^-24 * sc * P with P = sum of q * xq. The factor 2^24 goes into
//    the super-scale d, so the only float work per output and block is one fma with the
//    activation scale; d is applied once per super-block.
//  * The min term dmin * m * xd * S (S = sum of the block's codes) is a contraction over the
//    blocks of dmin * m (row, block) with -xd * S (block, vector), done on the float32 matrix
//    cores (v_mfma_f32_32x32x2f32, two blocks per instruction) straight into the accumulator.
//
// Work split: a workgroup of 4 waves takes 128 rows; each wave 32 rows (the MFMA's M) and every
// vector of its group (nt tiles of 32 vectors, the MFMA's N) over one column split. Per
// super-block the workgroup converts the group's codes for 256 columns to fp16 in LDS once
// (shared by the four waves) with -xd * S; every load of the next super-block (each wave's
// codes, 64 contiguous bytes per lane, and headers straight from HBM; the activation pieces)
// goes out before the current one's arithmetic.
//
// Lane layout of the 32x32x16 fp16 MFMA (checked on gfx950): lane l holds operand slots
// k = 8 (l / 32) .. + 7 of row (A) or column (B) l % 32, and result element i of row
// 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32. The sum over k does not depend on which column
// each (lane half, slot) stands for, as long as A and B agree; here, within each group of 8
// columns, slots 0..7 hold columns 0, 2, 1, 3, 4, 6, 5, 7 (the order the nibbles and bytes come
// out of a 32-bit word with two masks).
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16v_t __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kActStride = 264;   // fp16 per staged activation row: 256 columns + 8 (banks)

// Two signed bytes (bytes 0 and 2 of w, or 1 and 3 with shift 8) -> two exact fp16 values:
// the pattern 0x6600 + xq is the fp16 1536 + xq (ulp 1 in [1024, 2048)); subtracting 1536 in
// fp16 is exact.
template <int SHIFT>
__device__ __forceinline__ uint32_t codes_to_half2(uint32_t w_flipped) {
    const uint32_t pat = ((w_flipped >> SHIFT) & 0x00FF00FFu) + 0x65806580u;
    const half2_t h = __builtin_bit_cast(half2_t, pat) - half2_t{1536.0f16, 1536.0f16};
    return __builtin_bit_cast(uint32_t, h);
}

// Nibbles (bytes 0 and 2, or 1 and 3 with shift 8, low or high nibble with shift +4) times the
// sub-scale, as two fp16 bit patterns (integers below 1024 = subnormals).
template <int SHIFT>
__device__ __forceinline__ uint32_t nib_times(uint32_t w, uint32_t scpair) {
    const uint32_t n = (w >> SHIFT) & 0x000F000Fu;
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, n) *
                                            __builtin_bit_cast(u16x2_t, scpair));
}

template <int SHIFT>
__device__ __forceinline__ uint32_t nib(uint32_t w) {
    return (w >> SHIFT) & 0x000F000Fu;
}

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(half8_t, make_uint4(a, b, c, d));
}

template <int NT, bool DBG>
__global__ void __launch_bounds__(256) gemm_q4k_mfma_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) _Float16 act[NT * 32 * kActStride];
    __shared__ __attribute__((aligned(16))) float2 xdt[8 * NT * 32];     // (xd, -xd * S)
    __shared__ __attribute__((aligned(16))) float dd[4][32];             // d * 2^24 per wave

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int rows = a.rows, nb = a.nb, nvec = a.nvec;
    const int64_t cols = static_cast<int64_t>(nb) * 256;
    const int nbk = nb * 8;                           // 32-column blocks per row
    const int tok0 = blockIdx.y * NT * 32;
    const int sb0 = blockIdx.z * a.sb_per_split;
    const int sb1 = min(nb, sb0 + a.sb_per_split);
    const int wrow0 = blockIdx.x * kMcRows + wave * 32;
    // this lane's weight row (A operand), clamped so the last tile's loads stay in bounds
    const int arow = min(wrow0 + l32, rows - 1);
    const int64_t nblocks = static_cast<int64_t>(rows) * nb;
    const uint8_t *codes = a.w + (static_cast<int64_t>(arow) * nb) * 128 + 64 * h;
    const uint8_t *hdrs = a.w + nblocks * 128 + (static_cast<int64_t>(arow) * nb) * 16;
    // staging: thread -> (vector tid / 16 + 16 r, 16-byte piece tid % 16) in round r
    const int sp = tid & 15;
    const int sv = tid >> 4;

    float16v_t acc[NT];
    float t1[NT][16];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
            acc[t][i] = 0.0f;
            t1[t][i] = 0.0f;
        }

    // loads of one super-block: this lane's codes and header, this thread's activation pieces
    uint4 c[4], hdr, xqr[2 * NT];
    float xdr[2 * NT];
    auto issue = [&](int sb) {
#pragma unroll
        for (int k = 0; k < 4; k++)
            c[k] = load16_stream(codes + static_cast<int64_t>(sb) * 128 + 16 * k);
        hdr = load16(hdrs + static_cast<int64_t>(sb) * 16);
#pragma unroll
        for (int rnd = 0; rnd < 2 * NT; rnd++) {
            const int tok = tok0 + rnd * 16 + sv;
            xqr[rnd] = make_uint4(0u, 0u, 0u, 0u);
            xdr[rnd] = 0.0f;
            if (tok < nvec) {
                xqr[rnd] = load16(a.xq + static_cast<int64_t>(tok) * cols + sb * 256 + 16 * sp);
                if ((sp & 1) == 0) xdr[rnd] = a.xd[static_cast<int64_t>(tok) * nbk + sb * 8 + (sp >> 1)];
            }
        }
    };
    issue(sb0);

    for (int sb = sb0; sb < sb1; sb++) {
        // ---- this super-block's weights: codes to (dword 2h, 2h + 1) of every chunk ----
        uint32_t aw[8], bw[8];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const auto rx = __builtin_amdgcn_permlane32_swap(c[k].x, c[k].z, false, false);
            const auto ry = __builtin_amdgcn_permlane32_swap(c[k].y, c[k].w, false, false);
            const uint32_t x0 = rx[0], x1 = rx[1], y0 = ry[0], y1 = ry[1];
            aw[k] = x0;
            aw[k + 4] = x1;
            bw[k] = y0;
            bw[k + 4] = y1;
        }
        uint32_t sc[8];
        float cmin[4];      // dmin * m of blocks h, h + 2, h + 4, h + 6 of this lane's row
        {
            const float d = half_to_float(hdr.x & 0xFFFFu);
            const float dmin = half_to_float(hdr.x >> 16);
#pragma unroll
            for (int j = 0; j < 8; j++)
                sc[j] = ((hdr.y >> (8 * (j / 2) + 4 * (j % 2))) & 0xFu) |
                        (((hdr.w >> (8 * (j / 4) + 2 * (j % 4))) & 3u) << 4);
#pragma unroll
            for (int pp = 0; pp < 4; pp++) {
                // block 2 pp + h: low nibble of byte pp of the m field, high bits of byte
                // 14 + pp / 2 at bit 4 (pp % 2) + 2 h
                const uint32_t m = ((hdr.z >> (8 * pp + 4 * h)) & 0xFu) |
                                   (((hdr.w >> (16 + 8 * (pp / 2) + 4 * (pp % 2) + 2 * h)) & 3u) << 4);
                cmin[pp] = dmin * static_cast<float>(m);
            }
            if (h == 0) dd[wave][l32] = d * 16777216.0f;
        }

        // ---- the group's activation codes for these 256 columns, to fp16 in LDS ----
#pragma unroll
        for (int rnd = 0; rnd < 2 * NT; rnd++) {
            const int v = rnd * 16 + sv;
            const uint4 q = xqr[rnd];
            int s = byte_sum(q.x, byte_sum(q.y, byte_sum(q.z, byte_sum(q.w, 0))));
            s += __builtin_amdgcn_update_dpp(0, s, kDppXor1, 0xF, 0xF, false);
            const uint32_t fx = q.x ^ 0x80808080u, fy = q.y ^ 0x80808080u;
            const uint32_t fz = q.z ^ 0x80808080u, fw = q.w ^ 0x80808080u;
            uint4 *dst = reinterpret_cast<uint4 *>(act + v * kActStride + 16 * sp);
            dst[0] = make_uint4(codes_to_half2<0>(fx), codes_to_half2<8>(fx), codes_to_half2<0>(fy),
                                codes_to_half2<8>(fy));
            dst[1] = make_uint4(codes_to_half2<0>(fz), codes_to_half2<8>(fz), codes_to_half2<0>(fw),
                                codes_to_half2<8>(fw));
            if ((sp & 1) == 0) {
                const int j = sp >> 1;
                const float x = xdr[rnd];
                xdt[j * NT * 32 + v] = make_float2(x, -(x * static_cast<float>(s)));
                const int tok = tok0 + v;
                if (DBG && blockIdx.x == 0 && tok < nvec)
                    a.S[static_cast<int64_t>(tok) * nbk + sb * 8 + j] = s;
            }
        }
        // ---- the next super-block's loads go out now, to land during this one's work ----
        if (sb + 1 < sb1) issue(sb + 1);
        __syncthreads();

        // ---- eight 32-column blocks ----
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t scp = sc[j] * 0x00010001u;
            const uint32_t wa = aw[j], wb = bw[j];
            const half8_t A0 = as_half8(nib_times<0>(wa, scp), nib_times<8>(wa, scp),
                                        nib_times<0>(wb, scp), nib_times<8>(wb, scp));
            const half8_t A1 = as_half8(nib_times<4>(wa, scp), nib_times<12>(wa, scp),
                                        nib_times<4>(wb, scp), nib_times<12>(wb, scp));
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const _Float16 *brow = act + (t * 32 + l32) * kActStride + 32 * j + 8 * h;
                const half8_t B0 = *reinterpret_cast<const half8_t *>(brow);
                const half8_t B1 = *reinterpret_cast<const half8_t *>(brow + 16);
                const float xs = xdt[j * NT * 32 + t * 32 + l32].x;
                const float16v_t zero = {};
                float16v_t Q = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, B0, zero, 0, 0, 0);
                Q = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, B1, Q, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 16; i++) t1[t][i] = fmaf(xs, Q[i], t1[t][i]);
                if (DBG) {
                    const half8_t U0 = as_half8(nib<0>(wa), nib<8>(wa), nib<0>(wb), nib<8>(wb));
                    const half8_t U1 = as_half8(nib<4>(wa), nib<12>(wa), nib<4>(wb), nib<12>(wb));
                    float16v_t R = __builtin_amdgcn_mfma_f32_32x32x16_f16(U0, B0, zero, 0, 0, 0);
                    R = __builtin_amdgcn_mfma_f32_32x32x16_f16(U1, B1, R, 0, 0, 0);
                    const int tok = tok0 + t * 32 + l32;
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const int row = wrow0 + 8 * (i / 4) + 4 * h + (i % 4);
                        if (tok < nvec && row < rows)
                            a.P[(static_cast<int64_t>(tok) * rows + row) * nbk + sb * 8 + j] =
                                static_cast<int>(R[i] * 16777216.0f);
                    }
                }
            }
        }
        // ---- the min terms of the eight blocks on the float32 matrix cores: two blocks per
        //      32x32x2 product, A = dmin * m (row, block), B = -xd * S (block, vector) ----
#pragma unroll
        for (int pp = 0; pp < 4; pp++)
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const float tb = xdt[(2 * pp + h) * NT * 32 + t * 32 + l32].y;
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(cmin[pp], tb, acc[t], 0, 0, 0);
            }
        float ddv[16];
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
            const float4 f = *reinterpret_cast<const float4 *>(&dd[wave][8 * qq + 4 * h]);
            ddv[4 * qq] = f.x;
            ddv[4 * qq + 1] = f.y;
            ddv[4 * qq + 2] = f.z;
            ddv[4 * qq + 3] = f.w;
        }
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                acc[t][i] = fmaf(ddv[i], t1[t][i], acc[t][i]);
                t1[t][i] = 0.0f;
            }
        __syncthreads();   // the next super-block overwrites the staged codes and tables
    }

    if (DBG) return;
    float *out = a.out + static_cast<int64_t>(blockIdx.z) * nvec * rows;
    // 16-byte stores when every row group of 4 starts 16-byte aligned
    const bool vec4 = (rows & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int tok = tok0 + t * 32 + l32;
        if (tok >= nvec) continue;
        float *yv = out + static_cast<int64_t>(tok) * rows;
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
            const int row = wrow0 + 8 * qq + 4 * h;
            if (vec4 && row + 3 < rows) {
                *reinterpret_cast<float4 *>(yv + row) =
                    make_float4(acc[t][4 * qq], acc[t][4 * qq + 1], acc[t][4 * qq + 2],
                                acc[t][4 * qq + 3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (row + i < rows) yv[row + i] = acc[t][4 * qq + i];
            }
        }
    }
}

template <int NT>
hipError_t launch_nt(const GemmArgs &a, int row_tiles, int groups, int splits, bool debug,
                     hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(row_tiles), static_cast<unsigned>(groups),
                    static_cast<unsigned>(splits));
    if (debug)
        hipLaunchKernelGGL((gemm_q4k_mfma_kernel<NT, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_q4k_mfma_kernel<NT, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_q4k_mfma(const GemmArgs &a, int nt, int row_tiles, int groups, int splits,
                                bool debug, hipStream_t stream) {
    switch (nt) {
        case 1: return launch_nt<1>(a, row_tiles, groups, splits, debug, stream);
        case 2: return launch_nt<2>(a, row_tiles, groups, splits, debug, stream);
        case 3: return launch_nt<3>(a, row_tiles, groups, splits, debug, stream);
        case 4: return launch_nt<4>(a, row_tiles, groups, splits, debug, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
