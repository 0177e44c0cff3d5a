// Q4_K weights x 1..16 int8 activation vectors on the integer matrix cores
// (v_mfma_i32_16x16x64_i8).
//
// With several vectors the vector kernel's int8 4-way dot products, eight per 32-column block
// and vector, become the bulk of its work (oxinfer README, "Speculative decoding": the
// multi-token int8 decode variants are instruction-bound at Q4). The same exact integer
// sub-block products P = sum q * xq are formed here on the matrix cores, where one instruction
// does 16 rows x 64 columns x 16 outputs:
//
//  * The weight operand is the 4-bit codes themselves as int8 (two masks per 8 codes); the
//    activation operand is the int8 codes as stored. Nothing is scaled inside the product, so
//    the int32 result is P exactly.
//  * A product covers two 32-column blocks: the 16 output columns are 8 vectors x the two
//    blocks, and the activation operand holds zeros where a vector's block does not meet the
//    weight columns of the other block. Every output is then the P of one (vector, block, row).
//    With 9..16 vectors a second product per pair of blocks takes the second group of 8 from
//    the same weight operand.
//  * The float work per output and block is the exact integer sc * P, its conversion and one
//    fma with the activation scale; the super-scale d is applied once per super-block. The min
//    term dmin * m * xd * S (S = sum of the block's codes) is a contraction over the blocks of
//    dmin * m (block, row) with -xd * S (vector, block), done on the float32 matrix cores
//    (v_mfma_f32_16x16x4_f32, four blocks per instruction) straight into the accumulator.
//
// Work split: a workgroup of up to 4 waves takes row tiles of 16 rows in turn over one column
// split of up to 8 super-blocks, each wave two super-blocks; the waves' sums are added in LDS
// in wave order. The split's activation (codes in the operand order, scales, -xd * S) is staged
// in LDS once per workgroup, so the loop over row tiles reads only weights from memory: per
// lane and super-block two 16-byte code loads (the four lanes of a row read 64 contiguous
// bytes; one exchange between lane groups then gives each lane the half-chunks it multiplies)
// and the 16-byte header. The next tile's loads go out as soon as the current tile's
// arithmetic has read the registers, ahead of the sums over the waves and the stores.
//
// Lane layouts (16 x 16 products, checked on gfx950): lane l holds operand row / column l % 16,
// slots of lane group g = l / 16; result element i is row 4 g + i, column l % 16. Which column
// each (group, slot) stands for is free as long as both operands agree; here the weight lane of
// group g multiplies the 8 code bytes 8 (g % 2) .. + 7 of block 2 t + g / 2 of the pair t,
// slots 0..7 their low nibbles (columns 8 (g % 2) + 0..7) and 8..15 their high nibbles
// (columns 16 + 8 (g % 2) + 0..7). The staged activation of a block is stored in that order.
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kSbw = kI8SbPerWave;                  // super-blocks per wave

// LDS of a workgroup of `waves` waves (split of kSbw * waves super-blocks) for vg groups of 8
// vectors: 8 vg + 1 rows of codes (the vectors, then zeros) of pitch columns + 16 bytes (the 16
// spread the rows over the banks), the scales and -xd * S of the split's blocks (8 vg vectors
// each), and two slots of the waves' sums of a row tile (16 rows x 8 vg vectors per wave).
__host__ __device__ constexpr int code_pitch(int waves) { return waves * kSbw * 256 + 16; }
__host__ __device__ constexpr int lds_bytes(int waves, int vg) {
    return (8 * vg + 1) * code_pitch(waves) + 2 * (waves * kSbw * 8) * (8 * vg) * 4 +
           2 * waves * 16 * (8 * vg) * 4;
}

// Staging passes of the fused form at most: each group of 8 lanes quantizes one 32-column block
// per pass; 8 vectors x 8 nsb blocks over 8 waves groups, with nsb <= kSbw waves. The form from
// codes takes a block per 2 lanes, a quarter of the passes per group of 8 vectors.
constexpr int kStagePasses = 8 * kSbw;

// VG groups of 8 vectors per launch (nvec <= 8 VG): every group multiplies the same loaded
// weights (one product per group and pair of blocks).
// KEEP: the wave's activation operands stay in registers for the whole kernel (one group of 8
// vectors, a launch of at most two row tiles per workgroup); otherwise every product reads its
// operands from LDS as it goes, which leaves registers for more resident waves when each
// workgroup walks many tiles.
template <int MODE, int VG, int KEEP>
__global__ void __launch_bounds__(256) gemm_q4k_i8_kernel(GemmArgs a) {
    constexpr bool DBG = MODE == kModeDebug;
    constexpr bool FUSED = MODE == kModeFused;
    constexpr int NV = 8 * VG;      // vector slots
    static_assert(!FUSED || VG == 1, "the fused form takes up to 8 vectors");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_i8[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int waves = blockDim.x >> 6;
    const int pitch = code_pitch(waves);
    const int sblk = waves * kSbw * 8;
    uint8_t *const xq_s = lds_i8;                   // [NV + 1][pitch]: codes (block-permuted), zeros
    float *const xd_s = reinterpret_cast<float *>(lds_i8 + (NV + 1) * pitch);   // [sblk][NV]
    float *const xs_s = xd_s + sblk * NV;           // [sblk][NV]: -xd * S
    float *const red_s = xs_s + sblk * NV;          // [2][waves][16][NV]
    const int r = lane & 15;        // tile row of this lane's weights and outputs
    const int g = lane >> 4;        // lane group
    const int q = g >> 1;           // block of the pair this lane's weights and outputs are in
    const int rows = a.rows, nb = a.nb, nvec = a.nvec;
    const int nbk = nb * 8;
    const int row_tiles = a.row_tiles;
    const int sb_lo = blockIdx.y * a.sb_per_split;
    const int sb_hi = min(nb, sb_lo + a.sb_per_split);
    const int nsb = sb_hi - sb_lo;
    const int wsb = wave * kSbw;    // this wave's first super-block, relative to sb_lo
    const uint8_t *hplane = a.w + static_cast<int64_t>(rows) * nb * 128;

    int rt = blockIdx.x;
    if (rt >= row_tiles) return;    // the whole workgroup (never taken: grid <= row tiles)

    // One row tile's loads per super-block: two 16-byte code chunks and the header. The four
    // lanes of a row read the 64 bytes of chunks 4 i .. 4 i + 3 together (i = 0, 1): lane group
    // g takes chunk 4 i + pc, pc = 2 (g % 2) + g / 2, so the lanes of even groups hold the
    // chunks of pairs t = 0 and 2 and those of odd groups the chunks of pairs 1 and 3 (block
    // 2 t + g / 2 each); one exchange between the groups (in `products`) then gives every lane
    // the half it multiplies. A wave with fewer super-blocks than kSbw (the split's end) reloads
    // the split's last one, unused. Rows past the matrix read its last row (not stored).
    const int pc = 2 * (g & 1) + (g >> 1);
    auto issue = [&](int tile, uint4 (&c)[kSbw][2], uint4 (&h)[kSbw]) {
        const int row = min(tile * 16 + r, rows - 1);
#pragma unroll
        for (int k = 0; k < kSbw; k++) {
            const int sb = sb_lo + min(wsb + k, nsb - 1);
            const int64_t blk = static_cast<int64_t>(row) * nb + sb;
            const uint8_t *src = a.w + blk * 128 + 16 * pc;
            c[k][0] = load16(src);
            c[k][1] = load16(src + 64);
            h[k] = load16(hplane + blk * 16);
        }
    };
    // Two row tiles' weights go out before anything waits: this workgroup's tiles rt and
    // rt + stride (the second clamped to the last tile when the workgroup has only one), after
    // the staging's loads and before the staging's arithmetic, so the wait for the staged
    // activation never waits for the weights, and both tiles are in flight from the start.
    const int stride = static_cast<int>(gridDim.x);
    const int ntiles = (row_tiles - rt + stride - 1) / stride;      // this workgroup's tiles
    uint4 cwA[kSbw][2], cwB[kSbw][2];
    uint4 hdA[kSbw], hdB[kSbw];
    auto issue_first_two = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        issue(rt, cwA, hdA);
        issue(min(rt + stride, row_tiles - 1), cwB, hdB);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- the split's activation into LDS: codes permuted per block (columns 0-7, 16-23,
    //      8-15, 24-31), scales and -xd * S; zeros for vectors past nvec. All loads go out
    //      first. From codes: 2 lanes per block (16 columns each); the fused form quantizes
    //      the float32 block itself, 8 lanes per block (4 columns each), and the first
    //      workgroup of the split also stores the codes and scales ----
    for (int i = tid; i < pitch / 16; i += blockDim.x)
        *reinterpret_cast<uint4 *>(xq_s + NV * pitch + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
    {
        const int nblk = nsb * 8;
        const int items = NV * nblk;                    // (vector, block), vector-major
        for (int it = nvec * nblk + tid; it < items; it += blockDim.x) {
            const int v = it / nblk, b = it - v * nblk;
            xd_s[b * NV + v] = 0.0f;
            xs_s[b * NV + v] = 0.0f;
        }
        if constexpr (FUSED) {
            const int per_pass = static_cast<int>(blockDim.x) >> 3;
            const int passes = (nvec * nblk + per_pass - 1) / per_pass;   // <= kStagePasses
            const int j8 = tid & 7;
            // dword of the permuted block image holding columns 4 j8 .. 4 j8 + 3
            const int pd = j8 + ((j8 >> 1) == 1 ? 2 : ((j8 >> 1) == 2 ? -2 : 0));
            float4 xv[kStagePasses];
#pragma unroll
            for (int ps = 0; ps < kStagePasses; ps++) {
                const int item = ps * per_pass + (tid >> 3);
                const int v = item / nblk;
                const int64_t gb = static_cast<int64_t>(v) * nbk + sb_lo * 8 + (item - v * nblk);
                xv[ps] = ps < passes && v < nvec
                             ? *reinterpret_cast<const float4 *>(a.x + gb * 32 + 4 * j8)
                             : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
            issue_first_two();
#pragma unroll
            for (int ps = 0; ps < kStagePasses; ps++) {
                if (ps < passes) {            // the same in every lane of the workgroup
                    const int item = ps * per_pass + (tid >> 3);
                    const int v = item / nblk, b = item - v * nblk;
                    const int64_t gb = static_cast<int64_t>(v) * nbk + sb_lo * 8 + b;
                    const ActQuad aq = quantize_act_quad(xv[ps]);   // all lanes: DPP over 8
                    // the block's code sum: exact in float32 (|S| <= 4064)
                    const float s = group_sum<8>(static_cast<float>(byte_sum(aq.codes, 0)));
                    if (v < nvec) {
                        if (a.xq_out != nullptr && blockIdx.x == 0) {
                            reinterpret_cast<uint32_t *>(a.xq_out)[gb * 8 + j8] = aq.codes;
                            if (j8 == 0) a.xd_out[gb] = aq.scale;
                        }
                        *reinterpret_cast<uint32_t *>(xq_s + v * pitch + 32 * b + 4 * pd) = aq.codes;
                        if (j8 == 0) {
                            xd_s[b * NV + v] = aq.scale;
                            xs_s[b * NV + v] = -(aq.scale * s);
                        }
                    }
                }
            }
        } else {
            const int per_pass = static_cast<int>(blockDim.x) >> 1;
            const int passes = (nvec * nblk + per_pass - 1) / per_pass;   // <= VG kStagePasses / 4
            const int h = tid & 1;
            uint4 cv[VG * kStagePasses / 4];
            float sv[VG * kStagePasses / 4];
#pragma unroll
            for (int ps = 0; ps < VG * kStagePasses / 4; ps++) {
                const int item = ps * per_pass + (tid >> 1);
                const int v = item / nblk;
                const int64_t gb = static_cast<int64_t>(v) * nbk + sb_lo * 8 + (item - v * nblk);
                const bool live = ps < passes && v < nvec;
                cv[ps] = live ? load16(a.xq + gb * 32 + 16 * h) : make_uint4(0u, 0u, 0u, 0u);
                sv[ps] = live ? a.xd[gb] : 0.0f;
            }
            issue_first_two();
#pragma unroll
            for (int ps = 0; ps < VG * kStagePasses / 4; ps++) {
                if (ps < passes) {            // the same in every lane of the workgroup
                    const int item = ps * per_pass + (tid >> 1);
                    const int v = item / nblk, b = item - v * nblk;
                    const uint4 c = cv[ps];
                    // the block's code sum (the two halves added across the lane pair): exact
                    const int half = byte_sum(c.x, byte_sum(c.y, byte_sum(c.z, byte_sum(c.w, 0))));
                    const int s = half + __builtin_amdgcn_update_dpp(0, half, kDppXor1, 0xF, 0xF, false);
                    if (v < nvec) {
                        // columns 16 h .. + 7 to position 8 h, columns 16 h + 8 .. + 15 to 16 + 8 h
                        uint8_t *dst = xq_s + v * pitch + 32 * b;
                        *reinterpret_cast<uint2 *>(dst + 8 * h) = make_uint2(c.x, c.y);
                        *reinterpret_cast<uint2 *>(dst + 16 + 8 * h) = make_uint2(c.z, c.w);
                        if (h == 0) {
                            xd_s[b * NV + v] = sv[ps];
                            xs_s[b * NV + v] = -(sv[ps] * static_cast<float>(s));
                            if (DBG && blockIdx.x == 0)
                                a.S[static_cast<int64_t>(v) * nbk + sb_lo * 8 + b] = s;
                        }
                    }
                }
            }
        }
    }
    // (the staging's loads, used or not, were issued before the weights, so every wait for
    // the weights below also covers them)
    __syncthreads();

    // ---- where this lane reads its activation operands in LDS (for every row tile), per
    //      group gi of 8 vectors: the operand row of vector 8 gi + av, block ap of each pair
    //      (the zero row where the vector is past nvec or the block does not meet this lane
    //      group's weights), the scales of the output vectors 8 gi + 4 (g % 2) .. + 3, and the
    //      min-term operands ----
    const int av = lane & 7, ap = (lane >> 3) & 1;
    const uint8_t *arow[VG];
    const float *xrow[VG];
    float mina[VG][kSbw][2];
#pragma unroll
    for (int gi = 0; gi < VG; gi++) {
        const int v = 8 * gi + av;
        arow[gi] = xq_s + (((g >> 1) == ap && v < nvec) ? v : NV) * pitch + ap * 32 + 16 * (g & 1);
        xrow[gi] = xd_s + q * NV + 8 * gi + 4 * (g & 1);
        const int am = lane & 15;
#pragma unroll
        for (int k = 0; k < kSbw; k++) {
            const int sbl = min(wsb + k, nsb - 1);
#pragma unroll
            for (int u = 0; u < 2; u++)
                mina[gi][k][u] = am < 8 ? xs_s[(sbl * 8 + 4 * u + g) * NV + 8 * gi + am] : 0.0f;
        }
    }

    // This wave's activation operands (codes and scales of every pair of blocks it multiplies)
    // are the same for every row tile. With KEEP they are read from LDS once, all together (one
    // wait for the lot instead of one LDS round trip ahead of each product), into 64 registers
    // kept for the whole kernel (16384 x 2048 x 8: 8.1 against 8.7 us); that halves the resident
    // waves, so launches whose workgroups walk many tiles read them per product instead
    // (262144 x 1536 x 8: 50 against 57 us).
    struct ActOps {
        v4i_t A[kSbw][4];
        v4f_t X[kSbw][4];
    };
    ActOps ops;
    if constexpr (KEEP) {
#pragma unroll
        for (int k = 0; k < kSbw; k++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int blk = (wsb + k) * 8 + 2 * t;    // within the split's staged blocks
                ops.A[k][t] = *reinterpret_cast<const v4i_t *>(arow[0] + blk * 32);
                ops.X[k][t] = *reinterpret_cast<const v4f_t *>(xrow[0] + blk * NV);
            }
    }

    float *out = DBG ? nullptr : a.out + static_cast<int64_t>(blockIdx.y) * nvec * rows;
    int slot = 0;
    // Row tile `rt` from the loaded registers (cw, hd): its products, folded to this lane's two
    // outputs per group gi (vectors 8 gi + vv and 8 gi + vv + 2 of row r, vv = 4 (g % 2) + l / 32).
    auto products = [&](int rt, const uint4 (&cw)[kSbw][2], const uint4 (&hd)[kSbw],
                        float (&fold)[VG][2]) {
        v4f_t acc[VG];
#pragma unroll
        for (int gi = 0; gi < VG; gi++) acc[gi] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < kSbw; k++) {
            if (wsb + k < nsb) {            // the same in every lane of the wave
                const uint4 h = hd[k];
                const float d = half_to_float(h.x & 0xFFFFu);
                const float dmin = half_to_float(h.x >> 16);
                // sub-scale of block 2 t + q: low 4 bits at y bit 4 (2 t + q), high 2 bits at w bit
                // 2 (2 t + q)
                const uint32_t ysh = h.y >> (4 * q), wsh = h.w >> (2 * q);
                // The exchange: the half-chunks an even group sends (the upper halves of its
                // chunks) swap with those its odd neighbour sends (the lower halves of its
                // chunks), v_permlane16_swap pairing rows of 16 lanes 0-1 and 2-3. Afterwards
                // pair t's 8 code bytes are dwords 2 (t % 2), + 1 of chunk register t / 2.
                uint32_t pw[4][2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const auto s0 = __builtin_amdgcn_permlane16_swap(cw[k][i].x, cw[k][i].z, false, false);
                    const auto s1 = __builtin_amdgcn_permlane16_swap(cw[k][i].y, cw[k][i].w, false, false);
                    const uint32_t x = s0[0], z = s0[1], y = s1[0], w = s1[1];
                    pw[2 * i][0] = x;
                    pw[2 * i][1] = y;
                    pw[2 * i + 1][0] = z;
                    pw[2 * i + 1][1] = w;
                }
                // The four pairs' weight operands and sub-scales first, then their products
                // back to back into separate registers, then the float work on the results:
                // no product waits for the previous one's float work, and no float work waits
                // on the product just issued.
                v4i_t B[4];
                int sc[4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const uint2 c = make_uint2(pw[t][0], pw[t][1]);
                    B[t] = v4i_t{static_cast<int>(c.x & 0x0F0F0F0Fu),
                                 static_cast<int>(c.y & 0x0F0F0F0Fu),
                                 static_cast<int>((c.x >> 4) & 0x0F0F0F0Fu),
                                 static_cast<int>((c.y >> 4) & 0x0F0F0F0Fu)};
                    sc[t] = static_cast<int>(((ysh >> (8 * t)) & 15u) | (((wsh >> (4 * t)) & 3u) << 4));
                }
                v4i_t P[VG][4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const int blk = (wsb + k) * 8 + 2 * t;      // first block of the pair, in the split
#pragma unroll
                    for (int gi = 0; gi < VG; gi++) {
                        const v4i_t A = KEEP ? ops.A[k][t]
                                                : *reinterpret_cast<const v4i_t *>(arow[gi] + blk * 32);
                        const v4i_t zero = {0, 0, 0, 0};
                        P[gi][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B[t], zero, 0, 0, 0);
                    }
                }
                v4f_t tt[VG];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const int blk = (wsb + k) * 8 + 2 * t;
#pragma unroll
                    for (int gi = 0; gi < VG; gi++) {
                        const v4f_t xdv = KEEP ? ops.X[k][t]
                                                  : *reinterpret_cast<const v4f_t *>(xrow[gi] + blk * NV);
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const float ps = static_cast<float>(__mul24(sc[t], P[gi][t][i]));   // exact: < 2^22
                            tt[gi][i] = t == 0 ? xdv[i] * ps : fmaf(xdv[i], ps, tt[gi][i]);
                        }
                        if (DBG) {
                            const int row = rt * 16 + r;
                            const int gblk = sb_lo * 8 + blk + q;
#pragma unroll
                            for (int i = 0; i < 4; i++) {
                                const int v = 8 * gi + 4 * (g & 1) + i;
                                if (v < nvec && row < rows)
                                    a.P[(static_cast<int64_t>(v) * rows + row) * nbk + gblk] = P[gi][t][i];
                            }
                        }
                    }
                }
#pragma unroll
                for (int gi = 0; gi < VG; gi++)
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[gi][i] = fmaf(d, tt[gi][i], acc[gi][i]);
                // min terms of blocks 4 u + g: m low 4 bits at z bit 4 (4 u + g), high 2 bits at w
                // bit 16 + 2 (4 u + g)
                const uint32_t zsh = h.z >> (4 * g), wsh2 = h.w >> (16 + 2 * g);
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    const uint32_t m = ((zsh >> (16 * u)) & 15u) | (((wsh2 >> (8 * u)) & 3u) << 4);
                    const float dm = dmin * static_cast<float>(m);
#pragma unroll
                    for (int gi = 0; gi < VG; gi++)
                        acc[gi] = __builtin_amdgcn_mfma_f32_16x16x4f32(mina[gi][k][u], dm, acc[gi], 0, 0, 0);
                }
            }
        }

        // ---- the two blocks of each pair sit in lane groups g and g + 2 (lanes l, l + 32).
        //      One swap of the upper half of element 2 e with the lower half of element
        //      2 e + 1 leaves, after one add, element 2 e's pair sum in lanes 0-31 and element
        //      2 e + 1's in lanes 32-63: lane l then holds vectors vv and vv + 2 of row r, with
        //      vv = 4 (g % 2) + l / 32. The waves' sums are then added in LDS, in wave order ----
        // (The elements are copied to scalars first: __builtin_bit_cast of a vector element
        // read the vector's first element with this compiler.)
#pragma unroll
        for (int gi = 0; gi < VG; gi++)
#pragma unroll
            for (int e = 0; e < 2; e++) {
                const float lo = acc[gi][2 * e], hi = acc[gi][2 * e + 1];
                const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, lo),
                                                                 __builtin_bit_cast(uint32_t, hi),
                                                                 false, false);
                const uint32_t s0 = sw[0], s1 = sw[1];
                fold[gi][e] = __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
            }
    };
    // The sums over the workgroup's waves (in wave order) and the stores of row tile rt.
    auto finish = [&](int rt, const float (&fold)[VG][2]) {
        if (!DBG) {
            const int vv = 4 * (g & 1) + (lane >> 5);
#pragma unroll
            for (int gi = 0; gi < VG; gi++) {
                red_s[((slot * waves + wave) * 16 + r) * NV + 8 * gi + vv] = fold[gi][0];
                red_s[((slot * waves + wave) * 16 + r) * NV + 8 * gi + vv + 2] = fold[gi][1];
            }
            __syncthreads();
            // 16 NV outputs, output e by thread e % blockDim (a fixed number of stores per
            // lane, so the compiler can count the loads still in flight past them instead of
            // waiting for all of them)
#pragma unroll
            for (int i = 0; i < 2 * VG; i++) {
                const int e = tid + static_cast<int>(blockDim.x) * i;
                const int v = e >> 4, rr = e & 15;
                const int row = rt * 16 + rr;
                if (e < 16 * NV && v < nvec && row < rows) {
                    float y = red_s[((slot * waves) * 16 + rr) * NV + v];
#pragma unroll
                    for (int w = 1; w < kI8MaxWaves; w++)
                        if (w < waves) y += red_s[((slot * waves + w) * 16 + rr) * NV + v];
                    out[static_cast<int64_t>(v) * rows + row] = y;
                }
            }
            slot ^= 1;
        }
    };
    // One or two tiles: both are in flight already. More: tile 3 goes into the first set as
    // soon as tile 1's arithmetic has read it, and from then on each tile's successor goes out
    // into the same registers right after the tile's arithmetic, ahead of the sums over the
    // waves and the stores (past the last tile it reloads the last one, unused). The branches
    // are uniform over the workgroup and every wait in them counts only loads issued on the
    // same path.
    float fold[VG][2];
    if (ntiles <= 2) {
        __builtin_amdgcn_sched_barrier(0);
        products(rt, cwA, hdA, fold);
        __builtin_amdgcn_sched_barrier(0);
        finish(rt, fold);
        if (ntiles == 2) {
            __builtin_amdgcn_sched_barrier(0);
            products(rt + stride, cwB, hdB, fold);
            __builtin_amdgcn_sched_barrier(0);
            finish(rt + stride, fold);
        }
        return;
    }
    __builtin_amdgcn_sched_barrier(0);
    products(rt, cwA, hdA, fold);
    __builtin_amdgcn_sched_barrier(0);
    issue(rt + 2 * stride, cwA, hdA);
    __builtin_amdgcn_sched_barrier(0);
    finish(rt, fold);
    __builtin_amdgcn_sched_barrier(0);
    products(rt + stride, cwB, hdB, fold);
    __builtin_amdgcn_sched_barrier(0);
    finish(rt + stride, fold);
    rt += 2 * stride;
    while (true) {
        __builtin_amdgcn_sched_barrier(0);
        products(rt, cwA, hdA, fold);
        __builtin_amdgcn_sched_barrier(0);
        issue(min(rt + stride, row_tiles - 1), cwA, hdA);
        __builtin_amdgcn_sched_barrier(0);
        finish(rt, fold);
        rt += stride;
        if (rt >= row_tiles) break;
    }
}

}  // namespace

namespace {

template <int VG>
hipError_t launch_vg(const GemmArgs &a, int waves, bool debug, hipStream_t stream) {
    // Workgroups of this size resident at once (registers and LDS) times the CUs, looked up
    // once per form and size; each workgroup then takes an equal share of the row tiles, and at
    // least two (the staging is per workgroup, and a second tile's loads overlap the first
    // tile's arithmetic: 16384 x 2048 x 8 measured 9.6 us against 10.3 us with one tile per
    // workgroup). Concurrent first calls store the same values. The residency is that of the
    // form that walks many tiles (KEEP = 0). With one group of 8 vectors, at most two tiles per
    // workgroup and every workgroup resident at once in the form that keeps its operands in
    // registers (KEEP = 1, fewer resident workgroups), that form runs (32768 x 2048 x 8: two
    // rounds of it, 14.3 us, against one of the other, 13.7 us).
    static std::atomic<int> per_cu[3][kI8MaxWaves] = {};
    static std::atomic<int> per_cu_keep[3][kI8MaxWaves] = {};
    static std::atomic<int> cus{0};
    if (cus.load(std::memory_order_relaxed) == 0) {
        int dev = 0, n = 0;
        const bool ok = hipGetDevice(&dev) == hipSuccess &&
                        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                            hipSuccess &&
                        n > 0;
        cus.store(ok ? n : 256, std::memory_order_relaxed);
    }
    const int mode = debug ? kModeDebug : (a.x != nullptr ? kModeFused : kModePlain);
    if (mode == kModeFused && VG != 1) return hipErrorInvalidValue;
    const int threads = 64 * waves;
    const size_t lds = static_cast<size_t>(lds_bytes(waves, VG));
    std::atomic<int> &res = per_cu[mode][waves - 1];
    if (res.load(std::memory_order_relaxed) == 0) {
        int n = 0;
        hipError_t e;
        if (mode == kModeDebug)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_q4k_i8_kernel<kModeDebug, VG, 0>, threads, lds);
        else if (mode == kModeFused)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_q4k_i8_kernel<kModeFused, 1, 0>, threads, lds);
        else
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_q4k_i8_kernel<kModePlain, VG, 0>, threads, lds);
        res.store((e == hipSuccess && n > 0) ? n : 1, std::memory_order_relaxed);
    }
    std::atomic<int> &res_keep = per_cu_keep[mode][waves - 1];
    if (VG == 1 && mode != kModeDebug && res_keep.load(std::memory_order_relaxed) == 0) {
        int n = 0;
        const hipError_t e =
            mode == kModeFused
                ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_q4k_i8_kernel<kModeFused, 1, 1>, threads, lds)
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_q4k_i8_kernel<kModePlain, 1, 1>, threads, lds);
        res_keep.store((e == hipSuccess && n > 0) ? n : 1, std::memory_order_relaxed);
    }
    const int64_t cap = std::max<int64_t>(
        1, int64_t{res.load(std::memory_order_relaxed)} * cus.load(std::memory_order_relaxed) /
               a.splits);
    const int64_t per_wg = std::max<int64_t>(2, (a.row_tiles + cap - 1) / cap);
    const int64_t blocks = (a.row_tiles + per_wg - 1) / per_wg;
    const bool keep = VG == 1 && mode != kModeDebug && per_wg <= 2 &&
                      blocks * a.splits <= int64_t{res_keep.load(std::memory_order_relaxed)} *
                                               cus.load(std::memory_order_relaxed);
    const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(a.splits));
    const dim3 block(static_cast<unsigned>(threads));
    if (mode == kModeDebug)
        hipLaunchKernelGGL((gemm_q4k_i8_kernel<kModeDebug, VG, 0>), grid, block, lds, stream, a);
    else if (mode == kModeFused && keep)
        hipLaunchKernelGGL((gemm_q4k_i8_kernel<kModeFused, 1, 1>), grid, block, lds, stream, a);
    else if (mode == kModeFused)
        hipLaunchKernelGGL((gemm_q4k_i8_kernel<kModeFused, 1, 0>), grid, block, lds, stream, a);
    else if (keep)
        hipLaunchKernelGGL((gemm_q4k_i8_kernel<kModePlain, 1, 1>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((gemm_q4k_i8_kernel<kModePlain, VG, 0>), grid, block, lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_q4k_i8(const GemmArgs &a, int waves, bool debug, hipStream_t stream) {
    if (waves < 1 || waves > kI8MaxWaves || a.sb_per_split != kSbw * waves || a.nvec < 1 ||
        a.nvec > kI8MaxVec || a.row_tiles < 1 || a.splits < 1)
        return hipErrorInvalidValue;
    if (a.nvec <= 8) return launch_vg<1>(a, waves, debug, stream);
    return launch_vg<2>(a, waves, debug, stream);
}

}  // namespace qgemv
