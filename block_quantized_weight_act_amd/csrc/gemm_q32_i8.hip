// Q8_0, Q4_0, Q6_K and Q4_K weights x 1..16 int8 activation vectors on the integer matrix cores
// (v_mfma_i32_16x16x64_i8).
//
// With a few vectors the vector kernel's int8 4-way dot products, eight per 32-weight block and
// vector, bound it (oxinfer README, "Speculative decoding": the multi-token int8 variants are
// instruction-bound at Q4). Here the same exact block partials P are formed on the matrix
// cores:
//
//  * One product covers 16 rows x 64 columns x 16 output slots. Its 64 columns are four 16-code
//    halves, one per lane group g: the halves of blocks 4 i + g (g = 0..3) of the wave's 16
//    blocks, so a lane's weight operand is exactly the 16 bytes it loaded (Q8_0: one 16-byte
//    plane chunk; Q4_0: the low or the high nibbles of its block's 16 bytes, which hold weights
//    0..15 and 16..31). The 16 output slots are 4 blocks x 4 vectors: the activation operand
//    of slot (block g', vector v) holds the vector's codes at lane group g' and zeros in the
//    other three, so every output is one (row, vector, block) partial. Two products (the two
//    halves of the blocks) accumulate into one P; each further half of 4 vectors (up to 4)
//    takes another pair with the same weight operands.
//  * Q4_0 stores codes 0..15 for weights q - 8, and P = sum (q - 8) xq comes out exact, as the
//    vector kernel and the oracle define it, in one of two ways. With up to 8 vectors the
//    weight operand is the codes and the first product's accumulator input is -8 S (S the
//    activation block's code sum, kept in registers). With 9..16 the weight operand is
//    16 (q - 8) as int8 (each nibble moved to the high half of its byte with its top bit
//    flipped), so the products give 16 P with no accumulator input to read from LDS; the 16
//    stays in the float sums and comes out once per output when y is stored (scaling by a
//    power of two commutes with float32 rounding, so y is the one P itself gives wherever the
//    sums stay normal and finite, |y| below 2^123).
//  * Float work per output and block: (d * xd) and one fma with P converted, as in the vector
//    kernel, so y stays within the same bound.
//
// Work split: a workgroup of up to 4 waves stages the activation of one column split (16
// blocks per wave) in LDS once, then takes row tiles of 16 rows in turn; each wave multiplies
// its 16 blocks of the tile and the waves' sums are added in LDS in wave order. A lane (row r,
// lane group g) loads per tile and i = 0..3 the code chunk(s) of block 4 i + g of its row (the
// four lanes of a row read 64 contiguous bytes per plane) and that block's scale; the lane
// then holds the outputs of those blocks, so the scale is the one it loaded. Two tiles' loads
// are in flight from the start and each tile's successor goes out right after its arithmetic.
//
// Lane layouts of both 16 x 16 products (checked on gfx950 for the Q4_K kernel): operand lane
// l holds row (or column) l % 16, slots of lane group l / 16; result element e is row
// 4 (l / 16) + e, column l % 16. Here the activation is the row operand (slots) and the weights
// the column operand (rows of the tile).
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "gemm_mc.h"

namespace qgemv {

namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kBw = kQ32I8BlocksPerWave;

// LDS of a workgroup of `waves` waves and NV vector slots: NV rows of codes (the split's blocks)
// and a row of zeros, each of pitch bytes (the 16 spread the rows over the banks); the scales
// and Q4_0's -8 S or Q4_K's -xd S of the split's blocks [block][NV]; two slots of the waves'
// sums of a row tile.
__host__ __device__ constexpr int q32i8_pitch(int waves) { return waves * kBw * 32 + 16; }
__host__ __device__ constexpr int q32i8_lds_bytes(int waves, int nv) {
    return (nv + 1) * q32i8_pitch(waves) + 2 * waves * kBw * nv * 4 + 2 * waves * 16 * nv * 4;
}

// H halves of 4 vectors (nvec <= 4 H). VS: rows of whole groups of 4 blocks (cols a multiple of
// 128), so a lane's 4 scales are one aligned load (otherwise one load per block).
template <int FMT, int MODE, int H, bool VS>
__global__ void __launch_bounds__(256) gemm_q32_i8_kernel(GemmArgs a) {
    constexpr bool DBG = MODE == kModeDebug;
    constexpr bool Q40 = FMT == kTypeQ40;
    constexpr bool Q6 = FMT == kTypeQ6K;
    constexpr bool QK = FMT == kTypeQ4K;
    constexpr int NV = 4 * H;
    constexpr int NP = FMT == kTypeQ80 ? 2 : 1;    // 16-byte code chunks per block and lane
    // One tile in flight per wave from the start (SINGLE), or two (the first two tiles) with the
    // registers of a second set: with 5..8 Q6_K or Q4_0 vectors the second set costs more
    // resident waves than it gains (262144 x 1536 x 8: Q6_K 72.4 against 113.1 us, Q4_0 44.1
    // against 54.5 us); with 1..4 vectors, and for Q8_0, it gains (Q6_K x 4: 66.3 against 74.0,
    // Q8_0 x 8: 84.2 against 91.3 us).
    constexpr bool SINGLE = (H == 2 && FMT != kTypeQ80) || H >= 3;
    // With up to 8 vectors the activation scales (and Q4_0's -8 S) of the lane's outputs stay in
    // registers for the whole kernel; with more the scales are read from LDS per product, and
    // Q4_0's weight operand is 16 (q - 8) (X16: measured on 65536 x 2048, 16 vectors 25.9 ->
    // 23.3 us, 12 vectors 19.8 -> 19.2; with 8 on 262144 x 1536 it lost 2%).
    constexpr bool KEEP = H <= 2;
    constexpr bool X16 = Q40 && !KEEP;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_q32i8[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int threads = static_cast<int>(blockDim.x);
    const int waves = threads >> 6;
    const int pitch = q32i8_pitch(waves);
    const int nblk = waves * kBw;              // staged blocks of the split
    uint8_t *const xq_s = lds_q32i8;           // [NV + 1][pitch]: codes, then zeros
    float *const xd_s = reinterpret_cast<float *>(lds_q32i8 + (NV + 1) * pitch);   // [nblk][NV]
    float *const s8_s = xd_s + nblk * NV;      // [nblk][NV]: Q4_K: -xd S; Q4_0 (not X16): -8 S
    float *const red_s = reinterpret_cast<float *>(s8_s + nblk * NV);  // [2][waves][16][NV]
    const int r = lane & 15;                   // tile row of this lane's weights and outputs
    const int g = lane >> 4;                   // lane group: block 4 i + g of the wave's 16
    const int rows = a.rows, nb = a.nb, nvec = a.nvec;
    const int row_tiles = a.row_tiles;
    const int b_lo = blockIdx.y * a.sb_per_split;
    const int nsb = min(nb, b_lo + a.sb_per_split) - b_lo;   // blocks of this split
    const int wb0 = wave * kBw;                // this wave's first block, relative to b_lo
    const int64_t nblocks = static_cast<int64_t>(rows) * nb;
    const uint8_t *const hi_plane = a.w + nblocks * 16;        // Q8_0: codes 16..31; Q6_K: high bits
    const uint8_t *const d_plane = a.w + nblocks * (Q40 ? 16 : (Q6 ? 26 : 32));
    const uint8_t *const sc_plane = a.w + nblocks * (QK ? 16 : 24);  // Q6_K sub-scales; Q4_K headers

    int rt = blockIdx.x;
    if (rt >= row_tiles) return;               // the whole workgroup (never taken: grid <= tiles)

    // One row tile's loads: per i the chunk(s) of block wb0 + 4 i + g of row r (the split's last
    // block where that is past the split: loaded, never used), and the scales: with VS those of
    // blocks wb0 + 4 g .. + 3 in one load (a group past the split reads the split's last group,
    // unused; splits hold whole groups), exchanged between the lane groups in `products`, else
    // that of block wb0 + 4 i + g per i. Rows past the matrix read its last row (not stored).
    // (One load of a lane's four scales instead of four 2- or 4-byte loads: 262144 x 1536 Q4_0
    // with one vector took 50 us with the four loads, 36 us without any.)
    // Q6_K: per i also the 8 high-bit bytes of the block, and per tile the 16 sub-scales and
    // the super-scale of the wave's two super-blocks (a super-block past the split reads the
    // split's last one, unused).
    struct WTile {
        uint4 c[4][NP];
        uint32_t d[4];
        uint2 hb[Q6 ? 4 : 1];
        uint4 sc[Q6 || QK ? 2 : 1];
    };
    auto issue = [&](int tile, WTile &t) {
        const int64_t row = std::min<int64_t>(int64_t{tile} * 16 + r, rows - 1);
        const int64_t rb = row * nb + b_lo;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t blk = rb + min(wb0 + 4 * i + g, nsb - 1);
            t.c[i][0] = load16(a.w + blk * 16);
            if constexpr (Q6) t.hb[i] = *reinterpret_cast<const uint2 *>(hi_plane + blk * 8);
            if constexpr (!Q40 && !Q6) t.c[i][1] = load16(hi_plane + blk * 16);
            if constexpr (!VS && !Q6 && !QK) {
                if constexpr (Q40)
                    t.d[i] = reinterpret_cast<const uint16_t *>(d_plane)[blk];
                else
                    t.d[i] = reinterpret_cast<const uint32_t *>(d_plane)[blk];
            }
        }
        if constexpr (Q6 || QK) {
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const int64_t sbk = (rb + min(wb0 + 8 * q, nsb - 8)) >> 3;
                t.sc[q] = load16(sc_plane + sbk * 16);
                if constexpr (Q6) t.d[q] = reinterpret_cast<const uint16_t *>(d_plane)[sbk];
            }
        }
        if constexpr (VS && !Q6 && !QK) {
            const int64_t b4 = rb + min(wb0 + 4 * g, nsb - 4);
            if constexpr (Q40) {
                const uint2 v = *reinterpret_cast<const uint2 *>(d_plane + b4 * 2);
                t.d[0] = v.x;
                t.d[1] = v.y;
            } else {
                const uint4 v = load16(d_plane + b4 * 4);
                t.d[0] = v.x;
                t.d[1] = v.y;
                t.d[2] = v.z;
                t.d[3] = v.w;
            }
        }
    };
    const int stride = static_cast<int>(gridDim.x);
    WTile tA, tB;     // tB: the second tile of the first two (not with SINGLE)

    // ---- the split's activation into LDS: codes as stored (one (vector, block) item of 32
    //      bytes per thread and pass), scales, -xd S (Q4_K) or -8 S (Q4_0); zeros for vectors past nvec and blocks
    //      past the split. The staging's loads go out first, then both tiles' weights, then the
    //      staging's stores ----
    for (int i = tid; i < pitch / 16; i += threads)
        *reinterpret_cast<uint4 *>(xq_s + NV * pitch + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
    {
        uint4 cv[H][2];
        float sv[H];
#pragma unroll
        for (int p = 0; p < H; p++) {
            const int it = p * threads + tid;  // < NV * nblk = H * threads
            const int v = it / nblk, b = it - v * nblk;
            const bool live = v < nvec && b < nsb;
            const int64_t gb = static_cast<int64_t>(v) * nb + b_lo + b;
            cv[p][0] = live ? load16(a.xq + gb * 32) : make_uint4(0u, 0u, 0u, 0u);
            cv[p][1] = live ? load16(a.xq + gb * 32 + 16) : make_uint4(0u, 0u, 0u, 0u);
            sv[p] = live ? a.xd[gb] : 0.0f;
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(rt, tA);
        if constexpr (!SINGLE) issue(min(rt + stride, row_tiles - 1), tB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < H; p++) {
            const int it = p * threads + tid;
            const int v = it / nblk, b = it - v * nblk;
            const uint4 c0 = cv[p][0], c1 = cv[p][1];
            *reinterpret_cast<uint4 *>(xq_s + v * pitch + 32 * b) = c0;
            *reinterpret_cast<uint4 *>(xq_s + v * pitch + 32 * b + 16) = c1;
            xd_s[b * NV + v] = sv[p];
            if constexpr (QK || (Q40 && !X16) || DBG) {
                const int s = byte_sum(c0.x, byte_sum(c0.y, byte_sum(c0.z, byte_sum(c0.w,
                              byte_sum(c1.x, byte_sum(c1.y, byte_sum(c1.z, byte_sum(c1.w, 0))))))));
                if constexpr (QK) s8_s[b * NV + v] = -(sv[p] * static_cast<float>(s));
                if constexpr (Q40 && !X16) reinterpret_cast<int *>(s8_s)[b * NV + v] = -8 * s;
                if (DBG && blockIdx.x == 0 && v < nvec && b < nsb)
                    a.S[static_cast<int64_t>(v) * nb + b_lo + b] = s;
            }
        }
    }
    __syncthreads();

    // ---- this lane's operands from LDS, the same for every row tile: the activation rows it
    //      reads (slot r: block r / 4 of each group of 4, vector 4 h + r % 4; the zero row
    //      where r / 4 is not this lane group), and for its outputs (vectors 4 h .. 4 h + 3 of
    //      block wb0 + 4 i + g) the scales and Q4_0's -8 S ----
    const bool live = (r >> 2) == g;
    const uint8_t *abase[H];
#pragma unroll
    for (int h = 0; h < H; h++)
        abase[h] = xq_s + (live ? 4 * h + (r & 3) : NV) * pitch + (wb0 + g) * 32;
    v4f_t xdk[4][KEEP ? H : 1];
    v4i_t c8k[4][KEEP ? H : 1];
    float mink[4][H];   // Q4_K: the min-term product's row operand (slot r < 4: -xd S of vector
                        // 4 h + r, block wb0 + 4 i + g; 0 in the other slots)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int h = 0; h < H; h++) {
            const int o = (wb0 + 4 * i + g) * NV + 4 * h;
            if constexpr (KEEP) {
                xdk[i][h] = Q6 ? v4f_t{0.0f, 0.0f, 0.0f, 0.0f} : *reinterpret_cast<const v4f_t *>(xd_s + o);
                c8k[i][h] = Q40 ? *reinterpret_cast<const v4i_t *>(s8_s + o) : v4i_t{0, 0, 0, 0};
            }
            mink[i][h] = QK && r < 4 ? s8_s[(wb0 + 4 * i + g) * NV + 4 * h + r] : 0.0f;
            // (Q6_K reads its activation scales per product instead: its weight operands take
            // more registers)
        }

    auto xd_of = [&](int i, int h) -> v4f_t {
        if constexpr (KEEP) return xdk[i][h];
        else return *reinterpret_cast<const v4f_t *>(xd_s + (wb0 + 4 * i + g) * NV + 4 * h);
    };
    // Q4_0's -8 S as the first product's accumulator input (zeros for the other formats and X16)
    auto c8_of = [&](int i, int h) -> v4i_t {
        if constexpr (KEEP) return c8k[i][h];
        else return v4i_t{0, 0, 0, 0};
    };

    float *out = DBG ? nullptr : a.out + static_cast<int64_t>(blockIdx.y) * nvec * rows;
    int slot = 0;
    // Row tile `tile` from the loaded registers: its products, then the sums over the four
    // lane groups, leaving vectors 4 n + j0 (n < H) of row r in this lane, j0 = 2 (g % 2) + g / 2.
    auto products = [&](int tile, const WTile &t, float (&z)[H]) {
        v4f_t acc[H];
#pragma unroll
        for (int h = 0; h < H; h++) acc[h] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (QK) {
            // Q4_K: the super-scales of the wave's two super-blocks (d, dmin in the header's
            // first word), then per block the exact integer sc * P, one fma with d * xd, and the
            // min term -dmin * m * xd * S as a contraction over the four blocks of the product
            // (lane group g: dmin * m of block 4 i + g; slots 0-3: -xd * S) on the float32
            // matrix cores, straight into the accumulator
            float dq[2], dmq[2];
#pragma unroll
            for (int q = 0; q < 2; q++) {
                dq[q] = half_to_float(t.sc[q].x & 0xFFFFu);
                dmq[q] = half_to_float(t.sc[q].x >> 16);
            }
            const v4i_t zero = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint4 c = t.c[i][0];
                const v4i_t B0 = v4i_t{static_cast<int>(c.x & 0x0F0F0F0Fu), static_cast<int>(c.y & 0x0F0F0F0Fu),
                                       static_cast<int>(c.z & 0x0F0F0F0Fu), static_cast<int>(c.w & 0x0F0F0F0Fu)};
                const v4i_t B1 = v4i_t{static_cast<int>((c.x >> 4) & 0x0F0F0F0Fu),
                                       static_cast<int>((c.y >> 4) & 0x0F0F0F0Fu),
                                       static_cast<int>((c.z >> 4) & 0x0F0F0F0Fu),
                                       static_cast<int>((c.w >> 4) & 0x0F0F0F0Fu)};
                v4i_t P[H];
                v4f_t X[H];
#pragma unroll
                for (int h = 0; h < H; h++) {
                    const v4i_t A0 = *reinterpret_cast<const v4i_t *>(abase[h] + 128 * i);
                    const v4i_t A1 = *reinterpret_cast<const v4i_t *>(abase[h] + 128 * i + 16);
                    P[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B0, zero, 0, 0, 0);
                    P[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B1, P[h], 0, 0, 0);
                    X[h] = xd_of(i, h);
                }
                // sub-scale and min of block bs = 4 (i % 2) + g of super-block i / 2: low 4 bits
                // at bit 4 bs of the second (scales) and third (mins) words, high 2 bits at bit
                // 2 bs (scales) and 16 + 2 bs (mins) of the fourth
                const uint4 hd = t.sc[i >> 1];
                const int bs = 4 * (i & 1) + g;
                const int sc = static_cast<int>(((hd.y >> (4 * bs)) & 15u) | (((hd.w >> (2 * bs)) & 3u) << 4));
                const uint32_t m = ((hd.z >> (4 * bs)) & 15u) | (((hd.w >> (16 + 2 * bs)) & 3u) << 4);
                const bool bv = wb0 + 4 * i + g < nsb;
                const float d = bv ? dq[i >> 1] : 0.0f;
                const float dm = bv ? dmq[i >> 1] * static_cast<float>(m) : 0.0f;
#pragma unroll
                for (int h = 0; h < H; h++) {
#pragma unroll
                    for (int e = 0; e < 4; e++)     // sc * P exact: below 2^22
                        acc[h][e] = fmaf(X[h][e] * d, static_cast<float>(__mul24(sc, P[h][e])),
                                         acc[h][e]);
                    acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(mink[i][h], dm, acc[h], 0, 0, 0);
                    if (DBG) {
                        const int64_t row = int64_t{tile} * 16 + r;
                        const int blk = b_lo + wb0 + 4 * i + g;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int v = 4 * h + e;
                            if (v < nvec && row < rows && bv)
                                a.P[(int64_t{v} * rows + row) * nb + blk] = P[h][e];
                        }
                    }
                }
            }
        } else if constexpr (Q6) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // (one block at a time: hoisting every block's LDS operands ahead took all 256
                // registers with 5..8 vectors)
                __builtin_amdgcn_sched_barrier(0);
                // the two sub-blocks' weight operands q - 32 as int8: the low nibbles (columns
                // 0-15) or high nibbles (16-31) of the low-bit chunk, OR the two high bits h
                // (word s of the high-bit bytes shifted by 2 s) mapped by one byte permute to
                // the upper nibble of q - 32, (h - 2) * 16: 0xE0, 0xF0, 0x00, 0x10
                const uint4 c = t.c[i][0];
                const uint2 hb = t.hb[i];
                const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
                int b0[4], b1[4];
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    const uint32_t u0 = __builtin_amdgcn_perm(0u, 0x1000F0E0u, (hb.x >> (2 * w)) & 0x03030303u);
                    const uint32_t u1 = __builtin_amdgcn_perm(0u, 0x1000F0E0u, (hb.y >> (2 * w)) & 0x03030303u);
                    b0[w] = static_cast<int>((cw[w] & 0x0F0F0F0Fu) | u0);
                    b1[w] = static_cast<int>(((cw[w] >> 4) & 0x0F0F0F0Fu) | u1);
                }
                const v4i_t B0 = v4i_t{b0[0], b0[1], b0[2], b0[3]};
                const v4i_t B1 = v4i_t{b1[0], b1[1], b1[2], b1[3]};
                // P0, P1 = sum (q - 32) xq of the block's two sub-blocks
                v4i_t P0[H], P1[H];
                v4f_t X[H];
                const v4i_t zero = {0, 0, 0, 0};
#pragma unroll
                for (int h = 0; h < H; h++) {
                    const int o = (wb0 + 4 * i + g) * NV + 4 * h;
                    const v4i_t A0 = *reinterpret_cast<const v4i_t *>(abase[h] + 128 * i);
                    const v4i_t A1 = *reinterpret_cast<const v4i_t *>(abase[h] + 128 * i + 16);
                    P0[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B0, zero, 0, 0, 0);
                    P1[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B1, zero, 0, 0, 0);
                    X[h] = *reinterpret_cast<const v4f_t *>(xd_s + o);
                }
                // the sub-scales of block wb0 + 4 i + g: bytes 2 (g % 2), + 1 of dword
                // 2 (i % 2) + g / 2 of super-block i / 2's 16
                const uint4 sw = t.sc[i >> 1];
                const uint32_t word = (i & 1) ? ((g & 2) ? sw.w : sw.z) : ((g & 2) ? sw.y : sw.x);
                const int sh = 16 * (g & 1);
                const int sc0 = static_cast<int>(static_cast<int8_t>(word >> sh));
                const int sc1 = static_cast<int>(static_cast<int8_t>(word >> (sh + 8)));
                const bool bv = wb0 + 4 * i + g < nsb;
                const float d = bv ? half_to_float(t.d[i >> 1]) : 0.0f;
#pragma unroll
                for (int h = 0; h < H; h++) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        // exact: |sc P| < 2^23 for each sub-block, the sum below 2^24
                        const int T = __mul24(sc0, P0[h][e]) + __mul24(sc1, P1[h][e]);
                        acc[h][e] = fmaf(X[h][e] * d, static_cast<float>(T), acc[h][e]);
                    }
                    if (DBG) {
                        const int64_t row = int64_t{tile} * 16 + r;
                        const int blk = b_lo + wb0 + 4 * i + g;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int v = 4 * h + e;
                            if (v < nvec && row < rows && bv) {
                                int32_t *pp = a.P + (int64_t{v} * rows + row) * (2 * int64_t{nb}) + 2 * blk;
                                pp[0] = P0[h][e];
                                pp[1] = P1[h][e];
                            }
                        }
                    }
                }
            }
        } else {
            // dl[i]: the scale of block wb0 + 4 i + g
            float dl[4];
            if constexpr (VS) {
                // m[j] (lane group g) = scale of block wb0 + 4 g + j; dl[i] (lane group g) = m[g] of
                // lane group i: a 4 x 4 transpose over the lane groups of each row r, one swap of
                // halves (lanes l, l + 32) and one of rows of 16 (0-1, 2-3) per pair of registers
                float m[4];
                if constexpr (Q40) {
                    m[0] = half_to_float(t.d[0] & 0xFFFFu);
                    m[1] = half_to_float(t.d[0] >> 16);
                    m[2] = half_to_float(t.d[1] & 0xFFFFu);
                    m[3] = half_to_float(t.d[1] >> 16);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; j++) m[j] = __builtin_bit_cast(float, t.d[j]);
                }
                uint32_t x[4];
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, m[j]),
                                                                     __builtin_bit_cast(uint32_t, m[j + 2]),
                                                                     false, false);
                    x[j] = sw[0];
                    x[j + 2] = sw[1];
                }
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const auto sw = __builtin_amdgcn_permlane16_swap(x[2 * j], x[2 * j + 1], false, false);
                    const uint32_t lo = sw[0], hi = sw[1];
                    dl[2 * j] = __builtin_bit_cast(float, lo);
                    dl[2 * j + 1] = __builtin_bit_cast(float, hi);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    dl[i] = Q40 ? half_to_float(t.d[i]) : __builtin_bit_cast(float, t.d[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v4i_t B0, B1;
                if constexpr (Q40 && !X16) {
                    const uint4 c = t.c[i][0];
                    B0 = v4i_t{static_cast<int>(c.x & 0x0F0F0F0Fu), static_cast<int>(c.y & 0x0F0F0F0Fu),
                               static_cast<int>(c.z & 0x0F0F0F0Fu), static_cast<int>(c.w & 0x0F0F0F0Fu)};
                    B1 = v4i_t{static_cast<int>((c.x >> 4) & 0x0F0F0F0Fu),
                               static_cast<int>((c.y >> 4) & 0x0F0F0F0Fu),
                               static_cast<int>((c.z >> 4) & 0x0F0F0F0Fu),
                               static_cast<int>((c.w >> 4) & 0x0F0F0F0Fu)};
                } else if constexpr (X16) {
                    // 16 (q - 8) as int8: bit 3 of each nibble flipped, the nibble in the high
                    // half of its byte (low nibbles: weights 0..15, high: 16..31)
                    const uint32_t x0 = t.c[i][0].x ^ 0x88888888u, x1 = t.c[i][0].y ^ 0x88888888u;
                    const uint32_t x2 = t.c[i][0].z ^ 0x88888888u, x3 = t.c[i][0].w ^ 0x88888888u;
                    B0 = v4i_t{static_cast<int>((x0 << 4) & 0xF0F0F0F0u), static_cast<int>((x1 << 4) & 0xF0F0F0F0u),
                               static_cast<int>((x2 << 4) & 0xF0F0F0F0u), static_cast<int>((x3 << 4) & 0xF0F0F0F0u)};
                    B1 = v4i_t{static_cast<int>(x0 & 0xF0F0F0F0u), static_cast<int>(x1 & 0xF0F0F0F0u),
                               static_cast<int>(x2 & 0xF0F0F0F0u), static_cast<int>(x3 & 0xF0F0F0F0u)};
                } else {
                    B0 = __builtin_bit_cast(v4i_t, t.c[i][0]);
                    B1 = __builtin_bit_cast(v4i_t, t.c[i][1]);
                }
                v4i_t P[H];
                v4f_t X[H];
#pragma unroll
                for (int h = 0; h < H; h++) {
                    const v4i_t A0 = *reinterpret_cast<const v4i_t *>(abase[h] + 128 * i);
                    const v4i_t A1 = *reinterpret_cast<const v4i_t *>(abase[h] + 128 * i + 16);
                    P[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B0, c8_of(i, h), 0, 0, 0);
                    P[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B1, P[h], 0, 0, 0);
                    X[h] = xd_of(i, h);
                }
                // blocks past the split: P is 0 there, and so is d (whatever the loaded bits)
                const bool bv = wb0 + 4 * i + g < nsb;
                const float d = bv ? dl[i] : 0.0f;
#pragma unroll
                for (int h = 0; h < H; h++) {
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        acc[h][e] = fmaf(X[h][e] * d, static_cast<float>(P[h][e]), acc[h][e]);
                    if (DBG) {
                        const int64_t row = int64_t{tile} * 16 + r;
                        const int blk = b_lo + wb0 + 4 * i + g;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int v = 4 * h + e;
                            if (v < nvec && row < rows && bv)
                                a.P[(int64_t{v} * rows + row) * nb + blk] = X16 ? P[h][e] >> 4 : P[h][e];
                        }
                    }
                }
            }
        }
        // ---- sums over the lane groups: the vectors' values u[j] = acc[j / 4][j % 4]. Lanes
        //      l and l + 32 first: one swap of the upper half of u[2 m] with the lower half of
        //      u[2 m + 1], one add, leaves u[2 m] in lanes 0-31 and u[2 m + 1] in lanes 32-63;
        //      then rows of 16 lanes 0-1 and 2-3 the same way ----
        // (The elements are copied to scalars first: __builtin_bit_cast of a vector element
        // read the vector's first element with this compiler.)
        float w1[2 * H];
#pragma unroll
        for (int m = 0; m < 2 * H; m++) {
            const float lo = acc[m >> 1][2 * (m & 1)], hi = acc[m >> 1][2 * (m & 1) + 1];
            const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, lo),
                                                             __builtin_bit_cast(uint32_t, hi),
                                                             false, false);
            const uint32_t s0 = sw[0], s1 = sw[1];
            w1[m] = __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
        }
#pragma unroll
        for (int n = 0; n < H; n++) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, w1[2 * n]),
                                                             __builtin_bit_cast(uint32_t, w1[2 * n + 1]),
                                                             false, false);
            const uint32_t s0 = sw[0], s1 = sw[1];
            z[n] = __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
        }
    };
    // The sums over the workgroup's waves (in wave order) and the stores of row tile `tile`.
    const int j0 = 2 * (g & 1) + (g >> 1);
    auto finish = [&](int tile, const float (&z)[H]) {
        if (!DBG) {
#pragma unroll
            for (int n = 0; n < H; n++)
                red_s[((slot * waves + wave) * 16 + r) * NV + 4 * n + j0] = z[n];
            __syncthreads();
            // 16 NV outputs, output e by thread e % threads (a fixed number of stores per lane)
#pragma unroll
            for (int k = 0; k < (16 * NV + 63) / 64; k++) {
                const int e = tid + threads * k;
                const int v = e >> 4, rr = e & 15;
                const int64_t row = int64_t{tile} * 16 + rr;
                if (e < 16 * NV && v < nvec && row < rows) {
                    float y = red_s[((slot * waves) * 16 + rr) * NV + v];
#pragma unroll
                    for (int w = 1; w < kQ32I8MaxWaves; w++)
                        if (w < waves) y += red_s[((slot * waves + w) * 16 + rr) * NV + v];
                    out[static_cast<int64_t>(v) * rows + row] = X16 ? y * 0.0625f : y;
                }
            }
            slot ^= 1;
        }
    };
    // One or two tiles: both are in flight already. More: the third goes into the first set as
    // soon as the first tile's arithmetic has read it, and from then on each tile's successor
    // goes out into the same registers right after the tile's arithmetic, ahead of the sums over
    // the waves and the stores (past the last tile it reloads the last one, unused). The
    // branches are uniform over the workgroup. (Two sets alternating in the loop kept two tiles
    // in flight per wave but ran slower with 1-4 vectors: 262144 x 1536 Q8_0 x 1 in 87 against
    // 77 us.)
    float z[H];
    if constexpr (SINGLE) {
        while (true) {
            __builtin_amdgcn_sched_barrier(0);
            products(rt, tA, z);
            __builtin_amdgcn_sched_barrier(0);
            issue(min(rt + stride, row_tiles - 1), tA);
            __builtin_amdgcn_sched_barrier(0);
            finish(rt, z);
            rt += stride;
            if (rt >= row_tiles) break;
        }
        return;
    }
    const int ntiles = (row_tiles - rt + stride - 1) / stride;     // this workgroup's tiles
    if (ntiles <= 2) {
        __builtin_amdgcn_sched_barrier(0);
        products(rt, tA, z);
        __builtin_amdgcn_sched_barrier(0);
        finish(rt, z);
        if (ntiles == 2) {
            __builtin_amdgcn_sched_barrier(0);
            products(rt + stride, tB, z);
            __builtin_amdgcn_sched_barrier(0);
            finish(rt + stride, z);
        }
        return;
    }
    __builtin_amdgcn_sched_barrier(0);
    products(rt, tA, z);
    __builtin_amdgcn_sched_barrier(0);
    issue(rt + 2 * stride, tA);
    __builtin_amdgcn_sched_barrier(0);
    finish(rt, z);
    __builtin_amdgcn_sched_barrier(0);
    products(rt + stride, tB, z);
    __builtin_amdgcn_sched_barrier(0);
    finish(rt + stride, z);
    rt += 2 * stride;
    while (true) {
        __builtin_amdgcn_sched_barrier(0);
        products(rt, tA, z);
        __builtin_amdgcn_sched_barrier(0);
        issue(min(rt + stride, row_tiles - 1), tA);
        __builtin_amdgcn_sched_barrier(0);
        finish(rt, z);
        rt += stride;
        if (rt >= row_tiles) break;
    }
}

}  // namespace

namespace {

template <int FMT, int H, bool VS>
hipError_t launch_fh(const GemmArgs &a, int waves, bool debug, hipStream_t stream) {
    // Workgroups of this size resident at once (registers and LDS) times the CUs, looked up
    // once per form and size; each workgroup then takes an equal share of the row tiles, and at
    // least two (the staging is per workgroup, and the second tile's loads overlap the first
    // tile's arithmetic). Concurrent first calls store the same values.
    static std::atomic<int> per_cu[2][kQ32I8MaxWaves] = {};      // per instance (FMT, H, VS)
    static std::atomic<int> cus{0};
    if (cus.load(std::memory_order_relaxed) == 0) {
        int dev = 0, n = 0;
        const bool ok = hipGetDevice(&dev) == hipSuccess &&
                        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                            hipSuccess &&
                        n > 0;
        cus.store(ok ? n : 256, std::memory_order_relaxed);
    }
    const int threads = 64 * waves;
    const size_t lds = static_cast<size_t>(q32i8_lds_bytes(waves, 4 * H));
    std::atomic<int> &res = per_cu[debug ? 1 : 0][waves - 1];
    if (res.load(std::memory_order_relaxed) == 0) {
        int n = 0;
        const hipError_t e =
            debug ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &n, gemm_q32_i8_kernel<FMT, kModeDebug, H, VS>, threads, lds)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &n, gemm_q32_i8_kernel<FMT, kModePlain, H, VS>, threads, lds);
        res.store((e == hipSuccess && n > 0) ? n : 1, std::memory_order_relaxed);
    }
    const int64_t cap = std::max<int64_t>(
        1, int64_t{res.load(std::memory_order_relaxed)} * cus.load(std::memory_order_relaxed) /
               a.splits);
    const int64_t per_wg = std::max<int64_t>(2, (a.row_tiles + cap - 1) / cap);
    const int64_t blocks = (a.row_tiles + per_wg - 1) / per_wg;
    const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(a.splits));
    const dim3 block(static_cast<unsigned>(threads));
    if (debug)
        hipLaunchKernelGGL((gemm_q32_i8_kernel<FMT, kModeDebug, H, VS>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((gemm_q32_i8_kernel<FMT, kModePlain, H, VS>), grid, block, lds, stream, a);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_f(const GemmArgs &a, int waves, bool debug, hipStream_t stream) {
    // (Q6_K's super-block scales have loads of their own)
    const int h = (a.nvec + 3) / 4;     // halves of 4 vectors
    if constexpr (FMT == kTypeQ6K || FMT == kTypeQ4K) {
        switch (h) {
            case 1: return launch_fh<FMT, 1, false>(a, waves, debug, stream);
            case 2: return launch_fh<FMT, 2, false>(a, waves, debug, stream);
            case 3: return launch_fh<FMT, 3, false>(a, waves, debug, stream);
            default: return launch_fh<FMT, 4, false>(a, waves, debug, stream);
        }
    } else {
        const bool vs = a.nb % 4 == 0;
        switch (h) {
            case 1: return vs ? launch_fh<FMT, 1, true>(a, waves, debug, stream)
                              : launch_fh<FMT, 1, false>(a, waves, debug, stream);
            case 2: return vs ? launch_fh<FMT, 2, true>(a, waves, debug, stream)
                              : launch_fh<FMT, 2, false>(a, waves, debug, stream);
            case 3: return vs ? launch_fh<FMT, 3, true>(a, waves, debug, stream)
                              : launch_fh<FMT, 3, false>(a, waves, debug, stream);
            default: return vs ? launch_fh<FMT, 4, true>(a, waves, debug, stream)
                               : launch_fh<FMT, 4, false>(a, waves, debug, stream);
        }
    }
}

}  // namespace

hipError_t launch_gemm_q32_i8(int wtype, const GemmArgs &a, int waves, bool debug,
                              hipStream_t stream) {
    if (waves < 1 || waves > kQ32I8MaxWaves || a.sb_per_split != kBw * waves || a.nvec < 1 ||
        a.nvec > kQ32I8MaxVec || a.row_tiles < 1 || a.splits < 1 || a.nb < 1 ||
        static_cast<int64_t>(a.splits - 1) * a.sb_per_split >= a.nb ||
        static_cast<int64_t>(a.splits) * a.sb_per_split < a.nb ||
        static_cast<int64_t>(a.row_tiles) * 16 < a.rows ||
        static_cast<int64_t>(a.row_tiles - 1) * 16 >= a.rows || a.splits > 65535)
        return hipErrorInvalidValue;
    switch (wtype) {
        case kTypeQ80: return launch_f<kTypeQ80>(a, waves, debug, stream);
        case kTypeQ40: return launch_f<kTypeQ40>(a, waves, debug, stream);
        case kTypeQ6K:
            if (a.nb % 8 != 0) return hipErrorInvalidValue;
            return launch_f<kTypeQ6K>(a, waves, debug, stream);
        case kTypeQ4K:
            if (a.nb % 8 != 0) return hipErrorInvalidValue;
            return launch_f<kTypeQ4K>(a, waves, debug, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
