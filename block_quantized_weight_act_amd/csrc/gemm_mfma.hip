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
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16v_t __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

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

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4): lane l of the wave
// writes the 16 bytes at lds + 16 l; lds is the same for the whole wave (it goes in M0). The
// instruction is issued from inline assembly so that the compiler does not see an LDS write
// in flight: seeing one, it waits for every outstanding load before each LDS read, which
// would wait for the next super-block's loads too. The kernel waits for these copies
// explicitly (vmcnt) before the barrier that publishes them. Loads complete in order, so the
// compiler's own vmcnt waits, which do not count these copies, stay correct (only more
// conservative).
__device__ __forceinline__ void copy16_to_lds(const void *src, const void *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t base =
        __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(base), "v"(src)
                 : "memory", "m0");
#endif
}

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(half8_t, make_uint4(a, b, c, d));
}

// s_waitcnt immediate: no vector-memory load outstanding, the other counters not waited for
// (vmcnt bits 3:0 and 15:14, expcnt 6:4 at its maximum 7, lgkmcnt 11:8 at its maximum 15).
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);

// Bytes of one staged tile (one super-block of one vector group): the fp16 codes of 32 * NT
// vectors x 256 columns (512 bytes per vector), then (xd, -xd * S) for 8 blocks x the vectors.
template <int NT>
constexpr int tile_bytes() {
    return NT * 32 * 512 + 8 * NT * 32 * 8;
}

// Pre-pass: the activation codes of every (super-block, vector group) converted once to the
// fp16 image the main kernel copies into LDS; a workgroup per 16 vectors of a group. In a vector's 512 bytes, the 16-byte piece p
// (columns 8p .. 8p + 7 in the slot order above) sits at slot p ^ (vector % 32), so the 32
// vectors of a matrix-core operand read 32 different bank groups.
template <int NT, bool DBG>
__global__ void __launch_bounds__(256) mc_stage_kernel(GemmArgs a) {
    const int tid = threadIdx.x;
    const int sp = tid & 15;
    const int sv = tid >> 4;
    const int sb = blockIdx.x;
    const int nb = a.nb, nvec = a.nvec;
    const int64_t cols = static_cast<int64_t>(nb) * 256;
    const int nbk = nb * 8;
    const int tok0 = blockIdx.y * NT * 32;
    uint8_t *tile = a.tiles + (static_cast<int64_t>(sb) * gridDim.y + blockIdx.y) * tile_bytes<NT>();
    float2 *xdt = reinterpret_cast<float2 *>(tile + NT * 32 * 512);
    {
        const int rnd = blockIdx.z;     // 16 vectors per workgroup
        const int v = rnd * 16 + sv;
        const int tok = tok0 + v;
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        float x = 0.0f;
        if (tok < nvec) {
            q = load16(a.xq + static_cast<int64_t>(tok) * cols + sb * 256 + 16 * sp);
            x = a.xd[static_cast<int64_t>(tok) * nbk + sb * 8 + (sp >> 1)];
        }
        int s = byte_sum(q.x, byte_sum(q.y, byte_sum(q.z, byte_sum(q.w, 0))));
        s += __builtin_amdgcn_update_dpp(0, s, kDppXor1, 0xF, 0xF, false);
        const uint32_t fx = q.x ^ 0x80808080u, fy = q.y ^ 0x80808080u;
        const uint32_t fz = q.z ^ 0x80808080u, fw = q.w ^ 0x80808080u;
        uint8_t *row = tile + v * 512;
        const int sw = v & 31;
        *reinterpret_cast<uint4 *>(row + 16 * ((2 * sp) ^ sw)) =
            make_uint4(codes_to_half2<0>(fx), codes_to_half2<8>(fx), codes_to_half2<0>(fy),
                       codes_to_half2<8>(fy));
        *reinterpret_cast<uint4 *>(row + 16 * ((2 * sp + 1) ^ sw)) =
            make_uint4(codes_to_half2<0>(fz), codes_to_half2<8>(fz), codes_to_half2<0>(fw),
                       codes_to_half2<8>(fw));
        if ((sp & 1) == 0) {
            const int j = sp >> 1;
            xdt[j * NT * 32 + v] = make_float2(x, -(x * static_cast<float>(s)));
            if (DBG && tok < nvec) a.S[static_cast<int64_t>(tok) * nbk + sb * 8 + j] = s;
        }
    }
}

// One work item: a row tile (128 rows), a vector group (32 NT vectors), a column split.
struct Item {
    int wrow0;      // first row of this wave
    int tok0;       // first vector of the group
    int group;
    int split;
    int sb0, sb1;   // super-blocks of the split
};

// Persistent: the grid holds about as many workgroups as stay resident, and each takes items
// blockIdx.x, blockIdx.x + gridDim.x, ... (split fastest, then group, then row tile). The load
// pipeline runs on across items: the next item's first super-block is loaded while the current
// item's last one is computed.
template <int NT, bool DBG>
__global__ void __launch_bounds__(256) gemm_q4k_mfma_kernel(GemmArgs a) {
    constexpr int TB = tile_bytes<NT>();
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][TB];   // staged tiles, two in flight
    __shared__ __attribute__((aligned(16))) float dd[4][32];      // d * 2^24 per wave

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int rows = a.rows, nb = a.nb, nvec = a.nvec;
    const int nbk = nb * 8;                           // 32-column blocks per row
    const int groups = a.groups, splits = a.splits;
    const int items = a.row_tiles * groups * splits;
    const int64_t nblocks = static_cast<int64_t>(rows) * nb;
    const int64_t tile_stride = static_cast<int64_t>(groups) * TB;

    auto item_of = [&](int it) {
        Item m;
        m.split = it % splits;
        const int rest = it / splits;
        m.group = rest % groups;
        m.wrow0 = (rest / groups) * kMcRows + wave * 32;
        m.tok0 = m.group * NT * 32;
        m.sb0 = m.split * a.sb_per_split;
        m.sb1 = min(nb, m.sb0 + a.sb_per_split);
        return m;
    };
    // this lane's weight row (A operand), clamped so the last tile's loads stay in bounds
    auto codes_of = [&](const Item &m) {
        const int arow = min(m.wrow0 + l32, rows - 1);
        return a.w + (static_cast<int64_t>(arow) * nb) * 128 + 64 * h;
    };
    auto hdrs_of = [&](const Item &m) {
        const int arow = min(m.wrow0 + l32, rows - 1);
        return a.w + nblocks * 128 + (static_cast<int64_t>(arow) * nb) * 16;
    };

    // The next super-block's weights (registers) and staged tile (the other LDS buffer) are
    // loaded while the current one is computed; the tile copies go out first, and the barrier
    // waits for every load of the current super-block.
    uint4 c[4], hdr;
    auto issue_weights = [&](const uint8_t *codes, const uint8_t *hdrs, int sb) {
#pragma unroll
        for (int k = 0; k < 4; k++) c[k] = load16(codes + static_cast<int64_t>(sb) * 128 + 16 * k);
        hdr = load16(hdrs + static_cast<int64_t>(sb) * 16);
    };
    // a super-block's staged tile into LDS buffer `buf` (1 KB per wave instruction)
    auto issue_tile = [&](const Item &m, int sb, int buf) {
        const uint8_t *src = a.tiles + static_cast<int64_t>(m.group) * TB + sb * tile_stride;
        for (int k = wave; k < TB / 1024; k += 4)
            copy16_to_lds(src + k * 1024 + lane * 16, &lds[buf][k * 1024]);
    };

    int it = blockIdx.x;
    if (it >= items) return;
    Item cur = item_of(it);
    issue_weights(codes_of(cur), hdrs_of(cur), cur.sb0);
    issue_tile(cur, cur.sb0, 0);
    int buf = 0;

    while (true) {
        float16v_t acc[NT];
        float t1[NT][16];
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[t][i] = 0.0f;
        const int tok0 = cur.tok0, wrow0 = cur.wrow0;

        for (int sb = cur.sb0; sb < cur.sb1; sb++) {
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
            const uint4 hd = hdr;
            uint32_t sc[8];
            float cmin[4];      // dmin * m of blocks h, h + 2, h + 4, h + 6 of this lane's row
            {
                const float d = half_to_float(hd.x & 0xFFFFu);
                const float dmin = half_to_float(hd.x >> 16);
#pragma unroll
                for (int j = 0; j < 8; j++)
                    sc[j] = ((hd.y >> (8 * (j / 2) + 4 * (j % 2))) & 0xFu) |
                            (((hd.w >> (8 * (j / 4) + 2 * (j % 4))) & 3u) << 4);
#pragma unroll
                for (int pp = 0; pp < 4; pp++) {
                    // block 2 pp + h: low nibble of byte pp of the m field, high bits of byte
                    // 14 + pp / 2 at bit 4 (pp % 2) + 2 h
                    const uint32_t m = ((hd.z >> (8 * pp + 4 * h)) & 0xFu) |
                                       (((hd.w >> (16 + 8 * (pp / 2) + 4 * (pp % 2) + 2 * h)) & 3u)
                                        << 4);
                    cmin[pp] = dmin * static_cast<float>(m);
                }
                if (h == 0) dd[wave][l32] = d * 16777216.0f;
            }
            // Everything this super-block needs from its loaded registers is computed now (the
            // empty asm statements keep the compiler from recomputing it from them later), so
            // the next loads can reuse those registers without copies.
#pragma unroll
            for (int k = 0; k < 8; k++) asm volatile("" : "+v"(aw[k]), "+v"(bw[k]), "+v"(sc[k]));
#pragma unroll
            for (int pp = 0; pp < 4; pp++) asm volatile("" : "+v"(cmin[pp]));
            // this super-block's tile has landed in every wave's part, and every wave is done
            // with the buffer the next tile overwrites
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            __syncthreads();

            // ---- the next loads: the next super-block of this item, else the first of the next
            //      item of this workgroup (the weights unconditionally: without a next one they
            //      reload the current super-block, unused; a conditional load would make the
            //      register allocator copy the loaded registers, which waits for them) ----
            {
                const bool more = sb + 1 < cur.sb1;
                const bool next_item = !more && it + static_cast<int>(gridDim.x) < items;
                const Item nx = more ? cur : item_of(next_item ? it + gridDim.x : it);
                const int nsb = more ? sb + 1 : (next_item ? nx.sb0 : sb);
                if (more || next_item) issue_tile(nx, nsb, buf ^ 1);
                // the fences keep the scheduler from sinking the loads into the arithmetic
                __builtin_amdgcn_sched_barrier(0);
                issue_weights(codes_of(nx), hdrs_of(nx), nsb);
                __builtin_amdgcn_sched_barrier(0);
            }

            const uint8_t *act = lds[buf];
            const float2 *xdt = reinterpret_cast<const float2 *>(act + NT * 32 * 512);
            // ---- eight 32-column blocks. The operand reads from LDS go out two blocks ahead
            //      and the matrix products one block ahead of the float work that uses them,
            //      so neither waits on the previous step (for up to two vector tiles; with
            //      more, the registers are not there and each block is done in turn) ----
            struct BOps {
                half8_t b0[NT], b1[NT];
                float xs[NT];
            };
            auto read_b = [&](int j, BOps &o) {
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const uint8_t *brow = act + (t * 32 + l32) * 512;
                    o.b0[t] = *reinterpret_cast<const half8_t *>(brow + 16 * ((4 * j + h) ^ l32));
                    o.b1[t] = *reinterpret_cast<const half8_t *>(brow + 16 * ((4 * j + 2 + h) ^ l32));
                    o.xs[t] = xdt[j * NT * 32 + t * 32 + l32].x;
                }
            };
            auto product = [&](int j, const BOps &o, float16v_t (&Q)[NT]) {
                const uint32_t scp = sc[j] * 0x00010001u;
                const uint32_t wa = aw[j], wb = bw[j];
                const half8_t A0 = as_half8(nib_times<0>(wa, scp), nib_times<8>(wa, scp),
                                            nib_times<0>(wb, scp), nib_times<8>(wb, scp));
                const half8_t A1 = as_half8(nib_times<4>(wa, scp), nib_times<12>(wa, scp),
                                            nib_times<4>(wb, scp), nib_times<12>(wb, scp));
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const float16v_t zero = {};
                    Q[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, o.b0[t], zero, 0, 0, 0);
                    Q[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, o.b1[t], Q[t], 0, 0, 0);
                    if (DBG) {
                        const half8_t U0 = as_half8(nib<0>(wa), nib<8>(wa), nib<0>(wb), nib<8>(wb));
                        const half8_t U1 =
                            as_half8(nib<4>(wa), nib<12>(wa), nib<4>(wb), nib<12>(wb));
                        float16v_t R =
                            __builtin_amdgcn_mfma_f32_32x32x16_f16(U0, o.b0[t], zero, 0, 0, 0);
                        R = __builtin_amdgcn_mfma_f32_32x32x16_f16(U1, o.b1[t], R, 0, 0, 0);
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
            };
            auto scale = [&](int j, const BOps &o, const float16v_t (&Q)[NT]) {
#pragma unroll
                for (int t = 0; t < NT; t++)
#pragma unroll
                    for (int i = 0; i < 16; i++)
                        t1[t][i] = j == 0 ? o.xs[t] * Q[t][i] : fmaf(o.xs[t], Q[t][i], t1[t][i]);
            };
            if constexpr (NT <= 2) {
                BOps ob[3];
                float16v_t Qa[NT], Qb[NT];
                read_b(0, ob[0]);
                read_b(1, ob[1]);
                product(0, ob[0], Qa);
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    float16v_t(&cur_q)[NT] = (j & 1) ? Qb : Qa;
                    float16v_t(&nxt_q)[NT] = (j & 1) ? Qa : Qb;
                    if (j + 2 < 8) read_b(j + 2, ob[(j + 2) % 3]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (j + 1 < 8) product(j + 1, ob[(j + 1) % 3], nxt_q);
                    scale(j, ob[j % 3], cur_q);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    BOps o;
                    float16v_t Q[NT];
                    read_b(j, o);
                    product(j, o, Q);
                    scale(j, o, Q);
                }
            }
            // ---- the min terms of the eight blocks on the float32 matrix cores: two blocks
            //      per 32x32x2 product, A = dmin * m (row, block), B = -xd * S (block, vector) ----
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
                for (int i = 0; i < 16; i++) acc[t][i] = fmaf(ddv[i], t1[t][i], acc[t][i]);
            buf ^= 1;
        }

        if (!DBG) {
            float *out = a.out + static_cast<int64_t>(cur.split) * nvec * rows;
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
        it += gridDim.x;
        if (it >= items) break;
        cur = item_of(it);
    }
}

template <int NT>
hipError_t launch_nt(const GemmArgs &a, int row_tiles, int groups, int splits, bool debug,
                     hipStream_t stream) {
    const dim3 sgrid(static_cast<unsigned>(a.nb), static_cast<unsigned>(groups), 2 * NT);
    // Workgroups that stay resident at once: per CU (from the kernel's registers and LDS) times
    // the CUs. Looked up once; concurrent first calls store the same values. The grid size only
    // sets how many workgroups share the items, so any value gives the same results.
    static std::atomic<int> per_cu[2] = {{0}, {0}};
    static std::atomic<int> cus{0};
    if (cus.load(std::memory_order_relaxed) == 0) {
        int dev = 0, n = 0;
        const bool ok = hipGetDevice(&dev) == hipSuccess &&
                        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                            hipSuccess &&
                        n > 0;
        cus.store(ok ? n : 256, std::memory_order_relaxed);
    }
    std::atomic<int> &res = per_cu[debug ? 1 : 0];
    if (res.load(std::memory_order_relaxed) == 0) {
        int n = 0;
        const hipError_t e =
            debug ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_q4k_mfma_kernel<NT, true>, 256, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_q4k_mfma_kernel<NT, false>, 256, 0);
        res.store((e == hipSuccess && n > 0) ? n : 1, std::memory_order_relaxed);
    }
    const int resident = res.load(std::memory_order_relaxed);
    const int64_t items = static_cast<int64_t>(row_tiles) * groups * splits;
    const unsigned blocks = static_cast<unsigned>(
        std::min<int64_t>(items, int64_t{resident} * cus.load(std::memory_order_relaxed)));
    if (debug) {
        hipLaunchKernelGGL((mc_stage_kernel<NT, true>), sgrid, dim3(256), 0, stream, a);
        hipLaunchKernelGGL((gemm_q4k_mfma_kernel<NT, true>), dim3(blocks), dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL((mc_stage_kernel<NT, false>), sgrid, dim3(256), 0, stream, a);
        hipLaunchKernelGGL((gemm_q4k_mfma_kernel<NT, false>), dim3(blocks), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_q4k_mfma(const GemmArgs &a, int nt, int row_tiles, int groups, int splits,
                                bool debug, hipStream_t stream) {
    switch (nt) {
        case 1: return launch_nt<1>(a, row_tiles, groups, splits, debug, stream);
        case 2: return launch_nt<2>(a, row_tiles, groups, splits, debug, stream);
        case 3: return launch_nt<3>(a, row_tiles, groups, splits, debug, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
