// Per-lane building blocks of the GEMV kernels: where a lane sits in a row, one step of the
// Q4_K or Q6_K product over G row groups, and the reduction of a row's lane sums to y.
//
// genie-ai-runtime (jared-hpc.com), "The decode arc": the quantized matrix-vector product is
// done with int8 4-way dot products on whole 32-bit words of codes, a row shared by the lanes
// of a warp. Here a 64-lane wavefront holds 64 / T rows of T lanes; lane t of a row takes the
// row's 16-byte code chunks t, t + T, ... (NC of them, 32 columns each), so its columns never
// change and its activation slice stays in VGPRs.
//
// A step is G consecutive row groups of a wave (G = 4, 2, 1 for NC = 1, 2, >= 3). Its loads
// are unconditional: a row past the end of the matrix reads the last row (its result is not
// stored) and a chunk past the end of a row reads the row's first block against an all-zero
// activation slice, so it adds exactly zero.
#pragma once

#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

// Where this lane sits: row rsub of the wave's 64 / T rows, lane t of that row, and for each
// of its NC chunks the 32-column block index g, whether it exists (cv), and the super-block
// index within the row it falls in (blk; 0 for a chunk past the end).
template <int T, int NC>
struct LaneGeom {
    int lane, t, rsub, split, j;
    int g[NC];
    bool cv[NC];
    uint32_t blk[NC];

    // the lane's column chunk `split` (blockIdx.y unless given)
    __device__ __forceinline__ explicit LaneGeom(int nsub) : LaneGeom(nsub, blockIdx.y) {}
    __device__ __forceinline__ LaneGeom(int nsub, int split_) {
        lane = threadIdx.x & 63;
        t = lane & (T - 1);
        rsub = lane / T;
        split = split_;
        j = t & 7;                           // chunk inside the super-block
#pragma unroll
        for (int k = 0; k < NC; k++) {
            g[k] = split * T * NC + t + T * k;
            cv[k] = g[k] < nsub;
            blk[k] = cv[k] ? static_cast<uint32_t>(g[k] >> 3) : 0u;
        }
    }
};

// The lane sums of one row (per vector) to y: a log2(T)-step butterfly and a store by lane
// t = v; with one row per wave and 3-8 vectors, a reduce-scatter over the wave instead.
// out is [splits][V][rows]; nothing is stored for a row past the end (rv false).
template <int V, int T>
__device__ __forceinline__ void store_row(float (&acc)[V], float *out, int rows, int row, bool rv,
                                          int t, int lane, int split) {
    if constexpr (T == 64 && V >= 3) {
        const float o = wave_reduce_scatter8(acc);
        const int vi = scatter_index(lane);
        if (rv && (lane & 7) == 0 && vi < V)
            out[(static_cast<int64_t>(split) * V + vi) * rows + row] = o;
    } else {
#pragma unroll
        for (int v = 0; v < V; v++) acc[v] = group_sum<T>(acc[v]);
        if (rv && t < V) {
            float o = acc[0];
#pragma unroll
            for (int v = 1; v < V; v++)
                if (t == v) o = acc[v];
            out[(static_cast<int64_t>(split) * V + t) * rows + row] = o;
        }
    }
}

// The loaded data of one step: up to 9 dwords per (row group, chunk) in every format, so a
// kernel that mixes formats keeps one set of registers. Every format's issue writes all three
// fields (zeros where it has nothing), so that the branches of a mixed kernel define the same
// values and the register set is never demoted to scratch memory.
template <int G, int NC>
struct StepRegs {
    uint4 a[G][NC], b[G][NC];
    uint32_t c[G][NC];
};

// The activation terms the formats need besides the codes, all exact integers computed from
// the slice: the code sum of each 32-column block and of its two 16-column halves.
template <int V, int NC>
struct ActTerms {
    int sum[V][NC];
    int lo[V][NC], hi[V][NC];
    float sumf[V][NC];      // sum as float (exact: |sum| <= 4064)
};

template <int V, int NC>
__device__ __forceinline__ void act_terms(const uint32_t (&xw)[V][NC][8], ActTerms<V, NC> &a) {
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
            a.lo[v][k] = s0;
            a.hi[v][k] = s1;
            a.sum[v][k] = s0 + s1;
            a.sumf[v][k] = static_cast<float>(s0 + s1);
        }
    }
}

// ---------------------------------------------------------------------------------- Q4_K --
// Planar tensor: codes plane (128 bytes per super-block), then the header plane (16 bytes:
// fp16 d, fp16 dmin, packed 6-bit sub-scales and mins). One chunk = one 32-column sub-block j:
// its low nibbles meet activation bytes 0..15 and its high nibbles bytes 16..31.
//
// The float32 work per sub-block is xd * (d * (sc * P) - dmin * (m * S)). d * sc and dmin * m
// are exact in float32 (11-bit significand times a 6-bit integer) and shared by every vector;
// sc * P and m * S are exact integers below 2^24. The two products can nearly cancel, so the
// difference is formed with the exact rounding error of the min product (a TwoProduct through
// fmaf) and carries a relative error of about two float32 roundings of the sub-block's own
// value; a sub-block whose dequantized weights times activations are all zero adds exactly 0.
template <int V, int T, int NC>
struct Q4kTile {
    static constexpr int G = groups_per_step(NC);
    static constexpr int RPW = 64 / T;
    using Regs = StepRegs<G, NC>;           // a: the 16-byte header, b: 16 code bytes

    // The loads of step st of a matrix with `rows` rows (>= 1) and nb super-blocks per row:
    // 8 consecutive lanes read one block's 128 code bytes as one contiguous run (nontemporal:
    // no other load touches it); the 16-byte header is an ordinary load, the same address for
    // those 8 lanes, and stays cached for the neighbouring blocks that share its line.
    static __device__ __forceinline__ void issue(Regs &r, const uint8_t *w, int rows, int nb,
                                                 int st, const LaneGeom<T, NC> &L) {
        const uint8_t *hplane = w + static_cast<int64_t>(rows) * nb * 128;
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const int64_t brow = static_cast<int64_t>(row < rows ? row : rows - 1) * nb;
            const uint8_t *qrow = w + brow * 128;
            const uint8_t *hrow = hplane + brow * 16;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                r.a[gg][k] = load16(hrow + L.blk[k] * 16);
                r.b[gg][k] = load16_stream(qrow + L.blk[k] * 128 + 16 * L.j);
                r.c[gg][k] = 0u;
            }
        }
    }

    // The arithmetic of the step, its row reductions and stores (out [splits][V][rows]). The
    // debug form (DBG) writes the exact partials to P [V][rows][nsub] instead of y.
    template <bool DBG>
    static __device__ __forceinline__ void compute(const Regs &r, const uint32_t (&xw)[V][NC][8],
                                                   const float (&xs)[V][NC],
                                                   const ActTerms<V, NC> &at, float *out,
                                                   int rows, int st, const LaneGeom<T, NC> &L,
                                                   int32_t *P, int nsub) {
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const bool rv = row < rows;
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; v++) acc[v] = 0.0f;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const uint4 h = r.a[gg][k];
                const int j = L.j;
                const float d = half_to_float(h.x & 0xFFFFu);
                const float dmin = half_to_float(h.x >> 16);
                const int sc = static_cast<int>(((h.y >> (4 * j)) & 15u) | (((h.w >> (2 * j)) & 3u) << 4));
                const int m = static_cast<int>(((h.z >> (4 * j)) & 15u) |
                                               (((h.w >> (16 + 2 * j)) & 3u) << 4));
                const float dsc = d * static_cast<float>(sc);
                const float dm = dmin * static_cast<float>(m);
                const uint32_t q[4] = {r.b[gg][k].x, r.b[gg][k].y, r.b[gg][k].z, r.b[gg][k].w};
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    lo[i] = q[i] & 0x0F0F0F0Fu;
                    hi[i] = (q[i] >> 4) & 0x0F0F0F0Fu;
                }
#pragma unroll
                for (int v = 0; v < V; v++) {
                    int p = 0;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        p = dot4(lo[i], xw[v][k][i], p);
                        p = dot4(hi[i], xw[v][k][4 + i], p);
                    }
                    // pb is the rounded min product and eb its exact rounding error, so
                    // fmaf(d sc, P, -pb) - eb is the difference up to two roundings of
                    // quantities no larger than the result (plus eps^2 |pb|).
                    const float pb = dm * at.sumf[v][k];
                    const float eb = fmaf(dm, at.sumf[v][k], -pb);
                    const float diff = fmaf(dsc, static_cast<float>(p), -pb) - eb;
                    acc[v] = fmaf(xs[v][k], diff, acc[v]);
                    if (DBG && rv && L.cv[k])
                        P[(static_cast<int64_t>(v) * rows + row) * nsub + L.g[k]] = p;
                }
            }
            if (!DBG) store_row<V, T>(acc, out, rows, row, rv, L.t, L.lane, L.split);
        }
    }
};

// ---------------------------------------------------------------------------------- Q6_K --
// Planar tensor: low-bit plane (128 bytes per super-block), high-bit plane (64), sub-scale
// plane (16 int8), super-scale plane (fp16). A 16-byte low-bit chunk holds the low 4 bits of
// one 32-column activation block (sub-blocks 2k and 2k + 1 in its low and high nibbles); the 8
// matching high-bit bytes hold their high 2 bits, so one shift and mask of a 32-bit word lines
// them up under the 4 codes of the matching low-bit word. Codes q in [0, 63] are rebuilt with
// AND / shift / OR, dotted with the activation codes, and the offset of 32 is removed after:
// sum (q - 32) x = sum q x - 32 sum x, with the sums of each 16-column half in VGPRs. All of it
// is exact: |sc * P| < 2^23 per sub-block and the chunk's two sub-blocks stay below 2^24.
template <int V, int T, int NC>
struct Q6kTile {
    static constexpr int G = groups_per_step(NC);
    static constexpr int RPW = 64 / T;
    // a: 16 low-bit bytes; b: 8 high-bit bytes and the sub-scale word; c: the fp16 super-scale
    using Regs = StepRegs<G, NC>;

    // Low and high bits are contiguous runs that no other load touches (nontemporal); the
    // sub-scale word and the fp16 super-scale are ordinary loads that stay cached.
    static __device__ __forceinline__ void issue(Regs &r, const uint8_t *w, int rows, int nb,
                                                 int st, const LaneGeom<T, NC> &L) {
        const int64_t nblocks = static_cast<int64_t>(rows) * nb;
        const uint8_t *hplane = w + nblocks * 128;
        const uint8_t *splane = w + nblocks * 192;
        const uint16_t *dplane = reinterpret_cast<const uint16_t *>(w + nblocks * 208);
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const int64_t brow = static_cast<int64_t>(row < rows ? row : rows - 1) * nb;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const int64_t b = brow + L.blk[k];
                r.a[gg][k] = load16_stream(w + b * 128 + 16 * L.j);
                const uint2 h = load8_stream(hplane + b * 64 + 8 * L.j);
                const uint32_t sc = *reinterpret_cast<const uint32_t *>(splane + b * 16 +
                                                                        4 * (L.j >> 1));
                r.b[gg][k] = make_uint4(h.x, h.y, sc, 0u);
                r.c[gg][k] = dplane[b];
            }
        }
    }

    // As Q4kTile::compute; the debug partials are P [V][rows][2 nsub] (per 16 columns).
    template <bool DBG>
    static __device__ __forceinline__ void compute(const Regs &r, const uint32_t (&xw)[V][NC][8],
                                                   const float (&xs)[V][NC],
                                                   const ActTerms<V, NC> &at, float *out, int rows,
                                                   int st, const LaneGeom<T, NC> &L, int32_t *P,
                                                   int nsub) {
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const bool rv = row < rows;
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; v++) acc[v] = 0.0f;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const uint4 hb = r.b[gg][k];
                const float d = half_to_float(r.c[gg][k]);
                const int sh = 16 * (L.j & 1);
                const int sc_lo = static_cast<int>(static_cast<int8_t>(hb.z >> sh));
                const int sc_hi = static_cast<int>(static_cast<int8_t>(hb.z >> (sh + 8)));
                const uint4 l4 = r.a[gg][k];
                const uint2 h2 = make_uint2(hb.x, hb.y);
                const uint32_t w4[4] = {l4.x, l4.y, l4.z, l4.w};
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    lo[s] = (w4[s] & 0x0F0F0F0Fu) | (((h2.x >> (2 * s)) & 0x03030303u) << 4);
                    hi[s] = ((w4[s] >> 4) & 0x0F0F0F0Fu) | (((h2.y >> (2 * s)) & 0x03030303u) << 4);
                }
#pragma unroll
                for (int v = 0; v < V; v++) {
                    // the codes' offset as the dot products' starting values: -32 S of each
                    // sub-block is the same for every row this lane reads
                    int plo = -32 * at.lo[v][k], phi = -32 * at.hi[v][k];
#pragma unroll
                    for (int s = 0; s < 4; s++) {
                        plo = dot4(lo[s], xw[v][k][s], plo);
                        phi = dot4(hi[s], xw[v][k][4 + s], phi);
                    }
                    const int scp = sc_lo * plo + sc_hi * phi;
                    acc[v] = fmaf(xs[v][k] * d, static_cast<float>(scp), acc[v]);
                    if (DBG && rv && L.cv[k]) {
                        int32_t *pp = P + (static_cast<int64_t>(v) * rows + row) * (2 * nsub);
                        pp[2 * L.g[k]] = plo;
                        pp[2 * L.g[k] + 1] = phi;
                    }
                }
            }
            if (!DBG) store_row<V, T>(acc, out, rows, row, rv, L.t, L.lane, L.split);
        }
    }
};

// ----------------------------------------------------------------- Q4_0, Q8_0 --
// oxinfer README, "Build and run": GGUF-style Q4_0 (32 weights, 4-bit codes, one fp16 scale)
// and int8 weights in blocks of 32 with an f32 scale; "Pre-quantized checkpoints": codes and
// scales are separate tensors. Here: codes planes (Q4_0: one of 16 bytes per block; Q8_0: two,
// the first and the last 16 codes of each block) then a scale plane (fp16 or float32 per block);
// one 32-weight block is exactly one lane's chunk, so the lane loads its codes (one 16-byte load
// per plane, streamed) and its own scale. Q4_0 weight t is nibble
// (t >= 16) of code byte t mod 16, the same arrangement as a Q4_K chunk: the low nibbles meet
// activation bytes 0..15 and the high nibbles bytes 16..31. Per block the product is
// xd * d * P with P = sum (q - 8) x = sum q x - 8 S (Q4_0) or sum q x (Q8_0), exact integers
// below 2^24.
template <int V, int T, int NC>
struct Q40Tile {
    static constexpr int G = groups_per_step(NC);
    static constexpr int RPW = 64 / T;
    using Regs = StepRegs<G, NC>;           // a: 16 code bytes, c: fp16 d

    // nb = 32-weight blocks per row
    static __device__ __forceinline__ void issue(Regs &r, const uint8_t *w, int rows, int nb,
                                                 int st, const LaneGeom<T, NC> &L) {
        const uint16_t *dplane = reinterpret_cast<const uint16_t *>(
            w + static_cast<int64_t>(rows) * nb * 16);
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const int64_t brow = static_cast<int64_t>(row < rows ? row : rows - 1) * nb;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const int64_t b = brow + (L.cv[k] ? L.g[k] : 0);
                r.a[gg][k] = load16_stream(w + b * 16);
                r.b[gg][k] = make_uint4(0u, 0u, 0u, 0u);
                r.c[gg][k] = dplane[b];
            }
        }
    }

    template <bool DBG>
    static __device__ __forceinline__ void compute(const Regs &r, const uint32_t (&xw)[V][NC][8],
                                                   const float (&xs)[V][NC],
                                                   const ActTerms<V, NC> &at, float *out,
                                                   int rows, int st, const LaneGeom<T, NC> &L,
                                                   int32_t *P, int nsub) {
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const bool rv = row < rows;
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; v++) acc[v] = 0.0f;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const float d = half_to_float(r.c[gg][k]);
                const uint32_t q[4] = {r.a[gg][k].x, r.a[gg][k].y, r.a[gg][k].z, r.a[gg][k].w};
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    lo[i] = q[i] & 0x0F0F0F0Fu;
                    hi[i] = (q[i] >> 4) & 0x0F0F0F0Fu;
                }
#pragma unroll
                for (int v = 0; v < V; v++) {
                    // the offset of the codes as the dot products' starting value: -8 S is the
                    // same for every row this lane reads, so it costs nothing per row
                    int p = -8 * at.sum[v][k];
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        p = dot4(lo[i], xw[v][k][i], p);
                        p = dot4(hi[i], xw[v][k][4 + i], p);
                    }
                    acc[v] = fmaf(xs[v][k] * d, static_cast<float>(p), acc[v]);
                    if (DBG && rv && L.cv[k])
                        P[(static_cast<int64_t>(v) * rows + row) * nsub + L.g[k]] = p;
                }
            }
            if (!DBG) store_row<V, T>(acc, out, rows, row, rv, L.t, L.lane, L.split);
        }
    }
};

template <int V, int T, int NC>
struct Q80Tile {
    static constexpr int G = groups_per_step(NC);
    static constexpr int RPW = 64 / T;
    using Regs = StepRegs<G, NC>;           // a, b: the 32 int8 codes, c: float32 d

    // nb = 32-weight blocks per row. The two halves of a block's codes are in two planes, so
    // consecutive lanes read consecutive 16-byte words in both loads (one 32-byte block per
    // lane in one plane would leave every load half of each 32-byte span: 64.6 us against
    // 73.9 us for 262144 x 1536 on MI355X).
    static __device__ __forceinline__ void issue(Regs &r, const uint8_t *w, int rows, int nb,
                                                 int st, const LaneGeom<T, NC> &L) {
        const int64_t nblocks = static_cast<int64_t>(rows) * nb;
        const uint8_t *hi = w + nblocks * 16;
        const uint32_t *dplane = reinterpret_cast<const uint32_t *>(w + nblocks * 32);
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const int64_t brow = static_cast<int64_t>(row < rows ? row : rows - 1) * nb;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const int64_t b = brow + (L.cv[k] ? L.g[k] : 0);
                r.a[gg][k] = load16_stream(w + b * 16);
                r.b[gg][k] = load16_stream(hi + b * 16);
                r.c[gg][k] = dplane[b];
            }
        }
    }

    template <bool DBG>
    static __device__ __forceinline__ void compute(const Regs &r, const uint32_t (&xw)[V][NC][8],
                                                   const float (&xs)[V][NC],
                                                   const ActTerms<V, NC> &at, float *out,
                                                   int rows, int st, const LaneGeom<T, NC> &L,
                                                   int32_t *P, int nsub) {
        (void)at;
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            const int row = (st * G + gg) * RPW + L.rsub;
            const bool rv = row < rows;
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; v++) acc[v] = 0.0f;
#pragma unroll
            for (int k = 0; k < NC; k++) {
                const float d = __builtin_bit_cast(float, r.c[gg][k]);
                const uint32_t q[8] = {r.a[gg][k].x, r.a[gg][k].y, r.a[gg][k].z, r.a[gg][k].w,
                                       r.b[gg][k].x, r.b[gg][k].y, r.b[gg][k].z, r.b[gg][k].w};
#pragma unroll
                for (int v = 0; v < V; v++) {
                    int p = 0;
#pragma unroll
                    for (int i = 0; i < 8; i++) p = dot4(q[i], xw[v][k][i], p);
                    acc[v] = fmaf(xs[v][k] * d, static_cast<float>(p), acc[v]);
                    if (DBG && rv && L.cv[k])
                        P[(static_cast<int64_t>(v) * rows + row) * nsub + L.g[k]] = p;
                }
            }
            if (!DBG) store_row<V, T>(acc, out, rows, row, rv, L.t, L.lane, L.split);
        }
    }
};

}  // namespace qgemv
