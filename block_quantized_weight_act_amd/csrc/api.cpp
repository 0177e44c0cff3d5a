// C ABI of libqgemv: argument checks, the per-shape launch plan, and launches on the
// caller's stream. Declared in include/qgemv.h, which states each operation, its layouts,
// ownership and error behaviour.
#include <qgemv.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gemm_mc.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {
thread_local char g_last_error[256] = "";
}

int hip_fail(hipError_t e) {
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return QGEMV_EHIP;
}

int fail_with(int status, const char *text) {
    std::snprintf(g_last_error, sizeof g_last_error, "%s", text);
    return status;
}

}  // namespace qgemv

namespace {

using namespace qgemv;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

bool type_ok(int wtype) {
    return wtype == QGEMV_Q4K || wtype == QGEMV_Q6K || wtype == QGEMV_Q4_0 || wtype == QGEMV_Q8_0;
}

// Weights per block of a format: 256 for the super-block formats, 32 for Q4_0 and Q8_0.
int64_t block_cols(int wtype) { return wtype == QGEMV_Q4_0 || wtype == QGEMV_Q8_0 ? 32 : kQK; }

size_t weight_bytes(int wtype, int64_t rows, int64_t cols) {
    const int64_t nblocks = rows * (cols / block_cols(wtype));
    switch (wtype) {
        case QGEMV_Q4K: return static_cast<size_t>(nblocks) * kQ4KBytes;
        case QGEMV_Q6K: return static_cast<size_t>(nblocks) * (kQ6KBody + 2);
        case QGEMV_Q4_0: return static_cast<size_t>(nblocks) * 18;
        case QGEMV_Q8_0: return static_cast<size_t>(nblocks) * 36;
        default: return 0;
    }
}

// Shape limits common to every format: cols a positive multiple of 32 (the activation block).
bool shape_ok(int64_t rows, int64_t cols, int32_t nvec) {
    if (rows < 1 || cols < 32 || cols % 32 != 0 || nvec < 1 || nvec > kMaxVec) return false;
    if (rows > (int64_t{1} << 30) || cols > (int64_t{1} << 30)) return false;
    return rows * (cols / 32) < (int64_t{1} << 31);
}

// ... and of one format: a valid type and whole weight blocks per row.
bool shape_ok_t(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    return type_ok(wtype) && shape_ok(rows, cols, nvec) && cols % block_cols(wtype) == 0;
}

hipError_t launch_gemv_split(int wtype, const GemvArgs &a, const LaunchShape &s, int nvec,
                             hipStream_t stream) {
    switch (wtype) {
        case QGEMV_Q4K: return launch_gemv_split_q4k(a, s, nvec, stream);
        case QGEMV_Q6K: return launch_gemv_split_q6k(a, s, nvec, stream);
        case QGEMV_Q4_0: return launch_gemv_split_q40(a, s, nvec, stream);
        case QGEMV_Q8_0: return launch_gemv_split_q80(a, s, nvec, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(int wtype, const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                       hipStream_t stream) {
    switch (wtype) {
        case QGEMV_Q4K: return launch_gemv_q4k(a, s, nvec, debug, stream);
        case QGEMV_Q6K: return launch_gemv_q6k(a, s, nvec, debug, stream);
        case QGEMV_Q4_0: return launch_gemv_q40(a, s, nvec, debug, stream);
        case QGEMV_Q8_0: return launch_gemv_q80(a, s, nvec, debug, stream);
        default: return hipErrorInvalidValue;
    }
}

bool variant_exists(int lanes, int chunks, int nvec) {
    const bool lanes_ok = lanes == 8 || lanes == 16 || lanes == 32 || lanes == 64;
    return lanes_ok && chunks >= 1 && chunks <= 4 && nvec >= 1 && nvec <= kMaxVec &&
           nvec * chunks <= 8;
}

int splits_for(int lanes, int chunks, int64_t cols) {
    const int64_t nchunks = cols / 32;
    const int64_t per = static_cast<int64_t>(lanes) * chunks;
    return static_cast<int>((nchunks + per - 1) / per);
}

// Wavefronts a launch aims for. With one or two vectors a wave needs under 100 VGPRs, the GPU
// holds about 256 CUs x 20 waves, and a grid of 16384 waves (about three rounds) gave the best
// streaming rate on the 262144 x 1536 vocabulary projection. With more vectors the activation
// slice raises register use to ~120 VGPRs (16 waves per CU) and one round of 4096 waves is best.
int64_t target_waves(int32_t nvec) { return nvec <= 2 ? 256 * 64 : 256 * 16; }

// The per-shape plan. Lanes per row T and chunks per lane NC are chosen so that one pass of a
// wave covers a row's chunks with the least idle lanes, preferring more chunks per lane
// (more 16-byte loads in flight per lane) while the activation slice fits in VGPRs
// (nvec * NC <= 8). When a row has more than 256 chunks (cols > 8192) or rows alone are too
// few to give every CU work, the columns are split.
// Lanes per row and chunks per lane for a row of `cols` columns (see make_plan). With
// one_pass set, only geometries that cover the whole row in one pass; with fit_waves, only
// those whose passes (column chunks) a workgroup can split among its waves; false if there is
// none. With several_rule (the planners of one and of several matrices), two corrections
// measured with several vectors apply (explicit plans against the planner's, graph replay, cold, MI355X; the best
// of the T x NC plans within 3% on average, against 8% before):
//  * 2 vectors take at most 3 chunks per lane: 4 chunks (64 activation registers) ran
//    24-50% slower than 1-2 (16384 / 65536 x 2048 x 2: 7.2 / 22.7 us with T 16, NC 4, against
//    5.8 / 15.8 with T 32, NC 2; 16384 x 4096 x 2: 12.3 against 9.3 with T 64, NC 2);
//  * 5 or more vectors (one chunk per lane) weigh a split pass like 15% idle lanes, so a row
//    of 48 chunks takes one pass of 64 lanes with a quarter idle rather than three of 16
//    (262144 x 1536 x 8: 92.9 against 125.4 us; x 6: 78.2 against 84.4; 65536 x 1536 x 8:
//    26.9 against 36.2).
// In one multi-matrix launch the first gains alike (two 8192 x 2048 Q4_K matrices x 2: 6.02
// against 6.97 us; three 16384 x 2048: 13.2 against 15.9).
bool choose_geometry(int64_t cols, int32_t nvec, bool one_pass, int &best_t, int &best_nc,
                     bool fit_waves = false, bool several_rule = false) {
    const int64_t nchunks = cols / 32;
    bool found = false;
    double best_cost = 1e30;
    const double split_cost = several_rule && nvec >= 5 ? 0.15 : 0.02;
    for (int nc = 1; nc <= 4; nc++) {
        if (nvec * nc > 8) break;
        if (several_rule && nvec == 2 && nc > 3) break;
        for (int t : {8, 16, 32, 64}) {
            const int64_t per = static_cast<int64_t>(t) * nc;
            const int64_t passes = (nchunks + per - 1) / per;
            if (one_pass && passes > 1) continue;
            if (fit_waves && passes > gemv_max_waves(nvec, t, nc)) continue;
            const double waste = 1.0 - static_cast<double>(nchunks) / (passes * per);
            // idle lanes cost bandwidth in flight; split passes cost a workspace round trip
            const double cost = waste + split_cost * (passes - 1) - 0.01 * nc;
            if (cost < best_cost - 1e-12) {
                best_cost = cost;
                best_t = t;
                best_nc = nc;
                found = true;
            }
        }
    }
    return found;
}

qgemv_plan make_plan(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    int best_t = 64, best_nc = 1;
    choose_geometry(cols, nvec, false, best_t, best_nc, false, true);
    qgemv_plan p{};
    p.lanes_per_row = best_t;
    p.chunks_per_lane = best_nc;
    p.waves_per_block = 4;
    int splits = splits_for(best_t, best_nc, cols);
    // Too few rows to fill the GPU: split further (whole chunks per lane kept). Not for small
    // matrices, which are latency-bound: there the second (reduce) launch costs more than the
    // extra waves win (512 x 512: 3.7 us split against 2.0 us whole).
    const int64_t rows_per_wave = 64 / best_t;
    int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave * splits;
    const bool small = weight_bytes(wtype, rows, cols) < (size_t{16} << 20);
    while (!small && waves < target_waves(nvec) / 8 && best_nc > 1) {
        best_nc--;
        splits = splits_for(best_t, best_nc, cols);
        waves = (rows + rows_per_wave - 1) / rows_per_wave * splits;
    }
    p.chunks_per_lane = best_nc;
    p.splits = splits;
    const int64_t groups = (rows + rows_per_wave - 1) / rows_per_wave;
    const int64_t steps = (groups + groups_per_step(best_nc) - 1) / groups_per_step(best_nc);
    const int64_t waves_per_split = std::max<int64_t>(1, target_waves(nvec) / splits);
    const int64_t want = std::min(steps, waves_per_split);
    // A wide activation slice: every workgroup of the fused form quantizes the whole slice its
    // lanes read, so 8 waves per workgroup halve that work per lane and the slice's L2 reads
    // per wave (1536 x 6144, one vector: 3.9 us in one launch against 5.6 us with 4 waves).
    // Not when it would leave fewer than 128 workgroups (1536 x 2048: 3.4 us against 2.9 us);
    // the unfused form runs at the same speed either way.
    if (gemv_max_waves(nvec, best_t, best_nc) == 8 && want >= 8 * 128) p.waves_per_block = 8;
    p.blocks = static_cast<int32_t>(std::max<int64_t>(1, (want + p.waves_per_block - 1) /
                                                             p.waves_per_block));
    return p;
}

bool plan_ok(const qgemv_plan &p, int32_t nvec) {
    return variant_exists(p.lanes_per_row, p.chunks_per_lane, nvec) && p.waves_per_block >= 1 &&
           p.waves_per_block <= gemv_max_waves(nvec, p.lanes_per_row, p.chunks_per_lane) &&
           p.blocks >= 1 && p.blocks <= 65535 * 64;
}

size_t plan_ws_bytes(const qgemv_plan &p, int64_t rows, int64_t cols, int32_t nvec) {
    const int splits = splits_for(p.lanes_per_row, p.chunks_per_lane, cols);
    if (splits <= 1) return 0;
    return static_cast<size_t>(splits) * nvec * rows * sizeof(float);
}

int check_gemv_args(int wtype, const void *w, const int8_t *xq, const float *xd, const void *out,
                    size_t out_bytes, int64_t rows, int64_t cols, int32_t nvec) {
    if (!w || !xq || !xd || !out) return QGEMV_EINVAL;
    if (!shape_ok_t(wtype, rows, cols, nvec)) return QGEMV_EINVAL;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(out, 4))
        return QGEMV_EALIGN;
    const size_t wb = weight_bytes(wtype, rows, cols);
    const size_t xqb = static_cast<size_t>(nvec) * cols;
    const size_t xdb = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
    if (overlaps(out, out_bytes, w, wb) || overlaps(out, out_bytes, xq, xqb) ||
        overlaps(out, out_bytes, xd, xdb))
        return QGEMV_EINVAL;
    return QGEMV_OK;
}

// The activation of one GEMV launch: either quantized codes and scales (xq, xd), or the float32
// activation x that the kernel quantizes itself, optionally storing the codes and scales.
struct Activation {
    const int8_t *xq = nullptr;
    const float *xd = nullptr;
    const float *x = nullptr;
    int8_t *xq_out = nullptr;
    float *xd_out = nullptr;
};

int check_fused_act(const Activation &act, const void *w, size_t wbytes, const void *y,
                    size_t ybytes, int64_t cols, int32_t nvec) {
    if (!act.x) return QGEMV_EINVAL;
    if ((act.xq_out == nullptr) != (act.xd_out == nullptr)) return QGEMV_EINVAL;
    if (!aligned(act.x, 16)) return QGEMV_EALIGN;
    const size_t xb = static_cast<size_t>(nvec) * cols * sizeof(float);
    if (overlaps(y, ybytes, act.x, xb)) return QGEMV_EINVAL;
    if (act.xq_out) {
        if (!aligned(act.xq_out, 4) || !aligned(act.xd_out, 4)) return QGEMV_EALIGN;
        const size_t qb = static_cast<size_t>(nvec) * cols;
        const size_t db = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
        if (overlaps(act.xq_out, qb, act.x, xb) || overlaps(act.xq_out, qb, w, wbytes) ||
            overlaps(act.xq_out, qb, y, ybytes) || overlaps(act.xd_out, db, act.x, xb) ||
            overlaps(act.xd_out, db, w, wbytes) || overlaps(act.xd_out, db, y, ybytes) ||
            overlaps(act.xd_out, db, act.xq_out, qb))
            return QGEMV_EINVAL;
    }
    return QGEMV_OK;
}

// Waves per workgroup of the column split inside the workgroup: the plan's, when its sets of
// `splits` waves divide it, else as many whole sets as the kernel's wave limit allows.
int split_waves_per_block(const qgemv_plan &plan, int maxw) {
    return plan.splits <= maxw && plan.waves_per_block % plan.splits == 0
               ? plan.waves_per_block
               : plan.splits * std::max(1, maxw / plan.splits);
}

int run_gemv(int wtype, const void *w, const Activation &act, float *y, int64_t rows,
             int64_t cols, int32_t nvec, const qgemv_plan &plan_in, void *ws, size_t ws_bytes,
             hipStream_t stream) {
    const size_t ybytes = static_cast<size_t>(nvec) * rows * sizeof(float);
    int st;
    if (act.x) {
        // check the weights and y as for the unfused form (the codes' places are unused)
        if (!w || !y || !shape_ok_t(wtype, rows, cols, nvec)) return QGEMV_EINVAL;
        if (!aligned(w, 16) || !aligned(y, 4)) return QGEMV_EALIGN;
        if (overlaps(y, ybytes, w, weight_bytes(wtype, rows, cols))) return QGEMV_EINVAL;
        st = check_fused_act(act, w, weight_bytes(wtype, rows, cols), y, ybytes, cols, nvec);
    } else {
        st = check_gemv_args(wtype, w, act.xq, act.xd, y, ybytes, rows, cols, nvec);
    }
    if (st != QGEMV_OK) return st;
    if (!plan_ok(plan_in, nvec)) return QGEMV_EINVAL;
    qgemv_plan plan = plan_in;
    plan.splits = splits_for(plan.lanes_per_row, plan.chunks_per_lane, cols);
    const size_t need = plan_ws_bytes(plan, rows, cols, nvec);
    if (need > 0) {
        if (!ws || ws_bytes < need) return QGEMV_EWORKSPACE;
        if (!aligned(ws, 4)) return QGEMV_EALIGN;
        const size_t wb = weight_bytes(wtype, rows, cols);
        const size_t qb = static_cast<size_t>(nvec) * cols;
        const size_t db = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
        if (overlaps(ws, need, w, wb) || overlaps(ws, need, y, ybytes) ||
            (act.xq && overlaps(ws, need, act.xq, qb)) || (act.xd && overlaps(ws, need, act.xd, db)) ||
            (act.x && overlaps(ws, need, act.x, qb * sizeof(float))) ||
            (act.xq_out && (overlaps(ws, need, act.xq_out, qb) || overlaps(ws, need, act.xd_out, db))))
            return QGEMV_EINVAL;
    }
    GemvArgs a{};
    a.w = static_cast<const uint8_t *>(w);
    a.xq = act.xq;
    a.xd = act.xd;
    a.x = act.x;
    a.xq_out = act.xq_out;
    a.xd_out = act.xd_out;
    a.rows = static_cast<int32_t>(rows);
    a.nb = static_cast<int32_t>(cols / block_cols(wtype));
    a.nchunks = static_cast<int32_t>(cols / 32);
    // Column splits: the splits inside the workgroup (its waves in sets of `splits`, their row
    // sums added in LDS in chunk order), one launch and the same y bit for bit as the split-K
    // reduce, with as many waves in all as the plan's two-pass form but at most 4096 (one
    // resident round at 16 waves per CU, so every workgroup loops over its steps with the next
    // loads in flight: 4096 x 16384 from codes 8.7 us against 10.4 us with 8192 waves on
    // MI355X). In the fused form the workgroup quantizes every chunk of the row, so the slices
    // of all chunks must fit in LDS. The workspace is still required (the ABI's contract is
    // per shape), though not touched.
    const int maxw = gemv_max_waves(nvec, plan.lanes_per_row, plan.chunks_per_lane);
    const int wpb = split_waves_per_block(plan, maxw);
    const bool in_wg = need > 0 && plan.splits <= maxw &&
                       (!act.x || gemv_split_lds_bytes(nvec, plan.lanes_per_row, plan.chunks_per_lane,
                                                       true, plan.splits, wpb) <= kMaxSplitLds);
    if (in_wg) {
        const int64_t waves = std::min<int64_t>(
            static_cast<int64_t>(plan.blocks) * plan.splits * plan.waves_per_block, 4096);
        const int64_t blocks = std::min<int64_t>((waves + wpb - 1) / wpb, int64_t{65535} * 64);
        a.out = y;
        const LaunchShape s{plan.lanes_per_row, plan.chunks_per_lane, wpb,
                            static_cast<int>(blocks), plan.splits};
        const hipError_t e = launch_gemv_split(wtype, a, s, nvec, stream);
        return e == hipSuccess ? QGEMV_OK : hip_fail(e);
    }
    a.out = need > 0 ? static_cast<float *>(ws) : y;
    LaunchShape s{plan.lanes_per_row, plan.chunks_per_lane, plan.waves_per_block, plan.blocks,
                  plan.splits};
    hipError_t e = launch_gemv(wtype, a, s, nvec, false, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (need > 0) {
        e = launch_splitk_reduce(static_cast<const float *>(ws), y, static_cast<int64_t>(nvec) * rows,
                                 plan.splits, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return QGEMV_OK;
}

// More than kMaxVec vectors (Q4_K): the matrix-core kernel. Workgroups of 128 rows x one
// group of 32 * nt vectors; the super-blocks are split over more workgroups when rows and
// groups alone give fewer than two workgroups per CU (the splits are added by the ordered
// reduce, as for the vector kernels).
struct McPlan {
    int nt, row_tiles, groups, splits, sbps;
};

// check_gemv_args for any vector count (the shape itself checked by the caller)
int check_gemv_args_n(int wtype, const void *w, const int8_t *xq, const float *xd, const void *out,
                      size_t out_bytes, int64_t rows, int64_t cols, int32_t nvec) {
    if (!w || !xq || !xd || !out) return QGEMV_EINVAL;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(out, 4))
        return QGEMV_EALIGN;
    const size_t wb = weight_bytes(wtype, rows, cols);
    const size_t xqb = static_cast<size_t>(nvec) * cols;
    const size_t xdb = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
    if (overlaps(out, out_bytes, w, wb) || overlaps(out, out_bytes, xq, xqb) ||
        overlaps(out, out_bytes, xd, xdb))
        return QGEMV_EINVAL;
    return QGEMV_OK;
}

bool q32i8_many(int wtype, int64_t rows, int64_t cols, int32_t nvec);

// (Q4_K products with 9..16 vectors that the few-vector kernel takes are not this path's.)
bool mc_shape_ok(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    return wtype == QGEMV_Q4K && nvec > kMaxVec && nvec <= kMaxBatch && rows >= 1 &&
           rows <= (int64_t{1} << 30) && cols >= kQK && cols % kQK == 0 &&
           cols <= (int64_t{1} << 30) && rows * (cols / 32) < (int64_t{1} << 31) &&
           !q32i8_many(wtype, rows, cols, nvec);
}

McPlan make_mc_plan(int64_t rows, int64_t cols, int32_t nvec) {
    McPlan p{};
    const int64_t nb = cols / kQK;
    // Up to 96 vectors one group of ceil(nvec / 32) tiles; beyond, groups of 2 tiles (64
    // vectors): the 2-tile kernel keeps two waves per SIMD and pipelines its blocks, where 3 or 4
    // tiles leave one, and smaller groups pad less (262144 x 1536, graph replay on MI355X,
    // 2 / 3 / 4 tiles per group: 96 vectors 192 / 169 / 170 us; 128: 213 / 328 / 221; 160:
    // 287 / 327 / 427; 192: 298 / 327 / 427; 256: 400 / 478 / 430).
    p.nt = nvec <= 96 ? (nvec + 31) / 32 : 2;
    p.groups = (nvec + 32 * p.nt - 1) / (32 * p.nt);
    p.row_tiles = static_cast<int>((rows + kMcRows - 1) / kMcRows);
    const int64_t base = static_cast<int64_t>(p.row_tiles) * p.groups;
    const int64_t want = 2 * 256;
    int64_t splits = base < want ? std::min<int64_t>(nb, (want + base - 1) / base) : 1;
    p.sbps = static_cast<int>((nb + splits - 1) / splits);
    p.splits = static_cast<int>((nb + p.sbps - 1) / p.sbps);
    return p;
}

// Workspace of the matrix-core path: the staged tiles, then (when split) the partial outputs.
size_t mc_tiles_bytes(const McPlan &p, int64_t cols) {
    return static_cast<size_t>(cols / kQK) * p.groups * mc_tile_bytes(p.nt);
}

size_t mc_ws_bytes(const McPlan &p, int64_t rows, int64_t cols, int32_t nvec) {
    const size_t parts = p.splits > 1 ? static_cast<size_t>(p.splits) * nvec * rows * sizeof(float) : 0;
    return mc_tiles_bytes(p, cols) + parts;
}

int run_mc(const void *w, const int8_t *xq, const float *xd, float *y, int32_t *P, int32_t *S,
           int64_t rows, int64_t cols, int32_t nvec, void *ws, size_t ws_bytes,
           hipStream_t stream) {
    const bool debug = P != nullptr;
    if (!w || !xq || !xd || (!debug && !y)) return QGEMV_EINVAL;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xd, 4) || (y && !aligned(y, 4)))
        return QGEMV_EALIGN;
    const size_t wb = weight_bytes(QGEMV_Q4K, rows, cols);
    const size_t qb = static_cast<size_t>(nvec) * cols;
    const size_t db = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
    const size_t yb = static_cast<size_t>(nvec) * rows * sizeof(float);
    if (y && (overlaps(y, yb, w, wb) || overlaps(y, yb, xq, qb) || overlaps(y, yb, xd, db)))
        return QGEMV_EINVAL;
    McPlan p = make_mc_plan(rows, cols, nvec);
    if (debug) p.splits = 1;    // the debug form covers every super-block in one split
    const size_t tb = mc_tiles_bytes(p, cols);
    const size_t need = mc_ws_bytes(p, rows, cols, nvec);
    if (!ws || ws_bytes < need) return QGEMV_EWORKSPACE;
    if (!aligned(ws, 16)) return QGEMV_EALIGN;
    if (overlaps(ws, need, w, wb) || (y && overlaps(ws, need, y, yb)) || overlaps(ws, need, xq, qb) ||
        overlaps(ws, need, xd, db))
        return QGEMV_EINVAL;
    if (debug) {
        const size_t pb = static_cast<size_t>(nvec) * rows * (cols / 32) * sizeof(int32_t);
        const size_t sbb = static_cast<size_t>(nvec) * (cols / 32) * sizeof(int32_t);
        if (overlaps(ws, need, P, pb) || overlaps(ws, need, S, sbb)) return QGEMV_EINVAL;
    }
    GemmArgs a{};
    a.w = static_cast<const uint8_t *>(w);
    a.xq = xq;
    a.xd = xd;
    a.tiles = static_cast<uint8_t *>(ws);
    float *parts = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + tb);
    a.out = p.splits > 1 ? parts : y;
    a.P = P;
    a.S = S;
    a.rows = static_cast<int32_t>(rows);
    a.nb = static_cast<int32_t>(cols / kQK);
    a.nvec = nvec;
    a.sb_per_split = debug ? a.nb : p.sbps;
    a.row_tiles = p.row_tiles;
    a.groups = p.groups;
    a.splits = p.splits;
    hipError_t e = launch_gemm_q4k_mfma(a, p.nt, p.row_tiles, p.groups, p.splits, debug, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (!debug && p.splits > 1) {
        e = launch_splitk_reduce(parts, y, static_cast<int64_t>(nvec) * rows, p.splits, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return QGEMV_OK;
}

// Q8_0, Q4_0 and Q6_K with more than kMaxVec vectors: the integer matrix cores (gemm_q32.hip,
// gemm_q6k_mc.hip), one pass over the weights for up to 256 vectors. A workgroup covers vw
// tiles of 32 vectors (1, 2 or 4 for 1, 2, 3+ tiles) by mc32_rows_per_wg(vw) rows; the
// columns are split when the row tiles and vector groups alone give fewer than two workgroups
// per CU (the splits added by the ordered reduce).
bool mc32_ok(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    const bool fmt = wtype == QGEMV_Q8_0 || wtype == QGEMV_Q4_0 || wtype == QGEMV_Q6K;
    const bool few = (fmt || wtype == QGEMV_Q4K) && nvec >= 1 && nvec <= kQ32I8MaxVec;
    const bool many = fmt && nvec > kMaxVec && nvec <= kMaxBatch;
    return (few || many) && shape_ok_t(wtype, rows, cols, 1) &&
           static_cast<int64_t>(nvec) * cols < (int64_t{1} << 34);
}

// Where qgemv_batch takes that path. On a small tensor its staging, split and reduce cost a
// floor of 16-20 us, where the vector kernel on groups of 8 vectors (each group reading every
// weight) is ahead until the groups are many. Measured on MI355X (graph replay, cold weights;
// matrix cores against groups of 8): 2048 x 8192 Q6_K / Q8_0 / Q4_0 with 9 vectors 20.0 / 19.4
// / 18.9 us against 12.4 / 12.0 / 10.4, with 24 vectors 22.2 / 23.5 / 23.1 against 22.3 / 19.5
// / 19.1, with 32 vectors 22.9 / 25.0 / 24.6 against 29.3 / 25.7 / 25.2; 16384 x 2048 with 16
// vectors 19.2 / 17.9 / 18.3 against 21.2 / 20.2 / 16.9, with 24 vectors 20.0 / 19.3 / 20.2
// against 31.5 / 29.7 / 24.9; 65536 x 1536 with 9 vectors 38.4 / 30.7 / 30.2 against 55.4 /
// 48.4 / 38.5. The weight count (not the bytes) separates the formats: from 32 vectors
// always, from 16 vectors from 24 Mi weights, from 9 vectors from 48 Mi weights.
// Where qgemv_batch takes the few-vector kernel for Q8_0, Q4_0 and Q6_K (gemm_q32_i8.hip)
// instead of the vector kernel. It moves the same HBM bytes (FETCH_SIZE per dispatch equal) at
// about 85% of the vector kernel's rate, but its work per weight does not grow with the vector
// count, so it wins where the vector kernel's dot products bind, on rows of one split (up to
// 2048 columns; a second split and its reduce cost more than they save below 8 vectors):
// Q4_0 from 4 vectors on tensors of at least 32 Mi weights (3 from 256 Mi; with two splits 8);
// Q6_K from 4 vectors on 256 Mi weights, with 8 from 64 Mi; Q8_0 (twice the bytes per weight)
// with 8 vectors from 256 Mi weights; Q4_K with 4 vectors where its own integer kernel is not
// taken (below). Measured on MI355X (graph replay, cold; this kernel
// against the vector kernel, us):
//   Q4_0 262144 x 1536 x 2 / 3 / 4 / 8: 40.9 / 36.5, 40.6 / 44.8, 40.7 / 47.7, 43.8 / 97.8;
//        65536 x 2048 x 3 / 4 / 5 / 8: 17.1 / 15.2, 17.4 / 17.0, 17.7 / 19.5, 17.8 / 23.5;
//        16384 x 2048 x 3 / 4 / 8: 6.63 / 6.29, 6.63 / 7.07, 6.90 / 8.32;
//        16384 x 4096 x 6 / 8: 12.9 / 12.3, 13.1 / 13.8; 4096 x 4096 x 8: 8.0 / 6.4;
//   Q6_K 262144 x 1536 x 3 / 4 / 8: 66.2 / 64.6, 66.4 / 71.0, 73.4 / 140.8;
//        65536 x 2048 x 4 / 6 / 8: 26.9 / 25.1, 31.3 / 27.1, 31.2 / 32.1;
//        16384 x 2048 x 8: 10.6 / 10.7; 16384 x 4096 x 8: 23.3 / 20.1;
//   Q8_0 262144 x 1536 x 6 / 8: 86.0 / 84.2, 84.2 / 103.6; 65536 x 2048 x 8: 29.7 / 29.1.
int64_t i8_min_bytes(int32_t nvec);

bool q32i8_auto(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    constexpr int64_t Mi = int64_t{1} << 20;
    const int64_t weights = rows * cols;
    const bool one_split = cols <= int64_t{kQ32I8MaxWaves} * kQ32I8BlocksPerWave * 32;
    switch (wtype) {
        case QGEMV_Q4_0:
            if (!one_split) return weights >= 32 * Mi && nvec >= 8;
            return weights >= 32 * Mi && nvec >= (weights >= 256 * Mi ? 3 : 4);
        case QGEMV_Q6K:
            return one_split && ((weights >= 256 * Mi && nvec >= 4) ||
                                 (weights >= 64 * Mi && nvec >= 8));
        case QGEMV_Q8_0: return one_split && weights >= 256 * Mi && nvec >= 8;
        case QGEMV_Q4K: {
            // 4 vectors on tensors of 16-96 MiB, below the Q4_K integer kernel's threshold
            // (i8_min_bytes); measured against the vector kernel (planner's plan): 16384 /
            // 32768 / 65536 x 2048 x 4 in 7.09 / 10.7 / 17.7 against 8.15 / 12.3 / 20.9 us;
            // with 3, 5 or 6 vectors it was within a few % either way
            const int64_t bytes = static_cast<int64_t>(weight_bytes(wtype, rows, cols));
            return one_split && nvec == 4 && bytes >= (int64_t{16} << 20) &&
                   bytes < i8_min_bytes(4);
        }
        default: return false;
    }
}

// Whether 9..16 vectors run on the few-vector kernel (gemm_q32_i8.hip, 3 or 4 halves of 4
// vectors) rather than the 32 x 32 x 32 kernels, the vector kernel on groups of 8, or (Q4_K) the
// Q4_K integer kernel. Measured on MI355X (graph replay, cold; this kernel against what was
// taken before, us):
//   Q4_0 262144 x 1536 x 12 / 16: 52.2 / 81.1, 63.0 / 83.6; 65536 x 2048 x 12: 20.7 / 37.4;
//        16384 x 2048 x 12: 7.85 / 15.2 (groups of 8); 2048 x 8192 x 10: 9.42 / 10.8;
//   Q6_K 262144 x 1536 x 12: 86.2 / 99.8; 65536 x 2048 x 12: 30.2 / 42.0; 16384 x 2048 x 12:
//        11.5 / 19.6; 4096 x 4096 x 10: 11.4 / 11.5;
//   Q8_0 262144 x 1536 x 16: 90.9 / 107.2; 65536 x 2048 x 10 / 12 / 16: 35.8 / 33.4,
//        36.0 / 33.8, 32.9 / 34.4; 16384 x 2048 x 12: 11.4 / 18.9;
//   Q4_K 65536 x 2048 x 10 / 12 / 16: 23.9 / 25.2, 24.7 / 25.5, 31.0 / 26.3; 16384 x 2048 x
//        12: 9.11 / 10.0; 262144 x 1536 x 12: 62.9 / 61.0.
// Smaller tensors than 16 Mi weights were not measured and keep the earlier routes.
bool q32i8_many(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    if (nvec <= kMaxVec || nvec > kQ32I8MaxVec) return false;
    constexpr int64_t Mi = int64_t{1} << 20;
    const int64_t weights = rows * cols;
    if (weights < 16 * Mi) return false;
    switch (wtype) {
        case QGEMV_Q4_0:
        case QGEMV_Q6K: return true;
        case QGEMV_Q8_0: return nvec >= 16 || weights < 48 * Mi || weights >= 256 * Mi;
        case QGEMV_Q4K:
            return nvec <= 12 && static_cast<int64_t>(weight_bytes(wtype, rows, cols)) <
                                     (int64_t{128} << 20);
        default: return false;
    }
}

bool mc32_auto(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    if (!mc32_ok(wtype, rows, cols, nvec)) return false;
    const int64_t weights = rows * cols;
    constexpr int64_t Mi = int64_t{1} << 20;
    if (nvec <= kMaxVec) return q32i8_auto(wtype, rows, cols, nvec);
    if (q32i8_many(wtype, rows, cols, nvec)) return true;
    if (wtype == QGEMV_Q4K) return false;
    return nvec >= 32 || (nvec >= 16 && weights >= 24 * Mi) || weights >= 48 * Mi;
}

// Which kernel run_mc32 takes: the few-vector kernel for 1..8 vectors, for Q4_K, and for 9..16
// where q32i8_many says so; else the 32 x 32 x 32 kernels.
bool mc32_few_kernel(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    return nvec <= kMaxVec || wtype == QGEMV_Q4K || q32i8_many(wtype, rows, cols, nvec);
}

// More than kMaxVec vectors where the matrix-core path is not taken: the vector kernel on
// groups of up to kMaxVec vectors, one after another on the stream (not Q4_K, whose 9..16
// vectors take its integer kernel).
bool grouped_shape_ok(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    return wtype != QGEMV_Q4K && nvec > kMaxVec && mc32_ok(wtype, rows, cols, nvec) &&
           !mc32_auto(wtype, rows, cols, nvec);
}

// The plan of the few-vector kernel (gemm_q32_i8.hip): a split holds at most kQ32I8MaxWaves *
// kQ32I8BlocksPerWave blocks of 32 columns (the activation a workgroup stages in LDS); wider
// rows are split into equal parts of whole waves, added by the ordered reduce.
struct Q32I8Plan {
    int waves, splits, bps, row_tiles;
};

Q32I8Plan make_q32i8_plan(int64_t rows, int64_t cols) {
    Q32I8Plan p{};
    const int64_t nb = cols / 32;
    const int64_t most = int64_t{kQ32I8MaxWaves} * kQ32I8BlocksPerWave;
    const int64_t parts = (nb + most - 1) / most;
    const int64_t per = (nb + parts - 1) / parts;
    p.waves = static_cast<int>((per + kQ32I8BlocksPerWave - 1) / kQ32I8BlocksPerWave);
    p.bps = p.waves * kQ32I8BlocksPerWave;
    p.splits = static_cast<int>((nb + p.bps - 1) / p.bps);
    p.row_tiles = static_cast<int>((rows + 15) / 16);
    return p;
}

struct Mc32Plan {
    int vw, groups, row_tiles, splits, bps;
};

Mc32Plan make_mc32_plan(int64_t rows, int64_t cols, int32_t nvec) {
    Mc32Plan p{};
    const int vtiles = (nvec + 31) / 32;
    p.vw = vtiles >= 3 ? 4 : vtiles;
    const int wg_rows = mc32_rows_per_wg(p.vw);
    p.groups = (vtiles + p.vw - 1) / p.vw;
    p.row_tiles = static_cast<int>((rows + wg_rows - 1) / wg_rows);
    const int64_t nb = cols / 32;
    const int64_t steps = (nb + 7) / 8;               // the kernels' steps of 8 blocks
    const int64_t base = static_cast<int64_t>(p.row_tiles) * p.groups;
    const int64_t want = 2 * 256;
    const int64_t splits = base < want ? std::min<int64_t>(steps, (want + base - 1) / base) : 1;
    p.bps = static_cast<int>(8 * ((steps + splits - 1) / splits));
    p.splits = static_cast<int>((nb + p.bps - 1) / p.bps);
    return p;
}

// The workspace of run_mc32 for a shape mc32_ok accepts: partial sums of column splits.
size_t mc32_route_ws_bytes(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    const int splits = mc32_few_kernel(wtype, rows, cols, nvec)
                           ? make_q32i8_plan(rows, cols).splits
                           : make_mc32_plan(rows, cols, nvec).splits;
    return splits > 1 ? static_cast<size_t>(splits) * nvec * rows * sizeof(float) : 0;
}

// y (or, with P, the debug partials P and S) of a Q8_0, Q4_0 or Q6_K product with many vectors.
int run_mc32(int wtype, const void *w, const int8_t *xq, const float *xd, float *y, int32_t *P,
              int32_t *S, int64_t rows, int64_t cols, int32_t nvec, void *ws, size_t ws_bytes,
              hipStream_t stream) {
    const bool debug = P != nullptr;
    if (!mc32_ok(wtype, rows, cols, nvec)) return QGEMV_EINVAL;
    const size_t ybytes = static_cast<size_t>(nvec) * rows * sizeof(float);
    const int64_t nsub = wtype == QGEMV_Q6K ? cols / 16 : cols / 32;
    const size_t pbytes = static_cast<size_t>(nvec) * rows * nsub * sizeof(int32_t);
    int st = check_gemv_args_n(wtype, w, xq, xd, debug ? static_cast<const void *>(P) : y,
                               debug ? pbytes : ybytes, rows, cols, nvec);
    if (st != QGEMV_OK) return st;
    const size_t wb = weight_bytes(wtype, rows, cols);
    const size_t qb = static_cast<size_t>(nvec) * cols;
    const size_t db = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
    if (debug) {
        const size_t sbytes = static_cast<size_t>(nvec) * (cols / 32) * sizeof(int32_t);
        if (!S) return QGEMV_EINVAL;
        if (!aligned(S, 4)) return QGEMV_EALIGN;
        if (overlaps(S, sbytes, P, pbytes) || overlaps(S, sbytes, w, wb) ||
            overlaps(S, sbytes, xq, qb) || overlaps(S, sbytes, xd, db))
            return QGEMV_EINVAL;
    }
    const size_t need = debug ? 0 : mc32_route_ws_bytes(wtype, rows, cols, nvec);
    if (need > 0) {
        if (!ws || ws_bytes < need) return QGEMV_EWORKSPACE;
        if (!aligned(ws, 4)) return QGEMV_EALIGN;
        if (overlaps(ws, need, w, wb) || overlaps(ws, need, y, ybytes) || overlaps(ws, need, xq, qb) ||
            overlaps(ws, need, xd, db))
            return QGEMV_EINVAL;
    }
    GemmArgs a{};
    a.w = static_cast<const uint8_t *>(w);
    a.xq = xq;
    a.xd = xd;
    a.out = debug ? nullptr : (need > 0 ? static_cast<float *>(ws) : y);
    a.P = P;
    a.S = S;
    a.rows = static_cast<int32_t>(rows);
    a.nb = static_cast<int32_t>(cols / 32);
    a.nvec = nvec;
    hipError_t e;
    if (mc32_few_kernel(wtype, rows, cols, nvec)) {
        const Q32I8Plan p = make_q32i8_plan(rows, cols);
        a.sb_per_split = p.bps;
        a.row_tiles = p.row_tiles;
        a.groups = 1;
        a.splits = p.splits;
        e = launch_gemm_q32_i8(wtype, a, p.waves, debug, stream);
    } else {
        const Mc32Plan p = make_mc32_plan(rows, cols, nvec);
        a.sb_per_split = p.bps;
        a.row_tiles = p.row_tiles;
        a.groups = p.groups;
        a.splits = p.splits;
        e = wtype == QGEMV_Q6K ? launch_gemm_q6k_mc(a, p.vw, debug, stream)
                               : launch_gemm_q32_mc(wtype, a, p.vw, debug, stream);
    }
    if (e != hipSuccess) return hip_fail(e);
    if (need > 0) {
        e = launch_splitk_reduce(static_cast<const float *>(ws), y,
                                 static_cast<int64_t>(nvec) * rows, a.splits, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return QGEMV_OK;
}

// Several matrices with one activation (plain: act.xq / act.xd; fused: act.x and optionally
// act.xq_out / act.xd_out): every check, then the launch description in a and s.
// Q4_K with up to kMaxVec vectors on the integer matrix cores (gemm_i8.hip). The kernel takes
// any 1..kI8MaxVec vectors (qgemv_batch_i8mc); qgemv_batch routes to it where it was measured
// faster than the vector kernel: from 3 vectors on tensors of 128 MiB down to 8 vectors on
// 16 MiB (i8_min_bytes), and always for 9..16 vectors (faster than the float matrix-core
// kernel on every shape measured: 262144 x 1536 x 16 in 64 against 76 us, 16384 x 2048 x 16
// in 11 against 17 us). With few vectors the vector kernel's dot products hide under the
// weight stream; on small tensors the time is the latency of a few loads per wave, where the
// vector kernel (no activation staging) is ahead. A split holds at most
// kI8MaxWaves * kI8SbPerWave super-blocks (the activation a workgroup stages in LDS); wider
// rows are split into equal parts, added by the ordered reduce.
int64_t i8_min_bytes(int32_t nvec) {
    constexpr int64_t MiB = int64_t{1} << 20;
    switch (nvec) {
        case 3: return 128 * MiB;
        case 4: return 96 * MiB;
        case 5: return 48 * MiB;
        case 6: return 32 * MiB;
        case 7: return 24 * MiB;
        case 8: return 16 * MiB;
        default: return nvec > kMaxVec && nvec <= kI8MaxVec ? 0 : INT64_MAX;
    }
}

bool i8_ok(int64_t rows, int64_t cols, int32_t nvec) {
    return nvec >= 1 && nvec <= kI8MaxVec && shape_ok_t(QGEMV_Q4K, rows, cols, 1) &&
           static_cast<int64_t>(nvec) * cols < (int64_t{1} << 34);
}

bool i8_auto(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    return wtype == QGEMV_Q4K && i8_ok(rows, cols, nvec) &&
           static_cast<int64_t>(weight_bytes(QGEMV_Q4K, rows, cols)) >= i8_min_bytes(nvec) &&
           !q32i8_many(wtype, rows, cols, nvec);
}

struct I8Plan {
    int waves, splits, sbps, row_tiles;
};

I8Plan make_i8_plan(int64_t rows, int64_t cols) {
    I8Plan p{};
    const int64_t nb = cols / kQK;
    const int64_t most = int64_t{kI8MaxWaves} * kI8SbPerWave;
    const int64_t parts = (nb + most - 1) / most;
    const int64_t per = (nb + parts - 1) / parts;
    p.waves = static_cast<int>((per + kI8SbPerWave - 1) / kI8SbPerWave);
    p.sbps = p.waves * kI8SbPerWave;
    p.splits = static_cast<int>((nb + p.sbps - 1) / p.sbps);
    p.row_tiles = static_cast<int>((rows + 15) / 16);
    return p;
}

size_t i8_ws_bytes(const I8Plan &p, int64_t rows, int32_t nvec) {
    return p.splits > 1 ? static_cast<size_t>(p.splits) * nvec * rows * sizeof(float) : 0;
}

// y (or, with P, the debug partials P and S instead) of a Q4_K product on the integer matrix
// cores, from codes and scales or (act.x) from the float32 activation; arguments checked as
// for the vector kernels.
int run_i8(const void *w, const Activation &act, float *y, int32_t *P, int32_t *S, int64_t rows,
           int64_t cols, int32_t nvec, void *ws, size_t ws_bytes, hipStream_t stream) {
    const bool debug = P != nullptr;
    const size_t ybytes = static_cast<size_t>(nvec) * rows * sizeof(float);
    const size_t pbytes = static_cast<size_t>(nvec) * rows * (cols / 32) * sizeof(int32_t);
    const size_t wb = weight_bytes(QGEMV_Q4K, rows, cols);
    int st;
    if (act.x) {
        if (debug || !w || !y || !i8_ok(rows, cols, nvec) || nvec > kMaxVec) return QGEMV_EINVAL;
        if (!aligned(w, 16) || !aligned(y, 4)) return QGEMV_EALIGN;
        if (overlaps(y, ybytes, w, wb)) return QGEMV_EINVAL;
        st = check_fused_act(act, w, wb, y, ybytes, cols, nvec);
    } else {
        if (!i8_ok(rows, cols, nvec)) return QGEMV_EINVAL;
        st = check_gemv_args_n(QGEMV_Q4K, w, act.xq, act.xd,
                               debug ? static_cast<const void *>(P) : y, debug ? pbytes : ybytes,
                               rows, cols, nvec);
    }
    if (st != QGEMV_OK) return st;
    const int8_t *xq = act.xq;
    const float *xd = act.xd;
    const I8Plan p = make_i8_plan(rows, cols);
    const size_t need = debug ? 0 : i8_ws_bytes(p, rows, nvec);
    const size_t qb = static_cast<size_t>(nvec) * cols;
    const size_t db = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
    if (debug) {
        const size_t sbytes = static_cast<size_t>(nvec) * (cols / 32) * sizeof(int32_t);
        if (!aligned(S, 4)) return QGEMV_EALIGN;
        if (overlaps(S, sbytes, P, pbytes) || overlaps(S, sbytes, w, wb) ||
            overlaps(S, sbytes, xq, qb) || overlaps(S, sbytes, xd, db))
            return QGEMV_EINVAL;
    }
    if (need > 0) {
        if (!ws || ws_bytes < need) return QGEMV_EWORKSPACE;
        if (!aligned(ws, 4)) return QGEMV_EALIGN;
        if (overlaps(ws, need, w, wb) || overlaps(ws, need, y, ybytes) ||
            (xq && overlaps(ws, need, xq, qb)) || (xd && overlaps(ws, need, xd, db)) ||
            (act.x && overlaps(ws, need, act.x, qb * sizeof(float))) ||
            (act.xq_out && (overlaps(ws, need, act.xq_out, qb) || overlaps(ws, need, act.xd_out, db))))
            return QGEMV_EINVAL;
    }
    GemmArgs a{};
    a.w = static_cast<const uint8_t *>(w);
    a.xq = xq;
    a.xd = xd;
    a.x = act.x;
    a.xq_out = act.xq_out;
    a.xd_out = act.xd_out;
    a.out = need > 0 ? static_cast<float *>(ws) : y;
    a.P = P;
    a.S = S;
    a.rows = static_cast<int32_t>(rows);
    a.nb = static_cast<int32_t>(cols / kQK);
    a.nvec = nvec;
    a.sb_per_split = p.sbps;
    a.row_tiles = p.row_tiles;
    a.groups = 1;
    a.splits = p.splits;
    hipError_t e = launch_gemm_q4k_i8(a, p.waves, debug, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (need > 0) {
        e = launch_splitk_reduce(static_cast<const float *>(ws), y,
                                 static_cast<int64_t>(nvec) * rows, p.splits, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return QGEMV_OK;
}

// The lane geometry of a multi-matrix launch: one that covers the row in one pass if any
// (the fewest idle lanes), else by the one-matrix planner's rule among the geometries whose
// column chunks a workgroup can split among its waves (one wave per chunk).
bool multi_geometry(int64_t cols, int32_t nvec, int &t, int &nc, int &splits) {
    splits = 1;
    if (choose_geometry(cols, nvec, true, t, nc, false, true)) return true;
    if (!choose_geometry(cols, nvec, false, t, nc, true, true)) return false;
    splits = splits_for(t, nc, cols);
    return true;
}

int prepare_multi(const qgemv_matrix *mats, int32_t nmats, const Activation &act, int64_t cols,
                  int32_t nvec, MultiArgs &a, LaunchShape &s, double &wbytes) {
    if (!mats || nmats < 1 || nmats > kMaxMats || !shape_ok(1, cols, nvec)) return QGEMV_EINVAL;
    int t = 0, nc = 0, splits = 1;
    if (!multi_geometry(cols, nvec, t, nc, splits)) return QGEMV_EINVAL;
    const size_t qb = static_cast<size_t>(nvec) * cols;
    const size_t db = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
    const size_t xb = qb * sizeof(float);
    // the activation buffers (the fused form's are written, so they must not overlap)
    struct Buf {
        const void *p;
        size_t n;
    };
    Buf acts[3];
    int nacts = 0;
    if (act.x) {
        if ((act.xq_out == nullptr) != (act.xd_out == nullptr)) return QGEMV_EINVAL;
        if (!aligned(act.x, 16)) return QGEMV_EALIGN;
        acts[nacts++] = {act.x, xb};
        if (act.xq_out) {
            if (!aligned(act.xq_out, 4) || !aligned(act.xd_out, 4)) return QGEMV_EALIGN;
            acts[nacts++] = {act.xq_out, qb};
            acts[nacts++] = {act.xd_out, db};
        }
        for (int i = 0; i < nacts; i++)
            for (int k = i + 1; k < nacts; k++)
                if (overlaps(acts[i].p, acts[i].n, acts[k].p, acts[k].n)) return QGEMV_EINVAL;
    } else {
        if (!act.xq || !act.xd) return QGEMV_EINVAL;
        if (!aligned(act.xq, 16) || !aligned(act.xd, 4)) return QGEMV_EALIGN;
        acts[nacts++] = {act.xq, qb};
        acts[nacts++] = {act.xd, db};
    }
    for (int i = 0; i < nmats; i++) {
        const qgemv_matrix &m = mats[i];
        if (m.reserved != 0 || !m.w || !m.y || !shape_ok_t(m.wtype, m.rows, cols, nvec))
            return QGEMV_EINVAL;
        if (!aligned(m.w, 16) || !aligned(m.y, 4)) return QGEMV_EALIGN;
    }
    // each output overlaps no weights, no activation buffer and no other output; the fused
    // form's code outputs overlap no weights
    wbytes = 0;
    for (int i = 0; i < nmats; i++) {
        const size_t yb = static_cast<size_t>(nvec) * mats[i].rows * sizeof(float);
        const size_t wb = weight_bytes(mats[i].wtype, mats[i].rows, cols);
        wbytes += static_cast<double>(wb);
        for (int k = 0; k < nmats; k++) {
            if (overlaps(mats[i].y, yb, mats[k].w, weight_bytes(mats[k].wtype, mats[k].rows, cols)))
                return QGEMV_EINVAL;
            if (k != i && overlaps(mats[i].y, yb, mats[k].y,
                                   static_cast<size_t>(nvec) * mats[k].rows * sizeof(float)))
                return QGEMV_EINVAL;
        }
        for (int k = 0; k < nacts; k++) {
            if (overlaps(mats[i].y, yb, acts[k].p, acts[k].n)) return QGEMV_EINVAL;
            if (act.x && k > 0 && overlaps(acts[k].p, acts[k].n, mats[i].w, wb)) return QGEMV_EINVAL;
        }
    }
    // the step numbering and the grid
    const int rpw = 64 / t, g = groups_per_step(nc);
    a = MultiArgs{};
    a.act.xq = act.xq;
    a.act.xd = act.xd;
    a.act.x = act.x;
    a.act.xq_out = act.xq_out;
    a.act.xd_out = act.xd_out;
    a.act.nb = 0;                            // unused: each matrix has its own
    a.act.nchunks = static_cast<int32_t>(cols / 32);
    // descriptors ordered by format (stable), so each format's steps are consecutive
    int64_t steps = 0;
    int k = 0;
    for (int wt : {QGEMV_Q4K, QGEMV_Q6K, QGEMV_Q4_0, QGEMV_Q8_0}) {
        const int64_t first = steps;
        for (int i = 0; i < nmats; i++) {
            if (mats[i].wtype != wt) continue;
            MatDesc &d = a.m[k++];
            d.w = static_cast<const uint8_t *>(mats[i].w);
            d.out = mats[i].y;
            d.rows = static_cast<int32_t>(mats[i].rows);
            d.nb = static_cast<int32_t>(cols / block_cols(wt));
            d.wtype = wt;
            d.step0 = static_cast<int32_t>(steps);
            steps += ((mats[i].rows + rpw - 1) / rpw + g - 1) / g;
            if (steps >= (int64_t{1} << 30)) return QGEMV_EINVAL;
        }
        if (steps > first) {
            FmtGroup &fg = a.g[a.ngroups++];
            fg.wtype = wt;
            fg.step0 = static_cast<int32_t>(first);
            fg.steps = static_cast<int32_t>(steps - first);
        }
    }
    if (k != nmats) return QGEMV_EINVAL;
    a.nmats = nmats;
    a.steps = static_cast<int32_t>(steps);
    // The grid, then each format's share of it in proportion to its steps (at least one
    // workgroup each). A split row takes the one-matrix split's grid: workgroups of sets of
    // `splits` waves, at most 4096 waves in all.
    const int maxw = gemv_max_waves(nvec, t, nc);
    const int waves = splits > 1 ? splits * (maxw / splits) : 4;
    const int64_t want = splits > 1 ? std::min<int64_t>(steps * splits, 4096)
                                    : std::min<int64_t>(steps, target_waves(nvec));
    const int64_t total = (want + waves - 1) / waves;
    int32_t blocks = 0;
    for (int i = 0; i < a.ngroups; i++) {
        FmtGroup &fg = a.g[i];
        fg.block0 = blocks;
        fg.blocks = static_cast<int32_t>(std::max<int64_t>(1, (total * fg.steps + steps - 1) / steps));
        blocks += fg.blocks;
    }
    s = LaunchShape{t, nc, waves, blocks, splits};
    return QGEMV_OK;
}

// Matrices all of one format take that format's walk, whose first weights go out ahead of the
// activation slice (gate + up, 2 x 6144 x 1536 Q4_K, graph-replayed on MI355X: 4.7 us against
// 5.4 us); a mix of formats takes the kernel that branches on the format per step.
int launch_multi(const MultiArgs &a, const LaunchShape &s, int32_t nvec, hipStream_t stream) {
    bool one_format = true;
    for (int i = 1; i < a.nmats; i++) one_format = one_format && a.m[i].wtype == a.m[0].wtype;
    hipError_t e = hipErrorInvalidValue;
    if (s.splits > 1) {
        if (!one_format)
            e = launch_gemv_multi_split(a, s, nvec, stream);
        else if (a.m[0].wtype == QGEMV_Q4K)
            e = launch_gemv_multi_split_q4k(a, s, nvec, stream);
        else if (a.m[0].wtype == QGEMV_Q6K)
            e = launch_gemv_multi_split_q6k(a, s, nvec, stream);
        else if (a.m[0].wtype == QGEMV_Q4_0)
            e = launch_gemv_multi_split_q40(a, s, nvec, stream);
        else if (a.m[0].wtype == QGEMV_Q8_0)
            e = launch_gemv_multi_split_q80(a, s, nvec, stream);
    } else if (!one_format)
        e = launch_gemv_multi(a, s, nvec, stream);
    else if (a.m[0].wtype == QGEMV_Q4K)
        e = launch_gemv_multi_q4k(a, s, nvec, stream);
    else if (a.m[0].wtype == QGEMV_Q6K)
        e = launch_gemv_multi_q6k(a, s, nvec, stream);
    else if (a.m[0].wtype == QGEMV_Q4_0)
        e = launch_gemv_multi_q40(a, s, nvec, stream);
    else if (a.m[0].wtype == QGEMV_Q8_0)
        e = launch_gemv_multi_q80(a, s, nvec, stream);
    return e == hipSuccess ? QGEMV_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int qgemv_version(void) { return 100; }

const char *qgemv_status_string(int status) {
    switch (status) {
        case QGEMV_OK: return "ok";
        case QGEMV_EINVAL: return "invalid argument (null pointer, shape, type or overlap)";
        case QGEMV_EALIGN: return "pointer not aligned as required";
        case QGEMV_EWORKSPACE: return "workspace missing or too small";
        case QGEMV_EHIP: return "HIP runtime error (see qgemv_last_error)";
        default: return "unknown status";
    }
}

const char *qgemv_last_error(void) { return g_last_error; }

size_t qgemv_weight_bytes(int wtype, int64_t rows, int64_t cols) {
    if (!shape_ok_t(wtype, rows, cols, 1)) return 0;
    return weight_bytes(wtype, rows, cols);
}

int qgemv_quantize_act(const float *x, int8_t *xq, float *xd, int64_t cols, int32_t nvec,
                       hipStream_t stream) {
    if (!x || !xq || !xd || cols < 32 || cols % 32 != 0 || nvec < 1) return QGEMV_EINVAL;
    if (cols * static_cast<int64_t>(nvec) > (int64_t{1} << 34)) return QGEMV_EINVAL;
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(xd, 4)) return QGEMV_EALIGN;
    const size_t n = static_cast<size_t>(cols) * nvec;
    if (overlaps(xq, n, x, n * 4) || overlaps(xd, n / 8, x, n * 4) || overlaps(xq, n, xd, n / 8))
        return QGEMV_EINVAL;
    const hipError_t e = launch_quantize_act(x, xq, xd, static_cast<int64_t>(n / 32), stream);
    return e == hipSuccess ? QGEMV_OK : hip_fail(e);
}

size_t qgemv_workspace_bytes(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    if (i8_auto(wtype, rows, cols, nvec)) return i8_ws_bytes(make_i8_plan(rows, cols), rows, nvec);
    if (mc32_auto(wtype, rows, cols, nvec)) return mc32_route_ws_bytes(wtype, rows, cols, nvec);
    if (mc_shape_ok(wtype, rows, cols, nvec))
        return mc_ws_bytes(make_mc_plan(rows, cols, nvec), rows, cols, nvec);
    if (grouped_shape_ok(wtype, rows, cols, nvec)) {
        // groups of up to kMaxVec vectors, one after another on the stream, share the
        // workspace: the largest of the full groups' and the last, smaller group's (whose plan
        // may split the columns where the full groups' does not)
        const int32_t rest = nvec % kMaxVec;
        size_t need = plan_ws_bytes(make_plan(wtype, rows, cols, kMaxVec), rows, cols, kMaxVec);
        if (rest > 0)
            need = std::max(need, plan_ws_bytes(make_plan(wtype, rows, cols, rest), rows, cols, rest));
        return need;
    }
    if (!shape_ok_t(wtype, rows, cols, nvec)) return 0;
    return plan_ws_bytes(make_plan(wtype, rows, cols, nvec), rows, cols, nvec);
}

int qgemv_plan_for(int wtype, int64_t rows, int64_t cols, int32_t nvec, qgemv_plan *plan) {
    if (!plan || !shape_ok_t(wtype, rows, cols, nvec))
        return QGEMV_EINVAL;
    *plan = make_plan(wtype, rows, cols, nvec);
    return QGEMV_OK;
}

size_t qgemv_plan_workspace_bytes(const qgemv_plan *plan, int64_t rows, int64_t cols,
                                  int32_t nvec) {
    if (!plan || !shape_ok(rows, cols, nvec) || !plan_ok(*plan, nvec)) return 0;
    return plan_ws_bytes(*plan, rows, cols, nvec);
}

int qgemv_batch_plan(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                     int64_t rows, int64_t cols, int32_t nvec, const qgemv_plan *plan,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!plan) return QGEMV_EINVAL;
    Activation act;
    act.xq = xq;
    act.xd = xd;
    return run_gemv(wtype, w, act, y, rows, cols, nvec, *plan, workspace, workspace_bytes, stream);
}

int qgemv_fused_plan(int wtype, const void *w, const float *x, int8_t *xq_out, float *xd_out,
                     float *y, int64_t rows, int64_t cols, int32_t nvec, const qgemv_plan *plan,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!plan) return QGEMV_EINVAL;
    Activation act;
    act.x = x;
    act.xq_out = xq_out;
    act.xd_out = xd_out;
    return run_gemv(wtype, w, act, y, rows, cols, nvec, *plan, workspace, workspace_bytes, stream);
}

int qgemv_batch(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                int64_t rows, int64_t cols, int32_t nvec, void *workspace,
                size_t workspace_bytes, hipStream_t stream) {
    if (i8_auto(wtype, rows, cols, nvec)) {
        Activation act;
        act.xq = xq;
        act.xd = xd;
        return run_i8(w, act, y, nullptr, nullptr, rows, cols, nvec, workspace, workspace_bytes,
                      stream);
    }
    if (mc_shape_ok(wtype, rows, cols, nvec))
        return run_mc(w, xq, xd, y, nullptr, nullptr, rows, cols, nvec, workspace,
                      workspace_bytes, stream);
    if (mc32_auto(wtype, rows, cols, nvec))
        return run_mc32(wtype, w, xq, xd, y, nullptr, nullptr, rows, cols, nvec, workspace,
                         workspace_bytes, stream);
    if (grouped_shape_ok(wtype, rows, cols, nvec)) {
        // the vector kernel on groups of up to kMaxVec vectors (each group one pass over the
        // weights); every argument is checked for the whole product before the first launch
        const size_t ybytes = static_cast<size_t>(nvec) * rows * sizeof(float);
        int st = check_gemv_args_n(wtype, w, xq, xd, y, ybytes, rows, cols, nvec);
        if (st != QGEMV_OK) return st;
        const size_t need = qgemv_workspace_bytes(wtype, rows, cols, nvec);
        if (need > 0) {
            if (!workspace || workspace_bytes < need) return QGEMV_EWORKSPACE;
            if (!aligned(workspace, 4)) return QGEMV_EALIGN;
            if (overlaps(workspace, need, w, weight_bytes(wtype, rows, cols)) ||
                overlaps(workspace, need, y, ybytes) ||
                overlaps(workspace, need, xq, static_cast<size_t>(nvec) * cols) ||
                overlaps(workspace, need, xd, static_cast<size_t>(nvec) * (cols / 32) * sizeof(float)))
                return QGEMV_EINVAL;
        }
        for (int32_t v0 = 0; v0 < nvec; v0 += kMaxVec) {
            const int32_t g = std::min<int32_t>(kMaxVec, nvec - v0);
            Activation act;
            act.xq = xq + static_cast<int64_t>(v0) * cols;
            act.xd = xd + static_cast<int64_t>(v0) * (cols / 32);
            st = run_gemv(wtype, w, act, y + static_cast<int64_t>(v0) * rows, rows, cols, g,
                          make_plan(wtype, rows, cols, g), workspace, workspace_bytes, stream);
            if (st != QGEMV_OK) return st;
        }
        return QGEMV_OK;
    }
    if (!shape_ok_t(wtype, rows, cols, nvec))
        return QGEMV_EINVAL;
    Activation act;
    act.xq = xq;
    act.xd = xd;
    return run_gemv(wtype, w, act, y, rows, cols, nvec, make_plan(wtype, rows, cols, nvec),
                    workspace, workspace_bytes, stream);
}

int qgemv_batch_scratch(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                        int64_t rows, int64_t cols, int32_t nvec, hipStream_t stream) {
    if (qgemv_route(wtype, rows, cols, nvec) == 0 || !w || !xq || !xd || !y) return QGEMV_EINVAL;
    const size_t need = qgemv_workspace_bytes(wtype, rows, cols, nvec);
    if (need > kScratchBytes)
        return fail_with(QGEMV_EWORKSPACE, "the shape needs more workspace than the static scratch");
    void *ws = nullptr;
    const int st = scratch_address(&ws);
    if (st != QGEMV_OK) return st;
    return qgemv_batch(wtype, w, xq, xd, y, rows, cols, nvec, ws, kScratchBytes, stream);
}

int qgemv_fused_launches(int wtype, int64_t rows, int64_t cols, int32_t nvec, int with_outputs) {
    if (!shape_ok_t(wtype, rows, cols, nvec)) return 0;
    if (!with_outputs) return 1;
    // The integer matrix-core kernels: for Q4_K quantizing once (into the caller's code outputs)
    // and running the product from the codes was measured faster than every workgroup quantizing
    // the split's activation itself; the Q8_0 / Q4_0 few-vector kernel runs from codes only.
    if (i8_auto(wtype, rows, cols, nvec) || mc32_auto(wtype, rows, cols, nvec)) return 2;
    // Every workgroup of the fused kernel quantizes the whole activation slice its lanes read
    // (with the column split inside the workgroup: the whole row), blocks of 32 elements over
    // 4 lanes each. That costs more than a second launch (~1.9 us) past 32 elements per lane
    // (wide rows, several vectors), or when the workgroups together repeat it for more than 16K
    // elements per CU while the slice is over a tenth of a workgroup's share of the weight
    // bytes (many workgroups on a wide row that is not long enough to hide it): then, if the
    // caller gave places for the codes, the library quantizes once into them and runs the
    // product from them. Both forms give the same codes and the same y. Measured on MI355X, one
    // launch against two (elements per lane, per CU, slice over the share): 1536 x 6144 (12,
    // 4.6K, 0.22) 3.4 / 5.3 us; 8192 x 2048 x 8 vectors (32, 16K, 0.44) 7.6 / 8.2 us; 2048 x
    // 8192 x 2 vectors (32, 16K, 0.44) 6.0 / 6.5 us, Q6_K 7.2 / 7.1 us; 4096 x 8192 x 3 vectors,
    // split in two (48, 49K, 0.67) 11.7 / 9.2 us; 1536 x 6144 x 4 vectors, split in three (64)
    // 8.7 / 7.2 us; 16384 x 4096 x 2 vectors (16, 33K, 0.22) 14.7 / 14.2 us; 4096 x 16384, split
    // in two (32, 33K, 0.22) 10.6 / 10.6 us; 262144 x 1536 (6, 25K, 0.03) 34.7 / 36.3 us.
    const qgemv_plan plan = make_plan(wtype, rows, cols, nvec);
    // what each workgroup of the one-launch form quantizes, how many workgroups, how many lanes
    // (with the column split inside the workgroup, every workgroup quantizes the whole row)
    int64_t slice = static_cast<int64_t>(nvec) * plan.lanes_per_row * plan.chunks_per_lane * 32;
    int64_t lanes = 64 * static_cast<int64_t>(plan.waves_per_block);
    double wgs = static_cast<double>(plan.blocks) * plan.splits;
    if (plan.splits > 1) {
        const int maxw = gemv_max_waves(nvec, plan.lanes_per_row, plan.chunks_per_lane);
        const int wpb = split_waves_per_block(plan, maxw);
        if (plan.splits <= maxw &&
            gemv_split_lds_bytes(nvec, plan.lanes_per_row, plan.chunks_per_lane, true, plan.splits,
                                 wpb) <= kMaxSplitLds) {
            const int64_t waves = std::min<int64_t>(
                static_cast<int64_t>(plan.blocks) * plan.splits * plan.waves_per_block, 4096);
            slice = static_cast<int64_t>(nvec) * cols;
            lanes = 64 * static_cast<int64_t>(wpb);
            wgs = static_cast<double>((waves + wpb - 1) / wpb);
        }
    }
    if ((slice + lanes - 1) / lanes > 32) return 2;
    const double share = static_cast<double>(weight_bytes(wtype, rows, cols)) / wgs;
    return wgs * static_cast<double>(slice) / 256.0 > 16384.0 && slice > 0.1 * share ? 2 : 1;
}

int qgemv_fused(int wtype, const void *w, const float *x, int8_t *xq_out, float *xd_out, float *y,
                int64_t rows, int64_t cols, int32_t nvec, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
    if (!shape_ok_t(wtype, rows, cols, nvec))
        return QGEMV_EINVAL;
    const qgemv_plan plan = make_plan(wtype, rows, cols, nvec);
    Activation act;
    act.x = x;
    act.xq_out = xq_out;
    act.xd_out = xd_out;
    if (xq_out && xd_out && aligned(xq_out, 16) &&
        qgemv_fused_launches(wtype, rows, cols, nvec, 1) == 2) {
        int st = check_fused_act(act, w, weight_bytes(wtype, rows, cols), y,
                                 static_cast<size_t>(nvec) * rows * sizeof(float), cols, nvec);
        if (st != QGEMV_OK) return st;
        // the product's workspace is checked before the quantization goes out
        const size_t need = qgemv_workspace_bytes(wtype, rows, cols, nvec);
        if (need > 0 && (!workspace || workspace_bytes < need)) return QGEMV_EWORKSPACE;
        st = qgemv_quantize_act(x, xq_out, xd_out, cols, nvec, stream);
        if (st != QGEMV_OK) return st;
        Activation q;
        q.xq = xq_out;
        q.xd = xd_out;
        if (i8_auto(wtype, rows, cols, nvec))
            return run_i8(w, q, y, nullptr, nullptr, rows, cols, nvec, workspace, workspace_bytes,
                          stream);
        if (mc32_auto(wtype, rows, cols, nvec))
            return run_mc32(wtype, w, xq_out, xd_out, y, nullptr, nullptr, rows, cols, nvec,
                            workspace, workspace_bytes, stream);
        return run_gemv(wtype, w, q, y, rows, cols, nvec, plan, workspace, workspace_bytes, stream);
    }
    if (i8_auto(wtype, rows, cols, nvec))
        return run_i8(w, act, y, nullptr, nullptr, rows, cols, nvec, workspace, workspace_bytes,
                      stream);
    return run_gemv(wtype, w, act, y, rows, cols, nvec, plan, workspace, workspace_bytes, stream);
}

int qgemv_multi_geometry(int64_t cols, int32_t nvec, int32_t *lanes_per_row,
                         int32_t *chunks_per_lane) {
    int t = 0, nc = 0, splits = 1;
    if (!lanes_per_row || !chunks_per_lane || !shape_ok(1, cols, nvec) ||
        !multi_geometry(cols, nvec, t, nc, splits))
        return QGEMV_EINVAL;
    *lanes_per_row = t;
    *chunks_per_lane = nc;
    return QGEMV_OK;
}

int qgemv_multi(const qgemv_matrix *mats, int32_t nmats, const int8_t *xq, const float *xd,
                int64_t cols, int32_t nvec, hipStream_t stream) {
    Activation act;
    act.xq = xq;
    act.xd = xd;
    MultiArgs a;
    LaunchShape s;
    double wbytes = 0;
    const int st = prepare_multi(mats, nmats, act, cols, nvec, a, s, wbytes);
    return st != QGEMV_OK ? st : launch_multi(a, s, nvec, stream);
}

int qgemv_multi_fused(const qgemv_matrix *mats, int32_t nmats, const float *x, int8_t *xq_out,
                      float *xd_out, int64_t cols, int32_t nvec, hipStream_t stream) {
    if (!x) return QGEMV_EINVAL;
    Activation act;
    act.x = x;
    act.xq_out = xq_out;
    act.xd_out = xd_out;
    MultiArgs a;
    LaunchShape s;
    double wbytes = 0;
    int st = prepare_multi(mats, nmats, act, cols, nvec, a, s, wbytes);
    if (st != QGEMV_OK) return st;
    // As for one matrix: with code outputs (16-byte aligned, as the product reads them) and a
    // slice that is large next to a workgroup's share of the weights, quantize once and run
    // the product from the codes. A split row whose chunks' slices do not all fit in LDS
    // needs the codes.
    const double slice = static_cast<double>(nvec) * s.lanes * s.chunks * 32 * s.splits;
    const bool fits = s.splits == 1 || gemv_split_lds_bytes(nvec, s.lanes, s.chunks, true, s.splits,
                                                            s.waves) <= kMaxSplitLds;
    if (!fits && !(xq_out && aligned(xq_out, 16)))
        return fail_with(QGEMV_EINVAL, "the row's activation slices do not fit in LDS: pass 16-byte "
                                       "aligned code outputs");
    if (!fits || (xq_out && aligned(xq_out, 16) && slice > 0.15 * wbytes / s.blocks)) {
        st = qgemv_quantize_act(x, xq_out, xd_out, cols, nvec, stream);
        if (st != QGEMV_OK) return st;
        a.act.x = nullptr;
        a.act.xq_out = nullptr;
        a.act.xd_out = nullptr;
        a.act.xq = xq_out;
        a.act.xd = xd_out;
    }
    return launch_multi(a, s, nvec, stream);
}

int qgemv_route(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    if (i8_auto(wtype, rows, cols, nvec)) return QGEMV_ROUTE_I8MC;
    if (mc_shape_ok(wtype, rows, cols, nvec)) return QGEMV_ROUTE_MC;
    if (mc32_auto(wtype, rows, cols, nvec)) return QGEMV_ROUTE_MC32;
    if (grouped_shape_ok(wtype, rows, cols, nvec)) return QGEMV_ROUTE_GROUPED;
    if (shape_ok_t(wtype, rows, cols, nvec)) return QGEMV_ROUTE_VECTOR;
    return 0;
}

size_t qgemv_i8mc_workspace_bytes(int64_t rows, int64_t cols, int32_t nvec) {
    if (!i8_ok(rows, cols, nvec)) return 0;
    return i8_ws_bytes(make_i8_plan(rows, cols), rows, nvec);
}

int qgemv_batch_i8mc(const void *w, const int8_t *xq, const float *xd, float *y, int64_t rows,
                     int64_t cols, int32_t nvec, void *workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    Activation act;
    act.xq = xq;
    act.xd = xd;
    return run_i8(w, act, y, nullptr, nullptr, rows, cols, nvec, workspace, workspace_bytes,
                  stream);
}

size_t qgemv_mc32_workspace_bytes(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    if (!mc32_ok(wtype, rows, cols, nvec)) return 0;
    return mc32_route_ws_bytes(wtype, rows, cols, nvec);
}

int qgemv_batch_mc32(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                     int64_t rows, int64_t cols, int32_t nvec, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    return run_mc32(wtype, w, xq, xd, y, nullptr, nullptr, rows, cols, nvec, workspace,
                    workspace_bytes, stream);
}

int qgemv_debug_partials_i8mc(const void *w, const int8_t *xq, const float *xd, int32_t *P,
                              int32_t *S, int64_t rows, int64_t cols, int32_t nvec,
                              hipStream_t stream) {
    if (!P || !S) return QGEMV_EINVAL;
    Activation act;
    act.xq = xq;
    act.xd = xd;
    return run_i8(w, act, nullptr, P, S, rows, cols, nvec, nullptr, 0, stream);
}

int qgemv_mc32_tile(int wtype, int64_t rows, int64_t cols, int32_t nvec) {
    if (!mc32_ok(wtype, rows, cols, nvec)) return 0;
    return mc32_few_kernel(wtype, rows, cols, nvec) ? 16 : 32;
}

int qgemv_debug_partials_mc32(int wtype, const void *w, const int8_t *xq, const float *xd,
                              int32_t *P, int32_t *S, int64_t rows, int64_t cols, int32_t nvec,
                              hipStream_t stream) {
    if (!P || !S) return QGEMV_EINVAL;
    return run_mc32(wtype, w, xq, xd, nullptr, P, S, rows, cols, nvec, nullptr, 0, stream);
}

int qgemv_fused_i8mc(const void *w, const float *x, int8_t *xq_out, float *xd_out, float *y,
                     int64_t rows, int64_t cols, int32_t nvec, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    Activation act;
    act.x = x;
    act.xq_out = xq_out;
    act.xd_out = xd_out;
    return run_i8(w, act, y, nullptr, nullptr, rows, cols, nvec, workspace, workspace_bytes,
                  stream);
}

int qgemv_q4k(const void *w, const int8_t *xq, const float *xd, float *y, int64_t rows,
              int64_t cols, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return qgemv_batch(QGEMV_Q4K, w, xq, xd, y, rows, cols, 1, workspace, workspace_bytes, stream);
}

int qgemv_q6k(const void *w, const int8_t *xq, const float *xd, float *y, int64_t rows,
              int64_t cols, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return qgemv_batch(QGEMV_Q6K, w, xq, xd, y, rows, cols, 1, workspace, workspace_bytes, stream);
}

int qgemv_debug_partials(int wtype, const void *w, const int8_t *xq, const float *xd,
                         int32_t *P, int32_t *S, int64_t rows, int64_t cols, int32_t nvec,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!P || !S) return QGEMV_EINVAL;
    if (i8_auto(wtype, rows, cols, nvec)) {
        Activation act;
        act.xq = xq;
        act.xd = xd;
        return run_i8(w, act, nullptr, P, S, rows, cols, nvec, nullptr, 0, stream);
    }
    if (mc_shape_ok(wtype, rows, cols, nvec)) {
        const size_t pbytes = static_cast<size_t>(nvec) * rows * (cols / 32) * sizeof(int32_t);
        const size_t sbytes = static_cast<size_t>(nvec) * (cols / 32) * sizeof(int32_t);
        if (!aligned(P, 4) || !aligned(S, 4)) return QGEMV_EALIGN;
        const size_t wb = weight_bytes(wtype, rows, cols);
        const size_t qb = static_cast<size_t>(nvec) * cols;
        const size_t db = static_cast<size_t>(nvec) * (cols / 32) * sizeof(float);
        if (overlaps(P, pbytes, S, sbytes) || overlaps(P, pbytes, w, wb) ||
            overlaps(P, pbytes, xq, qb) || overlaps(P, pbytes, xd, db) ||
            overlaps(S, sbytes, w, wb) || overlaps(S, sbytes, xq, qb) || overlaps(S, sbytes, xd, db))
            return QGEMV_EINVAL;
        return run_mc(w, xq, xd, nullptr, P, S, rows, cols, nvec, workspace, workspace_bytes,
                      stream);
    }
    if (nvec > kMaxVec ? mc32_ok(wtype, rows, cols, nvec) : mc32_auto(wtype, rows, cols, nvec))
        return run_mc32(wtype, w, xq, xd, nullptr, P, S, rows, cols, nvec, nullptr, 0, stream);
    const int64_t nsub = wtype == QGEMV_Q6K ? cols / 16 : cols / 32;
    const size_t pbytes = static_cast<size_t>(nvec) * rows * nsub * sizeof(int32_t);
    int st = check_gemv_args(wtype, w, xq, xd, P, pbytes, rows, cols, nvec);
    if (st != QGEMV_OK) return st;
    const size_t sbytes = static_cast<size_t>(nvec) * (cols / 32) * sizeof(int32_t);
    if (!aligned(S, 4)) return QGEMV_EALIGN;
    if (overlaps(S, sbytes, P, pbytes) || overlaps(S, sbytes, w, weight_bytes(wtype, rows, cols)) ||
        overlaps(S, sbytes, xq, static_cast<size_t>(nvec) * cols))
        return QGEMV_EINVAL;
    // The production plan's kernel instance with the debug stores on; it writes no y.
    qgemv_plan plan = make_plan(wtype, rows, cols, nvec);
    GemvArgs a{};
    a.w = static_cast<const uint8_t *>(w);
    a.xq = xq;
    a.xd = xd;
    a.out = nullptr;
    a.P = P;
    a.S = S;
    a.rows = static_cast<int32_t>(rows);
    a.nb = static_cast<int32_t>(cols / block_cols(wtype));
    a.nchunks = static_cast<int32_t>(cols / 32);
    LaunchShape s{plan.lanes_per_row, plan.chunks_per_lane, plan.waves_per_block, plan.blocks,
                  splits_for(plan.lanes_per_row, plan.chunks_per_lane, cols)};
    const hipError_t e = launch_gemv(wtype, a, s, nvec, true, stream);
    return e == hipSuccess ? QGEMV_OK : hip_fail(e);
}

int qgemv_quantize_weights_rows(int wtype, const float *w, void *out, int64_t rows,
                                int64_t cols, int64_t row0, int64_t nrows, hipStream_t stream) {
    if (!w || !out || !shape_ok_t(wtype, rows, cols, 1) || row0 < 0 || nrows < 1 ||
        row0 > rows - nrows)
        return QGEMV_EINVAL;
    if (!aligned(w, 16) || !aligned(out, 16)) return QGEMV_EALIGN;
    const size_t ob = weight_bytes(wtype, rows, cols);
    if (overlaps(out, ob, w, static_cast<size_t>(nrows) * cols * sizeof(float))) return QGEMV_EINVAL;
    uint8_t *o = static_cast<uint8_t *>(out);
    hipError_t e = hipErrorInvalidValue;
    switch (wtype) {
        case QGEMV_Q4K: e = launch_quantize_q4k(w, o, rows, cols, row0, nrows, stream); break;
        case QGEMV_Q6K: e = launch_quantize_q6k(w, o, rows, cols, row0, nrows, stream); break;
        case QGEMV_Q4_0: e = launch_quantize_q40(w, o, rows, cols, row0, nrows, stream); break;
        case QGEMV_Q8_0: e = launch_quantize_q80(w, o, rows, cols, row0, nrows, stream); break;
        default: break;
    }
    return e == hipSuccess ? QGEMV_OK : hip_fail(e);
}

int qgemv_quantize_weights(int wtype, const float *w, void *out, int64_t rows, int64_t cols,
                           hipStream_t stream) {
    return qgemv_quantize_weights_rows(wtype, w, out, rows, cols, 0, rows, stream);
}

int qgemv_read_probe(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks,
                     hipStream_t stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20))
        return QGEMV_EINVAL;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return QGEMV_EALIGN;
    if (overlaps(sink, 4, buf, bytes)) return QGEMV_EINVAL;
    const hipError_t e =
        launch_read_probe(buf, static_cast<int64_t>(bytes), sink, blocks, stream);
    return e == hipSuccess ? QGEMV_OK : hip_fail(e);
}

}  // extern "C"
