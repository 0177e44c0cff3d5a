/*
 * qgemv — block-quantized weight x int8-activation matrix-vector products for
 * AMD Instinct MI355X (gfx950). C ABI.
 *
 * The operation is the decode-time product y = W x of a large language model:
 * one token per pass, so every weight byte is read once per product and the
 * product is bound by HBM bandwidth (oxinfer README, "Performance"; the
 * genie-ai-runtime post, "The decode arc"). W is stored in 256-weight
 * super-blocks, x is quantized to int8 codes in blocks of 32 with one float32
 * scale each (oxinfer README, "Build and run", --quant q8; "How it works",
 * quant.rs: per-matmul activation quantization). The product is formed from
 * exact int32 dot products of weight codes with activation codes per
 * sub-block, which are then scaled and summed in float32 (genie-ai-runtime,
 * "The decode arc": int8 dot products for Q4_K and Q6_K instead of
 * dequantizing to floating point; "v1.2.0": one q8_1 activation shared by
 * several products).
 *
 * Formats (all multi-byte fields little-endian):
 *
 *  A super-block covers 256 consecutive weights of a row; block i of a
 *  tensor is block b of row r with i = r * cols/256 + b, and N = rows *
 *  cols/256 is the number of blocks. Each field of a block lives in a plane of
 *  its own, in block order, so that every plane is read with aligned,
 *  contiguous loads.
 *
 *  Q4_K tensor (144 bytes per block): codes plane [0, 128 N), header plane
 *  [128 N, 144 N). Sub-block j (j = 0..7) is weights 32j .. 32j+31.
 *    header of block i, at 128 N + 16 i:
 *      [0,2)    d     fp16 super-scale of the sub-scales
 *      [2,4)    dmin  fp16 super-scale of the sub-mins
 *      [4,8)    low 4 bits of sc_j at byte 4 + j/2, bit 4*(j%2)
 *      [8,12)   low 4 bits of m_j  at byte 8 + j/2, bit 4*(j%2)
 *      [12,14)  high 2 bits of sc_j at byte 12 + j/4, bit 2*(j%4)
 *      [14,16)  high 2 bits of m_j  at byte 14 + j/4, bit 2*(j%4)
 *    codes of block i, at 128 i: weight 32j + 16h + t (h = 0,1; t < 16) is
 *      the low (h = 0) or high (h = 1) nibble of byte 16j + t
 *    weight = d * sc_j * q - dmin * m_j
 *
 *  Q6_K tensor (210 bytes per block): low-bit plane [0, 128 N), high-bit
 *  plane [128 N, 192 N), sub-scale plane [192 N, 208 N), super-scale plane
 *  [208 N, 210 N). Sub-block j (j = 0..15) is weights 16j .. 16j+15.
 *    low bits of block i, at 128 i: weight 32k + 16g + t (k < 8, g = 0,1,
 *      t < 16) is nibble g of byte 16k + t
 *    high bits of block i, at 128 N + 64 i: weight 32k + 16g + 4s + c
 *      (s, c < 4) is bits 2s .. 2s+1 of byte 8k + 4g + c
 *    sub-scales of block i, at 192 N + 16 i: sc_j, signed int8, at byte j
 *    d of block i: fp16 at 208 N + 2 i
 *    weight = d * sc_j * (q - 32), q in [0, 63]
 *
 *  The 32-weight formats (oxinfer README, "Build and run": --quant q4 is
 *  GGUF-style Q4_0, --quant q8 int8 blocks of 32 with f32 scales;
 *  "Pre-quantized checkpoints": codes and scales in separate tensors). Block i
 *  = block b of row r with i = r * cols/32 + b; N = rows * cols/32.
 *  Q4_0 tensor (18 bytes per block): codes plane [0, 16 N), scale plane
 *  [16 N, 18 N).
 *    codes of block i, at 16 i: weight t (t < 32) is the low (t < 16) or high
 *      (t >= 16) nibble of byte t mod 16
 *    d of block i: fp16 at 16 N + 2 i
 *    weight = d * (q - 8), q in [0, 15]
 *  Q8_0 tensor (36 bytes per block): two codes planes [0, 16 N) and
 *  [16 N, 32 N), scale plane [32 N, 36 N).
 *    codes of block i: weight t < 16 is the int8 at byte 16 i + t, weight
 *      t >= 16 the int8 at byte 16 N + 16 i + (t - 16)
 *    d of block i: float32 at 32 N + 4 i
 *    weight = d * q, q in [-127, 127]
 *
 *  Activations: codes xq int8 [nvec][cols] in [-127, 127] and scales xd
 *  float32 [nvec][cols/32]; element i of vector v stands for
 *  xd[v][i/32] * xq[v][i].
 *
 *  Output: y float32 [nvec][rows].
 *
 * Conventions for every entry point:
 *  - All data pointers are device pointers owned by the caller. The library
 *    allocates and frees nothing and never synchronizes; work is enqueued on
 *    `stream` (0 = the null stream) and runs asynchronously.
 *  - Arguments are checked on the host before anything is enqueued; on a
 *    failed check nothing is launched and an error status is returned.
 *    Launch failures return QGEMV_EHIP with the HIP message available from
 *    qgemv_last_error() (per thread). Faults inside a kernel surface at the
 *    caller's next synchronization.
 *  - Shapes: cols a positive multiple of 256 (Q4_K, Q6_K) or of 32 (Q4_0,
 *    Q8_0), 1 <= rows <= 2^30, 1 <= nvec <= 8, rows * cols / 32 < 2^31;
 *    qgemv_batch and qgemv_workspace_bytes also take 9 <= nvec <=
 *    QGEMV_MAX_BATCH vectors (Q4_K: the matrix-core paths), and so does
 *    qgemv_debug_partials for Q4_K; the qgemv_*_i8mc functions take
 *    1 <= nvec <= 16.
 *  - Alignment: w and xq 16 bytes, xd and y 4 bytes.
 *  - Outputs must not overlap inputs.
 *  - The functions are safe to call from several host threads.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum qgemv_status {
    QGEMV_OK = 0,
    QGEMV_EINVAL = 1,       /* null pointer, bad shape, bad type, overlapping buffers */
    QGEMV_EALIGN = 2,       /* pointer not aligned as required */
    QGEMV_EWORKSPACE = 3,   /* workspace smaller than qgemv_workspace_bytes() */
    QGEMV_EHIP = 4          /* the HIP runtime refused a launch */
};

enum qgemv_wtype {
    QGEMV_Q4K = 1,
    QGEMV_Q6K = 2,
    QGEMV_Q4_0 = 3,
    QGEMV_Q8_0 = 4
};

#define QGEMV_MAX_NVEC 8
#define QGEMV_MAX_BATCH 256

/* Library version, major * 10000 + minor * 100 + patch. */
int qgemv_version(void);

/* Static text for a status code. */
const char *qgemv_status_string(int status);

/* Text of the last HIP error seen by this thread, or of the reason of the last
 * refusal of a qgemv_graph_* call ("" if none). */
const char *qgemv_last_error(void);

/* Bytes of a weight tensor of the given type and shape (0 on a bad shape). */
size_t qgemv_weight_bytes(int wtype, int64_t rows, int64_t cols);

/*
 * Activation quantization (oxinfer README, "How it works": per-matmul
 * activation quantization; "Build and run": blocks of 32, f32 scales).
 * x float32 [nvec][cols] -> xq int8 [nvec][cols], xd float32 [nvec][cols/32].
 * Per block of 32: amax = max |x|, xd = amax / 127 (IEEE float32 division),
 * inverse 127 / amax (0 when that is not a finite float32: amax = 0, or amax
 * below 127 / FLT_MAX, about 3.7e-37), code = rint(x * inverse) with one
 * float32 multiply and round-to-nearest-even, clamped to [-127, 127].
 * Here cols only needs to be a positive multiple of 32. x 16-byte aligned,
 * xq 4-byte aligned, xd 4-byte aligned. Inputs must be finite.
 */
int qgemv_quantize_act(const float *x, int8_t *xq, float *xd, int64_t cols, int32_t nvec,
                       hipStream_t stream);

/*
 * Workspace needed by qgemv_q4k / qgemv_q6k / qgemv_batch for this shape, in
 * bytes; 0 when the chosen plan does not split the columns. The planner splits
 * the columns into S chunks of whole blocks when a row is wider than one pass
 * or rows alone cannot fill the GPU (genie-ai-runtime "v1.3.0": split-K, chosen
 * per shape). The S partial results per output are always added in ascending
 * chunk order, without atomics: from codes (S no larger than a workgroup's
 * waves) by the waves of one workgroup, through LDS, in the same launch;
 * otherwise (the one-launch fused form, larger S) through the workspace and a
 * second launch. The two give the same y bit for bit; the workspace is
 * required whenever this returns more than 0.
 */
size_t qgemv_workspace_bytes(int wtype, int64_t rows, int64_t cols, int32_t nvec);

/*
 * y = W x for one activation vector, W in Q4_K (genie-ai-runtime, "The decode
 * arc": int8 dot-product mat-vec for Q4_K). Per sub-block j of a super-block:
 * P = sum of q * xq over its 32 columns (exact int32), S = sum of xq over the
 * same 32 columns, and the term xd * (d * sc_j * P - dmin * m_j * S) is added
 * to y in float32. w: Q4_K tensor [rows][cols]; xq, xd: one quantized vector;
 * y: [rows]. workspace may be NULL when qgemv_workspace_bytes() is 0.
 */
int qgemv_q4k(const void *w, const int8_t *xq, const float *xd, float *y, int64_t rows,
              int64_t cols, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * y = W x for one activation vector, W in Q6_K (genie-ai-runtime, "The decode
 * arc": int8 dot-product mat-vec for Q6_K). Per sub-block j of 16 columns:
 * P = sum of (q - 32) * xq (exact int32) and the term xd * d * sc_j * P is
 * added to y in float32. Arguments as for qgemv_q4k.
 */
int qgemv_q6k(const void *w, const int8_t *xq, const float *xd, float *y, int64_t rows,
              int64_t cols, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same product for nvec = 1..8 activation vectors sharing one pass over
 * the weights (several sequences decoded together; oxinfer README, "How it
 * works": multi-token int8 decode variants). xq [nvec][cols],
 * xd [nvec][cols/32], y [nvec][rows]. wtype is one of enum qgemv_wtype.
 *
 * Q4_K with 9 <= nvec <= QGEMV_MAX_BATCH (many tokens verified or prefilled
 * at once; oxinfer README, "Speculative decoding": the many-token int8
 * variants are instruction-bound at Q4) runs on the matrix cores: 9..16
 * vectors on the integer matrix cores (qgemv_batch_i8mc below), 17 and more
 * on the float matrix cores. Both form the same exact integer sub-block
 * products P and sums S, then the same float32 scaling, so y lies within the
 * same bound of the exact product; the float path's workspace
 * (qgemv_workspace_bytes) holds the staged activation and, for matrices with
 * few rows, partial sums. Q8_0, Q4_0 and Q6_K with 9 <= nvec <= QGEMV_MAX_BATCH
 * run on the integer matrix cores too where qgemv_route says QGEMV_ROUTE_MC32
 * (qgemv_batch_mc32 below), one pass over the weights; their workspace holds
 * partial sums of column splits when the matrix has few rows. Elsewhere
 * (QGEMV_ROUTE_GROUPED) they run the vector kernels on groups of up to 8
 * vectors, one after another on the stream (one pass over the weights per
 * group; the workspace is that of 8 vectors, shared by the groups). Q4_0, Q6_K
 * and Q8_0 with 3..8 vectors on large tensors also take the integer matrix cores
 * (QGEMV_ROUTE_MC32; qgemv_route gives the sizes).
 */
int qgemv_batch(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                int64_t rows, int64_t cols, int32_t nvec, void *workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * qgemv_batch for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels
 * with the same results, bit for bit, but the workspace is the library's static
 * device scratch buffer of QGEMV_SCRATCH_BYTES, so the caller passes only inputs and
 * outputs. Shapes whose qgemv_workspace_bytes() exceeds QGEMV_SCRATCH_BYTES are
 * refused with QGEMV_EWORKSPACE before anything is enqueued. The call allocates and
 * frees nothing. Each GPU holds its own copy of the buffer from the library's first
 * launch on it until the process ends; the first call on a device looks up its
 * address there (once, host only), so under graph capture make one call on each
 * device before capturing. stream must belong to the current device. Every call on
 * one GPU shares that GPU's buffer and it keeps the last call's contents (nothing in
 * it needs to start at zero): calls that can overlap on one GPU (several streams,
 * several host threads) race and must be ordered by the caller.
 */
#define QGEMV_SCRATCH_BYTES (32u << 20)
int qgemv_batch_scratch(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                        int64_t rows, int64_t cols, int32_t nvec, hipStream_t stream);

/* Which kernels qgemv_batch (and qgemv_fused, qgemv_debug_partials) run for a
 * shape: the vector kernels, the integer matrix cores (qgemv_batch_i8mc), the
 * float matrix cores for 17..QGEMV_MAX_BATCH Q4_K vectors, the integer matrix
 * cores for 9..QGEMV_MAX_BATCH Q8_0, Q4_0 or Q6_K vectors (qgemv_batch_mc32;
 * QGEMV_ROUTE_MC32) with 9..16 vectors on tensors of at least 16 Mi weights, from
 * 32 vectors, from 16 vectors on tensors of at least 24 Mi weights and from 9
 * vectors on at least 48 Mi weights, or else for those formats the vector
 * kernels on groups of 8 vectors (QGEMV_ROUTE_GROUPED: on a small tensor they
 * stay ahead of the matrix-core path's 16-20 us floor until the groups are
 * many); Q4_K with 9..12 vectors on tensors of 16 Mi weights to 128 MiB there
 * too (QGEMV_ROUTE_MC32), else with 9..16 on its own integer kernel
 * (QGEMV_ROUTE_I8MC); with 1..8 vectors the integer matrix cores
 * (QGEMV_ROUTE_MC32) where the vector kernel's dot products bind, on rows of up
 * to 2048 columns: Q4_0 from 4 vectors on tensors of at least 32 Mi weights (3
 * from 256 Mi; 8 on wider rows), Q6_K from 4 vectors on 256 Mi weights and with
 * 8 from 64 Mi, Q8_0 with 8 vectors from 256 Mi, and Q4_K with 4 vectors on
 * tensors of 16 to 96 MiB (below QGEMV_ROUTE_I8MC's sizes); 0 for an invalid
 * type or shape. Host only. */
enum qgemv_route_kind {
    QGEMV_ROUTE_VECTOR = 1,
    QGEMV_ROUTE_I8MC = 2,
    QGEMV_ROUTE_MC = 3,
    QGEMV_ROUTE_GROUPED = 4,
    QGEMV_ROUTE_MC32 = 5
};
int qgemv_route(int wtype, int64_t rows, int64_t cols, int32_t nvec);

/*
 * Q8_0, Q4_0 or Q6_K with 1 <= nvec <= QGEMV_MAX_BATCH, and Q4_K with
 * 1 <= nvec <= 16, on the integer matrix cores, for any shape (qgemv_batch takes it
 * where QGEMV_ROUTE_MC32 says; oxinfer README, "Speculative decoding": the
 * multi-token int8 variants). With 17 or more vectors, and with 9..16 on tensors
 * of fewer than 16 Mi weights (and Q8_0 with 9..15 vectors on 48 to 256 Mi), one
 * product is 32 weight rows x 32 vectors over one 32-weight block (Q8_0: the
 * stored codes; Q4_0: the codes 0..15, then P = sum q * xq - 8 S in integer) or
 * over one 16-weight Q6_K sub-block (the operand q - 32); otherwise (1..16
 * vectors) one product is 16 weight rows x 4 blocks x 4 vectors over one
 * 16-weight half of each block
 * (v_mfma_i32_16x16x64_i8; for Q8_0, Q4_0 and Q4_K two accumulate into a block's
 * P, Q4_0's starting from -8 S; for Q6_K each half is a sub-block, the operand
 * q - 32). Either way the int32 result is the exact integer partial P of
 * qgemv_debug_partials for every (row, vector); then y is sum over blocks of
 * (d * xd) * P (Q6_K: xd * (sc0 * P0 + sc1 * P1) per block, the integer
 * combination exact, times d per half super-block; Q4_K: d * xd * (sc * P) and
 * the min term -dmin * m * xd * S) in float32, within the same
 * bound as the vector kernels' y. Arguments as for qgemv_batch; the workspace
 * (qgemv_mc32_workspace_bytes: partial sums when the columns are split: by the
 * 32 x 32 x 32 kernels because row tiles and vector groups give fewer than 512
 * workgroups, by the 16 x 16 x 64 kernel for rows wider than 2048 columns) may
 * be NULL when that is 0.
 */
size_t qgemv_mc32_workspace_bytes(int wtype, int64_t rows, int64_t cols, int32_t nvec);
int qgemv_batch_mc32(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                     int64_t rows, int64_t cols, int32_t nvec, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Which kernel qgemv_batch_mc32 runs for a shape: 16 for the 16 x 16 x 64 one (1..16
 * vectors), 32 for the 32 x 32 x 32 ones; 0 when it does not take the shape. Host only. */
int qgemv_mc32_tile(int wtype, int64_t rows, int64_t cols, int32_t nvec);

/* Tests only: the integer partials P [nvec][rows][cols/32] (Q6_K: [cols/16]) and
 * block sums S [nvec][cols/32] of qgemv_batch_mc32's kernels for any shape it
 * takes, as qgemv_debug_partials writes them; no y, no workspace. */
int qgemv_debug_partials_mc32(int wtype, const void *w, const int8_t *xq, const float *xd,
                              int32_t *P, int32_t *S, int64_t rows, int64_t cols, int32_t nvec,
                              hipStream_t stream);

/*
 * Q4_K with 1 <= nvec <= 16 on the integer matrix cores (v_mfma_i32_16x16x64_i8;
 * two groups of 8 vectors share each loaded weight from 9 vectors on), for any shape; qgemv_batch, qgemv_fused and qgemv_debug_partials take this path
 * by themselves where it was measured faster than the other kernels: tensors of at
 * least 128, 96, 48, 32, 24 and 16 MiB for 3, 4, 5, 6, 7 and 8 vectors (there the
 * vector kernel's 4-way dot products, one per 4 codes and vector, are the
 * bottleneck; qgemv_fused with code outputs then quantizes once and runs this path
 * from the codes), and every Q4_K product with 9..16 vectors.
 * The same exact integer sub-block products P = sum q * xq (the product's int32
 * results as they are), S = sum xq, then per block the float32 term
 * xd * (sc * P) (sc * P exact) summed over the super-block and scaled by d, and the
 * min terms dmin * m * (-xd * S) on the float32 matrix cores: y lies within the
 * same bound of the exact product as the vector kernel's, with other rounding.
 * Arguments as for qgemv_batch with wtype QGEMV_Q4K; the workspace
 * (qgemv_i8mc_workspace_bytes: 0 unless cols > 2048, then partial sums of
 * column splits of up to 2048 columns) may be NULL when that is 0.
 */
size_t qgemv_i8mc_workspace_bytes(int64_t rows, int64_t cols, int32_t nvec);
int qgemv_batch_i8mc(const void *w, const int8_t *xq, const float *xd, float *y, int64_t rows,
                     int64_t cols, int32_t nvec, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* The same from the float32 activation x (16-byte aligned; 1 <= nvec <= 8),
 * quantized inside the launch exactly as qgemv_quantize_act does (bit for bit);
 * xq_out / xd_out (both NULL or both set, 4-byte aligned) optionally receive the
 * codes and scales. */
int qgemv_fused_i8mc(const void *w, const float *x, int8_t *xq_out, float *xd_out, float *y,
                     int64_t rows, int64_t cols, int32_t nvec, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Tests only: the integer partials P [nvec][rows][cols/32] and block sums
 * S [nvec][cols/32] of this path, as qgemv_debug_partials writes them; no y, no
 * workspace. */
int qgemv_debug_partials_i8mc(const void *w, const int8_t *xq, const float *xd, int32_t *P,
                              int32_t *S, int64_t rows, int64_t cols, int32_t nvec,
                              hipStream_t stream);

/*
 * Activation quantization and the product in one launch: x float32 [nvec][cols]
 * is quantized exactly as qgemv_quantize_act does (the same codes and scales,
 * bit for bit) by each workgroup for the columns it reads, then y = W x as in
 * qgemv_batch. For the common decode step where one activation feeds one
 * matrix this saves the separate quantization launch (oxinfer README, "How it
 * works": per-matmul activation quantization). xq_out [nvec][cols] and xd_out
 * [nvec][cols/32] optionally receive the codes and scales (both NULL or both
 * set; 4-byte aligned). x 16-byte aligned. Other arguments as for qgemv_batch.
 * Each workgroup repeats the quantization of the columns it reads; when that
 * is large next to its share of the weights (wide rows, several vectors) and
 * xq_out / xd_out are given (xq_out 16-byte aligned), the library instead
 * quantizes once into them and runs the product from them (two launches,
 * identical results). So it does too for the shapes qgemv_batch runs on the
 * integer matrix cores (QGEMV_ROUTE_I8MC, QGEMV_ROUTE_MC32), whose y is then
 * qgemv_batch's; without code outputs those shapes run the one-launch vector
 * kernel (y within the same bound).
 */
int qgemv_fused(int wtype, const void *w, const float *x, int8_t *xq_out, float *xd_out, float *y,
                int64_t rows, int64_t cols, int32_t nvec, void *workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * How many kernel launches qgemv_fused makes for this shape: 1 (the one-launch
 * kernel) or 2 (qgemv_quantize_act, then the product); with_outputs says whether
 * xq_out / xd_out are given (without them it is always 1; with an xq_out that is
 * not 16-byte aligned it is 1 as well). 0 for an invalid type or shape. Host
 * only; no device work.
 */
int qgemv_fused_launches(int wtype, int64_t rows, int64_t cols, int32_t nvec, int with_outputs);

/*
 * Several matrices that multiply the same activation, in one launch
 * (genie-ai-runtime, "v1.2.0": the attention projections of a decode step share
 * one quantized activation). Every matrix has `cols` columns; formats may be
 * mixed. For each matrix m: y_m[v][r] = sum over columns of W_m[r][c] * x_v[c],
 * computed exactly as qgemv_batch does for W_m alone with the same lanes per row
 * and chunks per lane (so the integer partials are the same and y_m lies within
 * the same bound).
 *
 * mats: HOST array of nmats (1..QGEMV_MAX_MATRICES) descriptors, read during the
 * call only. Each: wtype (any of enum qgemv_wtype), reserved = 0, rows >= 1, w the
 * device planar tensor (16-byte aligned), y device float32 [nvec][rows]
 * (4-byte aligned; no y may overlap any weights, the activation or another y).
 * A row wider than one pass of lanes (8192 columns for 1-2 vectors, 4096 for
 * 3-4, 2048 for 5-8) is split into column chunks inside each workgroup, one
 * wave per chunk and the chunks' row sums added in LDS in ascending chunk
 * order (bit-identical to qgemv_batch_plan's split with the same geometry); at
 * most 8 chunks, so cols is at most 65536, 32768 and 16384 for those vector
 * counts (QGEMV_EINVAL beyond). No workspace.
 */
#define QGEMV_MAX_MATRICES 8
typedef struct qgemv_matrix {
    int32_t wtype;
    int32_t reserved;
    int64_t rows;
    const void *w;
    float *y;
} qgemv_matrix;

/* The lanes per row and chunks per lane a multi-matrix launch uses for this
 * row width: the fewest idle lanes among the geometries that cover a row in one
 * pass, more chunks per lane preferred; for a wider row, the one-matrix
 * planner's rule (fewest idle lanes with each further pass priced as 2% of the
 * lanes idle) among the geometries whose ceil(cols/32 / (lanes_per_row *
 * chunks_per_lane)) chunks are at most a workgroup's waves (8 when nvec *
 * lanes_per_row * chunks_per_lane >= 128, else 4). QGEMV_EINVAL when there is
 * none. Host only. */
int qgemv_multi_geometry(int64_t cols, int32_t nvec, int32_t *lanes_per_row,
                         int32_t *chunks_per_lane);

/* The product from codes and scales made by qgemv_quantize_act (xq 16-byte,
 * xd 4-byte aligned). */
int qgemv_multi(const qgemv_matrix *mats, int32_t nmats, const int8_t *xq, const float *xd,
                int64_t cols, int32_t nvec, hipStream_t stream);

/* The same from the float32 activation x (16-byte aligned) with the quantization
 * done inside, as qgemv_fused does for one matrix; xq_out / xd_out (both NULL or
 * both set, 4-byte aligned, overlapping no input) optionally receive the codes
 * and scales. With code outputs that are 16-byte aligned and an activation
 * slice that is large next to a workgroup's share of the weights, the library
 * quantizes once and runs qgemv_multi's kernel from them (two launches, the
 * same results). A split row's workgroup quantizes all of its chunks into LDS;
 * where those slices take more than 64 KiB (36 bytes per activation block per
 * chunk, e.g. 65536 columns x 1 vector, 16384 x 8) the code outputs are
 * required, 16-byte aligned, and the product runs from them (QGEMV_EINVAL
 * without them). */
int qgemv_multi_fused(const qgemv_matrix *mats, int32_t nmats, const float *x, int8_t *xq_out,
                      float *xd_out, int64_t cols, int32_t nvec, hipStream_t stream);

/*
 * Replay of a decode step (genie-ai-runtime, "v1.2.1": the per-token kernel
 * launches of a decode step captured once into a graph, then one graph launch
 * per token). Between qgemv_graph_begin and qgemv_graph_end on a stream, calls
 * of this library (and any other capturable work the caller enqueues on that
 * stream) are recorded, not run; qgemv_graph_end turns the record into a
 * graph that qgemv_graph_launch replays. A replay runs the recorded kernels
 * with the recorded arguments, in the recorded order, on the same buffers:
 * the caller writes each step's inputs into the captured buffers first. The
 * library's calls enqueue only kernels (no allocation, memset or
 * synchronization), so a recorded call behaves as the same call made
 * directly and its outputs are the same bit for bit.
 *
 * qgemv_graph_begin: stream must be a created stream (QGEMV_EINVAL for the
 * null stream or one already capturing). The capture is thread-local: on this
 * thread, a HIP call that cannot be recorded fails (and invalidates the
 * capture) instead of running outside the graph. A call that fails its
 * argument checks during the capture records nothing and leaves it valid.
 * qgemv_graph_end: ends the capture on the same stream and stores a new graph
 * in *graph (NULL on any error: QGEMV_EINVAL when the stream is not capturing
 * or the record holds a memset node, which this library refuses to replay;
 * QGEMV_EHIP when the runtime invalidated the capture or cannot instantiate
 * the graph). The capture ends in every case where the stream was capturing.
 * qgemv_graph_launch: enqueue one replay on `stream` (any stream, 0 = null
 * stream). Replays of one graph run one after another; a graph must not be
 * destroyed before its last replay has finished.
 * qgemv_graph_nodes: the recorded kernel launches and other nodes (copies,
 * event waits) of a graph.
 * qgemv_graph_destroy: free the graph (host call; NULL is accepted).
 * Graph creation and destruction allocate; a launch does not.
 */
typedef struct qgemv_graph qgemv_graph;
int qgemv_graph_begin(hipStream_t stream);
/* The check qgemv_graph_end makes of a record, on its node types alone (values of HIP's
 * hipGraphNodeType): QGEMV_EINVAL when one is a memset node (or on a null pointer), else
 * QGEMV_OK with the kernel nodes and the other nodes counted. Host only; no HIP call, so it
 * can be checked without a GPU and without ever recording a memset. */
int qgemv_graph_classify(const int32_t *types, int64_t n, int64_t *kernel_nodes,
                         int64_t *other_nodes);
int qgemv_graph_end(hipStream_t stream, qgemv_graph **graph);
int qgemv_graph_launch(const qgemv_graph *graph, hipStream_t stream);
int qgemv_graph_nodes(const qgemv_graph *graph, int64_t *kernel_nodes, int64_t *other_nodes);
int qgemv_graph_destroy(qgemv_graph *graph);

/*
 * Test hook: the exact integer partials of the same kernels (for Q4_K with
 * more than 8 vectors, of the matrix-core kernel, which needs the workspace of
 * qgemv_workspace_bytes(); elsewhere workspace may be NULL; Q8_0, Q4_0 and Q6_K
 * take 9..QGEMV_MAX_BATCH vectors here too, on the kernel of qgemv_batch_mc32,
 * whichever route qgemv_batch takes: every route forms the same exact integers).
 * For Q4_0 and Q8_0, P [nvec][rows][cols/32] is the block's sum of (q - 8) * xq
 * or q * xq.
 * P int32: Q4_K [nvec][rows][cols/32] (sum of q * xq per 32-column
 * sub-block), Q6_K [nvec][rows][cols/16] (sum of (q - 32) * xq per 16-column
 * sub-block). S int32 [nvec][cols/32]: sum of xq per activation block.
 * P and S 4-byte aligned. y is not written.
 */
int qgemv_debug_partials(int wtype, const void *w, const int8_t *xq, const float *xd,
                         int32_t *P, int32_t *S, int64_t rows, int64_t cols, int32_t nvec,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Load-time weight quantization, float32 [rows][cols] -> a tensor of any format
 * (oxinfer README, "How it works", quant.rs: weights are block-quantized when
 * the model is loaded). Not on the per-token path. Every decision is taken in
 * float32 with round-to-nearest-even:
 *  Q4_K, per sub-block of 32: lo = min(0, min w), hi = max w,
 *    s = (hi - lo) / 15, o = -lo; d = fp16(max s / 63), dmin = fp16(max o / 63);
 *    sc = clamp(rint(s / d), 0, 63), m = clamp(rint(o / dmin), 0, 63) (0 for a
 *    zero divisor); q = clamp(rint((w + dmin * m) / (d * sc)), 0, 15).
 *  Q6_K, per sub-block of 16: s = max |w| / 31; d = fp16(max s / 127);
 *    sc = clamp(rint(s / d), -128, 127); q = clamp(rint(w / (d * sc)), -32, 31) + 32
 *    (32 when sc = 0).
 *  Q4_0, per block of 32: m = the first weight of largest |w|; d = fp16(m / -8)
 *    (+0 for an all-zero block); q = clamp(rint(w / d) + 8, 0, 15) (8 when d = 0).
 *  Q8_0, per block of 32: the activation rule, d = amax / 127,
 *    q = clamp(rint(w * (127 / amax)), -127, 127) (0 when 127 / amax is not finite).
 * w 16-byte aligned, out 16-byte aligned with qgemv_weight_bytes() bytes.
 * Inputs must be finite and small enough for the fp16 super-scales.
 */
int qgemv_quantize_weights(int wtype, const float *w, void *out, int64_t rows, int64_t cols,
                           hipStream_t stream);

/*
 * The same quantization for rows [row0, row0 + nrows) of a rows x cols matrix, so
 * a large matrix can be loaded in pieces: w holds only those rows (float32
 * [nrows][cols], 16-byte aligned), out is the whole tensor (qgemv_weight_bytes(
 * wtype, rows, cols) bytes, 16-byte aligned) and only the bytes of those rows'
 * super-blocks are written, in every plane. The pieces of one matrix give the
 * same bytes as one call over all rows. QGEMV_EINVAL for an empty or
 * out-of-range row range.
 */
int qgemv_quantize_weights_rows(int wtype, const float *w, void *out, int64_t rows,
                                int64_t cols, int64_t row0, int64_t nrows, hipStream_t stream);

/*
 * Launch plan of the GEMV kernels. Each row is cut into 16-byte chunks of
 * weight codes (one 32-column activation block each); a group of
 * lanes_per_row lanes of a 64-lane wavefront shares a row, each lane taking
 * chunks_per_lane chunks, so one pass covers lanes_per_row * chunks_per_lane
 * chunks and the row is split into ceil(cols/32 / that) column chunks
 * ("splits"; > 1 needs a workspace, see qgemv_workspace_bytes). waves_per_block
 * wavefronts form a workgroup; blocks is the number of workgroups per column
 * chunk, each looping over row groups.
 */
typedef struct qgemv_plan {
    int32_t lanes_per_row;    /* 8, 16, 32 or 64 */
    int32_t chunks_per_lane;  /* 1 .. 4 */
    int32_t waves_per_block;  /* 1 .. 4; 1 .. 8 when nvec * lanes_per_row *
                                 chunks_per_lane >= 128 */
    int32_t blocks;           /* workgroups per column chunk, >= 1 */
    int32_t splits;           /* derived: column chunks (output of qgemv_plan_for) */
} qgemv_plan;

/* The plan the library uses for a shape (filled into *plan); nvec <= 8 only
 * (the matrix-core path for more vectors has no explicit plans). */
int qgemv_plan_for(int wtype, int64_t rows, int64_t cols, int32_t nvec, qgemv_plan *plan);

/* Workspace bytes for an explicit plan (0 when it does not split). */
size_t qgemv_plan_workspace_bytes(const qgemv_plan *plan, int64_t rows, int64_t cols,
                                  int32_t nvec);

/* qgemv_batch with an explicit plan (for tuning); splits is recomputed. */
int qgemv_batch_plan(int wtype, const void *w, const int8_t *xq, const float *xd, float *y,
                     int64_t rows, int64_t cols, int32_t nvec, const qgemv_plan *plan,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* qgemv_fused with an explicit plan (for tuning and tests): always the fused kernel,
 * each workgroup quantizing the columns it reads (xq_out / xd_out, both NULL or both
 * set, receive the codes and scales). A plan that splits the columns into at most a
 * workgroup's waves of chunks runs in one launch, the workgroup quantizing every chunk
 * into LDS and its waves' chunk sums added there, when those slices take at most
 * 64 KiB (36 bytes per activation block per chunk); otherwise each workgroup quantizes
 * its chunk, the partial sums go to the workspace (qgemv_plan_workspace_bytes, required
 * whenever the plan splits) and a second launch adds them. Either way the chunks are
 * added in ascending order, so y is bit-identical to qgemv_batch_plan with the same
 * plan on the codes of qgemv_quantize_act. */
int qgemv_fused_plan(int wtype, const void *w, const float *x, int8_t *xq_out, float *xd_out,
                     float *y, int64_t rows, int64_t cols, int32_t nvec, const qgemv_plan *plan,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Measurement: read `bytes` (a multiple of 16) of device memory once with 16-byte loads
 * and nothing else, on `blocks` workgroups of 256 threads (a grid-stride loop). Its rate
 * is the practical read ceiling the GEMV is compared with (oxinfer README, "Performance":
 * machine read bandwidth measured apart from the kernels). sink: one device uint32 that is
 * written only for an input whose XOR is a fixed unlikely value.
 */
int qgemv_read_probe(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
