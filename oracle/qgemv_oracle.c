/*
 * CPU oracle for the block-quantized weight x int8-activation GEMV y = W x.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library. The GPU library shares no code
 * with it: no headers, no helpers, no tables.
 *
 * It is written to be read against the sources, not to be fast: plain loops,
 * one element at a time, every weight code located by an index formula over the
 * byte layout (never by word masks), every integer partial in 64-bit with an
 * int32 range check, and the result y and its error bound in float64.
 *
 * Sources of the method (cited by page title and section):
 *  - genie-ai-runtime v1.1 -> v1.3.1 (jared-hpc.com), "The decode arc": the
 *    quantized matrix-vector product for Q4_K and Q6_K weights is done in int8
 *    with 4-way byte dot products instead of dequantizing to floating point;
 *    "v1.2.0": one int8 activation (q8_1) is shared by several such products.
 *  - oxinfer README (docs.rs), "How it works" (quant.rs): per-matmul activation
 *    quantization to int8; decode kernels take int8 dot products block by block.
 *    "Build and run" (--quant q8): activation blocks of 32 with one f32 scale.
 *  - The workload definitions: Q4_K = 256-weight super-blocks of 8 x 32, 6-bit
 *    sub-scales and sub-mins, fp16 d and dmin, 4-bit codes; Q6_K = 16 x 16,
 *    int8 sub-scales, fp16 d, 6-bit codes with offset -32; activations to int8
 *    blocks of 32 with an fp32 scale; exact int32 sub-block dot products, then
 *    scaling and reduction in floating point.
 *  - oxinfer README, "Build and run": --quant q4 is GGUF-style Q4_0 (blocks of
 *    32 weights, 4-bit codes, one fp16 scale), --quant q8 is int8 weights in
 *    blocks of 32 with one f32 scale; "Pre-quantized checkpoints": the codes
 *    (two nibbles per byte for Q4_0) and the scales are separate tensors.
 *
 * The pages fix neither byte layouts nor rounding rules. The readings taken
 * here (byte layouts, quantizer steps, round-to-nearest-even everywhere) are
 * listed with their reasons in the design notes; the layouts are restated in
 * the comments of the pack/unpack functions below.
 *
 * Pins (all in the CPU test suite): fp16 codec against numpy's IEEE binary16;
 * hand-derived layout fixtures; closed-form activation cases; quantizer
 * round-trip bounds and nearest-code optimality; integer GEMV against a
 * float64 brute force over dequantized weights; one-hot / constant / zero
 * inputs; extreme codes at the int32 bounds. Every function below is pinned.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define QK 256            /* weights per super-block */
#define Q4K_BYTES 144     /* bytes per Q4_K super-block */
#define Q6K_BODY 208      /* bytes per Q6_K super-block body (the fp16 d lives in a separate plane) */
#define ACT_BLOCK 32      /* activation elements per int8 block */
#define QB 32             /* weights per Q4_0 / Q8_0 block */

static void die(const char *what) {
    fprintf(stderr, "qgemv oracle: %s\n", what);
    abort();
}

/* ---------------------------------------------------------------- fp16 ---- */
/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * float -> half rounds to nearest, ties to even, keeping subnormals; overflow
 * gives infinity; NaN stays NaN. half -> float is exact. */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

uint16_t orc_f32_to_f16(float f) {
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x7F800000u)                       /* inf or NaN */
        return (uint16_t)(sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u));
    if (a < 0x00800000u)                        /* float32 subnormal or zero: below half's range */
        return sign;
    int e = (int)(a >> 23) - 127;               /* value = mant * 2^(e - 23), mant has 24 bits */
    uint32_t mant = (a & 0x007FFFFFu) | 0x00800000u;
    if (e > 15)
        return (uint16_t)(sign | 0x7C00u);
    int shift = 13;                             /* keep 11 significant bits for a normal half */
    if (e < -14) shift += -14 - e;              /* fewer for a subnormal half */
    if (shift > 25)
        return sign;                            /* below half the smallest subnormal */
    uint32_t kept = mant >> shift;
    uint32_t rest = mant & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rest > half || (rest == half && (kept & 1u)))
        kept += 1;                              /* may carry into the exponent: still correct */
    uint32_t h = (e < -14) ? kept : ((uint32_t)(e + 14) << 10) + kept;
    return (uint16_t)(sign | h);                /* e = 15 with carry lands on 0x7C00 = inf */
}

float orc_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m + 1024), e - 25);
    return sign ? -v : v;
}

void orc_f32_to_f16_array(const float *x, uint16_t *h, int64_t n) {
    for (int64_t i = 0; i < n; i++) h[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_array(const uint16_t *h, float *x, int64_t n) {
    for (int64_t i = 0; i < n; i++) x[i] = orc_f16_to_f32(h[i]);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }

static float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* ------------------------------------------------------- activations ---- */
/* Per block of 32 elements: amax = max |x|; scale xd = amax / 127 (float32
 * division); inverse id = 127 / amax, or 0 when that is not a finite float32
 * (amax = 0, or amax below 127 / FLT_MAX, about 3.7e-37: such a block's codes
 * are all 0); code qx = clamp(rint(x * id), -127, 127) with one float32
 * multiply and round-to-nearest-even. The codes never take -128. */
void orc_quantize_act(const float *x, int64_t cols, int32_t nvec, int8_t *xq, float *xd) {
    if (cols % ACT_BLOCK) die("cols must be a multiple of 32");
    for (int32_t v = 0; v < nvec; v++) {
        for (int64_t b = 0; b < cols / ACT_BLOCK; b++) {
            const float *xb = x + (int64_t)v * cols + b * ACT_BLOCK;
            float amax = 0.0f;
            for (int i = 0; i < ACT_BLOCK; i++) {
                if (!isfinite(xb[i])) die("non-finite activation");
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float scale = amax / 127.0f;
            float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
            if (!(inv <= FLT_MAX)) inv = 0.0f;
            for (int i = 0; i < ACT_BLOCK; i++) {
                float prod = xb[i] * inv;
                float code = clampf(rintf(prod), -127.0f, 127.0f);
                xq[(int64_t)v * cols + b * ACT_BLOCK + i] = (int8_t)code;
            }
            xd[(int64_t)v * (cols / ACT_BLOCK) + b] = scale;
        }
    }
}

/* ---------------------------------------------------------- Q4_K layout --- */
/* One Q4_K super-block of 256 weights (sub-block j = weights 32j..32j+31) is
 * 144 bytes, written here as its "block image": a 16-byte header, then 128
 * bytes of codes.
 *   image [0,2)    d    (fp16, little-endian)  super-scale of the sub-scales
 *   image [2,4)    dmin (fp16)                 super-scale of the sub-mins
 *   image [4,8)    low 4 bits of sc_j: byte 4 + j/2, bits 4*(j%2) .. +3
 *   image [8,12)   low 4 bits of m_j : byte 8 + j/2, bits 4*(j%2) .. +3
 *   image [12,14)  high 2 bits of sc_j: byte 12 + j/4, bits 2*(j%4) .. +1
 *   image [14,16)  high 2 bits of m_j : byte 14 + j/4, bits 2*(j%4) .. +1
 *   image [16,144) codes: weight i = 32j + 16h + t (h in {0,1}, t < 16) is
 *                  nibble h (h=0 low, h=1 high) of byte 16 + 16j + t.
 * Dequantized weight: d * sc_j * q_i - dmin * m_j.
 *
 * A Q4_K tensor of N = rows * cols/256 blocks (block i = r * cols/256 + b)
 * keeps the two parts in two planes: the 128 code bytes of block i at
 * 128 * i, then the 16 header bytes of block i at 128 * N + 16 * i.         */

static int q4k_sc(const uint8_t *blk, int j) {
    int lo = (blk[4 + j / 2] >> (4 * (j % 2))) & 15;
    int hi = (blk[12 + j / 4] >> (2 * (j % 4))) & 3;
    return lo | (hi << 4);
}

static int q4k_m(const uint8_t *blk, int j) {
    int lo = (blk[8 + j / 2] >> (4 * (j % 2))) & 15;
    int hi = (blk[14 + j / 4] >> (2 * (j % 4))) & 3;
    return lo | (hi << 4);
}

static int q4k_q(const uint8_t *blk, int i) {
    int j = i / 32, h = (i % 32) / 16, t = i % 16;
    return (blk[16 + 16 * j + t] >> (4 * h)) & 15;
}

void orc_q4k_pack_block(uint16_t d, uint16_t dmin, const uint8_t *sc, const uint8_t *m,
                        const uint8_t *q, uint8_t *blk) {
    memset(blk, 0, Q4K_BYTES);
    wr16(blk + 0, d);
    wr16(blk + 2, dmin);
    for (int j = 0; j < 8; j++) {
        if (sc[j] > 63 || m[j] > 63) die("6-bit scale out of range");
        blk[4 + j / 2] |= (uint8_t)((sc[j] & 15) << (4 * (j % 2)));
        blk[8 + j / 2] |= (uint8_t)((m[j] & 15) << (4 * (j % 2)));
        blk[12 + j / 4] |= (uint8_t)((sc[j] >> 4) << (2 * (j % 4)));
        blk[14 + j / 4] |= (uint8_t)((m[j] >> 4) << (2 * (j % 4)));
    }
    for (int i = 0; i < QK; i++) {
        if (q[i] > 15) die("4-bit code out of range");
        int j = i / 32, h = (i % 32) / 16, t = i % 16;
        blk[16 + 16 * j + t] |= (uint8_t)(q[i] << (4 * h));
    }
}

void orc_q4k_unpack_block(const uint8_t *blk, uint16_t *d, uint16_t *dmin, uint8_t *sc,
                          uint8_t *m, uint8_t *q) {
    *d = rd16(blk + 0);
    *dmin = rd16(blk + 2);
    for (int j = 0; j < 8; j++) { sc[j] = (uint8_t)q4k_sc(blk, j); m[j] = (uint8_t)q4k_m(blk, j); }
    for (int i = 0; i < QK; i++) q[i] = (uint8_t)q4k_q(blk, i);
}

/* ---------------------------------------------------------- Q6_K layout --- */
/* One Q6_K super-block (sub-block j = weights 16j..16j+15, signed scale
 * sc_j) is a 208-byte "body" plus an fp16 super-scale d:
 *   body [0,128)   low 4 bits: weight i = 32k + 16g + t (k < 8, g in {0,1},
 *                  t < 16) is nibble g of byte 16k + t
 *   body [128,192) high 2 bits: weight i = 32k + 16g + 4s + c (s, c < 4) is
 *                  bits 2s .. 2s+1 of byte 128 + 8k + 4g + c
 *   body [192,208) sc_j as int8 at byte 192 + j
 * Code q_i in [0, 63]; dequantized weight: d * sc_j * (q_i - 32).
 *
 * A Q6_K tensor of N blocks keeps four planes, 210 bytes per block in all:
 * low bits of block i at 128 * i, high bits at 128 * N + 64 * i, scales at
 * 192 * N + 16 * i, d at 208 * N + 2 * i.                                    */

static int q6k_q(const uint8_t *body, int i) {
    int k = i / 32, g = (i % 32) / 16, t = i % 16, s = t / 4, c = t % 4;
    int lo = (body[16 * k + t] >> (4 * g)) & 15;
    int hi = (body[128 + 8 * k + 4 * g + c] >> (2 * s)) & 3;
    return lo | (hi << 4);
}

static int q6k_sc(const uint8_t *body, int j) { return (int)(int8_t)body[192 + j]; }

void orc_q6k_pack_block(const int8_t *sc, const uint8_t *q, uint8_t *body) {
    memset(body, 0, Q6K_BODY);
    for (int i = 0; i < QK; i++) {
        if (q[i] > 63) die("6-bit code out of range");
        int k = i / 32, g = (i % 32) / 16, t = i % 16, s = t / 4, c = t % 4;
        body[16 * k + t] |= (uint8_t)((q[i] & 15) << (4 * g));
        body[128 + 8 * k + 4 * g + c] |= (uint8_t)((q[i] >> 4) << (2 * s));
    }
    for (int j = 0; j < 16; j++) body[192 + j] = (uint8_t)sc[j];
}

void orc_q6k_unpack_block(const uint8_t *body, int8_t *sc, uint8_t *q) {
    for (int j = 0; j < 16; j++) sc[j] = (int8_t)q6k_sc(body, j);
    for (int i = 0; i < QK; i++) q[i] = (uint8_t)q6k_q(body, i);
}


/* ------------------------------------------------ tensor planes <-> blocks - */
static void q4k_get(const uint8_t *t, int64_t N, int64_t i, uint8_t *img) {
    memcpy(img, t + 128 * N + 16 * i, 16);
    memcpy(img + 16, t + 128 * i, 128);
}

static void q4k_put(uint8_t *t, int64_t N, int64_t i, const uint8_t *img) {
    memcpy(t + 128 * N + 16 * i, img, 16);
    memcpy(t + 128 * i, img + 16, 128);
}

static void q6k_get(const uint8_t *t, int64_t N, int64_t i, uint8_t *body, uint16_t *d) {
    memcpy(body, t + 128 * i, 128);
    memcpy(body + 128, t + 128 * N + 64 * i, 64);
    memcpy(body + 192, t + 192 * N + 16 * i, 16);
    *d = rd16(t + 208 * N + 2 * i);
}

static void q6k_put(uint8_t *t, int64_t N, int64_t i, const uint8_t *body, uint16_t d) {
    memcpy(t + 128 * i, body, 128);
    memcpy(t + 128 * N + 64 * i, body + 128, 64);
    memcpy(t + 192 * N + 16 * i, body + 192, 16);
    wr16(t + 208 * N + 2 * i, d);
}

void orc_q4k_get_block(const uint8_t *t, int64_t nblocks, int64_t i, uint8_t *img) {
    q4k_get(t, nblocks, i, img);
}
void orc_q4k_put_block(uint8_t *t, int64_t nblocks, int64_t i, const uint8_t *img) {
    q4k_put(t, nblocks, i, img);
}
void orc_q6k_get_block(const uint8_t *t, int64_t nblocks, int64_t i, uint8_t *body, uint16_t *d) {
    q6k_get(t, nblocks, i, body, d);
}
void orc_q6k_put_block(uint8_t *t, int64_t nblocks, int64_t i, const uint8_t *body, uint16_t d) {
    q6k_put(t, nblocks, i, body, d);
}

/* ------------------------------------------------ Q4_0 and Q8_0 layouts - */
/* Q4_0: a block of 32 weights (weight t, t < 32) with one fp16 scale d and
 * codes q_t in [0, 15]; dequantized weight d * (q_t - 8). Its 18-byte image:
 *   image [0,2)   d (fp16, little-endian)
 *   image [2,18)  codes: weight t is nibble (t >= 16 ? high : low) of byte
 *                 2 + (t mod 16), i.e. weights t and t + 16 share a byte.
 * A Q4_0 tensor of N = rows * cols/32 blocks (block i = r * cols/32 + b) keeps
 * the codes of block i at 16 * i and its d at 16 * N + 2 * i.
 *
 * Q8_0: a block of 32 weights with one float32 scale d and int8 codes q_t;
 * dequantized weight d * q_t. Its 36-byte image: d (float32, little-endian) at
 * [0,4), then weight t's code at byte 4 + t. A Q8_0 tensor of N blocks keeps
 * the codes of weights 0..15 of block i at 16 * i, those of weights 16..31 at
 * 16 * N + 16 * i, and its d at 32 * N + 4 * i.                                */
#define Q40_BYTES 18
#define Q80_BYTES 36

static int q40_q(const uint8_t *img, int t) {
    uint8_t byte = img[2 + t % 16];
    return t < 16 ? (byte & 15) : (byte >> 4);
}

void orc_q40_pack_block(uint16_t d, const uint8_t *q, uint8_t *img) {
    memset(img, 0, Q40_BYTES);
    wr16(img, d);
    for (int t = 0; t < QB; t++) {
        if (q[t] > 15) die("Q4_0 code out of range");
        img[2 + t % 16] |= (uint8_t)(t < 16 ? q[t] : q[t] << 4);
    }
}

void orc_q40_unpack_block(const uint8_t *img, uint16_t *d, uint8_t *q) {
    *d = rd16(img);
    for (int t = 0; t < QB; t++) q[t] = (uint8_t)q40_q(img, t);
}

static float rdf32(const uint8_t *p) {
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                 ((uint32_t)p[3] << 24);
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static void wrf32(uint8_t *p, float f) {
    uint32_t u = f32_bits(f);
    for (int k = 0; k < 4; k++) p[k] = (uint8_t)(u >> (8 * k));
}

void orc_q80_pack_block(float d, const int8_t *q, uint8_t *img) {
    wrf32(img, d);
    for (int t = 0; t < QB; t++) img[4 + t] = (uint8_t)q[t];
}

void orc_q80_unpack_block(const uint8_t *img, float *d, int8_t *q) {
    *d = rdf32(img);
    for (int t = 0; t < QB; t++) q[t] = (int8_t)img[4 + t];
}

static void q40_get(const uint8_t *t, int64_t N, int64_t i, uint8_t *img) {
    memcpy(img, t + 16 * N + 2 * i, 2);
    memcpy(img + 2, t + 16 * i, 16);
}
static void q40_put(uint8_t *t, int64_t N, int64_t i, const uint8_t *img) {
    memcpy(t + 16 * N + 2 * i, img, 2);
    memcpy(t + 16 * i, img + 2, 16);
}
static void q80_get(const uint8_t *t, int64_t N, int64_t i, uint8_t *img) {
    memcpy(img, t + 32 * N + 4 * i, 4);
    memcpy(img + 4, t + 16 * i, 16);
    memcpy(img + 20, t + 16 * N + 16 * i, 16);
}
static void q80_put(uint8_t *t, int64_t N, int64_t i, const uint8_t *img) {
    memcpy(t + 32 * N + 4 * i, img, 4);
    memcpy(t + 16 * i, img + 4, 16);
    memcpy(t + 16 * N + 16 * i, img + 20, 16);
}

void orc_q40_get_block(const uint8_t *t, int64_t nblocks, int64_t i, uint8_t *img) {
    q40_get(t, nblocks, i, img);
}
void orc_q40_put_block(uint8_t *t, int64_t nblocks, int64_t i, const uint8_t *img) {
    q40_put(t, nblocks, i, img);
}
void orc_q80_get_block(const uint8_t *t, int64_t nblocks, int64_t i, uint8_t *img) {
    q80_get(t, nblocks, i, img);
}
void orc_q80_put_block(uint8_t *t, int64_t nblocks, int64_t i, const uint8_t *img) {
    q80_put(t, nblocks, i, img);
}

/* ------------------------------------------------------ weight quantizers - */
/* Used to make test data; the GEMV never quantizes weights. Every decision
 * that yields an integer is taken in float32 with round-to-nearest-even.
 *
 * Q4_K, per super-block, per sub-block j of 32 weights:
 *   lo_j = min(0, min w), hi_j = max w, s_j = (hi_j - lo_j) / 15, o_j = -lo_j
 *   d = fp16(max_j s_j / 63), dmin = fp16(max_j o_j / 63)
 *   sc_j = clamp(rint(s_j / d), 0, 63), m_j = clamp(rint(o_j / dmin), 0, 63)
 *          (0 when the divisor is 0)
 *   q_i = clamp(rint((w_i + dmin*m_j) / (d*sc_j)), 0, 15)  (0 when d*sc_j = 0)
 * so that the codes 0..15 span [lo_j, hi_j] on a grid of step d*sc_j.        */
void orc_quantize_q4k(const float *w, int64_t rows, int64_t cols, uint8_t *out) {
    if (cols % QK) die("cols must be a multiple of 256");
    int64_t nb = cols / QK;
    uint8_t sc[8], m[8], q[QK], img[Q4K_BYTES];
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *wb = w + r * cols + b * QK;
            float s[8], o[8], smax = 0.0f, omax = 0.0f;
            for (int j = 0; j < 8; j++) {
                float lo = 0.0f, hi = wb[32 * j];
                for (int i = 0; i < 32; i++) {
                    float v = wb[32 * j + i];
                    if (!isfinite(v)) die("non-finite weight");
                    if (v < lo) lo = v;
                    if (v > hi) hi = v;
                }
                s[j] = (hi - lo) / 15.0f;
                o[j] = -lo;
                if (s[j] > smax) smax = s[j];
                if (o[j] > omax) omax = o[j];
            }
            uint16_t dh = orc_f32_to_f16(smax / 63.0f);
            uint16_t mh = orc_f32_to_f16(omax / 63.0f);
            float d = orc_f16_to_f32(dh), dmin = orc_f16_to_f32(mh);
            if (!isfinite(d) || !isfinite(dmin)) die("super-scale overflows fp16");
            for (int j = 0; j < 8; j++) {
                sc[j] = (uint8_t)(d > 0.0f ? clampf(rintf(s[j] / d), 0.0f, 63.0f) : 0.0f);
                m[j] = (uint8_t)(dmin > 0.0f ? clampf(rintf(o[j] / dmin), 0.0f, 63.0f) : 0.0f);
                float step = d * (float)sc[j];          /* exact: 11 x 6 significant bits */
                float off = dmin * (float)m[j];         /* exact */
                for (int i = 0; i < 32; i++) {
                    float v = wb[32 * j + i];
                    q[32 * j + i] = (uint8_t)(step > 0.0f
                        ? clampf(rintf((v + off) / step), 0.0f, 15.0f) : 0.0f);
                }
            }
            orc_q4k_pack_block(dh, mh, sc, m, q, img);
            q4k_put(out, rows * nb, r * nb + b, img);
        }
    }
}

/* Q6_K, per super-block, per sub-block j of 16 weights:
 *   a_j = max |w|, s_j = a_j / 31, d = fp16(max_j s_j / 127)
 *   sc_j = clamp(rint(s_j / d), -128, 127)   (0 when d = 0)
 *   q_i = clamp(rint(w_i / (d*sc_j)), -32, 31) + 32   (32 when sc_j = 0)
 * negate_scales != 0 gives the equivalent encoding sc' = -sc, q' = 64 - q in
 * every sub-block that has no code 0 (same dequantized values; it exercises
 * negative scales).                                                          */
void orc_quantize_q6k(const float *w, int64_t rows, int64_t cols, uint8_t *out,
                      int negate_scales) {
    if (cols % QK) die("cols must be a multiple of 256");
    int64_t nb = cols / QK;
    int8_t sc[16];
    uint8_t q[QK], body[Q6K_BODY];
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *wb = w + r * cols + b * QK;
            float s[16], smax = 0.0f;
            for (int j = 0; j < 16; j++) {
                float a = 0.0f;
                for (int i = 0; i < 16; i++) {
                    float v = wb[16 * j + i];
                    if (!isfinite(v)) die("non-finite weight");
                    if (fabsf(v) > a) a = fabsf(v);
                }
                s[j] = a / 31.0f;
                if (s[j] > smax) smax = s[j];
            }
            uint16_t dh = orc_f32_to_f16(smax / 127.0f);
            float d = orc_f16_to_f32(dh);
            if (!isfinite(d)) die("super-scale overflows fp16");
            for (int j = 0; j < 16; j++) {
                sc[j] = (int8_t)(d > 0.0f ? clampf(rintf(s[j] / d), -128.0f, 127.0f) : 0.0f);
                float step = d * (float)sc[j];          /* exact: 11 x 8 significant bits */
                int has_zero = 0;
                for (int i = 0; i < 16; i++) {
                    float v = wb[16 * j + i];
                    int c = step != 0.0f ? (int)clampf(rintf(v / step), -32.0f, 31.0f) + 32 : 32;
                    q[16 * j + i] = (uint8_t)c;
                    if (c == 0) has_zero = 1;
                }
                if (negate_scales && !has_zero) {
                    sc[j] = (int8_t)(-sc[j]);
                    for (int i = 0; i < 16; i++) q[16 * j + i] = (uint8_t)(64 - q[16 * j + i]);
                }
            }
            orc_q6k_pack_block(sc, q, body);
            q6k_put(out, rows * nb, r * nb + b, body, dh);
        }
    }
}

/* Q4_0, per block of 32 weights (GGUF-style: the largest-magnitude weight sets
 * the scale, mapped to code 0):
 *   m = the weight of largest |w| (the first one in index order on ties; +0
 *       for an all-zero block)
 *   d = fp16(m / -8)  (+0 when m = 0)
 *   q_t = clamp(rint(w_t / d) + 8, 0, 15) with the stored d in float32
 *         (8 when d = 0)
 * so m itself is reproduced up to the rounding of d and the opposite extreme
 * -m is clipped to 7/8 of its magnitude. */
void orc_quantize_q40(const float *w, int64_t rows, int64_t cols, uint8_t *out) {
    if (cols % QB) die("cols must be a multiple of 32");
    int64_t nb = cols / QB;
    uint8_t q[QB], img[Q40_BYTES];
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *wb = w + r * cols + b * QB;
            float m = 0.0f;
            for (int t = 0; t < QB; t++) {
                if (!isfinite(wb[t])) die("non-finite weight");
                if (fabsf(wb[t]) > fabsf(m)) m = wb[t];
            }
            uint16_t dh = m != 0.0f ? orc_f32_to_f16(m / -8.0f) : 0;
            float d = orc_f16_to_f32(dh);
            if (!isfinite(d)) die("scale overflows fp16");
            for (int t = 0; t < QB; t++)
                q[t] = (uint8_t)(d != 0.0f ? clampf(rintf(wb[t] / d) + 8.0f, 0.0f, 15.0f) : 8.0f);
            orc_q40_pack_block(dh, q, img);
            q40_put(out, rows * nb, r * nb + b, img);
        }
    }
}

/* Q8_0, per block of 32 weights: the rule of the activation quantizer,
 *   amax = max |w|, d = amax / 127, id = 127 / amax (0 when that is not a
 *   finite float32), q_t = clamp(rint(w_t * id), -127, 127). */
void orc_quantize_q80(const float *w, int64_t rows, int64_t cols, uint8_t *out) {
    if (cols % QB) die("cols must be a multiple of 32");
    int64_t nb = cols / QB;
    int8_t q[QB];
    uint8_t img[Q80_BYTES];
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *wb = w + r * cols + b * QB;
            float amax = 0.0f;
            for (int t = 0; t < QB; t++) {
                if (!isfinite(wb[t])) die("non-finite weight");
                if (fabsf(wb[t]) > amax) amax = fabsf(wb[t]);
            }
            float d = amax / 127.0f;
            float id = amax > 0.0f ? 127.0f / amax : 0.0f;
            if (!(id <= FLT_MAX)) id = 0.0f;
            for (int t = 0; t < QB; t++) q[t] = (int8_t)clampf(rintf(wb[t] * id), -127.0f, 127.0f);
            orc_q80_pack_block(d, q, img);
            q80_put(out, rows * nb, r * nb + b, img);
        }
    }
}

/* ------------------------------------------------------------ dequantize -- */
void orc_dequant_q4k(const uint8_t *w, int64_t rows, int64_t cols, double *out) {
    int64_t nb = cols / QK;
    uint8_t blk[Q4K_BYTES];
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            q4k_get(w, rows * nb, r * nb + b, blk);
            double d = orc_f16_to_f32(rd16(blk)), dmin = orc_f16_to_f32(rd16(blk + 2));
            for (int i = 0; i < QK; i++) {
                int j = i / 32;
                out[r * cols + b * QK + i] = d * q4k_sc(blk, j) * q4k_q(blk, i) - dmin * q4k_m(blk, j);
            }
        }
}

void orc_dequant_q6k(const uint8_t *w, int64_t rows, int64_t cols, double *out) {
    int64_t nb = cols / QK;
    uint8_t body[Q6K_BODY];
    uint16_t dh;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            q6k_get(w, rows * nb, r * nb + b, body, &dh);
            double d = orc_f16_to_f32(dh);
            for (int i = 0; i < QK; i++)
                out[r * cols + b * QK + i] = d * q6k_sc(body, i / 16) * (q6k_q(body, i) - 32);
        }
}

void orc_dequant_q40(const uint8_t *w, int64_t rows, int64_t cols, double *out) {
    int64_t nb = cols / QB;
    uint8_t img[Q40_BYTES];
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            q40_get(w, rows * nb, r * nb + b, img);
            double d = orc_f16_to_f32(rd16(img));
            for (int t = 0; t < QB; t++) out[r * cols + b * QB + t] = d * (q40_q(img, t) - 8);
        }
}

void orc_dequant_q80(const uint8_t *w, int64_t rows, int64_t cols, double *out) {
    int64_t nb = cols / QB;
    uint8_t img[Q80_BYTES];
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            q80_get(w, rows * nb, r * nb + b, img);
            double d = rdf32(img);
            for (int t = 0; t < QB; t++) out[r * cols + b * QB + t] = d * (int8_t)img[4 + t];
        }
}

/* ----------------------------------------------------------- integer GEMV - */
static int32_t checked32(int64_t v) {
    if (v > INT32_MAX || v < INT32_MIN) die("integer partial leaves int32");
    return (int32_t)v;
}

/* Q4_K: for vector v, row r and sub-block j (32 columns, the same columns as
 * activation block j):
 *   P[v][r][j] = sum_i q_i * qx_i        (exact integer)
 *   S[v][j]    = sum_i qx_i              (exact integer)
 *   y[v][r]    = sum_j xd_j * (d * sc_j * P - dmin * m_j * S)    (float64)
 *   bound[v][r] = sum_i |dequantized w_i| * |xd_j * qx_i|        (float64)
 * P (or S, bound) may be NULL. xq is [nvec][cols], xd [nvec][cols/32], y and
 * bound [nvec][rows], P [nvec][rows][cols/32], S [nvec][cols/32]. */
void orc_gemv_q4k(const uint8_t *w, int64_t rows, int64_t cols, int32_t nvec,
                  const int8_t *xq, const float *xd, int32_t *P, int32_t *S,
                  double *y, double *bound) {
    if (cols % QK) die("cols must be a multiple of 256");
    int64_t nb = cols / QK, ns = cols / 32;
    for (int32_t v = 0; v < nvec; v++) {
        const int8_t *xv = xq + (int64_t)v * cols;
        const float *dv = xd + (int64_t)v * ns;
        if (S)
            for (int64_t j = 0; j < ns; j++) {
                int64_t sum = 0;
                for (int i = 0; i < 32; i++) sum += xv[32 * j + i];
                S[(int64_t)v * ns + j] = checked32(sum);
            }
        for (int64_t r = 0; r < rows; r++) {
            double acc = 0.0, bnd = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                uint8_t blk[Q4K_BYTES];
                q4k_get(w, rows * nb, r * nb + b, blk);
                double d = orc_f16_to_f32(rd16(blk)), dmin = orc_f16_to_f32(rd16(blk + 2));
                for (int j = 0; j < 8; j++) {
                    int64_t col0 = b * QK + 32 * j;
                    int sc = q4k_sc(blk, j), m = q4k_m(blk, j);
                    int64_t p = 0, s = 0;
                    for (int i = 0; i < 32; i++) {
                        int q = q4k_q(blk, 32 * j + i);
                        p += (int64_t)q * xv[col0 + i];
                        s += xv[col0 + i];
                    }
                    double scale = dv[col0 / 32];
                    acc += scale * (d * sc * (double)checked32(p) - dmin * m * (double)checked32(s));
                    if (P) P[((int64_t)v * rows + r) * ns + col0 / 32] = (int32_t)p;
                    if (bound)
                        for (int i = 0; i < 32; i++) {
                            double wh = d * sc * q4k_q(blk, 32 * j + i) - dmin * m;
                            bnd += fabs(wh) * fabs(scale * xv[col0 + i]);
                        }
                }
            }
            y[(int64_t)v * rows + r] = acc;
            if (bound) bound[(int64_t)v * rows + r] = bnd;
        }
    }
}

/* Q6_K: for vector v, row r and sub-block j (16 columns, the half j%2 of
 * activation block j/2):
 *   P[v][r][j] = sum_i (q_i - 32) * qx_i                     (exact integer)
 *   y[v][r]    = sum_j xd_{j/2} * d * sc_j * P               (float64)
 * P is [nvec][rows][cols/16]; the other arrays as for Q4_K. */
void orc_gemv_q6k(const uint8_t *w, int64_t rows, int64_t cols, int32_t nvec,
                  const int8_t *xq, const float *xd, int32_t *P, double *y, double *bound) {
    if (cols % QK) die("cols must be a multiple of 256");
    int64_t nb = cols / QK, ns = cols / 16;
    for (int32_t v = 0; v < nvec; v++) {
        const int8_t *xv = xq + (int64_t)v * cols;
        const float *dv = xd + (int64_t)v * (cols / 32);
        for (int64_t r = 0; r < rows; r++) {
            double acc = 0.0, bnd = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                uint8_t body[Q6K_BODY];
                uint16_t dh;
                q6k_get(w, rows * nb, r * nb + b, body, &dh);
                double d = orc_f16_to_f32(dh);
                for (int j = 0; j < 16; j++) {
                    int64_t col0 = b * QK + 16 * j;
                    int sc = q6k_sc(body, j);
                    int64_t p = 0;
                    for (int i = 0; i < 16; i++)
                        p += (int64_t)(q6k_q(body, 16 * j + i) - 32) * xv[col0 + i];
                    double scale = dv[col0 / 32];
                    acc += scale * d * sc * (double)checked32(p);
                    if (P) P[((int64_t)v * rows + r) * ns + col0 / 16] = (int32_t)p;
                    if (bound)
                        for (int i = 0; i < 16; i++) {
                            double wh = d * sc * (q6k_q(body, 16 * j + i) - 32);
                            bnd += fabs(wh) * fabs(scale * xv[col0 + i]);
                        }
                }
            }
            y[(int64_t)v * rows + r] = acc;
            if (bound) bound[(int64_t)v * rows + r] = bnd;
        }
    }
}

/* Q4_0 and Q8_0: for vector v, row r and block j (32 columns, the columns of
 * activation block j):
 *   P[v][r][j] = sum_t c_t * qx_t       (exact integer; c_t = q_t - 8 for Q4_0,
 *                                         q_t for Q8_0)
 *   y[v][r]    = sum_j xd_j * d_j * P   (float64)
 * P is [nvec][rows][cols/32]; the other arrays as for Q4_K. */
static void gemv_q32(int is_q8, const uint8_t *w, int64_t rows, int64_t cols, int32_t nvec,
                     const int8_t *xq, const float *xd, int32_t *P, double *y, double *bound) {
    if (cols % QB) die("cols must be a multiple of 32");
    int64_t nb = cols / QB;
    for (int32_t v = 0; v < nvec; v++) {
        const int8_t *xv = xq + (int64_t)v * cols;
        const float *dv = xd + (int64_t)v * nb;
        for (int64_t r = 0; r < rows; r++) {
            double acc = 0.0, bnd = 0.0;
            for (int64_t j = 0; j < nb; j++) {
                uint8_t img[Q80_BYTES];
                double d;
                int c[QB];
                if (is_q8) {
                    q80_get(w, rows * nb, r * nb + j, img);
                    d = rdf32(img);
                    for (int t = 0; t < QB; t++) c[t] = (int8_t)img[4 + t];
                } else {
                    q40_get(w, rows * nb, r * nb + j, img);
                    d = orc_f16_to_f32(rd16(img));
                    for (int t = 0; t < QB; t++) c[t] = q40_q(img, t) - 8;
                }
                int64_t p = 0;
                for (int t = 0; t < QB; t++) p += (int64_t)c[t] * xv[QB * j + t];
                double scale = dv[j];
                acc += scale * d * (double)checked32(p);
                if (P) P[((int64_t)v * rows + r) * nb + j] = (int32_t)p;
                if (bound)
                    for (int t = 0; t < QB; t++) bnd += fabs(d * c[t]) * fabs(scale * xv[QB * j + t]);
            }
            y[(int64_t)v * rows + r] = acc;
            if (bound) bound[(int64_t)v * rows + r] = bnd;
        }
    }
}

void orc_gemv_q40(const uint8_t *w, int64_t rows, int64_t cols, int32_t nvec,
                  const int8_t *xq, const float *xd, int32_t *P, double *y, double *bound) {
    gemv_q32(0, w, rows, cols, nvec, xq, xd, P, y, bound);
}

void orc_gemv_q80(const uint8_t *w, int64_t rows, int64_t cols, int32_t nvec,
                  const int8_t *xq, const float *xd, int32_t *P, double *y, double *bound) {
    gemv_q32(1, w, rows, cols, nvec, xq, xd, P, y, bound);
}

/* -------------------------------------------------------------- brute force */
/* y[v][r] = sum_i what[r][i] * (xd_{i/32} * qx_i), float64, straight from a
 * dequantized matrix. Checks the integer formulation above. */
void orc_bruteforce(const double *what, int64_t rows, int64_t cols, int32_t nvec,
                    const int8_t *xq, const float *xd, double *y) {
    for (int32_t v = 0; v < nvec; v++)
        for (int64_t r = 0; r < rows; r++) {
            double acc = 0.0;
            for (int64_t i = 0; i < cols; i++)
                acc += what[r * cols + i] * ((double)xd[(int64_t)v * (cols / 32) + i / 32] *
                                             xq[(int64_t)v * cols + i]);
            y[(int64_t)v * rows + r] = acc;
        }
}
