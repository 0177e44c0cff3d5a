// Load-time weight quantization into the Q4_K and Q6_K layouts (oxinfer README, "How it
// works", quant.rs: weights are block-quantized once when the model is loaded). Not on the
// per-token path; written for clarity: one 64-lane wavefront per 256-weight super-block,
// 4 consecutive weights per lane. A launch may cover a range of rows: w holds those rows,
// blk0 is the index of their first super-block in the whole tensor and ntotal the tensor's
// super-block count, which fixes where each plane starts.
//
// Every decision that yields an integer (a code, a sub-scale, an fp16 super-scale) is an
// IEEE float32 operation with round-to-nearest-even, so the bytes are reproducible on any
// IEEE machine. Maxima and minima start from +0 and never produce -0, so the fp16
// super-scale of an all-zero block is +0.
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// Q4_K: sub-block j (32 weights) = lanes 8j .. 8j+7.
__global__ void __launch_bounds__(256) quantize_q4k_kernel(const float *__restrict__ w,
                                                           uint8_t *__restrict__ out,
                                                           int64_t nblocks, int nb, int64_t cols,
                                                           int64_t blk0, int64_t ntotal) {
    const int lane = threadIdx.x & 63;
    const int64_t local = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (local >= nblocks) return;                    // uniform over the wavefront
    const int64_t row = local / nb, b = local % nb;
    const int64_t blk = blk0 + local;                // index in the whole tensor
    const float4 v4 = *reinterpret_cast<const float4 *>(w + row * cols + b * kQK + 4 * lane);
    const float v[4] = {v4.x, v4.y, v4.z, v4.w};
    const int j = lane >> 3;

    // sub-block range: lo = min(0, min w), hi = max w
    float lo = 0.0f, hi = v[0];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lo = v[i] < lo ? v[i] : lo;
        hi = v[i] > hi ? v[i] : hi;
    }
    lo = group_min<8>(lo);
    hi = group_max<8>(hi);
    const float s = (hi - lo) / 15.0f;
    const float o = -lo;
    // super-scales from the largest sub-block step and offset (compared against +0)
    const float smax = group_max<64>(s > 0.0f ? s : 0.0f);
    const float omax = group_max<64>(o > 0.0f ? o : 0.0f);
    const uint32_t dh = float_to_half(smax / 63.0f);
    const uint32_t mh = float_to_half(omax / 63.0f);
    const float d = half_to_float(dh), dmin = half_to_float(mh);
    const int sc = static_cast<int>(d > 0.0f ? clampf(rintf(s / d), 0.0f, 63.0f) : 0.0f);
    const int m = static_cast<int>(dmin > 0.0f ? clampf(rintf(o / dmin), 0.0f, 63.0f) : 0.0f);
    const float step = d * static_cast<float>(sc);    // exact
    const float off = dmin * static_cast<float>(m);   // exact
    uint32_t codes = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float q = step > 0.0f ? clampf(rintf((v[i] + off) / step), 0.0f, 15.0f) : 0.0f;
        codes |= static_cast<uint32_t>(q) << (8 * i);
    }
    // Codes plane: block blk's 128 code bytes at 128 * blk. Weights 32j + 4(lane%8) + i: lanes
    // with lane%8 < 4 hold the low nibbles (columns 32j + t, t < 16) and their partner lane + 4
    // the high nibbles (32j + 16 + t) of the same 4 code bytes 16j + 4(lane%4) .. +3.
    uint8_t *codes_out = out + blk * 128;
    const uint32_t partner = __shfl_xor(codes, 4, 64);
    if ((lane & 4) == 0)
        *reinterpret_cast<uint32_t *>(codes_out + 16 * j + 4 * (lane & 3)) = codes | (partner << 4);
    // Header: sc/m low nibbles at bits 4j of words 1 and 2, high 2 bits at bits 2j and
    // 16 + 2j of word 3. Lane 8j holds sub-block j's values.
    const bool lead = (lane & 7) == 0;
    const uint32_t wa = group_or<64>(lead ? (static_cast<uint32_t>(sc) & 15u) << (4 * j) : 0u);
    const uint32_t wb = group_or<64>(lead ? (static_cast<uint32_t>(m) & 15u) << (4 * j) : 0u);
    const uint32_t wc = group_or<64>(
        lead ? ((static_cast<uint32_t>(sc) >> 4) << (2 * j)) |
                   ((static_cast<uint32_t>(m) >> 4) << (16 + 2 * j))
             : 0u);
    // Header plane: block blk's 16 header bytes at 128 * ntotal + 16 * blk.
    if (lane == 0)
        *reinterpret_cast<uint4 *>(out + ntotal * 128 + blk * 16) =
            make_uint4(dh | (mh << 16), wa, wb, wc);
}

// Q6_K: sub-block j (16 weights) = lanes 4j .. 4j+3.
__global__ void __launch_bounds__(256) quantize_q6k_kernel(const float *__restrict__ w,
                                                           uint8_t *__restrict__ out,
                                                           int64_t nblocks, int nb, int64_t cols,
                                                           int64_t blk0, int64_t ntotal) {
    const int lane = threadIdx.x & 63;
    const int64_t local = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (local >= nblocks) return;
    const int64_t row = local / nb, b = local % nb;
    const int64_t blk = blk0 + local;
    const float4 v4 = *reinterpret_cast<const float4 *>(w + row * cols + b * kQK + 4 * lane);
    const float v[4] = {v4.x, v4.y, v4.z, v4.w};

    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) a = fabsf(v[i]) > a ? fabsf(v[i]) : a;
    a = group_max<4>(a);
    const float s = a / 31.0f;
    const float smax = group_max<64>(s);
    const uint32_t dh = float_to_half(smax / 127.0f);
    const float d = half_to_float(dh);
    const int sc = static_cast<int>(d > 0.0f ? clampf(rintf(s / d), -128.0f, 127.0f) : 0.0f);
    const float step = d * static_cast<float>(sc);    // exact
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        q[i] = step != 0.0f ? static_cast<int>(clampf(rintf(v[i] / step), -32.0f, 31.0f)) + 32 : 32;

    // Planes of block blk: low bits at 128 * blk, high bits at 128 N + 64 * blk, sub-scales at
    // 192 N + 16 * blk, d at 208 N + 2 * blk (N = ntotal).
    uint8_t *low_out = out + blk * 128;
    uint8_t *high_out = out + ntotal * 128 + blk * 64;
    uint8_t *sc_out = out + ntotal * 192 + blk * 16;
    // Weight 4*lane + i = 32k + 16g + t with k = lane/8, g = (lane%8)/4, t = 4(lane%4) + i.
    const int k = lane >> 3, g = (lane >> 2) & 1, s4 = lane & 3;
    uint32_t low = 0, high = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        low |= static_cast<uint32_t>(q[i] & 15) << (8 * i);
        // high 2 bits of weight 32k + 16g + 4*s4 + i: bits 2*s4 of high-bit byte 8k + 4g + i
        high |= static_cast<uint32_t>((q[i] >> 4) & 3) << (8 * i + 2 * s4);
    }
    const uint32_t partner = __shfl_xor(low, 4, 64);
    if (g == 0) *reinterpret_cast<uint32_t *>(low_out + 16 * k + 4 * s4) = low | (partner << 4);
    high = group_or<4>(high);
    if (s4 == 0) *reinterpret_cast<uint32_t *>(high_out + 8 * k + 4 * g) = high;
    // sub-scales: lane 4j holds sc_j, sub-scale byte j; four per 32-bit word
    const int jj = lane >> 2;
    const uint32_t scb = group_or<16>((lane & 3) == 0
                                          ? (static_cast<uint32_t>(sc) & 0xFFu) << (8 * (jj & 3))
                                          : 0u);
    if ((lane & 15) == 0) *reinterpret_cast<uint32_t *>(sc_out + 4 * (lane >> 4)) = scb;
    if (lane == 0) reinterpret_cast<uint16_t *>(out + ntotal * 208)[blk] = static_cast<uint16_t>(dh);
}

hipError_t launch_quantize_q4k(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream) {
    const int64_t nb = cols / kQK, nblocks = nrows * nb;
    const int waves = 4;
    const int64_t grid = (nblocks + waves - 1) / waves;
    hipLaunchKernelGGL(quantize_q4k_kernel, dim3(static_cast<unsigned>(grid)), dim3(64 * waves), 0,
                       stream, w, out, nblocks, static_cast<int>(nb), cols, row0 * nb, rows * nb);
    return hipGetLastError();
}

hipError_t launch_quantize_q6k(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream) {
    const int64_t nb = cols / kQK, nblocks = nrows * nb;
    const int waves = 4;
    const int64_t grid = (nblocks + waves - 1) / waves;
    hipLaunchKernelGGL(quantize_q6k_kernel, dim3(static_cast<unsigned>(grid)), dim3(64 * waves), 0,
                       stream, w, out, nblocks, static_cast<int>(nb), cols, row0 * nb, rows * nb);
    return hipGetLastError();
}

// The 32-weight formats: 8 lanes per block, 4 consecutive weights per lane (lane l of a block
// holds weights 4l .. 4l + 3). w holds the rows' floats; block `local` of the launch is weights
// 32 local .. 32 local + 31 of w and block blk0 + local of the tensor of ntotal blocks.

// Q8_0: the activation rule on each block (quantize_act_quad: the same codes and scale). Lanes
// 0..3 of a block write its first 16 codes into the first codes plane, lanes 4..7 the other 16
// into the second.
__global__ void __launch_bounds__(256) quantize_q80_kernel(const float4 *__restrict__ w,
                                                           uint8_t *__restrict__ out,
                                                           int64_t nblocks, int64_t blk0,
                                                           int64_t ntotal) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t local = gid >> 3;
    const bool valid = local < nblocks;       // the same for the block's 8 lanes
    const float4 v = valid ? w[gid] : make_float4(0.f, 0.f, 0.f, 0.f);
    const ActQuad q = quantize_act_quad(v);
    if (valid) {
        const int64_t blk = blk0 + local;
        const int l = static_cast<int>(gid & 7);
        const int64_t at = l < 4 ? 16 * blk + 4 * l : 16 * ntotal + 16 * blk + 4 * (l - 4);
        *reinterpret_cast<uint32_t *>(out + at) = q.codes;
        if ((gid & 7) == 0) *reinterpret_cast<float *>(out + 32 * ntotal + 4 * blk) = q.scale;
    }
}

// Q4_0: m = the block's first weight of largest magnitude (a lane keeps the first of its four
// on ties; across lanes the larger magnitude wins, then the smaller index); d = fp16(m / -8),
// +0 for an all-zero block; q = clamp(rint(w / d) + 8, 0, 15), 8 when d = 0. Codes of weights
// t and t + 16 share byte t: lane l < 4 packs its codes with those of lane l + 4.
__global__ void __launch_bounds__(256) quantize_q40_kernel(const float4 *__restrict__ w,
                                                           uint8_t *__restrict__ out,
                                                           int64_t nblocks, int64_t blk0,
                                                           int64_t ntotal) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t local = gid >> 3;
    const int l = static_cast<int>(gid & 7);
    const bool valid = local < nblocks;
    const float4 v4 = valid ? w[gid] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float e[4] = {v4.x, v4.y, v4.z, v4.w};
    float mag = fabsf(e[0]), val = e[0];
    int idx = 4 * l;
#pragma unroll
    for (int i = 1; i < 4; i++) {
        if (fabsf(e[i]) > mag) {
            mag = fabsf(e[i]);
            val = e[i];
            idx = 4 * l + i;
        }
    }
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
        const float pm = __shfl_xor(mag, off, 64);
        const float pv = __shfl_xor(val, off, 64);
        const int pi = __shfl_xor(idx, off, 64);
        if (pm > mag || (pm == mag && pi < idx)) {
            mag = pm;
            val = pv;
            idx = pi;
        }
    }
    const uint32_t dh = val != 0.0f ? float_to_half(val / -8.0f) : 0u;
    const float d = half_to_float(dh);
    uint32_t codes = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float q = d != 0.0f ? clampf(rintf(e[i] / d) + 8.0f, 0.0f, 15.0f) : 8.0f;
        codes |= static_cast<uint32_t>(q) << (8 * i);
    }
    const uint32_t partner = __shfl_xor(codes, 4, 64);
    if (valid) {
        const int64_t blk = blk0 + local;
        if (l < 4) *reinterpret_cast<uint32_t *>(out + 16 * blk + 4 * l) = codes | (partner << 4);
        if (l == 0) reinterpret_cast<uint16_t *>(out + 16 * ntotal)[blk] = static_cast<uint16_t>(dh);
    }
}

hipError_t launch_quantize_q40(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream) {
    const int64_t nb = cols / 32, nblocks = nrows * nb;
    const int64_t grid = (nblocks * 8 + 255) / 256;
    hipLaunchKernelGGL(quantize_q40_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(w), out, nblocks, row0 * nb, rows * nb);
    return hipGetLastError();
}

hipError_t launch_quantize_q80(const float *w, uint8_t *out, int64_t rows, int64_t cols,
                               int64_t row0, int64_t nrows, hipStream_t stream) {
    const int64_t nb = cols / 32, nblocks = nrows * nb;
    const int64_t grid = (nblocks * 8 + 255) / 256;
    hipLaunchKernelGGL(quantize_q80_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(w), out, nblocks, row0 * nb, rows * nb);
    return hipGetLastError();
}

}  // namespace qgemv
