// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgemv {

// Four signed byte products summed into c (v_dot4_i32_i8): the integer core of every
// sub-block dot product. Exact: |sum| stays far inside int32 for the formats here.
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Sum of the four signed bytes of a word.
__device__ __forceinline__ int byte_sum(uint32_t a, int c) { return dot4(a, 0x01010101u, c); }

// IEEE binary16 bits -> float (exact, subnormals kept).
__device__ __forceinline__ float half_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// float -> IEEE binary16 bits, round to nearest even, subnormals kept.
__device__ __forceinline__ uint32_t float_to_half(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Lane permutations inside a row of 16 lanes (DPP): each is a modifier on one VALU op.
enum : int {
    kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141,  // lane i <-> 7 - i inside each half row of 8
    kDppMirror = 0x140,      // lane i <-> 15 - i inside each row of 16
    kDppRowRor8 = 0x128,     // rotate by 8 inside each row of 16 (lane i <-> i ^ 8)
};

template <int ctrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of `width` consecutive lanes (width 8, 16, 32 or 64); every lane of
// the group receives the same sum. Within a row of 16 the butterfly uses DPP (xor 1, xor 2,
// then the two mirrors, which pair every partial sum with the one it lacks); across rows it
// uses one ds_swizzle (xor 16) and, for the whole wave, the two half-wave sums read as
// scalars. Every pairwise add is commutative, so all lanes hold bit-identical results.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(width == 8 || width == 16 || width == 32 || width == 64, "group width");
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    if constexpr (width >= 16) v += dpp<kDppMirror>(v);
    if constexpr (width >= 32)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                   0x401F));  // xor 16
    if constexpr (width == 64) {
        const int b = __builtin_bit_cast(int, v);
        v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    }
    return v;
}

// Sums of up to 8 values per lane over all 64 lanes, scattered: afterwards lane l holds the
// full sum of value number scatter_index(l) (all 8 lanes of each aligned group of 8 agree).
// Step 1 swaps the upper half of value k with the lower half of value k + 4
// (v_permlane32_swap), so one add leaves value k's pair sum in lanes 0-31 and value k + 4's
// in lanes 32-63; step 2 does the same between odd and even rows of 16 (v_permlane16_swap);
// step 3 exchanges across 8 lanes inside a row (DPP row rotate by 8) keeping one value per
// lane; the last three DPP steps sum the remaining 8 lanes. 18 VALU ops instead of 8 full
// butterflies; values past `n` are taken as zero.
__device__ __forceinline__ int scatter_index(int lane) {
    return 4 * ((lane >> 5) & 1) + 2 * ((lane >> 3) & 1) + ((lane >> 4) & 1);
}

template <int n>
__device__ __forceinline__ float wave_reduce_scatter8(const float (&v)[n]) {
    static_assert(n >= 1 && n <= 8, "at most 8 values");
    float u[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const float a = k < n ? v[k] : 0.0f;
        const float b = k + 4 < n ? v[k + 4] : 0.0f;
        const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, a),
                                                        __builtin_bit_cast(int, b), false, false);
        // copy the two results to scalars first: bit-casting r[0] and r[1] in place has been
        // compiled as r[0] + r[0] by this toolchain
        const int r0 = r[0], r1 = r[1];
        u[k] = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    }
    float w[2];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, u[2 * k]),
                                                        __builtin_bit_cast(int, u[2 * k + 1]),
                                                        false, false);
        const int r0 = r[0], r1 = r[1];
        w[k] = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    }
    const bool upper8 = (__lane_id() & 8) != 0;
    const float keep = upper8 ? w[1] : w[0];
    const float send = upper8 ? w[0] : w[1];
    float z = keep + dpp<kDppRowRor8>(send);
    z += dpp<kDppXor1>(z);
    z += dpp<kDppXor2>(z);
    z += dpp<kDppHalfMirror>(z);
    return z;
}

template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int off = width / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

template <int width>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
    for (int off = width / 2; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
    return v;
}

template <int width>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
#pragma unroll
    for (int off = width / 2; off >= 1; off >>= 1) v |= __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ uint4 load16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Activation quantization (oxinfer README, "How it works": per-matmul activation quantization;
// "Build and run": blocks of 32 with an f32 scale): amax over the block, scale = amax / 127,
// inverse 127 / amax (0 when that is not a finite float32: amax = 0, or amax below 127 / FLT_MAX,
// whose block's codes are then all 0), code = clamp(rint(x * inverse), -127, 127). Both
// divisions are IEEE float32 divisions, the product one float32 multiply, rint rounds to nearest
// even: the codes are the same on every IEEE machine, whichever lanes hold the block.
//
// The inverse scale, or 0 where 127 / amax is not finite (amax = 0 included).
__device__ __forceinline__ float act_inverse(float amax) {
    const float r = 127.0f / amax;
    return r <= 3.40282347e38f ? r : 0.0f;
}

// act_code_bits returns a float32 whose low byte is the code: the product is clamped first (the
// same as clamping after rounding, since +-127 are integers), then 1.5 * 2^23 is added, which
// rounds it to the nearest integer, ties to even, into the low mantissa bits (|value| <= 127 <
// 2^22) in two's complement.
__device__ __forceinline__ uint32_t act_code_bits(float e, float inv) {
    const float c = fminf(fmaxf(e * inv, -127.0f), 127.0f);
    return __builtin_bit_cast(uint32_t, c + 12582912.0f);
}

// The low bytes of four words, element a in the low byte of the result.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    // v_perm_b32 picks bytes of {src0 : src1}: selector 0-3 = src1's bytes, 4-7 = src0's, 12 = 0
    return __builtin_amdgcn_perm(b, a, 0x0C0C0400u) | __builtin_amdgcn_perm(d, c, 0x04000C0Cu);
}

__device__ __forceinline__ uint32_t act_codes4(const float4 v, float inv) {
    return pack_low_bytes(act_code_bits(v.x, inv), act_code_bits(v.y, inv),
                          act_code_bits(v.z, inv), act_code_bits(v.w, inv));
}

// One block held by 8 consecutive lanes, 4 elements each. All 64 lanes of the wave must call it.
struct ActQuad {
    uint32_t codes;   // 4 int8 codes, element 0 in the low byte
    float scale;      // the block's scale (the same in all 8 lanes)
};

__device__ __forceinline__ ActQuad quantize_act_quad(const float4 v) {
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    // the maximum over the block's 8 lanes: xor 1, xor 2, then the half-row mirror pairs
    // each quad with the other one
    amax = fmaxf(amax, dpp<kDppXor1>(amax));
    amax = fmaxf(amax, dpp<kDppXor2>(amax));
    amax = fmaxf(amax, dpp<kDppHalfMirror>(amax));
    const float scale = amax / 127.0f;
    const float inv = act_inverse(amax);
    return {act_codes4(v, inv), scale};
}

// One block held by the 4 lanes of a DPP quad, 8 consecutive elements each (a then b): the
// divisions and the cross-lane maximum are shared by twice the elements of the form above.
// All 64 lanes of the wave must call it.
struct ActOct {
    uint32_t lo, hi;  // 8 int8 codes, element 0 in the low byte of lo
    float scale;      // the block's scale (the same in all 4 lanes)
};

__device__ __forceinline__ ActOct quantize_act_oct(const float4 a, const float4 b) {
    float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                       fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    amax = fmaxf(amax, dpp<kDppXor1>(amax));
    amax = fmaxf(amax, dpp<kDppXor2>(amax));
    const float scale = amax / 127.0f;
    const float inv = act_inverse(amax);
    return {act_codes4(a, inv), act_codes4(b, inv), scale};
}

// 16-byte load marked nontemporal: the weights are read once per product, so they are
// streamed past the caches instead of displacing the activation slice and other data.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load8_stream(const void *p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load4_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ uint32_t load2_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}

}  // namespace qgemv
