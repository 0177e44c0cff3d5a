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

// Sum over aligned groups of `width` consecutive lanes (width a power of two <= 64); every
// lane of the group receives the group's sum.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = width / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
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

}  // namespace qgemv
