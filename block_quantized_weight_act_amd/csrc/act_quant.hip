// Activation quantization: float32 -> int8 codes in blocks of 32 with one float32 scale.
//
// oxinfer README, "How it works" (quant.rs): the activation is quantized to int8 for each
// matmul; "Build and run" (--quant q8): blocks of 32 with f32 scales. genie-ai-runtime,
// "v1.2.0": one quantized activation is shared by several matrix-vector products.
//
// Per block: amax = max |x|, scale = amax / 127, inverse = 127 / amax (0 when amax = 0),
// code = clamp(rint(x * inverse), -127, 127). Both divisions are IEEE float32 divisions
// (hipcc's default correctly rounded divide), the product is one float32 multiply and
// rint rounds to nearest even, so the codes are the same on every IEEE machine.
//
// Mapping: 8 lanes per block of 32, 4 elements per lane (one 16-byte load, one 4-byte
// store of codes); the block maximum is a 3-step butterfly inside the 8 lanes.
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

__global__ void __launch_bounds__(256) quantize_act_kernel(const float4 *__restrict__ x,
                                                           uint32_t *__restrict__ xq,
                                                           float *__restrict__ xd,
                                                           int64_t nblocks) {
    const int64_t lane_id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t blk = lane_id >> 3;
    const bool valid = blk < nblocks;   // uniform over each group of 8 lanes
    float4 v = valid ? x[lane_id] : make_float4(0.f, 0.f, 0.f, 0.f);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = group_max<8>(amax);
    const float scale = amax / 127.0f;
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float code = fminf(fmaxf(rintf(e[i] * inv), -127.0f), 127.0f);
        packed |= (static_cast<uint32_t>(static_cast<int>(code)) & 0xFFu) << (8 * i);
    }
    if (valid) {
        xq[lane_id] = packed;
        if ((lane_id & 7) == 0) xd[blk] = scale;
    }
}

hipError_t launch_quantize_act(const float *x, int8_t *xq, float *xd, int64_t nblocks32,
                               hipStream_t stream) {
    const int64_t lanes = nblocks32 * 8;
    const int threads = 256;
    const int64_t grid = (lanes + threads - 1) / threads;
    hipLaunchKernelGGL(quantize_act_kernel, dim3(static_cast<unsigned>(grid)), dim3(threads), 0,
                       stream, reinterpret_cast<const float4 *>(x),
                       reinterpret_cast<uint32_t *>(xq), xd, nblocks32);
    return hipGetLastError();
}

}  // namespace qgemv
