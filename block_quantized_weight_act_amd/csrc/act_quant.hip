// Activation quantization: float32 -> int8 codes in blocks of 32 with one float32 scale.
//
// oxinfer README, "How it works" (quant.rs): the activation is quantized to int8 for each
// matmul; "Build and run" (--quant q8): blocks of 32 with f32 scales. genie-ai-runtime,
// "v1.2.0": one quantized activation is shared by several matrix-vector products.
//
// The arithmetic is quantize_act_quad (device_common.h), shared with the GEMV kernels that
// quantize their own activation slice. Mapping: 8 lanes per block of 32, 4 elements per lane
// (one 16-byte load, one 4-byte store of codes); the block maximum is a 3-step butterfly
// inside the 8 lanes.
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
    const float4 v = valid ? x[lane_id] : make_float4(0.f, 0.f, 0.f, 0.f);
    const ActQuad q = quantize_act_quad(v);
    if (valid) {
        xq[lane_id] = q.codes;
        if ((lane_id & 7) == 0) xd[blk] = q.scale;
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
