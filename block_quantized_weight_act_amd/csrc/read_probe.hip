// Streaming-read probe: reads a buffer once with 16-byte loads, as fast as the memory
// system allows, and does nothing else. Its bandwidth is the practical ceiling for any
// kernel that must read the same bytes, the way oxinfer's membench measures the machine's
// read bandwidth before judging its decode kernels (oxinfer README, "Performance").
//
// Each lane keeps four independent 16-byte loads in flight per step of a grid-stride loop;
// the XOR of everything read is stored only if it equals a value that random data does not
// produce, which keeps the loads alive without adding write traffic.
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

__global__ void __launch_bounds__(256) read_probe_kernel(const uint4 *__restrict__ buf,
                                                         int64_t n16, uint32_t *__restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
               d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = buf[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, int blocks,
                             hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const uint4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace qgemv
