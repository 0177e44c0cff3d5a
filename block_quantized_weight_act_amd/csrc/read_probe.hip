// Streaming-read probe: reads a buffer once with 16-byte loads, as fast as the memory
// system allows, and does nothing else. Its bandwidth is the practical ceiling for any
// kernel that must read the same bytes, the way oxinfer's membench measures the machine's
// read bandwidth before judging its decode kernels (oxinfer README, "Performance").
//
// Each wave reads kRuns runs of 64 consecutive 16-byte words (8 KB) per iteration, all
// issued before any is used and marked nontemporal, and the waves stride over the buffer: the
// access pattern of the GEMV's code plane without its arithmetic. The XOR of everything read is
// stored only if it equals a value that random data does not produce, which keeps the loads
// alive without adding write traffic.
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

constexpr int kRuns = 8;

__global__ void __launch_bounds__(256) read_probe_kernel(const uint4 *__restrict__ buf,
                                                         int64_t n16, uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
    uint32_t acc = 0;
    for (int64_t base = wave * (kRuns * 64); base < n16; base += nwaves * (kRuns * 64)) {
        uint4 v[kRuns];
#pragma unroll
        for (int u = 0; u < kRuns; u++) {
            const int64_t idx = base + u * 64 + lane;
            v[u] = idx < n16 ? load16_stream(buf + idx) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kRuns; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
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
