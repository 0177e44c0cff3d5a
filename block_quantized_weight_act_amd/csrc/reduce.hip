// Second pass of a split-K GEMV: y = sum over column chunks s = 0 .. splits-1 of the
// partial outputs, added in ascending s (genie-ai-runtime, "v1.3.0": partial results of a
// split reduction dimension combined by a separate reduce kernel). No atomics, so the
// result is the same on every run.
#include "device_common.h"
#include "qgemv_internal.h"

namespace qgemv {

__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *__restrict__ part,
                                                            float *__restrict__ y, int64_t n,
                                                            int splits) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float acc = part[i];
    for (int s = 1; s < splits; s++) acc += part[static_cast<int64_t>(s) * n + i];
    y[i] = acc;
}

hipError_t launch_splitk_reduce(const float *part, float *y, int64_t n, int splits,
                                hipStream_t stream) {
    const int threads = 256;
    const int64_t grid = (n + threads - 1) / threads;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(grid)), dim3(threads), 0,
                       stream, part, y, n, splits);
    return hipGetLastError();
}

}  // namespace qgemv
