// The library's static device scratch buffer: the workspace of qgemv_batch_scratch, for callers
// that cannot allocate device memory (code under graph capture, tight serving loops, harnesses
// that forbid allocation). The array lives in the library's code object, so every GPU the
// library runs on holds its own copy, at its own address, from the first launch until the
// process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address on
// the current GPU comes from hipGetSymbolAddress, taken once per device and kept; the kernels
// receive that address like any caller-provided workspace.
#include <qgemv.h>

#include <mutex>

#include "qgemv_internal.h"

namespace qgemv {

namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kMaxDevices];   // device address of `scratch` on each device (set once)

}  // namespace

int scratch_address(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices)
        return fail_with(QGEMV_EINVAL, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (p == nullptr) return fail_with(QGEMV_EHIP, "no device address for the scratch buffer");
        g_scratch_addr[dev] = p;
    }
    *ptr = g_scratch_addr[dev];
    return QGEMV_OK;
}

}  // namespace qgemv
