// The GEMV for Q4_0 (32-weight blocks: fp16 d, 4-bit codes with offset -8):
// the instances of the shared wave walk (gemv_walk.h) with this format's tile (tile.h), for one
// matrix and for several of this format sharing one activation; one translation unit per
// format to keep builds parallel.
#include "gemv_walk.h"

namespace qgemv {

hipError_t launch_gemv_q40(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream) {
    return GemvLaunch<Q40>::launch(a, s, nvec, debug, stream);
}

hipError_t launch_gemv_multi_q40(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q40>::launch_multi(a, s, nvec, stream);
}

hipError_t launch_gemv_split_q40(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q40>::launch_split(a, s, nvec, stream);
}

hipError_t launch_gemv_multi_split_q40(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream) {
    return GemvLaunch<Q40>::launch_multi_split(a, s, nvec, stream);
}

}  // namespace qgemv
