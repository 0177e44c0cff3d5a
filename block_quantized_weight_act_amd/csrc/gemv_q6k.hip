// The GEMV for Q6_K (256-weight super-blocks: int8 sub-scales, fp16 d, 6-bit codes
// with offset -32):
// the instances of the shared wave walk (gemv_walk.h) with this format's tile (tile.h), for one
// matrix and for several of this format sharing one activation; one translation unit per
// format to keep builds parallel.
#include "gemv_walk.h"

namespace qgemv {

hipError_t launch_gemv_q6k(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream) {
    return GemvLaunch<Q6K>::launch(a, s, nvec, debug, stream);
}

hipError_t launch_gemv_multi_q6k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q6K>::launch_multi(a, s, nvec, stream);
}

hipError_t launch_gemv_split_q6k(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q6K>::launch_split(a, s, nvec, stream);
}

hipError_t launch_gemv_multi_split_q6k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream) {
    return GemvLaunch<Q6K>::launch_multi_split(a, s, nvec, stream);
}

}  // namespace qgemv
