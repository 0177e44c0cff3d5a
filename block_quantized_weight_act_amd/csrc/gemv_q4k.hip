// The GEMV for Q4_K (256-weight super-blocks: 6-bit sub-scales and mins, fp16 d
// and dmin, 4-bit codes):
// the instances of the shared wave walk (gemv_walk.h) with this format's tile (tile.h), for one
// matrix and for several of this format sharing one activation; one translation unit per
// format to keep builds parallel.
#include "gemv_walk.h"

namespace qgemv {

hipError_t launch_gemv_q4k(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream) {
    return GemvLaunch<Q4K>::launch(a, s, nvec, debug, stream);
}

hipError_t launch_gemv_multi_q4k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q4K>::launch_multi(a, s, nvec, stream);
}

hipError_t launch_gemv_split_q4k(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q4K>::launch_split(a, s, nvec, stream);
}

hipError_t launch_gemv_multi_split_q4k(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream) {
    return GemvLaunch<Q4K>::launch_multi_split(a, s, nvec, stream);
}

}  // namespace qgemv
