// The GEMV for Q8_0 (32-weight blocks: float32 d, int8 codes):
// the instances of the shared wave walk (gemv_walk.h) with this format's tile (tile.h), for one
// matrix and for several of this format sharing one activation; one translation unit per
// format to keep builds parallel.
#include "gemv_walk.h"

namespace qgemv {

hipError_t launch_gemv_q80(const GemvArgs &a, const LaunchShape &s, int nvec, bool debug,
                           hipStream_t stream) {
    return GemvLaunch<Q80>::launch(a, s, nvec, debug, stream);
}

hipError_t launch_gemv_multi_q80(const MultiArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q80>::launch_multi(a, s, nvec, stream);
}

hipError_t launch_gemv_split_q80(const GemvArgs &a, const LaunchShape &s, int nvec,
                                 hipStream_t stream) {
    return GemvLaunch<Q80>::launch_split(a, s, nvec, stream);
}

hipError_t launch_gemv_multi_split_q80(const MultiArgs &a, const LaunchShape &s, int nvec,
                                       hipStream_t stream) {
    return GemvLaunch<Q80>::launch_multi_split(a, s, nvec, stream);
}

}  // namespace qgemv
