// qk_verify.hip -- few-column verify GEMV (ncols 2..8) on matrix cores.
#include "qk_launch.h"

namespace qk {

hipError_t launch_gemv_multi(int, const void *, const void *, void *, int64_t, int64_t, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace qk
