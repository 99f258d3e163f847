// qk_verify_iq4xs.hip -- the IQ4_XS instances of the verify kernels (qk_verify.h).
#include "qk_verify.h"

namespace qk {

hipError_t launch_verify_iq4xs(const void *W, const void *x, void *y, int64_t N, int64_t K, int ncols,
                               const Epilogue &ep, hipStream_t stream) {
    return verify_type<IQ4_XS>(W, x, y, N, K, ncols, ep, stream);
}

}  // namespace qk
