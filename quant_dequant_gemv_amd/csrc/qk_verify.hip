// qk_verify.hip -- type dispatch of the few-column verify GEMV; the kernels
// are in qk_verify.h, instantiated per quant type in qk_verify_q{4,5,6}k.hip
// and qk_verify_iq4xs.hip.
#include "qk_format.h"
#include "qk_launch.h"

namespace qk {

hipError_t launch_verify_q4k(const void *, const void *, void *, int64_t, int64_t, int, const Epilogue &, hipStream_t);
hipError_t launch_verify_q5k(const void *, const void *, void *, int64_t, int64_t, int, const Epilogue &, hipStream_t);
hipError_t launch_verify_q6k(const void *, const void *, void *, int64_t, int64_t, int, const Epilogue &, hipStream_t);
hipError_t launch_verify_iq4xs(const void *, const void *, void *, int64_t, int64_t, int, const Epilogue &,
                               hipStream_t);

hipError_t launch_gemv_multi(int type, const void *W, const void *x, void *y, int64_t N, int64_t K, int ncols,
                             const Epilogue &ep, hipStream_t stream) {
    switch (type) {
    case Q4_K: return launch_verify_q4k(W, x, y, N, K, ncols, ep, stream);
    case Q5_K: return launch_verify_q5k(W, x, y, N, K, ncols, ep, stream);
    case Q6_K: return launch_verify_q6k(W, x, y, N, K, ncols, ep, stream);
    case IQ4_XS: return launch_verify_iq4xs(W, x, y, N, K, ncols, ep, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qk
