// qk_launch.h -- internal launch entry points (C++ linkage) behind the C ABI.
// Arguments are validated by the callers in qk_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

// Layout flag carried in the type argument (QK_PLANAR of the C ABI).
constexpr int PLANAR_FLAG = 0x100;

// ncols == 1: the streaming GEMV.
hipError_t launch_gemv1(int type, const void *W, const void *x, void *y, int64_t N, int64_t K,
                        hipStream_t stream);

// Independent one-column GEMVs in one launch (at most MAX_BATCH).
constexpr int MAX_BATCH = 16;
struct BatchEntry {
    int type;
    const void *W;
    const void *x;
    void *y;
    int64_t N, K;
};
hipError_t launch_gemv_batch(const BatchEntry *entries, int count, hipStream_t stream);

// ncols in 2..8: the few-column verify form (matrix cores).
hipError_t launch_gemv_multi(int type, const void *W, const void *x, void *y, int64_t N, int64_t K,
                             int ncols, hipStream_t stream);

// fp32 dequantisation of the whole tensor (either layout).
hipError_t launch_dequant(int type, const void *W, void *out, int64_t N, int64_t K, hipStream_t stream);

// GGUF rows -> PLANAR rows (type without the flag).
hipError_t launch_repack(int type, const void *W, void *Wp, int64_t N, int64_t K, hipStream_t stream);

}  // namespace qk
