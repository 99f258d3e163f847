// qk_epilogue.h -- the fused epilogue at the store of y, shared by the
// one-column and the verify kernels (see Epilogue in qk_launch.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qk_launch.h"

namespace qk {

// silu(z) = z * sigmoid(z) = z / (1 + e^-z), fp32 with the device library's
// expf; e^-z overflows to +inf for z < -88.7 and the quotient is then -0.
__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

// y[i] = v, stored as fp32 or fp16 (RNE).
__device__ __forceinline__ void store_y(void *y, bool f16, size_t i, float v) {
    if (f16)
        reinterpret_cast<_Float16 *>(y)[i] = (_Float16)v;
    else
        reinterpret_cast<float *>(y)[i] = v;
}

// The residual is read early: a load issued at the store would add a full
// memory latency to every workgroup's tail.  The lane that stores row r
// reads res[r] before its own store of y[r], and no other workgroup touches
// row r, so res may be y itself.

}  // namespace qk
