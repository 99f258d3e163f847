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

// y[i] = v (+ res[i]), stored as fp32 or fp16 (RNE).  res may alias y: the
// same lane reads res[i] before it writes y[i].
__device__ __forceinline__ void store_y(void *y, const Epilogue &ep, size_t i, float v) {
    if (ep.res) v += ep.res[i];
    if (ep.f16)
        reinterpret_cast<_Float16 *>(y)[i] = (_Float16)v;
    else
        reinterpret_cast<float *>(y)[i] = v;
}

}  // namespace qk
