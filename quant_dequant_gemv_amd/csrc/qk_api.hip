// qk_api.hip -- the C ABI declared in include/qkgemv.h: argument checks,
// type x ncols dispatch, launch on the caller's stream.
#include <stdint.h>
#include <stdio.h>

#include "../../include/qkgemv.h"
#include "qk_launch.h"

#ifndef QKGEMV_VERSION
#define QKGEMV_VERSION "0.1.0"
#endif

namespace {

thread_local char g_launch_msg[256] = "launch failed";

static_assert(QK_PLANAR == qk::PLANAR_FLAG, "layout flag of the C ABI and the kernels");

int block_bytes(int type) {
    switch (type) {
    case QK_Q4_K: return 144;
    case QK_Q5_K: return 176;
    case QK_Q6_K: return 210;
    default: return -1;
    }
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Bytes of one row in the layout the type flags name, or -1.
int64_t row_bytes_of(int type, int64_t K) {
    const int bb = block_bytes(type & ~QK_PLANAR);
    if (bb < 0 || (type & ~(QK_PLANAR | 0xff)) != 0 || K < 256 || (K % 256) != 0) return -1;
    const int64_t b = (K / 256) * bb;
    return (type & QK_PLANAR) ? (b + 15) / 16 * 16 : b;
}

// Shared shape check.  Rows and columns must keep every byte offset inside
// int64 and every per-launch index inside the kernels' 32-bit ranges.
int check_shape(int type, int64_t N, int64_t K, int ncols) {
    if (block_bytes(type & ~QK_PLANAR) < 0 || (type & ~(QK_PLANAR | 0xff)) != 0) return QK_EINVAL_TYPE;
    if (N < 1 || K < 256 || (K % 256) != 0) return QK_EINVAL_SHAPE;
    if (ncols < 1 || ncols > QK_MAX_NCOLS) return QK_EINVAL_SHAPE;
    if ((type & QK_PLANAR) && ncols != 1) return QK_EINVAL_TYPE;
    if (K > (int64_t)1 << 30 || N > ((int64_t)1 << 31) - 1) return QK_EINVAL_SHAPE;
    const int64_t row_bytes = row_bytes_of(type, K);
    if (N > INT64_MAX / row_bytes) return QK_EINVAL_SHAPE;
    if (N > INT64_MAX / ((int64_t)K * 4)) return QK_EINVAL_SHAPE;
    return QK_OK;
}

int launched(hipError_t e);

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Pointer checks of the GEMV entry points (y fp32 or, with QK_Y_F16, fp16;
// the residual may be y itself only when y is fp32).
int check_io(const void *x, void *y, const void *res, int64_t N, int ncols, int flags) {
    if (!x || !y || !aligned(x, 16)) return QK_EINVAL_PTR;
    const bool f16 = (flags & QK_Y_F16) != 0;
    if (!aligned(y, f16 ? 2 : 4)) return QK_EINVAL_PTR;
    if (res) {
        if (!aligned(res, 4)) return QK_EINVAL_PTR;
        const int64_t n = N * ncols;
        if (!(res == y && !f16) && overlap(res, 4 * n, y, (f16 ? 2 : 4) * n)) return QK_EINVAL_PTR;
    }
    return QK_OK;
}

int gemv_launch(int type, const void *W, const void *W2, const void *x, void *y, int64_t N, int64_t K,
                int ncols, const void *residual, int flags, void *stream) {
    const qk::Epilogue ep{W2, (const float *)residual, (flags & QK_Y_F16) ? 1 : 0};
    hipStream_t st = (hipStream_t)stream;
    if (ncols == 1) return launched(qk::launch_gemv1(type, W, x, y, N, K, ep, st));
    return launched(qk::launch_gemv_multi(type, W, x, y, N, K, ncols, ep, st));
}

int launched(hipError_t e) {
    if (e == hipSuccess) return QK_OK;
    snprintf(g_launch_msg, sizeof g_launch_msg, "launch failed: %s", hipGetErrorString(e));
    return QK_ELAUNCH;
}

}  // namespace

extern "C" {

int qk_block_bytes(int type) { return block_bytes(type); }

int64_t qk_row_bytes(int type, int64_t K) { return row_bytes_of(type, K); }

int qk_gemv(int type, const void *W, const void *x, void *y, int64_t N, int64_t K, int ncols, void *stream) {
    return qk_gemv_ex(type, W, x, y, N, K, ncols, nullptr, 0, stream);
}

int qk_gemv_ex(int type, const void *W, const void *x, void *y, int64_t N, int64_t K, int ncols,
               const void *residual, int flags, void *stream) {
    int rc = check_shape(type, N, K, ncols);
    if (rc) return rc;
    if (flags & ~QK_Y_F16) return QK_EINVAL_FLAGS;
    if (!W || !aligned(W, 16)) return QK_EINVAL_PTR;
    if ((rc = check_io(x, y, residual, N, ncols, flags))) return rc;
    return gemv_launch(type, W, nullptr, x, y, N, K, ncols, residual, flags, stream);
}

int qk_gemv_swiglu(int type, const void *Wg, const void *Wu, const void *x, void *y, int64_t N, int64_t K,
                   int ncols, int flags, void *stream) {
    int rc = check_shape(type, N, K, ncols);
    if (rc) return rc;
    if (flags & ~QK_Y_F16) return QK_EINVAL_FLAGS;
    if (!Wg || !Wu || !aligned(Wg, 16) || !aligned(Wu, 16)) return QK_EINVAL_PTR;
    if ((rc = check_io(x, y, nullptr, N, ncols, flags))) return rc;
    return gemv_launch(type, Wg, Wu, x, y, N, K, ncols, nullptr, flags, stream);
}

int qk_gemv_batch(const qk_gemv_item *items, int count, void *stream) {
    if (!items || count < 1 || count > QK_MAX_BATCH || count > qk::MAX_BATCH) return QK_EINVAL_SHAPE;
    qk::BatchEntry e[qk::MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        const qk_gemv_item &it = items[i];
        const int rc = check_shape(it.type, it.N, it.K, 1);
        if (rc) return rc;
        if (!it.W || !it.x || !it.y || !aligned(it.W, 16) || !aligned(it.x, 16) || !aligned(it.y, 4))
            return QK_EINVAL_PTR;
        e[i] = qk::BatchEntry{it.type, it.W, it.x, it.y, it.N, it.K};
    }
    return launched(qk::launch_gemv_batch(e, count, (hipStream_t)stream));
}

int qk_dequant(int type, const void *W, void *out, int64_t N, int64_t K, void *stream) {
    const int rc = check_shape(type, N, K, 1);
    if (rc) return rc;
    if (!W || !out || !aligned(W, 16) || !aligned(out, 4)) return QK_EINVAL_PTR;
    return launched(qk::launch_dequant(type, W, out, N, K, (hipStream_t)stream));
}

int qk_repack(int type, const void *W, void *Wp, int64_t N, int64_t K, void *stream) {
    if (type & QK_PLANAR) return QK_EINVAL_TYPE;
    const int rc = check_shape(type, N, K, 1);
    if (rc) return rc;
    if (!W || !Wp || !aligned(W, 16) || !aligned(Wp, 16)) return QK_EINVAL_PTR;
    const uintptr_t a0 = (uintptr_t)W, a1 = a0 + (uintptr_t)(N * row_bytes_of(type, K));
    const uintptr_t b0 = (uintptr_t)Wp, b1 = b0 + (uintptr_t)(N * row_bytes_of(type | QK_PLANAR, K));
    if (a0 < b1 && b0 < a1) return QK_EINVAL_PTR;
    return launched(qk::launch_repack(type, W, Wp, N, K, (hipStream_t)stream));
}

const char *qk_strerror(int code) {
    switch (code) {
    case QK_OK: return "ok";
    case QK_EINVAL_TYPE:
        return "invalid type: expected QK_Q4_K (12), QK_Q5_K (13) or QK_Q6_K (14), optionally | QK_PLANAR "
               "(0x100) with ncols = 1 (qk_repack takes the type without the flag)";
    case QK_EINVAL_SHAPE: return "invalid shape: need N >= 1, K a positive multiple of 256, 1 <= ncols <= 32";
    case QK_EINVAL_PTR:
        return "invalid pointer: NULL, or W/x not 16-byte aligned, or y/out/residual not 4-byte aligned (fp16 y: 2), "
               "or a residual that overlaps y without being y (fp32 y)";
    case QK_EINVAL_FLAGS: return "invalid flags: the only epilogue flag is QK_Y_F16 (0x1)";
    case QK_ELAUNCH: return g_launch_msg;
    default: return "unknown error code";
    }
}

const char *qk_version(void) { return "qkgemv " QKGEMV_VERSION " gfx950"; }

}  // extern "C"
