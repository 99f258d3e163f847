// qk_api.hip -- the C ABI declared in include/qkgemv.h: argument checks,
// type x ncols dispatch, launch on the caller's stream.
#include <stdint.h>
#include <stdio.h>

#include <new>

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
    case QK_IQ4_XS: return 136;
    default: return -1;
    }
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Bytes of one row in the layout the type flags name, or -1.
int64_t row_bytes_of(int type, int64_t K) {
    const int bb = block_bytes(type & ~QK_PLANAR);
    if (bb < 0 || (type & ~(QK_PLANAR | 0xff)) != 0 || K < 256 || (K % 256) != 0) return -1;
    if (type == (QK_IQ4_XS | QK_PLANAR)) return -1;  // the k-quants only
    const int64_t b = (K / 256) * bb;
    return (type & QK_PLANAR) ? (b + 15) / 16 * 16 : b;
}

// Shared shape check.  Rows and columns must keep every byte offset inside
// int64 and every per-launch index inside the kernels' 32-bit ranges.
int check_shape(int type, int64_t N, int64_t K, int ncols) {
    if (block_bytes(type & ~QK_PLANAR) < 0 || (type & ~(QK_PLANAR | 0xff)) != 0) return QK_EINVAL_TYPE;
    if (N < 1 || K < 256 || (K % 256) != 0) return QK_EINVAL_SHAPE;
    if (ncols < 1 || ncols > QK_MAX_NCOLS) return QK_EINVAL_SHAPE;
    if ((type & QK_PLANAR) && (ncols != 1 || (type & ~QK_PLANAR) == QK_IQ4_XS)) return QK_EINVAL_TYPE;
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
// the residual may be y itself only when y is fp32).  y is written while W
// and x are still being read by other workgroups, so y may overlap neither.
int check_io(int type, const void *W, const void *x, void *y, const void *res, int64_t N, int64_t K, int ncols,
             int flags) {
    if (!x || !y || !aligned(x, 16)) return QK_EINVAL_PTR;
    const bool f16 = (flags & QK_Y_F16) != 0;
    if (!aligned(y, f16 ? 2 : 4)) return QK_EINVAL_PTR;
    const int64_t n = N * ncols, ybytes = (f16 ? 2 : 4) * n;
    if (overlap(y, ybytes, W, N * row_bytes_of(type, K)) || overlap(y, ybytes, x, 2 * K * ncols))
        return QK_EINVAL_PTR;
    if (res) {
        if (!aligned(res, 4)) return QK_EINVAL_PTR;
        if (!(res == y && !f16) && overlap(res, 4 * n, y, ybytes)) return QK_EINVAL_PTR;
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
    if ((rc = check_io(type, W, x, y, residual, N, K, ncols, flags))) return rc;
    return gemv_launch(type, W, nullptr, x, y, N, K, ncols, residual, flags, stream);
}

int qk_gemv_swiglu(int type, const void *Wg, const void *Wu, const void *x, void *y, int64_t N, int64_t K,
                   int ncols, int flags, void *stream) {
    int rc = check_shape(type, N, K, ncols);
    if (rc) return rc;
    if (flags & ~QK_Y_F16) return QK_EINVAL_FLAGS;
    if (!Wg || !Wu || !aligned(Wg, 16) || !aligned(Wu, 16)) return QK_EINVAL_PTR;
    if ((rc = check_io(type, Wg, x, y, nullptr, N, K, ncols, flags))) return rc;
    if (overlap(y, ((flags & QK_Y_F16) ? 2 : 4) * N * ncols, Wu, N * row_bytes_of(type, K))) return QK_EINVAL_PTR;
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
    // the entries run concurrently: no y may overlap any entry's W, x or y
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j) {
            const qk_gemv_item &a = items[i], &b = items[j];
            if (overlap(a.y, 4 * a.N, b.W, b.N * row_bytes_of(b.type, b.K)) || overlap(a.y, 4 * a.N, b.x, 2 * b.K) ||
                (i != j && overlap(a.y, 4 * a.N, b.y, 4 * b.N)))
                return QK_EINVAL_PTR;
        }
    return launched(qk::launch_gemv_batch(e, count, (hipStream_t)stream));
}

int64_t qk_chain_plan_bytes(int nsteps, int nentries) {
    if (nsteps < 1 || nentries < nsteps) return -1;
    return qk::chain_plan_bytes(nsteps, nentries);
}

int qk_chain_plan(const qk_chain_entry *entries, int nentries, const int *step_sizes, int nsteps, void *plan,
                  int64_t plan_bytes) {
    if (!entries || !step_sizes || nsteps < 1 || nentries < nsteps) return QK_EINVAL_SHAPE;
    if (!plan || plan_bytes < qk::chain_plan_bytes(nsteps, nentries)) return QK_EINVAL_SHAPE;
    static_assert(sizeof(qk_chain_entry) == 64, "qk_chain_entry layout");
    int sum = 0;
    for (int s = 0; s < nsteps; ++s) {
        if (step_sizes[s] < 1 || step_sizes[s] > QK_MAX_BATCH) return QK_EINVAL_SHAPE;
        sum += step_sizes[s];
    }
    if (sum != nentries) return QK_EINVAL_SHAPE;
    // each entry as qk_gemv_ex / qk_gemv_swiglu with one column
    for (int i = 0; i < nentries; ++i) {
        const qk_chain_entry &e = entries[i];
        int rc = check_shape(e.type, e.N, e.K, 1);
        if (rc) return rc;
        if (e.flags & ~QK_Y_F16) return QK_EINVAL_FLAGS;
        if (e.W2 && (e.type & ~QK_PLANAR) != QK_Q4_K) return QK_EINVAL_TYPE;  // SwiGLU pairs: Q4_K
        if (e.type == QK_IQ4_XS) return QK_EINVAL_TYPE;                       // k-quants only
        if (!e.W || !aligned(e.W, 16) || (e.W2 && !aligned(e.W2, 16))) return QK_EINVAL_PTR;
        if ((rc = check_io(e.type, e.W, e.x, e.y, e.residual, e.N, e.K, 1, e.flags))) return rc;
        if (e.W2 && overlap(e.y, ((e.flags & QK_Y_F16) ? 2 : 4) * e.N, e.W2, e.N * row_bytes_of(e.type, e.K)))
            return QK_EINVAL_PTR;
    }
    // the entries of a step run concurrently: no y may overlap anything
    // another entry of the step reads or writes
    for (int s = 0, e0 = 0; s < nsteps; e0 += step_sizes[s], ++s)
        for (int i = e0; i < e0 + step_sizes[s]; ++i)
            for (int j = e0; j < e0 + step_sizes[s]; ++j) {
                if (i == j) continue;
                const qk_chain_entry &a = entries[i], &b = entries[j];
                const int64_t ya = ((a.flags & QK_Y_F16) ? 2 : 4) * a.N, yb = ((b.flags & QK_Y_F16) ? 2 : 4) * b.N;
                const int64_t wb = b.N * row_bytes_of(b.type, b.K);
                if (overlap(a.y, ya, b.W, wb) || (b.W2 && overlap(a.y, ya, b.W2, wb)) ||
                    overlap(a.y, ya, b.x, 2 * b.K) || overlap(a.y, ya, b.y, yb) ||
                    (b.residual && overlap(a.y, ya, b.residual, 4 * b.N)))
                    return QK_EINVAL_PTR;
            }
    qk::ChainEntryIn in_stack[64];
    qk::ChainEntryIn *in = nentries <= 64 ? in_stack : new (std::nothrow) qk::ChainEntryIn[nentries];
    if (!in) return QK_ELAUNCH;
    for (int i = 0; i < nentries; ++i) {
        const qk_chain_entry &e = entries[i];
        in[i] = qk::ChainEntryIn{e.type, (e.flags & QK_Y_F16) ? 1 : 0, e.W, e.W2, e.x, e.y, e.residual, e.N, e.K,
                                 row_bytes_of(e.type, e.K)};
    }
    const hipError_t err = qk::chain_plan(in, nentries, step_sizes, nsteps, plan, plan_bytes);
    if (in != in_stack) delete[] in;
    return err == hipSuccess ? QK_OK : QK_EINVAL_SHAPE;
}

int64_t qk_chain_workspace_bytes(int nsteps) {
    if (nsteps < 1) return -1;
    return ((int64_t)(nsteps + 2) * 4 + 255) / 256 * 256;
}

int qk_gemv_chain(const void *plan, const void *plan_dev, void *workspace, int64_t workspace_bytes,
                  int64_t timeout_us, void *stream) {
    if (!plan || !plan_dev || !workspace || !aligned(plan_dev, 16) || !aligned(workspace, 4)) return QK_EINVAL_PTR;
    const int nsteps = qk::chain_steps(plan);
    if (nsteps < 1) return QK_EINVAL_SHAPE;
    if (workspace_bytes < qk_chain_workspace_bytes(nsteps)) return QK_EINVAL_SHAPE;
    const hipError_t e = qk::launch_chain(plan, plan_dev, static_cast<uint32_t *>(workspace), workspace_bytes / 4,
                                          timeout_us, (hipStream_t)stream);
    if (e == hipSuccess) return QK_OK;
    snprintf(g_launch_msg, sizeof g_launch_msg, "launch failed (%s): %s", qk::chain_stage(), hipGetErrorString(e));
    return QK_ELAUNCH;
}

int qk_gemv_chain_noalloc(const void *plan, const void *plan_dev, void *status, int64_t timeout_us, void *stream) {
    static_assert(QK_CHAIN_NOALLOC_MAX_STEPS + 2 <= qk::CHAIN_SCRATCH_WORDS, "chain scratch size");
    if (!plan || !plan_dev || !aligned(plan_dev, 16) || !aligned(status, 4)) return QK_EINVAL_PTR;
    const int nsteps = qk::chain_steps(plan);
    if (nsteps < 1 || nsteps > QK_CHAIN_NOALLOC_MAX_STEPS) return QK_EINVAL_SHAPE;
    const hipError_t e = qk::launch_chain_noalloc(plan, plan_dev, status, timeout_us, (hipStream_t)stream);
    if (e == hipSuccess) return QK_OK;
    snprintf(g_launch_msg, sizeof g_launch_msg, "launch failed (%s): %s", qk::chain_stage(), hipGetErrorString(e));
    return QK_ELAUNCH;
}

int qk_dequant(int type, const void *W, void *out, int64_t N, int64_t K, void *stream) {
    const int rc = check_shape(type, N, K, 1);
    if (rc) return rc;
    if (!W || !out || !aligned(W, 16) || !aligned(out, 4)) return QK_EINVAL_PTR;
    if (overlap(out, 4 * N * K, W, N * row_bytes_of(type, K))) return QK_EINVAL_PTR;
    return launched(qk::launch_dequant(type, W, out, N, K, (hipStream_t)stream));
}

int qk_repack(int type, const void *W, void *Wp, int64_t N, int64_t K, void *stream) {
    if ((type & QK_PLANAR) || type == QK_IQ4_XS) return QK_EINVAL_TYPE;
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
        return "invalid type: expected QK_Q4_K (12), QK_Q5_K (13), QK_Q6_K (14) or QK_IQ4_XS (23); the k-quants "
               "optionally | QK_PLANAR (0x100) with ncols = 1 (qk_repack takes the type without the flag); "
               "qk_repack and chains take the k-quants only, chain SwiGLU pairs Q4_K only";
    case QK_EINVAL_SHAPE:
        return "invalid shape: need N >= 1, K a positive multiple of 256, 1 <= ncols <= 32; a chain needs 1.."
               "QK_MAX_BATCH entries per step, a workspace of qk_chain_workspace_bytes, and for "
               "qk_gemv_chain_noalloc at most QK_CHAIN_NOALLOC_MAX_STEPS (4094) steps";
    case QK_EINVAL_PTR:
        return "invalid pointer: NULL, or W/x not 16-byte aligned, or y/out/residual not 4-byte aligned (fp16 y: 2), "
               "or an output that overlaps an input (y with W or x, out with W, a batch entry's y with any entry's "
               "W, x or y, Wp with W), or a residual that overlaps y without being y (fp32 y)";
    case QK_EINVAL_FLAGS: return "invalid flags: the only epilogue flag is QK_Y_F16 (0x1)";
    case QK_ELAUNCH: return g_launch_msg;
    default: return "unknown error code";
    }
}

const char *qk_version(void) { return "qkgemv " QKGEMV_VERSION " gfx950"; }

}  // extern "C"
