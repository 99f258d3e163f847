/* C99 client of include/qkgemv.h, built and run by tests/test_c_abi.py on
 * the CPU: it links libqkgemv.so like any C program would and calls only
 * what needs no GPU -- sizes, strings and the argument checks that return
 * before anything is enqueued.  Exit status 0 = every check held; otherwise
 * the number of failed checks (each is printed). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qkgemv.h"

static int failures = 0;

static void expect(int ok, const char *what) {
    if (!ok) {
        printf("FAIL: %s\n", what);
        ++failures;
    }
}

int main(void) {
    /* 16-byte aligned stand-ins: the checks below fail before any access */
    static uint8_t buf[4096] __attribute__((aligned(16)));
    void *W = buf, *x = buf + 1024, *y = buf + 2048;
    const qk_gemv_item bad_type = {99, buf, buf + 1024, buf + 2048, 4, 256};
    qk_gemv_item items[2];

    expect(qk_block_bytes(QK_Q4_K) == 144, "Q4_K block bytes");
    expect(qk_block_bytes(QK_Q5_K) == 176, "Q5_K block bytes");
    expect(qk_block_bytes(QK_Q6_K) == 210, "Q6_K block bytes");
    expect(qk_block_bytes(7) == -1, "unknown type block bytes");
    expect(qk_row_bytes(QK_Q6_K, 5120) == 20 * 210, "Q6_K GGUF row bytes");
    expect(qk_row_bytes(QK_Q6_K | QK_PLANAR, 5120) == 4208, "Q6_K PLANAR row bytes (padded to 16)");
    expect(qk_row_bytes(QK_Q4_K, 300) == -1, "K not a multiple of 256");
    expect(qk_version() != NULL && strstr(qk_version(), "gfx950") != NULL, "version names the target");
    expect(strcmp(qk_strerror(QK_OK), "ok") == 0, "strerror(ok)");
    expect(qk_strerror(QK_EINVAL_SHAPE) != NULL && qk_strerror(12345) != NULL, "strerror never NULL");

    expect(qk_gemv(99, W, x, y, 4, 256, 1, NULL) == QK_EINVAL_TYPE, "gemv: bad type");
    expect(qk_gemv(QK_Q4_K, W, x, y, 0, 256, 1, NULL) == QK_EINVAL_SHAPE, "gemv: N = 0");
    expect(qk_gemv(QK_Q4_K, W, x, y, 4, 200, 1, NULL) == QK_EINVAL_SHAPE, "gemv: K % 256");
    expect(qk_gemv(QK_Q4_K, W, x, y, 4, 256, QK_MAX_NCOLS + 1, NULL) == QK_EINVAL_SHAPE, "gemv: ncols");
    expect(qk_gemv(QK_Q4_K | QK_PLANAR, W, x, y, 4, 256, 2, NULL) == QK_EINVAL_TYPE, "gemv: PLANAR, ncols 2");
    expect(qk_gemv(QK_Q4_K, NULL, x, y, 4, 256, 1, NULL) == QK_EINVAL_PTR, "gemv: NULL W");
    expect(qk_gemv(QK_Q4_K, buf + 8, x, y, 4, 256, 1, NULL) == QK_EINVAL_PTR, "gemv: misaligned W");
    expect(qk_gemv_ex(QK_Q4_K, W, x, y, 4, 256, 1, NULL, 0x2, NULL) == QK_EINVAL_FLAGS, "gemv_ex: flags");
    expect(qk_gemv_ex(QK_Q4_K, W, x, y, 4, 256, 1, buf + 2052, 0, NULL) == QK_EINVAL_PTR,
           "gemv_ex: residual overlapping y");
    expect(qk_gemv_swiglu(QK_Q4_K, W, NULL, x, y, 4, 256, 1, 0, NULL) == QK_EINVAL_PTR, "swiglu: NULL Wu");
    expect(qk_dequant(QK_Q6_K, W, y, 4, 100, NULL) == QK_EINVAL_SHAPE, "dequant: K % 256");
    expect(qk_repack(QK_Q4_K | QK_PLANAR, W, y, 4, 256, NULL) == QK_EINVAL_TYPE, "repack: flagged type");
    expect(qk_repack(QK_Q4_K, W, W, 4, 256, NULL) == QK_EINVAL_PTR, "repack: W and Wp overlap");
    expect(qk_gemv_batch(NULL, 1, NULL) == QK_EINVAL_SHAPE, "batch: NULL items");
    items[0] = bad_type;
    items[1] = bad_type;
    expect(qk_gemv_batch(items, 0, NULL) == QK_EINVAL_SHAPE, "batch: count 0");
    expect(qk_gemv_batch(items, QK_MAX_BATCH + 1, NULL) == QK_EINVAL_SHAPE, "batch: count too large");
    expect(qk_gemv_batch(items, 2, NULL) == QK_EINVAL_TYPE, "batch: bad entry type");

    /* IQ4_XS: a type of its own, no PLANAR layout */
    expect(qk_block_bytes(QK_IQ4_XS) == 136, "IQ4_XS block bytes");
    expect(qk_row_bytes(QK_IQ4_XS, 5120) == 20 * 136, "IQ4_XS row bytes");
    expect(qk_row_bytes(QK_IQ4_XS | QK_PLANAR, 5120) == -1, "IQ4_XS has no PLANAR rows");
    expect(qk_gemv(QK_IQ4_XS | QK_PLANAR, W, x, y, 4, 256, 1, NULL) == QK_EINVAL_TYPE, "gemv: IQ4_XS | PLANAR");
    expect(qk_repack(QK_IQ4_XS, W, y, 4, 256, NULL) == QK_EINVAL_TYPE, "repack: IQ4_XS");

    /* chains: sizes and the checks made before anything reaches the GPU */
    {
        qk_chain_entry ce = {QK_IQ4_XS, 0, W, NULL, x, y, NULL, 4, 256};
        int one = 1;
        static unsigned char plan[4096];
        expect(qk_chain_plan_bytes(0, 1) == -1 && qk_chain_plan_bytes(1, 0) == -1, "chain plan bytes: empty");
        expect(qk_chain_plan_bytes(1, 1) > 0 && qk_chain_plan_bytes(1, 1) <= (int64_t)sizeof plan,
               "chain plan bytes: one entry");
        expect(qk_chain_workspace_bytes(0) == -1 && qk_chain_workspace_bytes(10) == 256, "chain workspace bytes");
        expect(qk_chain_plan(&ce, 1, &one, 1, plan, (int64_t)sizeof plan) == QK_EINVAL_TYPE, "chain: IQ4_XS entry");
        ce.type = QK_Q4_K;
        one = QK_MAX_BATCH + 1;
        expect(qk_chain_plan(&ce, 1, &one, 1, plan, (int64_t)sizeof plan) == QK_EINVAL_SHAPE, "chain: step size");
        expect(qk_gemv_chain(NULL, W, W, 256, 0, NULL) == QK_EINVAL_PTR, "chain: NULL plan");
        expect(qk_gemv_chain_noalloc(NULL, W, NULL, 0, NULL) == QK_EINVAL_PTR, "chain noalloc: NULL plan");
        expect(qk_gemv_chain_noalloc(plan, buf + 8, NULL, 0, NULL) == QK_EINVAL_PTR,
               "chain noalloc: misaligned plan_dev");
        memset(plan, 0, sizeof plan);  /* not a plan */
        expect(qk_gemv_chain_noalloc(plan, W, NULL, 0, NULL) == QK_EINVAL_SHAPE, "chain noalloc: not a plan");
    }

    if (failures == 0) printf("c_abi_check: all checks held\n");
    return failures;
}
