/*
 * qk_oracle.c -- CPU oracle for the k-quant dequantisation and GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU product path
 * never calls it, links it or includes anything from this directory, and this
 * file includes nothing from the GPU path.
 *
 * It is deliberately plain: one weight at a time, scalar code, no blocking,
 * no fusion, no reordering of the sums.  Build it with -ffp-contract=off so
 * that every float operation is the one written here.
 *
 * Sources (the pages this follows):
 *  [T4-design]  "HARDWARE GROUND TRUTH: 2x NVIDIA Tesla T4 (Kaggle)", engine
 *               design-doc prompt, section "QUANTIZATION MIX": the Q4_K
 *               superblock struct { half d; half dmin; uint8 scales[12];
 *               uint8 qs[128]; } holding 256 weights in 144 bytes, and the
 *               dequantisation w = d * (sc * q4) - dmin * m.
 *  [T4-gemv]    Same dossier, "Mixed-Quant GEMV" kernel prompt, section
 *               "SPEC": the operation y[N] = dequant(W[N,K]) @ x[K] with fp16
 *               x, a per-tensor type flag selecting Q4_K / Q5_K, and the
 *               statement that the reference is the standard GGML
 *               dequantisation logic.
 *  [T4-design]  section "PHYSICS & CONTRACT": fp32 accumulation for all
 *               reductions.
 *  [T4-design]  section "QUANTIZATION MIX" also lists IQ4_XS among the mixed
 *               quants ("4-bit with specific superblock packing"), and
 *               [T4-gemv] "SPEC" asks for it beside Q4_K and Q5_K under the
 *               same type flag, with GGML's dequantisation as the reference.
 *  [DP4A-issue] "DP4A Q4K/Q6K GEMV profile is catastrophic through the Gated
 *               DeltaNet recurrence", issue description: GEMV error is
 *               measured against an exact f64 dot of the dequantised weights.
 *
 * Readings where the pages are silent (the pages give only the Q4_K struct
 * and formula; Q5_K and Q6_K are named but not laid out):
 *  - The 6-bit scale/min packing of scales[12], the nibble order of qs, the
 *    Q5_K high-bit plane and the whole Q6_K layout follow the GGML k-quant
 *    format that [T4-gemv] points to (field offsets are written out next to
 *    each function below).
 *  - Dequantised weights are fp32 values.  For Q4_K/Q5_K the products
 *    d*(sc*q) and dmin*m are exact in fp32 for every finite fp16 d, dmin
 *    (at most 11+6+5 significant bits), so the only rounding is the one
 *    fp32 subtraction, round-to-nearest-even.  For Q6_K, d*(sc*(q-32)) is
 *    exact (at most 11+7+5 bits): no rounding at all.
 *  - IQ4_XS follows GGML's block_iq4_xs (136 bytes: fp16 d, a 16-bit word
 *    and 4 bytes of 6-bit sub-block scales, 128 bytes of 4-bit indices into
 *    GGML's 16-entry non-linear int8 codebook shared with IQ4_NL); offsets
 *    and bit positions are written out below.  w = d * (ls - 32) * kv[idx]:
 *    |ls - 32| <= 32 and |kv| <= 127 make the integer factor at most 12
 *    significant bits, so with d's 11 the product is exact in fp32.
 *  - fp16 widening is exact, subnormals included (no flush to zero).
 *  - The GEMV reference is the f64 sum over k in ascending order of
 *    f64(w[n,k]) * f64(x[k,c]); alongside it the oracle returns
 *    S[n,c] = sum_k |w[n,k] * x[k,c]|, the scale of the per-row tolerance.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* GGUF tensor-type ids of the formats. */
#define ORACLE_Q4_K 12
#define ORACLE_Q5_K 13
#define ORACLE_Q6_K 14
#define ORACLE_IQ4_XS 23

#define ORACLE_QK 256 /* weights per superblock */

int oracle_block_bytes(int type)
{
    switch (type) {
    case ORACLE_Q4_K: return 144; /* 2 + 2 + 12 + 128 */
    case ORACLE_Q5_K: return 176; /* 2 + 2 + 12 + 32 + 128 */
    case ORACLE_Q6_K: return 210; /* 128 + 64 + 16 + 2 */
    case ORACLE_IQ4_XS: return 136; /* 2 + 2 + 4 + 128 */
    default: return -1;
    }
}

/* IEEE binary16 -> binary32, exact.  value = (-1)^s * 2^(e-15) * (1 + m/1024)
 * for 0 < e < 31, (-1)^s * 2^-14 * (m/1024) for e == 0, inf/NaN for e == 31. */
float oracle_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);
    return sign ? -v : v;
}

void oracle_half_to_float_n(const uint16_t *h, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_half_to_float(h[i]);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Q4_K / Q5_K 6-bit scale and min of sub-block j (0..7) from scales[12].
 * Bytes 0..3 hold sc_0..3 in their low 6 bits, bytes 4..7 hold m_0..3;
 * bytes 8..11 hold the low nibbles of sc_4..7 (low half) and m_4..7 (high
 * half); the spare top 2 bits of bytes 0..3 / 4..7 carry bits 4..5 of
 * sc_4..7 / m_4..7. */
void oracle_k_scale_min(const uint8_t *scales, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = scales[j] & 63;
        *m = scales[j + 4] & 63;
    } else {
        *sc = (scales[j + 4] & 0x0f) | ((scales[j - 4] >> 6) << 4);
        *m = (scales[j + 4] >> 4) | ((scales[j] >> 6) << 4);
    }
}

/* Integer quant of weight i (0..255) of one superblock.
 *  Q4_K: qs[128] at byte 16.  Weights come in 4 chunks of 64; chunk c uses
 *        qs[32c .. 32c+31]; its first 32 weights are the low nibbles, the
 *        next 32 the high nibbles.  q in 0..15.
 *  Q5_K: qh[32] at byte 16, qs[128] at byte 48.  Low 4 bits as Q4_K, bit 4
 *        is bit j of qh[i mod 32], j = i/32 the sub-block.  q in 0..31.
 *  Q6_K: ql[128] at 0, qh[64] at 128.  Weights come in 2 halves of 128, each
 *        in 4 quarters t of 32; quarter t of half n takes its low 4 bits from
 *        ql[64n + 32(t mod 2) + l] (low nibble for t < 2, high for t >= 2)
 *        and its high 2 bits from bits 2t, 2t+1 of qh[32n + l].  q in 0..63,
 *        returned before the -32 offset.
 *  IQ4_XS: qs[128] at byte 8, 16 bytes per sub-block ib = i/32: weight
 *        32ib + l takes the low nibble of qs[16ib + l] for l < 16 and the
 *        high nibble of qs[16ib + l - 16] for l >= 16.  The 4-bit index into
 *        the codebook (oracle_iq4nl_value), 0..15. */
int oracle_quant(int type, const uint8_t *sb, int i)
{
    int l = i % 32;
    if (type == ORACLE_Q4_K || type == ORACLE_Q5_K) {
        const uint8_t *qs = sb + (type == ORACLE_Q4_K ? 16 : 48);
        int c = i / 64, h = (i / 32) % 2;
        int q = (qs[32 * c + l] >> (4 * h)) & 0x0f;
        if (type == ORACLE_Q5_K) {
            const uint8_t *qh = sb + 16;
            int j = i / 32;
            q |= ((qh[l] >> j) & 1) << 4;
        }
        return q;
    }
    if (type == ORACLE_Q6_K) {
        const uint8_t *ql = sb, *qh = sb + 128;
        int n = i / 128, t = (i % 128) / 32;
        int lo = (ql[64 * n + 32 * (t % 2) + l] >> (4 * (t / 2))) & 0x0f;
        int hi = (qh[32 * n + l] >> (2 * t)) & 3;
        return lo | (hi << 4);
    }
    if (type == ORACLE_IQ4_XS) {
        const uint8_t *qs = sb + 8;
        int ib = i / 32;
        return (qs[16 * ib + (l % 16)] >> (4 * (l / 16))) & 0x0f;
    }
    return -1;
}

/* Q6_K signed 8-bit scale of weight i: scales[16] at byte 192, one per 16
 * consecutive weights. */
int oracle_q6k_scale(const uint8_t *sb, int i) { return (int8_t)sb[192 + i / 16]; }

/* IQ4_XS: d fp16 @0, scales_h (16 bits, little-endian) @2, scales_l[4] @4,
 * qs[128] @8.  Sub-block ib (0..7) holds weights 32ib .. 32ib+31 and the
 * 6-bit scale ls: its low 4 bits are nibble (ib mod 2) of scales_l[ib/2]
 * (low nibble for even ib), its high 2 bits are bits 2ib, 2ib+1 of
 * scales_h. */
int oracle_iq4xs_scale(const uint8_t *sb, int ib)
{
    int lo = (sb[4 + ib / 2] >> (4 * (ib % 2))) & 0x0f;
    int hi = (rd16(sb + 2) >> (2 * ib)) & 3;
    return lo | (hi << 4);
}

/* The non-linear codebook of the 4-bit indices (IQ4_NL / IQ4_XS). */
static const int iq4nl_codebook[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                       1,    13,   25,  38,  53,  69,  89,  113};

int oracle_iq4nl_value(int idx) { return (idx >= 0 && idx < 16) ? iq4nl_codebook[idx] : 0; }

/* Dequantise one superblock into out[256]. */
static void dequant_block(int type, const uint8_t *sb, float *out)
{
    if (type == ORACLE_Q4_K || type == ORACLE_Q5_K) {
        float d = oracle_half_to_float(rd16(sb + 0));
        float dmin = oracle_half_to_float(rd16(sb + 2));
        for (int i = 0; i < ORACLE_QK; i++) {
            int sc, m;
            oracle_k_scale_min(sb + 4, i / 32, &sc, &m);
            int q = oracle_quant(type, sb, i);
            /* w = d * (sc * q) - dmin * m: both products exact, one rounding. */
            float a = d * (float)(sc * q);
            float b = dmin * (float)m;
            out[i] = a - b;
        }
    } else if (type == ORACLE_Q6_K) {
        float d = oracle_half_to_float(rd16(sb + 208));
        for (int i = 0; i < ORACLE_QK; i++) {
            int sc = oracle_q6k_scale(sb, i);
            int q = oracle_quant(type, sb, i);
            out[i] = d * (float)(sc * (q - 32)); /* exact */
        }
    } else { /* ORACLE_IQ4_XS: d is the first field */
        float d = oracle_half_to_float(rd16(sb));
        for (int i = 0; i < ORACLE_QK; i++) {
            int ls = oracle_iq4xs_scale(sb, i / 32);
            int kv = oracle_iq4nl_value(oracle_quant(type, sb, i));
            out[i] = d * (float)((ls - 32) * kv); /* exact */
        }
    }
}

/* One row of K weights: superblocks stored back to back. */
static void dequant_row(int type, const uint8_t *row, int64_t K, float *out)
{
    int bb = oracle_block_bytes(type);
    for (int64_t s = 0; s < K / ORACLE_QK; s++)
        dequant_block(type, row + s * bb, out + s * ORACLE_QK);
}

static int check_args(int type, int64_t N, int64_t K, int ncols)
{
    if (oracle_block_bytes(type) < 0) return -1;
    if (N < 0 || K < 0 || K % ORACLE_QK != 0) return -2;
    if (ncols < 1) return -2;
    return 0;
}

/* ---- row-parallel driver (plain pthreads, contiguous row ranges) ---- */

typedef struct {
    int type;
    const uint8_t *W;
    const double *xd; /* x widened to f64, [K][ncols] */
    int64_t K;
    int ncols;
    int64_t r0, r1;
    float *deq_out; /* dequant mode: [N][K] */
    double *y, *S;  /* gemv mode: [N][ncols] */
} job_t;

static void *dequant_worker(void *arg)
{
    job_t *j = (job_t *)arg;
    int64_t rb = (j->K / ORACLE_QK) * oracle_block_bytes(j->type);
    for (int64_t n = j->r0; n < j->r1; n++)
        dequant_row(j->type, j->W + n * rb, j->K, j->deq_out + n * j->K);
    return NULL;
}

static void *gemv_worker(void *arg)
{
    job_t *j = (job_t *)arg;
    int64_t rb = (j->K / ORACLE_QK) * oracle_block_bytes(j->type);
    float *w = (float *)malloc(sizeof(float) * (size_t)(j->K > 0 ? j->K : 1));
    if (!w) return (void *)1;
    for (int64_t n = j->r0; n < j->r1; n++) {
        dequant_row(j->type, j->W + n * rb, j->K, w);
        for (int c = 0; c < j->ncols; c++) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < j->K; k++) {
                double p = (double)w[k] * j->xd[k * j->ncols + c];
                acc += p;
                mag += fabs(p);
            }
            j->y[n * j->ncols + c] = acc;
            j->S[n * j->ncols + c] = mag;
        }
    }
    free(w);
    return NULL;
}

static int run_rows(void *(*fn)(void *), job_t *tmpl, int64_t N, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > N) nthreads = (int)(N > 0 ? N : 1);
    pthread_t tid[256];
    job_t jobs[256];
    int rc = 0;
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = *tmpl;
        jobs[t].r0 = N * t / nthreads;
        jobs[t].r1 = N * (t + 1) / nthreads;
    }
    if (nthreads == 1) {
        if (fn(&jobs[0]) != NULL) rc = -5;
        return rc;
    }
    for (int t = 0; t < nthreads; t++)
        if (pthread_create(&tid[t], NULL, fn, &jobs[t]) != 0) {
            /* fall back to running the rest inline */
            for (int u = t; u < nthreads; u++)
                if (fn(&jobs[u]) != NULL) rc = -5;
            nthreads = t;
            break;
        }
    for (int t = 0; t < nthreads; t++) {
        void *ret = NULL;
        pthread_join(tid[t], &ret);
        if (ret != NULL) rc = -5;
    }
    return rc;
}

/* out[N][K] = dequantised weights (fp32).  Returns 0, or a negative code for
 * an unknown type (-1) or a bad shape (-2). */
int oracle_dequant(int type, const uint8_t *W, int64_t N, int64_t K, float *out, int nthreads)
{
    int rc = check_args(type, N, K, 1);
    if (rc) return rc;
    job_t j = {0};
    j.type = type; j.W = W; j.K = K; j.deq_out = out;
    return run_rows(dequant_worker, &j, N, nthreads);
}

/* y[N][ncols] = sum_k f64(w[n,k]) * f64(x[k,c]) in ascending k, and
 * S[N][ncols] = sum_k |f64(w[n,k]) * f64(x[k,c])|.  x is fp16 [K][ncols]. */
int oracle_gemv(int type, const uint8_t *W, const uint16_t *x, int64_t N, int64_t K, int ncols,
                double *y, double *S, int nthreads)
{
    int rc = check_args(type, N, K, ncols);
    if (rc) return rc;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(K * ncols > 0 ? K * ncols : 1));
    if (!xd) return -5;
    for (int64_t i = 0; i < K * ncols; i++)
        xd[i] = (double)oracle_half_to_float(x[i]);
    job_t j = {0};
    j.type = type; j.W = W; j.xd = xd; j.K = K; j.ncols = ncols; j.y = y; j.S = S;
    rc = run_rows(gemv_worker, &j, N, nthreads);
    free(xd);
    return rc;
}
