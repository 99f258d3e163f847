/*
 * qkgemv.h -- C ABI of libqkgemv.so, the MI355X (gfx950) mixed k-quant GEMV.
 *
 * Operation.  y = dequant(W[N, K]) @ x[K, ncols] for weights stored in GGML
 * k-quant superblocks, the format chosen per tensor by a type flag.  This is
 * the "Mixed-Quant GEMV" of the T4 dossier's kernel prompt ("HARDWARE GROUND
 * TRUTH: 2x NVIDIA Tesla T4 (Kaggle)", section SPEC: y[N] = dequant(W[N,K]) @
 * x[K] with fp16 x and a tensor-type flag), widened to a few columns for the
 * batched verification of drafted tokens that the same dossier asks for
 * (design-doc prompt, deliverable 3, "MTP Verify Plan") and that the B70 plan
 * ("Qwen3.6 27B Single-B70 Maximum-Speed Requirements And Execution Plan",
 * Phase 3 item 7 "multi-row equivalents for verifier widths", Phase 4 "True
 * Xe2 Batched Verification") builds.
 *
 * Dequantisation (design-doc prompt, section QUANTIZATION MIX; the other
 * layouts per the GGML logic the kernel prompt names as the reference):
 *   Q4_K (144 B / 256 w):  w = d * (sc * q) - dmin * m,  q 4-bit, sc/m 6-bit
 *   Q5_K (176 B / 256 w):  the same with 5-bit q
 *   Q6_K (210 B / 256 w):  w = d * sc * (q - 32),  q 6-bit, sc int8 per 16 w
 *   IQ4_XS (136 B / 256 w): w = d * (ls - 32) * kv[q],  q 4-bit, ls 6-bit per
 *          32 w, kv GGML's 16-entry non-linear int8 codebook (kernel prompt,
 *          SPEC: IQ4_XS beside Q4_K under the same type flag)
 * Accumulation is fp32 throughout (design-doc prompt, "PHYSICS & CONTRACT").
 *
 * Memory layout (all little-endian, all buffers on the device):
 *   W  row-major superblocks: superblock s of row n starts at byte
 *      (n * K/256 + s) * qk_block_bytes(type).  GGUF prints a projection as
 *      [K_in, N_out]; that tensor is W[N, K] here.
 *   x  fp16, row-major [K][ncols]  (ncols == 1: a plain vector of K halves)
 *   y  fp32, row-major [N][ncols]
 *
 * Ownership.  Every pointer is owned by the caller; the library keeps no
 * device state, allocates nothing and never synchronises.  `stream` is a
 * hipStream_t (NULL = the null stream); every call only enqueues work on it
 * and returns.  The host side caches, per device, the compute-unit count and
 * each kernel's opt-in to large LDS, filled on first use of that device.
 * Calls are thread-safe, from any number of threads and devices.  Results are deterministic: the same inputs give the
 * same bits on every call (no atomics, fixed summation order).
 *
 * Errors.  Arguments are checked before anything is enqueued; a bad argument
 * returns a negative code and launches nothing.  A launch failure returns
 * QK_ELAUNCH.  Faults inside a kernel surface at the caller's next
 * synchronisation on the stream.  qk_strerror() names every code.
 */
#ifndef QKGEMV_H
#define QKGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tensor-type flag: the GGUF / GGML type ids of the four formats. */
enum {
    QK_Q4_K = 12,
    QK_Q5_K = 13,
    QK_Q6_K = 14,
    QK_IQ4_XS = 23
};

/* Return codes. */
enum {
    QK_OK = 0,
    QK_EINVAL_TYPE = -1,  /* type is not one of QK_Q4_K / QK_Q5_K / QK_Q6_K /
                             QK_IQ4_XS, or a flag the call does not take       */
    QK_EINVAL_SHAPE = -2, /* N < 1, K < 256, K % 256 != 0, ncols not in 1..32,
                             or a size whose byte count overflows int64          */
    QK_EINVAL_PTR = -3,   /* a NULL pointer, W or x not 16-byte aligned, y /
                             out not 4-byte aligned, or an output that overlaps
                             an input                                             */
    QK_ELAUNCH = -4,      /* the HIP launch failed (message via qk_strerror)      */
    QK_EINVAL_FLAGS = -5  /* an epilogue flag other than QK_Y_F16                 */
};

#define QK_MAX_NCOLS 32

/*
 * Row layout flag, OR'ed into a type argument: QK_Q4_K | QK_PLANAR names a
 * Q4_K tensor whose rows are in the PLANAR layout that qk_repack writes.
 * PLANAR keeps every byte of a GGUF row but groups them into planes so that
 * the pieces consecutive lanes read are consecutive in memory (S = K/256
 * superblocks, U = 4S units of 64 weights, unit u = 4s + q of superblock s):
 *   Q4_K  H[S][16] (d, dmin, scales[12] of superblock s)
 *         A[U][16] = qs[32q .. 32q+15]   B[U][16] = qs[32q+16 .. 32q+31]
 *   Q5_K  H[S][16]  QH0[S][16] = qh[0..15]  QH1[S][16] = qh[16..31]  A[U][16]  B[U][16]
 *   Q6_K  A[U][16] = ql[64n+16b ..]  B[U][16] = ql[64n+32+16b ..]  C[U][16] = qh[32n+16b ..]
 *         SC[U][4] = scales[8n+b], scales[8n+2+b], scales[8n+4+b], scales[8n+6+b]
 *         D[S][2] = d;  (q = 2n+b), then zero padding to a multiple of 16 bytes
 * Planes follow one another in the order listed; rows are
 * qk_row_bytes(type | QK_PLANAR, K) bytes apart.  This is a repack for this
 * GPU, not a format of the pages; the B70 plan ("Qwen3.6 27B Single-B70
 * Maximum-Speed Requirements And Execution Plan", Non-Negotiable Requirements,
 * item 7) allows GPU-native weight packs that are built once and kept
 * resident.  qk_gemv (ncols = 1), qk_gemv_batch and qk_dequant accept it;
 * qk_gemv with ncols > 1 does not (QK_EINVAL_TYPE).  IQ4_XS has no PLANAR
 * layout (QK_IQ4_XS | QK_PLANAR gives QK_EINVAL_TYPE everywhere).
 */
#define QK_PLANAR 0x100

/*
 * qk_gemv -- y[n][c] = sum_k dequant(W)[n][k] * x[k][c], fp32 accumulation.
 *
 *   type   QK_Q4_K, QK_Q5_K, QK_Q6_K or QK_IQ4_XS (one flag for the whole
 *          tensor); the k-quants optionally | QK_PLANAR (then ncols must be 1)
 *   W      device pointer to N rows of K/256 superblocks, 16-byte aligned
 *   x      device pointer to K*ncols fp16 values, 16-byte aligned
 *   y      device pointer to N*ncols fp32 values, 4-byte aligned (written)
 *   N      rows (output features), >= 1
 *   K      columns of W (input features), a multiple of 256
 *   ncols  columns of x and y, 1..32: 1 is the decode GEMV, 2..32 the
 *          few-column verify form with W read once per call (the B70
 *          plan's checklist asks for verifier widths up to 17)
 *   stream hipStream_t to enqueue on
 *
 * y must not overlap W or x (QK_EINVAL_PTR): other workgroups are still
 * reading them while y is written.
 *
 * Accuracy: |y - y_exact| <= 1e-4 * sum_k |w * x| for every (n, c) and every
 * input (all finite fp16 d / dmin, subnormals and signs included; any int8
 * Q6_K scale), where y_exact is the f64 dot of the dequantised weights; x is
 * never quantised.  Each 32-weight (Q6_K: 16) scale group is summed as
 * a * sum (q - c) x + (a*c - b) * sum x with a = d*sc, b = dmin*m (Q6_K:
 * b = 32 a) and an integer c nearest b/a, q - c formed exactly per weight:
 * no term exceeds three times its weight's |w x|, so the fp32 error stays
 * below about 3 * 40 * 2^-24 * sum |w x| (< 1e-5 of it), and a row whose
 * weights are all zero (d*sc*q = dmin*m) gives exactly 0.  IQ4_XS needs no
 * shift: each 32-weight group is d*(ls - 32) * sum kv[q] x with the signed
 * codebook values exact per weight, so every term is its own |w x|.
 */
int qk_gemv(int type, const void *W, const void *x, void *y,
            int64_t N, int64_t K, int ncols, void *stream);

/* Epilogue flag: y is written as fp16 (the fp32 result rounded to nearest
 * even; beyond the fp16 range it becomes +-inf) -- the fp16 y of the T4
 * kernel prompt's SPEC, for a consumer that reads fp16. */
#define QK_Y_F16 0x1

/*
 * qk_gemv_ex -- qk_gemv with a fused epilogue at the store of y:
 *
 *   y[n][c] = residual[n][c] + sum_k dequant(W)[n][k] * x[k][c]
 *
 * the output projection with its residual add in one pass (the B70 plan,
 * "Phase 3: Maximum Useful Fusion", family 1: attention / DeltaNet output and
 * FFN down with a residual epilogue).  W is still read once; the epilogue
 * adds N*ncols reads and nothing else.
 *
 *   residual  NULL, or device pointer to N*ncols fp32 values, 4-byte
 *             aligned, row-major like y.  It may be y itself (y += W x in
 *             place) when y is fp32; any other overlap with y is
 *             QK_EINVAL_PTR.
 *   flags     0 or QK_Y_F16 (y is then N*ncols fp16 values, 2-byte aligned)
 *   others    as for qk_gemv (PLANAR types with ncols = 1)
 *
 * The residual is added in fp32 to the fp32 dot product (one rounding),
 * then y is stored.  Accuracy: |y - (residual + y_exact)| <=
 * 1e-4 * sum_k |w * x| + 2^-24 |y| (fp32 y) or + 2^-11 |y| + 2^-25 (fp16 y,
 * its rounding).  qk_gemv(...) is qk_gemv_ex(..., NULL, 0, stream).
 */
int qk_gemv_ex(int type, const void *W, const void *x, void *y,
               int64_t N, int64_t K, int ncols,
               const void *residual, int flags, void *stream);

/*
 * qk_gemv_swiglu -- the gate and up projections with the SiLU gating fused,
 * in one launch:
 *
 *   g = dequant(Wg) @ x,  u = dequant(Wu) @ x,  y[n][c] = silu(g[n][c]) * u[n][c]
 *   silu(z) = z / (1 + e^-z)
 *
 * (the B70 plan, "Phase 3: Maximum Useful Fusion", family 3: the combined
 * gate/up projection with SiLU and the multiply fused; family 7 asks for the
 * same at verifier widths, hence ncols 1..32).  Every workgroup streams the
 * same rows of both tensors, so g and u never leave the chip.
 *
 *   type   one type (and layout) for both tensors, as for qk_gemv
 *   Wg, Wu device pointers to the gate and up tensors, N x K each, 16-byte
 *          aligned (they may be the same tensor)
 *   x, y, N, K, ncols, stream   as for qk_gemv; flags 0 or QK_Y_F16
 *
 * g and u are each the fp32 GEMV of qk_gemv (within 1e-4 * S_g and 1e-4 *
 * S_u of their exact values, S = sum_k |w * x|); silu uses fp32 expf.  Since
 * |silu'| <= 1.1, |y - silu(g_exact) * u_exact| <= 1.1e-4 S_g (|u| + 1e-4
 * S_u) + 1e-4 S_u (|silu(g)| + 1.1e-4 S_g) + 2^-20 |y|, plus the fp16
 * rounding with QK_Y_F16.
 */
int qk_gemv_swiglu(int type, const void *Wg, const void *Wu, const void *x, void *y,
                   int64_t N, int64_t K, int ncols, int flags, void *stream);

/*
 * qk_dequant -- out[n][k] = dequant(W)[n][k] as fp32, bit-exact: for Q4_K and
 * Q5_K the two products are exact and the subtraction is rounded once to
 * nearest-even; Q6_K values are exact.  The check path for the unpacking the
 * GEMV kernels use; not on the timed path.
 *
 *   out    device pointer to N*K fp32 values, 4-byte aligned (written),
 *          not overlapping W (QK_EINVAL_PTR)
 *   other arguments as for qk_gemv
 */
int qk_dequant(int type, const void *W, void *out, int64_t N, int64_t K, void *stream);

#define QK_MAX_BATCH 16

/* One entry of qk_gemv_batch: a one-column GEMV, fields as for qk_gemv. */
typedef struct qk_gemv_item {
    int type;
    const void *W;
    const void *x;
    void *y;
    int64_t N;
    int64_t K;
} qk_gemv_item;

/*
 * qk_gemv_batch -- `count` independent one-column GEMVs in one launch:
 * y_i = dequant(W_i) @ x_i for every entry i.  The merged launch for the
 * projections that read the same activations (q/k/v, or gate and up, of one
 * layer), or for any other set of GEMVs with no dependence between them: the
 * B70 plan asks for the fewest practical device submissions ("Non-Negotiable
 * Requirements" item 4) and puts the gap between its observed pass and the
 * Q4 read floor on per-submission overhead ("Performance Model And North
 * Star"; "Phase 2: Full Device Replay", "Phase 3: Maximum Useful Fusion").
 *
 *   items  host array of `count` entries, read during the call only
 *   count  1..QK_MAX_BATCH
 *   stream hipStream_t to enqueue on
 *
 * Adjacent entries of the same type and K that read the same x (the same
 * pointer) are streamed with the geometry of one launch of all their rows,
 * each entry taking its share of the workgroups (performance only: results
 * are as below).
 *
 * Entries may share W and x.  No entry's y may overlap any entry's W, x or y
 * (checked: QK_EINVAL_PTR).
 * Every y_i is bit-identical to what qk_gemv(type_i, W_i, x_i, y_i, N_i, K_i,
 * 1, stream) writes; the accuracy bound is that of qk_gemv.  Every entry is
 * checked before anything is enqueued, with qk_gemv's codes; a count outside
 * 1..QK_MAX_BATCH or a NULL `items` gives QK_EINVAL_SHAPE.  Nothing is
 * allocated: the entries travel in the kernel arguments.
 */
int qk_gemv_batch(const qk_gemv_item *items, int count, void *stream);

/* One GEMV of a chain step (one column): as qk_gemv_ex, or as
 * qk_gemv_swiglu when W2 is set. */
typedef struct qk_chain_entry {
    int type;             /* QK_Q4_K / QK_Q5_K / QK_Q6_K, optionally | QK_PLANAR
                             (QK_IQ4_XS: QK_EINVAL_TYPE)                          */
    int flags;            /* 0 or QK_Y_F16                                          */
    const void *W;        /* N rows of superblocks, 16-byte aligned                 */
    const void *W2;       /* NULL, or the up tensor of a SwiGLU pair (Q4_K only):
                             y = silu(W x) * (W2 x)                                 */
    const void *x;        /* K fp16 values, 16-byte aligned                         */
    void *y;              /* N fp32 values (fp16 with QK_Y_F16)                     */
    const void *residual; /* NULL or N fp32 values added at the store; may be y     */
    int64_t N;
    int64_t K;
} qk_chain_entry;

/*
 * The decode token as one launch: a chain of steps, each a set of up to
 * QK_MAX_BATCH independent one-column GEMVs (qk_chain_entry), run in order.
 * A step may read (as x or residual) what an earlier step wrote: between
 * consecutive steps every workgroup of the launch waits until all of them
 * have stored their results (a device-wide barrier), exactly as back-to-back
 * launches on one stream would order them.  The weights of a step do not
 * depend on earlier steps, so each workgroup issues the first of them before
 * it waits: the fill of one GEMV overlaps the end of the previous one instead
 * of following it (the B70 plan, "Performance Model And North Star" and
 * "Phase 2: Full Device Replay", puts the gap between its observed pass and
 * the Q4 read floor on per-submission overhead; Non-Negotiable Requirements
 * item 4 asks for the fewest practical device submissions).
 *
 * Every y is bit-identical to what qk_gemv_ex / qk_gemv_swiglu write for the
 * same entry, with the same accuracy bound.
 *
 * Speed: on MI355X a step runs about twice as long as the same GEMV as a
 * launch of its own (one 1024-thread workgroup per CU, bodies sharing one
 * register budget), so a 448-GEMV decode token (14.6 GB of weights) takes
 * 8.0 ms as a chain against 4.2 ms as a captured graph of qk_gemv_batch /
 * qk_gemv_swiglu launches.  The chain is for callers that want one
 * submission per token and cannot capture graphs.
 *
 * Use: qk_chain_plan (host only) writes a plan of qk_chain_plan_bytes into
 * caller host memory; the caller copies it, unchanged, to device memory
 * (plan_dev, 16-byte aligned) and passes both to qk_gemv_chain, as often as
 * it likes while the tensors it names stay where they are.  The plan is made
 * for the current device (its compute-unit count) and refuses another.
 */

/* Bytes of a plan of nsteps steps and nentries entries, or -1. */
int64_t qk_chain_plan_bytes(int nsteps, int nentries);

/*
 *   entries     host array of nentries entries, step after step
 *   step_sizes  host array of nsteps counts, each 1..QK_MAX_BATCH, summing to
 *               nentries: step s runs the next step_sizes[s] entries
 *   plan        host memory of plan_bytes >= qk_chain_plan_bytes (written)
 * Every entry is checked as qk_gemv_ex / qk_gemv_swiglu check theirs, and no
 * y may overlap what another entry of the same step reads or writes
 * (QK_EINVAL_PTR).  A bad count or size, or a step the launch geometry cannot
 * place, gives QK_EINVAL_SHAPE.  Nothing touches the GPU.
 */
int qk_chain_plan(const qk_chain_entry *entries, int nentries, const int *step_sizes, int nsteps,
                  void *plan, int64_t plan_bytes);

/* Bytes of the synchronisation workspace of a chain of nsteps steps, or -1. */
int64_t qk_chain_workspace_bytes(int nsteps);

/*
 * qk_gemv_chain -- run a planned chain on `stream`: one small kernel clears
 * the workspace, then one cooperative launch with a workgroup per compute
 * unit runs every step.
 *
 *   plan        the host plan qk_chain_plan wrote (read during the call)
 *   plan_dev    the same bytes in device memory, 16-byte aligned
 *   workspace   device memory of workspace_bytes >= qk_chain_workspace_bytes
 *               (nsteps), 4-byte aligned, used by this call only: concurrent
 *               chains need workspaces of their own
 *   timeout_us  bound on each wait at a barrier (<= 0: 2 s)
 * Every wait is bounded: if one expires, the workgroup sets bit 0 of the
 * first 32-bit word of the workspace (QK_CHAIN_TIMEOUT) and every workgroup
 * abandons the chain at its next wait -- the outputs are then incomplete.
 * Read that word after synchronising to check a run.  Returns QK_OK, an
 * argument error, or QK_ELAUNCH (including a grid the device cannot hold).
 */
#define QK_CHAIN_TIMEOUT 0x1
int qk_gemv_chain(const void *plan, const void *plan_dev, void *workspace, int64_t workspace_bytes,
                  int64_t timeout_us, void *stream);

/*
 * qk_gemv_chain_noalloc -- qk_gemv_chain for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results, with the barrier
 * counters in a 16 KiB array the library holds on each GPU until the process
 * ends instead of a caller workspace.  Nothing is allocated per call.
 *
 *   plan, plan_dev, timeout_us, stream   as for qk_gemv_chain
 *   status      NULL, or a 4-byte aligned device word that receives the
 *               run's flag word (QK_CHAIN_TIMEOUT) once the chain has run
 * A plan of more than QK_CHAIN_NOALLOC_MAX_STEPS steps gives QK_EINVAL_SHAPE
 * before anything is launched.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must not be made; each call clears the words it uses before its chain.
 */
#define QK_CHAIN_NOALLOC_MAX_STEPS 4094
int qk_gemv_chain_noalloc(const void *plan, const void *plan_dev, void *status, int64_t timeout_us, void *stream);

/*
 * qk_repack -- rewrite N GGUF rows of `type` (no flag) as PLANAR rows: Wp is
 * then a valid QK_PLANAR tensor with the same weights.  One-time, outside the
 * decode loop; every y and every dequantised weight computed from Wp is
 * bit-identical to the one computed from W.
 *
 *   W      device pointer to N GGUF rows, 16-byte aligned (read)
 *   Wp     device pointer to N * qk_row_bytes(type | QK_PLANAR, K) bytes,
 *          16-byte aligned, not overlapping W (written)
 * Errors as for qk_dequant; overlapping W and Wp give QK_EINVAL_PTR; type
 * QK_IQ4_XS gives QK_EINVAL_TYPE (it has no PLANAR layout).
 */
int qk_repack(int type, const void *W, void *Wp, int64_t N, int64_t K, void *stream);

/* Bytes per 256-weight superblock: 144 / 176 / 210, or -1 for a bad type. */
int qk_block_bytes(int type);

/* Bytes per row of K weights: (K/256) * qk_block_bytes(type) for a GGUF type;
 * for type | QK_PLANAR the PLANAR row (the same, rounded up to 16 bytes for
 * Q6_K); -1 for a bad type or a K that is not a positive multiple of 256. */
int64_t qk_row_bytes(int type, int64_t K);

/* Static description of a return code; for QK_ELAUNCH the HIP error text of
 * the calling thread's last failed launch.  Never NULL. */
const char *qk_strerror(int code);

/* Library version string, e.g. "qkgemv 0.1.0 gfx950". */
const char *qk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QKGEMV_H */
