// qk_verify.hip -- few-column verify GEMV (ncols 2..8) on gfx950 matrix cores.
//
// y[n][c] = sum_k dequant(W)[n][k] * x[k][c] for c < ncols <= 8: the batched
// verification of drafted tokens (T4 dossier design-doc prompt, deliverable 3
// "MTP Verify Plan"; B70 plan, Phase 3 item 7 and Phase 4 "True Xe2 Batched
// Verification").  W is read from HBM once per call whatever ncols is.
//
// Matrix-core mapping (v_mfma_f32_4x4x4_16b_f16: 16 independent 4x4x4
// blocks, block = 4 consecutive lanes; lane 4b+j supplies row j of A and
// column j of B and receives D[0..3][j]):
//   B column j = W row (4*quad + j): the quant patterns of one 32-bit quant
//                word (pairs A and B, weights (l, l+2, l+1, l+3)) -- exact
//                fp16 values p * 2^-24, as in the one-column kernel;
//   A row j    = x column (4*cb + j) at the same four weights, from LDS;
//   D[i][j]    = sum over the word of x_i * q_j, accumulated in fp32 over a
//                sub-block (8 words), then scaled per row by d*sc (and the
//                min term dmin*m*sum(x) subtracted) in fp32.
// So a lane ends up with all columns of its own row.  The 16 blocks of a
// wave are 16 consecutive units of the same four rows; their partial sums are
// reduced across the blocks at the end of each work item.
#include "qk_format.h"
#include "qk_launch.h"

namespace qk {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int VSLOT = 36;  // dwords per unit slot: 32 of x pairs + 4 of padding

__device__ __forceinline__ float4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, float4_t c) {
    const half4_t a = __builtin_bit_cast(half4_t, make_uint2(a0, a1));
    const half4_t b = __builtin_bit_cast(half4_t, make_uint2(b0, b1));
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0);
}

template <int T>
__host__ __device__ constexpr int groups_per_unit() { return T == Q6_K ? 4 : 2; }

// Position of weight k (tile-relative, k < kt) in the LDS x planes: unit slot
// u and half index within the slot.  Q4_K/Q5_K: unit u = weights 64u..64u+63
// in order; Q6_K: unit 4s+2n+b holds quarter t at halves 16t..16t+15.  Groups
// of four halves are stored in the order (0, 2, 1, 3).  g = scale group.
template <int T>
__device__ __forceinline__ void x_place(int k, int &u, int &pos, int &g) {
    int r, base;
    if constexpr (T == Q6_K) {
        const int s = k >> 8, kk = k & 255;
        const int n = kk >> 7, t = (kk >> 5) & 3, b = (kk >> 4) & 1, l = kk & 15;
        u = 4 * s + 2 * n + b;
        base = 16 * t + (l & ~3);
        r = l & 3;
        g = t;
    } else {
        u = k >> 6;
        const int kk = k & 63;
        base = kk & ~3;
        r = kk & 3;
        g = kk >> 5;
    }
    const int perm = (r == 0) ? 0 : (r == 1) ? 2 : (r == 2) ? 1 : 3;
    pos = base + perm;
}

// Stage x[k0 .. k0+kt)[0..nc) into per-column planes of unit slots, then the
// fp32 sums of each scale group (fixed order).  planes: nc * units * VSLOT
// dwords; sums: nc * units * G floats.
template <int T>
__device__ void stage_xv(const uint16_t *__restrict__ x, int k0, int kt, int nc, uint32_t *planes, float *sums) {
    const int units = kt >> 6;
    uint16_t *ph = reinterpret_cast<uint16_t *>(planes);
    for (int e = (int)threadIdx.x; e < kt * nc; e += (int)blockDim.x) {
        const int k = e / nc, c = e - k * nc;
        int u, pos, g;
        x_place<T>(k, u, pos, g);
        ph[2 * VSLOT * (c * units + u) + pos] = x[(size_t)(k0 + k) * nc + c];
    }
    __syncthreads();
    constexpr int G = groups_per_unit<T>();
    constexpr int GW = 64 / G;  // weights per group
    for (int e = (int)threadIdx.x; e < nc * units * G; e += (int)blockDim.x) {
        const int c = e / (units * G), rem = e - c * units * G, u = rem / G, g = rem - u * G;
        const uint32_t *src = planes + VSLOT * (c * units + u) + (GW / 2) * g;
        float s = 0.f;
        for (int i = 0; i < GW / 2; ++i) s += f16_lo(src[i]) + f16_hi(src[i]);
        sums[(c * units + u) * G + g] = s;
    }
    __syncthreads();
}

// One work item = (row quad, step of 16 units).  Accumulates this lane's
// contribution for its row into acc[4*NCB] (columns 4*cb + i in acc[4*cb+i]).
template <int T, int NCB>
__device__ __forceinline__ void item_dot(const Unit<T> &U, int q, const KScaleSel &sel, const uint32_t *planes,
                                         const float *sums, int units, int u, int j, int nc, float *acc) {
    constexpr int G = groups_per_unit<T>();
    // A operands come from the planes of columns 4*cb + j (zero when past nc)
    const uint32_t *xa[NCB];
    bool colok[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int c = 4 * cb + j;
        colok[cb] = c < nc;
        xa[cb] = planes + VSLOT * ((colok[cb] ? c : 0) * units + u);
    }
    if constexpr (T == Q6_K) {
        float4_t D[NCB][4];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int t = 0; t < 4; ++t) D[cb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t p[8];
            U.patterns(i, q, p);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const uint2 xv = *reinterpret_cast<const uint2 *>(xa[cb] + 8 * t + 2 * i);
                    const uint32_t a0 = colok[cb] ? xv.x : 0u, a1 = colok[cb] ? xv.y : 0u;
                    D[cb][t] = mfma4(a0, a1, p[2 * t], p[2 * t + 1], D[cb][t]);
                }
        }
        const float d = f16_lo(U.d);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float ds = d * (float)U.scale(t, q);
            const float k = t < 2 ? 0x1p24f : 0x1p20f;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * cb + i;
                    const float xs = c < nc ? sums[(c * units + u) * G + t] : 0.f;
                    acc[4 * cb + i] += ds * (D[cb][t][i] * k - 32.f * xs);
                }
        }
    } else {
        float4_t Dl[NCB], Dh[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Dl[cb] = Dh[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t p[4];
            U.patterns(i, q, p);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const uint2 xl = *reinterpret_cast<const uint2 *>(xa[cb] + 2 * i);
                const uint2 xh = *reinterpret_cast<const uint2 *>(xa[cb] + 16 + 2 * i);
                Dl[cb] = mfma4(colok[cb] ? xl.x : 0u, colok[cb] ? xl.y : 0u, p[0], p[1], Dl[cb]);
                Dh[cb] = mfma4(colok[cb] ? xh.x : 0u, colok[cb] ? xh.y : 0u, p[2], p[3], Dh[cb]);
            }
        }
        const uint4 h = U.header();
        const KScales s = k_scales(h, sel);
        const float d = f16_lo(h.x), dmin = f16_hi(h.x);
        const float fl = d * (float)s.sc_lo * 0x1p24f, fh = d * (float)s.sc_hi * 0x1p20f;
        const float ml = dmin * (float)s.m_lo, mh = dmin * (float)s.m_hi;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 4 * cb + i;
                const float2 xs = c < nc ? *reinterpret_cast<const float2 *>(sums + (c * units + u) * 2)
                                         : make_float2(0.f, 0.f);
                acc[4 * cb + i] += fl * Dl[cb][i] + fh * Dh[cb][i] - (ml * xs.x + mh * xs.y);
            }
    }
}

// Work items of a workgroup: rows [r0, r1) in quads of 4, each row's units in
// steps of 16 (one unit per block).  Wave w takes the contiguous item range
// [w*per, (w+1)*per): consecutive items are consecutive steps of one quad, so
// the lane accumulates its row's sums across them and the 16 blocks are
// reduced only when the quad changes.  The run total goes to LDS at
// part[(row*nc + c)*steps_max + first step of the run] (other slots stay 0);
// at the end each (row, c) adds its slots in step order.  Loads go through a
// two-deep ring, unconditional with clamped addresses (exact load counting).
template <int T, int NCB>
__global__ void __launch_bounds__(512) verify_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ x,
                                                    float *__restrict__ y, int N, int K, int nc, int KT, int steps_max) {
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    constexpr int BB = Fmt<T>::bytes, G = groups_per_unit<T>();
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = (int)blockDim.x >> 6;
    const int blk = lane >> 2, j = lane & 3;
    const int r0 = (int)((int64_t)blockIdx.x * N / gridDim.x);
    const int r1 = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x);
    const int R = r1 - r0, quads = (R + 3) >> 2;
    const size_t row_bytes = (size_t)(K >> 8) * BB;
    const int units_kt = KT >> 6;
    float *part = reinterpret_cast<float *>(smem);  // [R][nc][steps_max]
    uint32_t *planes = smem + (size_t)R * nc * steps_max;
    float *sums = reinterpret_cast<float *>(planes + (size_t)nc * units_kt * VSLOT);
    for (int e = tid; e < R * nc * steps_max; e += (int)blockDim.x) part[e] = 0.f;

    for (int k0 = 0; k0 < K; k0 += KT) {
        const int kt = min(KT, K - k0), units = kt >> 6, ub = k0 >> 6;
        const int steps = (units + 15) >> 4;
        const int items = quads * steps;
        const int per = (items + nwaves - 1) / nwaves;
        const int i0 = min(wave * per, items), i1 = min(i0 + per, items);
        if (k0 > 0) __syncthreads();
        stage_xv<T>(x, k0, kt, nc, planes, sums);  // ends with a barrier

        auto addr = [&](int item) {
            const int it = min(item, items - 1);
            const int quad = it / steps, step = it - quad * steps;
            const int row = min(4 * quad + j, R - 1);
            const int u_raw = 16 * step + blk;
            const int u = min(u_raw, units - 4 + (u_raw & 3));
            return W + (size_t)(r0 + row) * row_bytes + (size_t)((ub + u) >> 2) * BB;
        };
        const int qq = blk & 3;  // unit index within the superblock (u & 3 == blk & 3)
        const KScaleSel sel(qq);
        const UnitAddr<T, GGUF> ua(0, qq);  // offsets from the superblock start
        Unit<T> buf[2];
        buf[0].template load<false, GGUF>(addr(i0), 0u, ua);
        buf[1].template load<false, GGUF>(addr(i0 + 1), 0u, ua);

        float acc[4 * NCB];
#pragma unroll
        for (int i = 0; i < 4 * NCB; ++i) acc[i] = 0.f;
        int run_step = -1;
        for (int item0 = i0; item0 < i1; item0 += 2) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int item = item0 + p;
                if (item < i1) {
                    const int quad = item / steps, step = item - quad * steps;
                    const int row = 4 * quad + j;
                    const int u_raw = 16 * step + blk;
                    if (run_step < 0) run_step = step;
                    // every lane runs the matrix-core path (a block reads the A rows of
                    // all four lanes); lanes past the rows or units only drop the result
                    const int u_c = min(u_raw, units - 4 + (u_raw & 3));
                    float tmp[4 * NCB];
#pragma unroll
                    for (int i = 0; i < 4 * NCB; ++i) tmp[i] = 0.f;
                    item_dot<T, NCB>(buf[p], qq, sel, planes, sums, units, u_c, j, nc, tmp);
                    const bool ok = row < R && u_raw < units;
#pragma unroll
                    for (int i = 0; i < 4 * NCB; ++i) acc[i] += ok ? tmp[i] : 0.f;
                    // end of a run: next item is another quad, or the range ends
                    const bool last = item + 1 >= i1 || (item + 1) / steps != quad;
                    if (last) {
#pragma unroll
                        for (int i = 0; i < 4 * NCB; ++i) {
                            float v = acc[i];
                            v += __shfl_xor(v, 4);
                            v += __shfl_xor(v, 8);
                            v += __shfl_xor(v, 16);
                            v += __shfl_xor(v, 32);
                            acc[i] = 0.f;
                            if (blk == 0 && row < R && i < nc)
                                part[((size_t)row * nc + i) * steps_max + (k0 >> 10) + run_step] = v;
                        }
                        run_step = -1;
                    }
                }
                buf[p].template load<false, GGUF>(addr(item + 2), 0u, ua);
            }
        }
    }
    __syncthreads();
    const int total_steps = ((K >> 6) + 15) >> 4;
    for (int e = tid; e < R * nc; e += (int)blockDim.x) {
        const float *pp = part + (size_t)e * steps_max;
        float s = 0.f;
        for (int i = 0; i < total_steps; ++i) s += pp[i];
        const int row = e / nc, c = e - row * nc;
        y[(size_t)(r0 + row) * nc + c] = s;
    }
}

// ---------------------------------------------------------------------------
// Launch: one workgroup per CU (more if the per-row partial sums would not fit
// in LDS); waves per workgroup chosen so every wave gets the same number of
// (quad, step) items; K tiled so that the x planes fit next to the partials.
// ---------------------------------------------------------------------------
constexpr size_t VLDS = 160 * 1024;

static int cus_v() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cus = v;
        else
            cus = 256;
    }
    return cus;
}

template <int T, int NCB>
static hipError_t launch_v(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc, hipStream_t st) {
    const int U = (int)(K / 64);
    const int steps_max = (U + 15) / 16;
    int64_t G = N < cus_v() ? N : cus_v();
    const size_t part_budget = 64 * 1024;
    while ((size_t)((N + G - 1) / G) * nc * steps_max * 4 > part_budget && G < N) G *= 2;
    if (G > N) G = N;
    const int64_t R = (N + G - 1) / G;
    const size_t part_bytes = (size_t)R * nc * steps_max * 4;
    // x planes + sums per unit of the tile
    const size_t per_unit = (size_t)nc * (VSLOT * 4 + groups_per_unit<T>() * 4);
    int KT = (int)(((VLDS - part_bytes) / per_unit) * 64);
    KT -= KT % 1024;  // whole 16-unit steps
    if (KT <= 0) return hipErrorInvalidValue;
    if (KT > K) KT = (int)K;
    const size_t lds = part_bytes + (size_t)(KT / 64) * per_unit;
    // waves: the fewest items per wave, then the fewest waves
    const int64_t items = ((R + 3) / 4) * ((KT / 64 + 15) / 16);
    int best_w = 8;
    int64_t best_t = INT64_MAX;
    for (int w = 1; w <= 8; ++w) {
        const int64_t t = (items + w - 1) / w;
        if (t < best_t) { best_t = t; best_w = w; }
    }
    static bool lds_opt_in = false;  // allow more than 64 KB of dynamic LDS
    if (!lds_opt_in) {
        const hipError_t e = hipFuncSetAttribute((const void *)verify_kernel<T, NCB>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)VLDS);
        if (e != hipSuccess) return e;
        lds_opt_in = true;
    }
    hipLaunchKernelGGL((verify_kernel<T, NCB>), dim3((unsigned)G), dim3(64 * best_w), lds, st,
                       (const uint8_t *)W, (const uint16_t *)x, (float *)y, (int)N, (int)K, nc, KT, steps_max);
    return hipGetLastError();
}

template <int T>
static hipError_t verify_dispatch(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc, hipStream_t st) {
    if (nc <= 4) return launch_v<T, 1>(W, x, y, N, K, nc, st);
    return launch_v<T, 2>(W, x, y, N, K, nc, st);
}

hipError_t launch_gemv_multi(int type, const void *W, const void *x, void *y, int64_t N, int64_t K, int ncols,
                             hipStream_t stream) {
    switch (type) {
    case Q4_K: return verify_dispatch<Q4_K>(W, x, y, N, K, ncols, stream);
    case Q5_K: return verify_dispatch<Q5_K>(W, x, y, N, K, ncols, stream);
    case Q6_K: return verify_dispatch<Q6_K>(W, x, y, N, K, ncols, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qk
