// qk_verify.h -- few-column verify GEMV (ncols 2..32) on gfx950 matrix cores.
// Included by one translation unit per quant type (qk_verify_q4k.hip, ...),
// which compile in parallel; qk_verify.hip dispatches on the type.
//
// y[n][c] = sum_k dequant(W)[n][k] * x[k][c] for c < ncols: the batched
// verification of drafted tokens (T4 dossier design-doc prompt, deliverable 3
// "MTP Verify Plan"; B70 plan, Phase 3 item 7 and Phase 4 "True Xe2 Batched
// Verification"; its checklist names verifier widths up to 17).  Up to 8
// columns W is streamed once per call; wider calls take the columns in
// groups of at most 8 inside the one launch, each group streaming the
// workgroup's rows again (mostly from the caches after the first).
//
// Same skeleton as the one-column kernel (x-stationary, rows balanced over
// the CUs, a ring of units in flight, partial sums in LDS, a fixed-order
// final sum), with the column products on the matrix cores:
//   v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4x4x4 blocks; block b is
//   the 4 lanes 4b..4b+3, lane 4b+j supplies row j of A and column j of B and
//   receives D[0..3][j].  Here block b is one unit column (64 weights of a
//   superblock) of four rows, lane j being row j of a row quad:
//     B column j = the quant patterns of row j for one 32-bit quant word,
//                  shifted by the row's integer c of the scale group (exact
//                  fp16 values s*(q-c)*2^-24, weights (l, l+2, l+1, l+3);
//                  c = 32 for Q6_K, see KShift in qk_format.h; IQ4_XS: the
//                  signed codebook values kv*2^-24, nothing to shift),
//     A row i    = x column 4*cb + i at the same four weights, held in
//                  registers by lane i of the block for the whole segment,
//     D[i][j]    = sum over the word of x_i * q_j.
//   D is accumulated over a scale group, then each lane scales its own row's
//   four columns by d*sc (and adds (d*sc*c - dmin*m) times the x sums) in fp32.
// A wave covers 16 consecutive unit columns of a row quad; the unit columns
// of one K segment form a phase of useg/16 waves, and P phases take the row
// quads of the workgroup in turn.  Per row quad the 16 blocks of a wave are
// folded with DPP rotations inside each 16-lane row and the 4 results per
// wave and column go to LDS; at the end each (row, column) adds its slots in
// a fixed order.
#pragma once

#include "qk_epilogue.h"
#include "qk_format.h"
#include "qk_launch.h"
#include "qk_verify16.h"

#include <algorithm>

namespace qk {

typedef f32x4 float4_t;

// a from the lane that the DPP control names
template <int CTRL>
__device__ __forceinline__ float vdpp(float a) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), CTRL, 0xf, 0xf, false));
}

// Largest workgroup: 12 waves (3 per SIMD, 168 registers each) for one
// column block; 8 waves (2 per SIMD, 256 registers) for two, whose x alone
// takes 64 registers.
template <int NCB>
__host__ __device__ constexpr int v_max_threads() { return NCB == 1 ? 768 : 512; }
constexpr int V_MAX_RL = 8;  // quads per straight-line round, at most
// Plain launches of two column blocks in short rounds fit 168 registers
// without spills, so they may take 12 waves (two row phases at K = 5120):
// Q4_K and IQ4_XS in rounds of up to 3 quads, Q5_K and Q6_K of one (measured
// 4-5% faster for Q4_K at 17408 x 5120, 6 and 8 columns).  The epilogue
// variants would spill there.
template <int T>
__host__ __device__ constexpr int v_short_rl() { return T == Q4_K || T == IQ4_XS ? 3 : 1; }
template <int T, int NCB, int RL, bool PAIR, bool EPI>
constexpr int v_bound() {
    return NCB == 2 && RL <= v_short_rl<T>() && !PAIR && !EPI ? 768 : v_max_threads<NCB>();
}
// LDS for the x planes of one segment: 112 KB for launches of up to 8
// columns, so that 5120 x 6144 takes one segment instead of two and
// 5120 x 17408 three instead of four at 8 columns (Q5_K 17.0 -> 13.3 us,
// Q6_K 44.5 -> 37.7 us).
constexpr int V_RAW_BUDGET = 112 * 1024;
constexpr int V_LDS_MAX = 160 * 1024;

template <int T>
__host__ __device__ constexpr int vgroups() { return T == Q6_K ? 4 : 2; }  // scale groups per unit

// x of one K segment in LDS, transposed into one plane per column: the 64
// x values unit ul of the segment multiplies sit in block ul of column c's
// plane, at c*ps + ul*144 (128 bytes + a 16-byte pad per block, so the 16
// unit columns of a wave read different banks).  For Q4_K and Q5_K that is
// k = 64*ul .. 64*ul+63 in order; for Q6_K the unit's four 16-value quarters.
constexpr int VXSTRIDE = 144;

__device__ __forceinline__ uint4 xplane16(const uint8_t *pl, int kb, int off) {
    return *reinterpret_cast<const uint4 *>(pl + kb * VXSTRIDE + off);
}

// Sixteen halves (two 16-byte vectors) -> 8 pair dwords in the pattern order
// (0, 2), (1, 3) per group of four, + their fp32 sum.
__device__ __forceinline__ float vx_pairs16(const uint4 &v0, const uint4 &v1, uint32_t *o) {
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        o[2 * g] = (w[2 * g] & 0xffffu) | (w[2 * g + 1] << 16);
        o[2 * g + 1] = (w[2 * g] >> 16) | (w[2 * g + 1] & 0xffff0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot2(w[i], 0x3c003c00u, s);  // (1, 1) pairs
    return s;
}

// Column plane pl at the unit's 64 weights (segment-relative unit ul), in
// the register order of the quant patterns; plus the fp32 sum of each scale
// group (16 weights for Q6_K, 32 otherwise).
template <int T>
__device__ __forceinline__ void gather_x(const uint8_t *pl, int ul, uint32_t *xr, float *sums) {
    float s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) s[m] = vx_pairs16(xplane16(pl, ul, 32 * m), xplane16(pl, ul, 32 * m + 16), xr + 8 * m);
    if constexpr (T == Q6_K) {
#pragma unroll
        for (int m = 0; m < 4; ++m) sums[m] = s[m];
    } else {
        sums[0] = s[0] + s[1];
        sums[1] = s[2] + s[3];
    }
}

// Copy ns blocks of 64 rows of x (NCV columns, row-major) into the column
// planes: each task takes 8 rows, contiguous in x (NCV 16-byte loads),
// transposes them in registers and writes one 16-byte vector per column.
// For Q6_K the plane block of unit ul holds the unit's four quarters in
// order instead (the same 16-byte reads then serve every type).
template <int T, int NCV>
__device__ __forceinline__ void stage_planes(const uint8_t *xg, uint8_t *planes, int ps, int ns, int tid) {
    const int ntask = ns * 8;
    for (int t = tid; t < ntask; t += (int)blockDim.x) {
        uint32_t h[4 * NCV];
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xg + ((size_t)t * NCV + i) * 16);
            h[4 * i] = v.x; h[4 * i + 1] = v.y; h[4 * i + 2] = v.z; h[4 * i + 3] = v.w;
        }
        // half e of the task is x[8t + e / NCV][e % NCV]
        auto half = [&](int e) -> uint32_t { return (h[e >> 1] >> (16 * (e & 1))) & 0xffffu; };
        int off;
        if constexpr (T == Q6_K) {
            // rows 8t..8t+7: superblock t/32, 16-row group g = (t/2)%16 of it
            // (quarter (g/2)%4 of unit 4*(t/32) + 2*(g/8) + g%2), half t%2 of the group
            const int g = (t >> 1) & 15;
            off = (4 * (t >> 5) + 2 * (g >> 3) + (g & 1)) * VXSTRIDE + 32 * ((g >> 1) & 3) + 16 * (t & 1);
        } else {
            off = (t >> 3) * VXSTRIDE + 16 * (t & 7);
        }
        uint8_t *dst = planes + off;
#pragma unroll
        for (int c = 0; c < NCV; ++c) {
            uint4 o;
            o.x = half(0 * NCV + c) | (half(1 * NCV + c) << 16);
            o.y = half(2 * NCV + c) | (half(3 * NCV + c) << 16);
            o.z = half(4 * NCV + c) | (half(5 * NCV + c) << 16);
            o.w = half(6 * NCV + c) | (half(7 * NCV + c) << 16);
            *reinterpret_cast<uint4 *>(dst + c * ps) = o;
        }
    }
}

// DPP quad_perm broadcast of lane J of each quad (J = 0..3)
template <int J>
__device__ __forceinline__ float quad_bcast(float a) { return vdpp<J | (J << 2) | (J << 4) | (J << 6)>(a); }

// v_mfma_f32_4x4x1_16b_f32: in each of the 16 blocks (lanes 4b..4b+3) lane
// 4b+j supplies a = A[j][0] and b = B[0][j] and receives D[0..3][j] +=
// A[i][0] * B[0][j], the same lane roles as mfma4.
__device__ __forceinline__ float4_t mfma1f32(float a, float b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// PAIR (the SwiGLU epilogue): the workgroup's rows of W and then of ep.W2
// form one schedule of 2R rows; row r's outputs combine the sums of rows r
// and R + r.  EPI: the store applies ep's residual / fp16 options (else it is
// the plain fp32 store).  x is [K][nc], y (and the residual) [N][nc], nc at
// most 4 * NCB.
template <int T, int NCB, int RL, int D, bool PAIR, bool EPI>
__global__ void __launch_bounds__((v_bound<T, NCB, RL, PAIR, EPI>())) verify_kernel(const uint8_t *__restrict__ W,
                                                               const uint16_t *__restrict__ x, void *y,
                                                               int N, int K, int nc, int useg, int P,
                                                               const Epilogue ep) {
    extern __shared__ __attribute__((aligned(16))) float vsm[];
    constexpr int G = vgroups<T>(), NC = 4 * NCB;
    constexpr int DD = D < RL ? D : RL;
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int blk = lane >> 2, j = lane & 3;
    const int wpp = useg >> 4;  // waves per phase
    const int ph = small_div(wave, wpp), wip = wave - ph * wpp;
    const int uc = 16 * wip + blk;  // unit column within the segment
    const RowSplit split(N, (int)blockIdx.x, (int)gridDim.x);
    const int r0 = split.r0, r1 = split.r1;
    const int R = r1 - r0, RV = PAIR ? 2 * R : R, Q = (RV + 3) >> 2;
    const int quads_lane = small_div(Q + P - 1, P);
    const int U = K >> 6;
    const size_t row_bytes = (size_t)(K >> 8) * Fmt<T>::bytes;
    const int nslot = 4 * wpp;  // partial slots per (row, column): 4 per wave of a phase
    // LDS: partial sums [row][slot][NC] (rows of every quad a phase visits),
    // then the x planes of a segment
    float *part = vsm;
    uint8_t *planes = reinterpret_cast<uint8_t *>(vsm + (size_t)quads_lane * P * 4 * nslot * NC);
    const int ps = useg * VXSTRIDE;  // bytes per column plane
    const int slot = 4 * wip + (blk >> 2);  // this lane's slot if it writes (blk % 4 == 0)
    // the residuals of the first row this lane stores (lane 0 of each 16)
    constexpr bool RES0 = EPI;
    float res0[RES0 ? NC : 1];
#pragma unroll
    for (int c = 0; c < (RES0 ? NC : 1); ++c) res0[c] = 0.f;
    if constexpr (RES0)
        if (ep.res && (tid & 15) == 0 && (tid >> 4) < R)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (c < nc) res0[c] = ep.res[(size_t)(r0 + (tid >> 4)) * nc + c];

    for (int s0 = 0; s0 < U; s0 += useg) {
        const int ns = min(useg, U - s0);
        const bool col_ok = uc < ns;
        const int u = s0 + min(uc, ns - 4 + (uc & 3));  // clamped, same q
        const int q = u & 3;
        const KScaleSel sel(q);

        // x of the segment into the column planes
        if (s0 > 0) __syncthreads();  // the previous segment's x is in registers everywhere
        const uint8_t *xg = reinterpret_cast<const uint8_t *>(x + (size_t)s0 * 64 * nc);
        switch (nc) {
        case 2: stage_planes<T, 2>(xg, planes, ps, ns, tid); break;
        case 3: if constexpr (NC >= 4) stage_planes<T, 3>(xg, planes, ps, ns, tid); break;
        case 4: if constexpr (NC >= 4) stage_planes<T, 4>(xg, planes, ps, ns, tid); break;
        case 5: if constexpr (NC >= 8) stage_planes<T, 5>(xg, planes, ps, ns, tid); break;
        case 6: if constexpr (NC >= 8) stage_planes<T, 6>(xg, planes, ps, ns, tid); break;
        case 7: if constexpr (NC >= 8) stage_planes<T, 7>(xg, planes, ps, ns, tid); break;
        default: if constexpr (NC >= 8) stage_planes<T, 8>(xg, planes, ps, ns, tid); break;
        }
        __syncthreads();
        // The segment's first ring of weight loads is issued here, before
        // the x reads of the planes (2-7% faster at 2-8 columns).
        const UnitAddr<T, GGUF> ua(K >> 8, u);
        auto load_quad = [&](Unit<T> &dst, int qi) {  // qi: the lane's quad index
            if constexpr (PAIR) {
                const int v = min(4 * (ph + P * qi) + j, RV - 1);  // row of the schedule
                const uint8_t *base = v < R ? W + (size_t)(r0 + v) * row_bytes
                                            : reinterpret_cast<const uint8_t *>(ep.W2) +
                                                  (size_t)(r0 + v - R) * row_bytes;
                dst.template load<false, GGUF>(base, ua);
            } else {
                const int row = min(r0 + 4 * (ph + P * qi) + j, r1 - 1);
                dst.template load<false, GGUF>(W + (size_t)row * row_bytes, ua);
            }
        };
        Unit<T> buf[DD];
#pragma unroll
        for (int p = 0; p < DD; ++p) load_quad(buf[p], p);
        // this lane's columns j, j+4 in registers; group sums of all columns of the unit
        uint32_t xr[NCB][32];
        // Q4_K/Q5_K: the sums of this lane's own columns (4cb + j) over the
        // unit's two sub-blocks, pre-scaled for the 2^-48 units of the partials
        float xs[NCB][2];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int c = 4 * cb + j;
            float own[G];
            if (c < nc) {
                gather_x<T>(planes + c * ps, u - s0, xr[cb], own);
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) xr[cb][i] = 0u;
#pragma unroll
                for (int g = 0; g < G; ++g) own[g] = 0.f;
            }
            xs[cb][0] = own[0] * 0x1p-24f;
            xs[cb][1] = own[1] * 0x1p-24f;
        }
        // one column block: every lane keeps the four columns' sums (quad
        // broadcasts), and the min terms are four fmas per column
        float xq[NCB == 1 ? 4 : 1][2];
        if constexpr (NCB == 1) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                xq[0][g] = quad_bcast<0>(xs[0][g]);
                xq[1][g] = quad_bcast<1>(xs[0][g]);
                xq[2][g] = quad_bcast<2>(xs[0][g]);
                xq[3][g] = quad_bcast<3>(xs[0][g]);
            }
        }
        for (int i0 = 0; i0 < quads_lane; i0 += RL) {
            if (i0 > 0)
#pragma unroll
                for (int p = 0; p < DD; ++p) load_quad(buf[p], i0 + p);
#pragma unroll
            for (int p = 0; p < RL; ++p) {
                const Unit<T> &Un = buf[p % DD];
                float val[NC];
                // each quant word's patterns once, multiplied into every
                // column block's accumulators
                if constexpr (T == IQ4_XS) {
                    // signed codebook patterns kv*2^-24 (exact), d*2^24*(ls-32)
                    // per sub-block; x pairs as in the one-column kernel
                    const float d = Un.d24();
                    const float fl = d * (float)Un.scale(q, 0), fh = d * (float)Un.scale(q, 1);
                    float4_t Dl[NCB], Dh[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) Dl[cb] = Dh[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t pl[4], ph[4];
                        Un.patterns(i, q, pl);
                        Un.patterns(i + 4, q, ph);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) {
                            Dl[cb] = mfma4(xr[cb][2 * i], xr[cb][2 * i + 1], pl[0], pl[1], Dl[cb]);
                            Dh[cb] = mfma4(xr[cb][2 * (i + 8)], xr[cb][2 * (i + 8) + 1], ph[0], ph[1], Dh[cb]);
                            Dl[cb] = mfma4(xr[cb][2 * (i + 4)], xr[cb][2 * (i + 4) + 1], pl[2], pl[3], Dl[cb]);
                            Dh[cb] = mfma4(xr[cb][2 * (i + 12)], xr[cb][2 * (i + 12) + 1], ph[2], ph[3], Dh[cb]);
                        }
                    }
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) val[4 * cb + i] = __builtin_fmaf(fl, Dl[cb][i], fh * Dh[cb][i]);
                } else if constexpr (T == Q6_K) {
                    const float d = f16_lo(Un.d);
                    float f[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) f[t] = d * (float)Un.scale(t, q);
                    float4_t Dq[NCB][4];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int t = 0; t < 4; ++t) Dq[cb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t pt[8];
                        Un.patterns(i, q, pt);
                        // q - 32 on the patterns (exact): no sum of x to subtract
#pragma unroll
                        for (int t = 0; t < 8; ++t) pt[t] = padd(pt[t], t < 4 ? Q6_OFF_LO : Q6_OFF_HI);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                Dq[cb][t] = mfma4(xr[cb][8 * t + 2 * i], xr[cb][8 * t + 2 * i + 1], pt[2 * t],
                                                  pt[2 * t + 1], Dq[cb][t]);
                    }
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float a = 0.f;
#pragma unroll
                            for (int t = 0; t < 4; ++t)  // patterns hold (q-32)*2^-24 (t < 2) or 16(q-32)*2^-24
                                a = __builtin_fmaf(f[t], Dq[cb][t][i] * (t < 2 ? 0x1p24f : 0x1p20f), a);
                            val[4 * cb + i] = a;
                        }
                } else {
                    // the shifted form of the one-column kernel (KShift), units of
                    // 2^-48: sc and m read as fp16 patterns are sc*2^-24 and m*2^-24,
                    // the patterns hold s*(q - c)*2^-24, the x sums are held times 2^-24
                    constexpr int QMAX = T == Q4_K ? 15 : 31;
                    const uint4 h = Un.header();
                    const KScales sk = k_scales(h, sel);
                    auto pat = [](uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)v); };
                    const float d = f16_lo(h.x), dmin = f16_hi(h.x);
                    const KShift kL = k_shift<QMAX, 1>(d, dmin, pat(sk.sc_lo), pat(sk.m_lo));
                    const KShift kH = k_shift<QMAX, 16>(d, dmin, pat(sk.sc_hi), pat(sk.m_hi));
                    const float fh = kH.a * 0x1p-4f;
                    float4_t Dl[NCB], Dh[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) Dl[cb] = Dh[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        uint32_t pt[4];
                        Un.patterns(i, q, pt);
                        pt[0] = padd(pt[0], kL.neg);
                        pt[1] = padd(pt[1], kL.neg);
                        pt[2] = padd(pt[2], kH.neg);
                        pt[3] = padd(pt[3], kH.neg);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) {
                            Dl[cb] = mfma4(xr[cb][2 * i], xr[cb][2 * i + 1], pt[0], pt[1], Dl[cb]);
                            Dh[cb] = mfma4(xr[cb][16 + 2 * i], xr[cb][17 + 2 * i], pt[2], pt[3], Dh[cb]);
                        }
                    }
                    // the min terms e_L * sum x_lo + e_H * sum x_hi of every (row j,
                    // column i) of a block.  Two column blocks: a rank-2 outer
                    // product of the rows' e and the columns' x sums on the matrix
                    // cores in fp32 (the broadcast sums of eight columns would not
                    // fit the registers of 12-wave launches: measured 10% faster
                    // at 5-8 columns); one block: fmas on the broadcast sums (2%
                    // faster there).
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        float4_t E;
                        if constexpr (NCB == 1) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) E[i] = __builtin_fmaf(kL.e, xq[i][0], kH.e * xq[i][1]);
                        } else {
                            E = mfma1f32(xs[cb][0], kL.e, float4_t{0.f, 0.f, 0.f, 0.f});
                            E = mfma1f32(xs[cb][1], kH.e, E);
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            val[4 * cb + i] = __builtin_fmaf(kL.a, Dl[cb][i], __builtin_fmaf(fh, Dh[cb][i], E[i]));
                    }
                }
                if (p + DD < RL) load_quad(buf[p % DD], i0 + p + DD);
                // fold the 4 blocks of each 16-lane row (same row j, consecutive units)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    float v = col_ok ? val[c] : 0.f;
                    v += vdpp<0x124>(v);  // row_ror:4
                    v += vdpp<0x128>(v);  // row_ror:8
                    val[c] = v;
                }
                // quads past quads_lane (RL need not divide it) have no slot rows
                if ((blk & 3) == 0 && i0 + p < quads_lane) {
                    const int row = 4 * (ph + P * (i0 + p)) + j;  // slot row (rows >= R are never read)
                    float4 *d4 = reinterpret_cast<float4 *>(part + ((size_t)row * nslot + slot) * NC);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const float4 v = make_float4(val[4 * cb], val[4 * cb + 1], val[4 * cb + 2], val[4 * cb + 3]);
                        if (s0 == 0) {
                            d4[cb] = v;
                        } else {
                            const float4 o = d4[cb];
                            d4[cb] = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    // y[row][c] = sum over the slots, fixed order: 16 lanes per row, lane s
    // adds slots s, s+16, ..., then a DPP fold of the 16 lanes per column
    const int s16 = tid & 15;
    constexpr float oscale = T == Q6_K || T == IQ4_XS ? 1.f : 0x1p48f;
    // the sums of schedule row v per column (every lane of the 16 takes part)
    auto row_sums = [&](int v, bool ok, float *a) {
        const float *pr = part + (size_t)(ok ? v : 0) * nslot * NC;
#pragma unroll
        for (int c = 0; c < NC; ++c) a[c] = 0.f;
        for (int sl = s16; sl < nslot; sl += 16) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const float4 w = reinterpret_cast<const float4 *>(pr + (size_t)sl * NC)[cb];
                a[4 * cb] += w.x;
                a[4 * cb + 1] += w.y;
                a[4 * cb + 2] += w.z;
                a[4 * cb + 3] += w.w;
            }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float t = a[c];
            t += vdpp<0xb1>(t);   // quad_perm [1,0,3,2]
            t += vdpp<0x4e>(t);   // quad_perm [2,3,0,1]
            t += vdpp<0x141>(t);  // row_half_mirror
            t += vdpp<0x140>(t);  // row_mirror
            a[c] = t * oscale;
        }
    };
    for (int rr = tid >> 4; rr - (tid >> 4) < R; rr += (int)blockDim.x >> 4) {
        const bool rok = rr < R;
        float a[NC];
        row_sums(rr, rok, a);
        if constexpr (PAIR) {
            float b[NC];
            row_sums(R + rr, rok, b);
#pragma unroll
            for (int c = 0; c < NC; ++c) a[c] = silu(a[c]) * b[c];
        }
        if (rok && s16 == 0) {
            const size_t o = (size_t)(r0 + rr) * nc;
            if constexpr (EPI) {
                const bool first = RES0 && rr == (tid >> 4);
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    if (c < nc) {
                        float v = a[c];
                        if (ep.res) v += first ? res0[RES0 ? c : 0] : ep.res[o + c];
                        store_y(y, ep.f16, o + c, v);
                    }
            } else {
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    if (c < nc) reinterpret_cast<float *>(y)[o + c] = a[c];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch geometry.  useg: unit columns per segment, a multiple of 16 (one
// wave per 16), at most 192 and with the x planes within their budget; the
// segments of K are made as even as possible.  G: one workgroup per CU unless
// the LDS does not fit.  P phases and RL quads per straight-line round as
// ranked below.
// ---------------------------------------------------------------------------
struct VGeo { int G, useg, P, RL, threads; size_t lds; };

static int cus_v() { return device_cus(); }

// mult = 2: each workgroup streams its rows of two tensors (SwiGLU).
// short_threads: the largest workgroup for rounds of at most short_rl
// quads (at least the general limit).
static bool vgeo(int64_t N, int64_t K, int nc, int ncb, int mult, int short_threads, int short_rl, int max_rl,
                 VGeo &g) {
    const int64_t U = K / 64;
    const int64_t xs = (int64_t)VXSTRIDE * nc;  // plane bytes per unit column
    const int long_threads = ncb == 1 ? v_max_threads<1>() : v_max_threads<2>();
    short_threads = std::max(short_threads, long_threads);
    const int max_waves = long_threads / 64;
    const int cap = (int)std::min<int64_t>(16 * max_waves, V_RAW_BUDGET / xs) / 16 * 16;
    if (cap < 16) return false;
    const int64_t nseg = (U + cap - 1) / cap;
    g.useg = (int)(((U + nseg - 1) / nseg + 15) / 16 * 16);
    const int wpp = g.useg / 16;
    const int pmax = std::max(1, (short_threads / 64) / wpp);
    // one workgroup per CU, also for a pair of tensors (each workgroup stages
    // x for its columns once: more workgroups would stage it more often;
    // measured slower for the pair at ncols = 4)
    for (int64_t G = std::min<int64_t>(N, cus_v());; G *= 2) {
        if (G > N) G = N;
        g.G = (int)G;
        const int64_t R = mult * ((N + G - 1) / G), Q = (R + 3) / 4;
        // Each lane's quads run in straight-line rounds of RL <= V_MAX_RL; a
        // round starts with an empty load ring, so the fewest rounds come
        // first, then the fewest quad slots in all (P lanes' worth, the
        // wasted ones included), then the fewest per lane.  Fewer than 4
        // waves leave SIMDs idle: avoided wherever the segment allows.
        const int min_waves = std::min(4, pmax * wpp);
        int64_t best[4] = {INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX};
        for (int p = 1; p <= pmax; ++p) {
            // above the general limit only short rounds fit the registers
            const int maxrl = p * wpp * 64 <= long_threads ? max_rl : short_rl;
            const int64_t ql = (Q + p - 1) / p;
            const int64_t rounds = (ql + maxrl - 1) / maxrl;
            const int rl = (int)((ql + rounds - 1) / rounds);
            const int64_t lane = rounds * rl;
            const int64_t key[4] = {p * wpp < min_waves ? 1 : 0, rounds, p * lane, lane};
            if (std::lexicographical_compare(key, key + 4, best, best + 4)) {
                std::copy(key, key + 4, best);
                g.P = p;
                g.RL = rl;
            }
        }
        const int64_t ql = (Q + g.P - 1) / g.P;
        g.threads = g.P * wpp * 64;
        g.lds = (size_t)(ql * g.P * 4 * (4 * wpp) * (4 * ncb)) * 4 + (size_t)g.useg * xs;
        if (g.lds <= (size_t)V_LDS_MAX) return true;
        if (G == N) return false;
    }
}

template <auto Kernel>
static hipError_t v_allow_lds() {
    return lds_opt_in<Kernel>(V_LDS_MAX);
}

template <int T, int NCB, int RL, bool PAIR, bool EPI>
static hipError_t launch_ve(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc, const VGeo &g,
                            const Epilogue &ep, hipStream_t st) {
    constexpr int D = 2;
    if (g.threads > v_bound<T, NCB, RL, PAIR, EPI>()) return hipErrorInvalidValue;
    const hipError_t e = v_allow_lds<verify_kernel<T, NCB, RL, D, PAIR, EPI>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((verify_kernel<T, NCB, RL, D, PAIR, EPI>), dim3((unsigned)g.G), dim3(g.threads), g.lds,
                       st, (const uint8_t *)W, (const uint16_t *)x, y, (int)N, (int)K, nc, g.useg, g.P, ep);
    return hipGetLastError();
}

// Plain launches run a body without the epilogue's store options.
template <int T, int NCB, int RL, bool PAIR>
static hipError_t launch_v(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc, const VGeo &g,
                           const Epilogue &ep, hipStream_t st) {
    static_assert(NCB == 1 || NCB == 2, "one or two column blocks");
    if (nc > 8) return hipErrorInvalidValue;
    if (!PAIR && !ep.res && !ep.f16) return launch_ve<T, NCB, RL, false, false>(W, x, y, N, K, nc, g, ep, st);
    return launch_ve<T, NCB, RL, PAIR, true>(W, x, y, N, K, nc, g, ep, st);
}

// Up to 8 columns: one or two column blocks of 4 (wider calls run on the
// 16x16x16 tiles of qk_verify16.h).

// Rounds of up to 8 quads.
template <int T, int NCB>
constexpr int v_max_rl() {
    return V_MAX_RL;
}

template <int T, int NCB, bool PAIR>
static hipError_t verify_dispatch(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc,
                                  const Epilogue &ep, hipStream_t st) {
    VGeo g;
    // plain launches of up to 8 columns may take the larger workgroups of short rounds
    const bool plain = !PAIR && !ep.res && !ep.f16 && nc <= 8;
    const int short_threads = plain ? v_bound<T, NCB, 1, false, false>() : v_max_threads<NCB>();
    if (!vgeo(N, K, nc, NCB, PAIR ? 2 : 1, short_threads, v_short_rl<T>(), v_max_rl<T, NCB>(), g))
        return hipErrorInvalidValue;
    constexpr int MRL = v_max_rl<T, NCB>();
    switch (g.RL) {
    case 1: return launch_v<T, NCB, 1, PAIR>(W, x, y, N, K, nc, g, ep, st);
    case 2: if constexpr (MRL >= 2) return launch_v<T, NCB, 2, PAIR>(W, x, y, N, K, nc, g, ep, st); break;
    case 3: if constexpr (MRL >= 3) return launch_v<T, NCB, 3, PAIR>(W, x, y, N, K, nc, g, ep, st); break;
    case 4: if constexpr (MRL >= 4) return launch_v<T, NCB, 4, PAIR>(W, x, y, N, K, nc, g, ep, st); break;
    default: break;
    }
    if constexpr (MRL > 4) {
        switch (g.RL) {
        case 5: return launch_v<T, NCB, 5, PAIR>(W, x, y, N, K, nc, g, ep, st);
        case 6: return launch_v<T, NCB, 6, PAIR>(W, x, y, N, K, nc, g, ep, st);
        case 7: return launch_v<T, NCB, 7, PAIR>(W, x, y, N, K, nc, g, ep, st);
        default: return launch_v<T, NCB, 8, PAIR>(W, x, y, N, K, nc, g, ep, st);
        }
    }
    return hipErrorInvalidValue;
}

template <int T>
static hipError_t verify_type(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc,
                              const Epilogue &ep, hipStream_t st) {
    // 9-32 columns, every epilogue: one pass on 16x16x16 tiles
    if constexpr (T == Q4_K || T == Q5_K)
        if (nc > 8 && nc <= 32) return launch_v16<T>(W, x, y, N, K, nc, ep, st);
    if constexpr (T == Q6_K || T == IQ4_XS)
        if (nc >= V16Q6_MIN && nc <= 32) return launch_v16q6<T>(W, x, y, N, K, nc, ep, st);
    if (nc < 2 || nc > 8) return hipErrorInvalidValue;
    const int ncb = nc > 4 ? 2 : 1;
    if (ep.W2)
        return ncb == 1 ? verify_dispatch<T, 1, true>(W, x, y, N, K, nc, ep, st)
                        : verify_dispatch<T, 2, true>(W, x, y, N, K, nc, ep, st);
    return ncb == 1 ? verify_dispatch<T, 1, false>(W, x, y, N, K, nc, ep, st)
                    : verify_dispatch<T, 2, false>(W, x, y, N, K, nc, ep, st);
}

}  // namespace qk
