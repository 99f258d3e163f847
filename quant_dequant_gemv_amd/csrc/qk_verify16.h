// qk_verify16.h -- 9 to 32 columns in one pass on 16x16x16 matrix tiles, every
// type (Q4_K / Q5_K: v16_kernel; Q6_K / IQ4_XS: v16q6_kernel, further down) (the verify form of drafted tokens: B70 plan, "Phase 4: True Xe2
// Batched Verification", and its checklist's verifier widths up to 17).
//
// v_mfma_f32_16x16x16_f16 (probed on the box: A[i][k] from lane i + 16(k/4),
// element k % 4; B[k][j] from lane j + 16(k/4); D[i][j] to lane j + 16(i/4),
// element i % 4).  Here A is x (i = column of x, up to 16) and B the weights
// (j = row), so D[column][row]: lane l holds row l % 16 and columns
// 4(l / 16) .. +3 -- its own row's outputs, so the per-row scales of the
// shifted form apply in the lane that unpacked them.
//
// A workgroup owns whole tiles of 16 rows; a wave owns one tile and a share
// of the superblocks of each K segment.  Per superblock lane l = r + 16g
// loads the header of row r and, for each of the four units, bytes 8g ..
// 8g+7 of the unit's 32 quant bytes (low nibbles: 8 weights of the low
// sub-block, high nibbles: the same positions of the high one), forms the
// exact fp16 patterns s(q - c)2^-24 of the one-column kernel and issues, per
// unit, two matrix instructions per sub-block (16 of its 32 weights each) and
// two more per sub-block on the same x operands against fp16 ones: the sums
// of x per column that the min terms take (exact products, fp32 sums).  The
// x operands come from LDS planes staged per segment in exactly that order
// (2 KB per unit: 80 units, all of K = 5120, fit the 160 KB), so each lane
// reads them as two 16-byte vectors.  Every (row, column) is accumulated by
// one lane per share, in unit order; the shares of a tile are added in a
// fixed order at the end.  Weights are read once; the first ring of each
// segment is issued before its x is staged.  (This paragraph describes the
// Q4_K / Q5_K kernel; the Q6_K / IQ4_XS one is described above it.)
#pragma once

#include "qk_epilogue.h"
#include "qk_format.h"
#include "qk_launch.h"

namespace qk {

constexpr int V16_UB = 2048;        // LDS bytes per unit and group of 16 columns: their x operands
constexpr int V16_PLANES = 160 * 1024;  // LDS for the planes of a segment
constexpr int V16_D = 2;             // superblocks in flight per lane

typedef _Float16 v16_half4 __attribute__((ext_vector_type(4)));
typedef float v16_f4 __attribute__((ext_vector_type(4)));
constexpr uint32_t V16_ONES = 0x3c003c00u;  // the fp16 pair (1, 1)

__device__ __forceinline__ v16_f4 mfma16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, v16_f4 c) {
    const uint2 a = make_uint2(a0, a1), b = make_uint2(b0, b1);
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v16_half4, a), __builtin_bit_cast(v16_half4, b),
                                                  c, 0, 0, 0);
}

// A lane's share of one superblock of its row: the header and, for each of
// the four units, its 8 quant bytes.
struct V16Sb {
    uint4 h;
    uint2 q[4];
    uint2 qh;  // Q5_K: bytes 8g .. 8g+7 of qh (bit 2u / 2u + 1: the fifth bit of unit u's sub-blocks)
};

// Superblock geometry of the k-quants with 32-weight sub-blocks and a min
template <int T> struct V16Fmt;
template <> struct V16Fmt<Q4_K> { static constexpr int bytes = 144, qs = 16, qmax = 15; };
template <> struct V16Fmt<Q5_K> { static constexpr int bytes = 176, qs = 48, qmax = 31; };

// Stage the x of units [s0, s0 + ns) (all nc columns; columns nc..15 zero)
// into the planes.  Unit ul at ul * V16_UB: [sb * 1024 + l * 16, +16) holds
// the x operands of lane l = c + 16g for sub-block sb -- halves 0..3 of the
// first instruction (weights 8g + 0, 2, 1, 3 of the sub-block), halves 4..7
// of the second (8g + 4, 6, 5, 7).
template <int NCV, bool CP = false>
__device__ __forceinline__ void v16_copy(const uint16_t *__restrict__ x, int s0, int ns, uint8_t *planes, int tid,
                                         int nthr) {
    constexpr int NG = NCV > 16 ? 2 : 1;  // groups of 16 columns
    // task: (unit, sub-block, group[, half]): RPT consecutive rows of x,
    // contiguous (NCV loads of 2 * RPT bytes), transposed in registers into
    // RPT halves of each column's operand vector (rows 0, 2, 1, 3 within each
    // four: the pattern order).  Eight rows (whole 16-byte vectors) up to 16
    // columns; four (half vectors) beyond, for the registers.
    constexpr int RPT = NG == 1 ? 8 : 4;
    const int ntask = ns * 8 * (8 / RPT);
    for (int t = tid; t < ntask; t += nthr) {
        const int hf = RPT == 8 ? 0 : t & 1, tt = RPT == 8 ? t : t >> 1;
        const int g = tt & 3, sb = (tt >> 2) & 1, ul = tt >> 3;
        const uint8_t *src = reinterpret_cast<const uint8_t *>(x) +
                             (size_t)(64 * (s0 + ul) + 32 * sb + 8 * g + 4 * hf) * NCV * 2;
        uint32_t h[RPT / 2 * NCV];
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            if constexpr (RPT == 8) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src + 16 * i);
                h[4 * i] = v.x; h[4 * i + 1] = v.y; h[4 * i + 2] = v.z; h[4 * i + 3] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2 *>(src + 8 * i);
                h[2 * i] = v.x; h[2 * i + 1] = v.y;
            }
        }
        // half e of the task is x[RPT rows][NCV]: row e / NCV, column e % NCV
        auto half = [&](int e) -> uint32_t { return (h[e >> 1] >> (16 * (e & 1))) & 0xffffu; };
        if constexpr (CP) {  // compact: NCV vectors per (sub-block, g), 128 NCV bytes per unit
            uint8_t *dst = planes + (size_t)ul * 128 * NCV + (sb * 4 + g) * NCV * 16;
#pragma unroll
            for (int c = 0; c < NCV; ++c)
                *reinterpret_cast<uint4 *>(dst + c * 16) =
                    make_uint4(half(0 * NCV + c) | (half(2 * NCV + c) << 16), half(1 * NCV + c) | (half(3 * NCV + c) << 16),
                               half(4 * NCV + c) | (half(6 * NCV + c) << 16), half(5 * NCV + c) | (half(7 * NCV + c) << 16));
            continue;
        }
        uint8_t *dst = planes + (size_t)ul * NG * V16_UB + sb * 1024 + 16 * g * 16 + 8 * hf;
#pragma unroll
        for (int c = 0; c < 16 * NG; ++c) {
            uint8_t *o = dst + (c >> 4) * V16_UB + (c & 15) * 16;
            if constexpr (RPT == 8) {
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (c < NCV) {
                    v.x = half(0 * NCV + c) | (half(2 * NCV + c) << 16);
                    v.y = half(1 * NCV + c) | (half(3 * NCV + c) << 16);
                    v.z = half(4 * NCV + c) | (half(6 * NCV + c) << 16);
                    v.w = half(5 * NCV + c) | (half(7 * NCV + c) << 16);
                }
                *reinterpret_cast<uint4 *>(o) = v;
            } else {
                uint2 v = make_uint2(0u, 0u);
                if (c < NCV) {
                    v.x = half(0 * NCV + c) | (half(2 * NCV + c) << 16);
                    v.y = half(1 * NCV + c) | (half(3 * NCV + c) << 16);
                }
                *reinterpret_cast<uint2 *>(o) = v;
            }
        }
    }
}

template <int NG, bool CP>
__device__ __forceinline__ void v16_stage(const uint16_t *__restrict__ x, int nc, int s0, int ns, uint8_t *planes,
                                          int tid, int nthr) {
#define V16_CASE(n) case n: v16_copy<n, CP>(x, s0, ns, planes, tid, nthr); break;
    if constexpr (NG == 1) {
        switch (nc) {
        V16_CASE(9) V16_CASE(10) V16_CASE(11) V16_CASE(12) V16_CASE(13) V16_CASE(14) V16_CASE(15)
        default: v16_copy<16>(x, s0, ns, planes, tid, nthr); break;  // (16 columns: never compact)
        }
    } else {
        switch (nc) {
        V16_CASE(17) V16_CASE(18) V16_CASE(19) V16_CASE(20) V16_CASE(21) V16_CASE(22) V16_CASE(23) V16_CASE(24)
        V16_CASE(25) V16_CASE(26) V16_CASE(27) V16_CASE(28) V16_CASE(29) V16_CASE(30) V16_CASE(31)
        default: v16_copy<32>(x, s0, ns, planes, tid, nthr); break;
        }
    }
#undef V16_CASE
}

template <int T_, int NG, bool CP>
__global__ void __launch_bounds__(768) v16_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ x,
                                                   void *__restrict__ y, int N, int K, int nc, int useg, int T,
                                                   int UG, Epilogue ep) {
    static_assert(T_ == Q4_K || T_ == Q5_K, "Q4_K and Q5_K");
    constexpr int SBB = V16Fmt<T_>::bytes, QSO = V16Fmt<T_>::qs, QMAX = V16Fmt<T_>::qmax;
    constexpr int DD = T_ == Q5_K ? 1 : V16_D;  // superblocks in flight (Q5_K: its qh bits take the registers)
    extern __shared__ __attribute__((aligned(16))) uint8_t v16sm[];
    const int tid = (int)threadIdx.x, nthr = (int)blockDim.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (wave-uniform)
    const int tile = wave % T, ug = wave / T;
    // SwiGLU pair: waves of tiles TH..T-1 stream the same rows of ep.W2
    const int TH = ep.W2 ? T >> 1 : T;
    const bool second = tile >= TH;  // (wave-uniform)
    const int trow = second ? tile - TH : tile;
    const uint8_t *Wt = second ? reinterpret_cast<const uint8_t *>(ep.W2) : W;
    const int r = lane & 15, g = lane >> 4;
    // whole 16-row tiles per workgroup (the last tile of the tensor may be
    // short): ceil(N / 16) tiles split as evenly as possible
    const RowSplit split((N + 15) >> 4, (int)blockIdx.x, (int)gridDim.x);
    const int r0 = 16 * split.r0, r1 = min(16 * split.r1, N);
    const int row = r0 + 16 * trow + r;
    const bool tile_ok = r0 + 16 * trow < r1;  // (wave-uniform)
    const uint8_t *wrow = Wt + (size_t)min(row, r1 - 1) * (size_t)((K >> 8) * SBB);
    const int U = K >> 6;
    uint8_t *planes = v16sm;
    // CP (one group, fewer than 16 columns): compact planes of nc columns;
    // the lanes of columns nc..15 read a zero vector after them (written
    // here, ordered by the first segment's barrier)
    uint8_t *zero16 = planes + (size_t)useg * 128 * nc;
    if (CP && tid == 0) *reinterpret_cast<uint4 *>(zero16) = make_uint4(0u, 0u, 0u, 0u);
    v16_f4 acc[NG];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) acc[cg] = v16_f4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < U; s0 += useg) {
        const int ns = min(useg, U - s0);
        // this wave's share of the segment's superblocks (segments start at
        // superblock boundaries); its first ring is issued before the x of
        // the segment is staged (the weights do not depend on it)
        const int nsb = ns >> 2;
        const int b0 = ug * nsb / UG, b1 = (ug + 1) * nsb / UG;
        const bool busy = tile_ok && b0 < b1;  // (wave-uniform)
        const uint8_t *wseg = wrow + SBB * (s0 >> 2);
        auto load = [&](V16Sb &d, int sbl) {
            const uint8_t *p = wseg + SBB * min(sbl, b1 - 1);
            d.h = *reinterpret_cast<const uint4 *>(p);
#pragma unroll
            for (int k = 0; k < 4; ++k) d.q[k] = *reinterpret_cast<const uint2 *>(p + QSO + 32 * k + 8 * g);
            if constexpr (T_ == Q5_K) d.qh = *reinterpret_cast<const uint2 *>(p + 16 + 8 * g);
        };
        V16Sb buf[DD];
        if (busy)
#pragma unroll
            for (int k = 0; k < DD; ++k) load(buf[k], b0 + k);
        if (s0 > 0) __syncthreads();  // every wave is done with the previous segment's planes
        v16_stage<NG, CP>(x, nc, s0, ns, planes, tid, nthr);
        __syncthreads();
        if (!busy) continue;
        for (int i0 = b0; i0 < b1; i0 += DD) {
#pragma unroll
            for (int kk = 0; kk < DD; ++kk) {
                const int sbl = i0 + kk;
                const V16Sb sb = buf[kk];
                load(buf[kk], sbl + DD);
                if (sbl < b1) {  // (wave-uniform)
                    const float d = f16_lo(sb.h.x), dmin = f16_hi(sb.h.x);
                    auto pat = [](uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)v); };
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        // the shifted form of each sub-block (KShift), units of 2^-48
                        const KScales sk = k_scales(sb.h, KScaleSel(k));
                        const KShift kL = k_shift<QMAX, 1>(d, dmin, pat(sk.sc_lo), pat(sk.m_lo));
                        const KShift kH = k_shift<QMAX, 16>(d, dmin, pat(sk.sc_hi), pat(sk.m_hi));
                        const uint32_t w0 = sb.q[k].x, w1 = sb.q[k].y, t0 = w0 >> 8, t1 = w1 >> 8;
                        // Q5_K: the fifth bits (bit 0 / 1 of each qh byte after the
                        // shift: low / high sub-block), as the one-column kernel sets them
                        const uint32_t H0 = T_ == Q5_K ? sb.qh.x >> (2 * k) : 0u, H1 = T_ == Q5_K ? sb.qh.y >> (2 * k) : 0u;
                        const float fh = kH.a * 0x1p-4f, eL = kL.e * 0x1p-24f, eH = kH.e * 0x1p-24f;
#pragma unroll
                        for (int cg = 0; cg < NG; ++cg) {  // each group of 16 columns
                            uint4 xl, xh;
                            if constexpr (CP) {
                                const uint8_t *ub = planes + (size_t)(4 * sbl + k) * 128 * nc + (g * nc + r) * 16;
                                xl = *reinterpret_cast<const uint4 *>(r < nc ? ub : zero16);
                                xh = *reinterpret_cast<const uint4 *>(r < nc ? ub + 64 * nc : zero16);
                            } else {
                                const uint8_t *blk = planes + ((size_t)(4 * sbl + k) * NG + cg) * V16_UB;
                                xl = *reinterpret_cast<const uint4 *>(blk + lane * 16);
                                xh = *reinterpret_cast<const uint4 *>(blk + 1024 + lane * 16);
                            }
                            // low sub-block: weights (8g, 8g+2), (8g+1, 8g+3) of w0, then
                            // of w1 (the patterns formed again per group: fewer live
                            // registers)
                            v16_f4 DL = {0.f, 0.f, 0.f, 0.f}, DH = {0.f, 0.f, 0.f, 0.f};
                            DL = mfma16(xl.x, xl.y, padd((w0 & 0x000f000fu) | ((H0 << 4) & 0x00100010u), kL.neg),
                                        padd((t0 & 0x000f000fu) | ((H0 >> 4) & 0x00100010u), kL.neg), DL);
                            DH = mfma16(xh.x, xh.y, padd((w0 & 0x00f000f0u) | ((H0 << 7) & 0x01000100u), kH.neg),
                                        padd((t0 & 0x00f000f0u) | ((H0 >> 1) & 0x01000100u), kH.neg), DH);
                            DL = mfma16(xl.z, xl.w, padd((w1 & 0x000f000fu) | ((H1 << 4) & 0x00100010u), kL.neg),
                                        padd((t1 & 0x000f000fu) | ((H1 >> 4) & 0x00100010u), kL.neg), DL);
                            DH = mfma16(xh.z, xh.w, padd((w1 & 0x00f000f0u) | ((H1 << 7) & 0x01000100u), kH.neg),
                                        padd((t1 & 0x00f000f0u) | ((H1 >> 1) & 0x01000100u), kH.neg), DH);
                            // the sums of x per sub-block and column, for the min
                            // terms: the same operands against fp16 ones (exact
                            // products)
                            v16_f4 SL = {0.f, 0.f, 0.f, 0.f}, SH = {0.f, 0.f, 0.f, 0.f};
                            SL = mfma16(xl.x, xl.y, V16_ONES, V16_ONES, SL);
                            SH = mfma16(xh.x, xh.y, V16_ONES, V16_ONES, SH);
                            SL = mfma16(xl.z, xl.w, V16_ONES, V16_ONES, SL);
                            SH = mfma16(xh.z, xh.w, V16_ONES, V16_ONES, SH);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float E = __builtin_fmaf(eL, SL[e], eH * SH[e]);
                                acc[cg][e] += __builtin_fmaf(kL.a, DL[e], __builtin_fmaf(fh, DH[e], E));
                            }
                        }
                    }
                }
            }
        }
    }
    // the residual of the lane's outputs, read before the shares are added
    // (res may be y itself: each element is read and written by one lane)
    float rv[NG][4];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * cg + 4 * g + e;
            rv[cg][e] = ep.res && ug == 0 && !second && tile_ok && row < r1 && c < nc ? ep.res[(size_t)row * nc + c] : 0.f;
        }
    // the shares of each tile, added in share order
    __syncthreads();
    float4 *part = reinterpret_cast<float4 *>(v16sm);
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) part[cg * nthr + tid] = make_float4(acc[cg][0], acc[cg][1], acc[cg][2], acc[cg][3]);
    __syncthreads();
    if (ug == 0 && !second && tile_ok && row < r1) {
#pragma unroll
        for (int cg = 0; cg < NG; ++cg) {
            float o[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < UG; ++s) {
                const float4 v = part[cg * nthr + (s * T + tile) * 64 + lane];
                o[0] += v.x;
                o[1] += v.y;
                o[2] += v.z;
                o[3] += v.w;
                if (ep.W2) {  // the same rows of W2: tile + TH
                    const float4 w = part[cg * nthr + (s * T + tile + TH) * 64 + lane];
                    u[0] += w.x;
                    u[1] += w.y;
                    u[2] += w.z;
                    u[3] += w.w;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * cg + 4 * g + e;
                float v = o[e] * 0x1p48f;
                if (ep.W2) v = silu(v) * (u[e] * 0x1p48f);
                if (ep.res) v += rv[cg][e];
                if (c < nc) store_y(y, ep.f16, (size_t)row * nc + c, v);
            }
        }
    }
}

// Whole 16-row tiles per workgroup, at most 8; one workgroup per CU unless
// N has fewer tiles (or more than 8 per CU); 1, 2 or 4 shares per tile (at
// most 12 waves: 168 registers); segments of at most 160 KB of planes, as
// even as possible, in whole superblocks.
template <int T_, int NG, bool CP>
static hipError_t launch_v16g(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc,
                              const Epilogue &ep, hipStream_t st) {
    const int cus = device_cus();
    const int64_t tiles = (N + 15) / 16;
    const int tmax = ep.W2 ? 6 : 8;  // (the pair streams each tile twice)
    const int64_t G = std::max<int64_t>(std::min<int64_t>(cus, tiles), (tiles + tmax - 1) / tmax);
    const int T = (int)((tiles + G - 1) / G) * (ep.W2 ? 2 : 1);  // tiles of the largest workgroup
    const int UG = T <= 3 ? 4 : T <= 6 ? 2 : 1;  // at most 12 waves (168 registers)
    const int threads = 64 * T * UG;
    const int64_t U = K / 64;
    // bytes per unit: compact 128 per column (then a zero vector), else 2 KB per group of 16 columns
    const int64_t ubb = CP ? 128 * nc : NG * V16_UB, extra = CP ? 16 : 0;
    const int64_t smax = (V16_PLANES - extra) / ubb / 4 * 4;  // units per segment at most
    const int64_t nseg = (U + smax - 1) / smax;
    const int useg = (int)(((U + nseg - 1) / nseg + 3) / 4 * 4);  // whole superblocks
    const size_t lds = std::max<size_t>((size_t)(useg * ubb + extra), (size_t)threads * 16 * NG);  // (planes, then the shares)
    if (T < 1 || T > 12 || threads > 768 || lds > 160 * 1024) return hipErrorInvalidValue;
    const hipError_t e = lds_opt_in<v16_kernel<T_, NG, CP>>(160 * 1024);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((v16_kernel<T_, NG, CP>), dim3((unsigned)G), dim3(threads), lds, st, (const uint8_t *)W,
                       (const uint16_t *)x, y, (int)N, (int)K, nc, useg, T, UG, ep);
    return hipGetLastError();
}

// 9-16 columns: one group; 17-32: two groups sharing each unit's patterns
template <int T_>
static hipError_t launch_v16(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc, const Epilogue &ep,
                             hipStream_t st) {
    if (nc > 16) return launch_v16g<T_, 2, false>(W, x, y, N, K, nc, ep, st);
    // compact planes only where they save K segments (their addressing costs
    // 1-4% where the segment count is the same)
    const int64_t U = K / 64;
    auto nseg = [&](int64_t ubb, int64_t extra) {
        const int64_t smax = (V16_PLANES - extra) / ubb / 4 * 4;
        return (U + smax - 1) / smax;
    };
    if (nc < 16 && nseg(128 * nc, 16) < nseg(V16_UB, 0)) return launch_v16g<T_, 1, true>(W, x, y, N, K, nc, ep, st);
    return launch_v16g<T_, 1, false>(W, x, y, N, K, nc, ep, st);
}

// ---------------------------------------------------------------------------
// Q6_K on the same tiles.  w = d * sc * (q - 32) with an int8 scale per 16
// weights, so each matrix instruction covers one scale group: group (n, t, h)
// of a superblock is its weights 128n + 32t + 16h + 0..15 (half n, quarter t,
// half-quarter h); they sit in the 16 ql bytes 64n + 32(t % 2) + 16h + 0..15
// (nibble t / 2) and the 16 qh bytes 32n + 16h + 0..15 (bits 2t, 2t + 1).
// Lane l = r + 16g of a tile supplies weights 4g..4g+3 of a group: dword g of
// its ql and qh chunks.  The four lanes of a row (g = 0..3) each read whole
// 16-byte chunks (ql chunks g and 4 + g, qh chunk g) and a 4 x 4 transpose
// across them (two rounds of lane-row swaps) hands every lane dword g of
// every chunk.  The patterns hold s(q - 32)2^-24 (s = 1 for the low nibbles,
// 16 for the high ones, as in the one-column kernel); no min term.  x planes:
// 8 KB per superblock and group of 16 columns, [n][t][lane][h][4 halves].
// ---------------------------------------------------------------------------
constexpr int V16Q6_SB = 8192;  // LDS bytes per superblock and group of 16 columns
constexpr int V16Q6_MIN = 9;  // fewest columns a Q6_K call takes on the tiles (at 5-8 the 4x4x4 form is faster)

struct V16Q6Sb {
    uint4 ql0, ql1, qh;  // ql chunks g and 4 + g, qh chunk g (lane row g)
    uint4 sc;            // the 16 int8 scales
    uint32_t d;          // fp16 d in the low half
};

// Lane row g (lanes 16g..16g+15) holds dwords R0..R3 of a 16-byte chunk of
// its own; afterwards dword m of lane row g is dword g of row m's chunk.
// v_permlane32_swap exchanges rows 2-3 of its first operand with rows 0-1 of
// its second, v_permlane16_swap rows 1, 3 of the first with rows 0, 2 of the
// second.
__device__ __forceinline__ uint4 v16_xpose(uint4 v) {
    const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return make_uint4(c[0], c[1], e[0], e[1]);
}

template <int NCV>
__device__ __forceinline__ void v16q6_copy(const uint16_t *__restrict__ x, int sb0, int nsb, uint8_t *planes, int tid,
                                           int nthr) {
    constexpr int NG = NCV > 16 ? 2 : 1;
    // task: (superblock, n, t, h, g): rows 128n + 32t + 16h + 4g + 0..3,
    // contiguous (NCV loads of 8 bytes), into half a 16-byte vector per column
    const int ntask = nsb * 64;
    for (int t = tid; t < ntask; t += nthr) {
        const int g = t & 3, h = (t >> 2) & 1, qt = (t >> 3) & 3, n = (t >> 5) & 1, sbl = t >> 6;
        const uint8_t *src = reinterpret_cast<const uint8_t *>(x) +
                             (size_t)(256 * (sb0 + sbl) + 128 * n + 32 * qt + 16 * h + 4 * g) * NCV * 2;
        uint32_t hv[2 * NCV];
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const uint2 v = *reinterpret_cast<const uint2 *>(src + 8 * i);
            hv[2 * i] = v.x;
            hv[2 * i + 1] = v.y;
        }
        auto half = [&](int e) -> uint32_t { return (hv[e >> 1] >> (16 * (e & 1))) & 0xffffu; };
        if constexpr (NG == 1 && NCV < 16) {  // compact: NCV vectors per (n, t, g), 512 NCV bytes per superblock
            uint8_t *dst = planes + (size_t)sbl * 512 * NCV + ((n * 4 + qt) * 4 + g) * NCV * 16 + 8 * h;
#pragma unroll
            for (int c = 0; c < NCV; ++c)  // rows 0, 2, 1, 3: the pattern order
                *reinterpret_cast<uint2 *>(dst + c * 16) =
                    make_uint2(half(0 * NCV + c) | (half(2 * NCV + c) << 16), half(1 * NCV + c) | (half(3 * NCV + c) << 16));
        } else {
            uint8_t *dst = planes + (size_t)sbl * NG * V16Q6_SB + ((n * 4 + qt) * 64 + 16 * g) * 16 + 8 * h;
#pragma unroll
            for (int c = 0; c < 16 * NG; ++c) {
                uint2 v = make_uint2(0u, 0u);
                if (c < NCV) {  // rows 0, 2, 1, 3: the pattern order
                    v.x = half(0 * NCV + c) | (half(2 * NCV + c) << 16);
                    v.y = half(1 * NCV + c) | (half(3 * NCV + c) << 16);
                }
                *reinterpret_cast<uint2 *>(dst + (c >> 4) * V16Q6_SB + (c & 15) * 16) = v;
            }
        }
    }
}

template <int NG>
__device__ __forceinline__ void v16q6_stage(const uint16_t *__restrict__ x, int nc, int sb0, int nsb, uint8_t *planes,
                                            int tid, int nthr) {
#define V16_CASE(n) \
    case n: v16q6_copy<n>(x, sb0, nsb, planes, tid, nthr); break;
    if constexpr (NG == 1) {
        switch (nc) {
        V16_CASE(5) V16_CASE(6) V16_CASE(7) V16_CASE(8) V16_CASE(9) V16_CASE(10) V16_CASE(11) V16_CASE(12)
        V16_CASE(13) V16_CASE(14) V16_CASE(15)
        default: v16q6_copy<16>(x, sb0, nsb, planes, tid, nthr); break;
        }
    } else {
        switch (nc) {
        V16_CASE(17) V16_CASE(18) V16_CASE(19) V16_CASE(20) V16_CASE(21) V16_CASE(22) V16_CASE(23) V16_CASE(24)
        V16_CASE(25) V16_CASE(26) V16_CASE(27) V16_CASE(28) V16_CASE(29) V16_CASE(30) V16_CASE(31)
        default: v16q6_copy<32>(x, sb0, nsb, planes, tid, nthr); break;
        }
    }
#undef V16_CASE
}

// Workgroups, tiles and shares as in v16_kernel; segments of whole
// superblocks (segsb of them, at most 160 KB of planes).
//
// IQ4_XS on the same kernel: sub-block ib (weights 32ib + 0..31, one 6-bit
// scale) is qs chunk ib (16 bytes: weight j in the low nibble of byte j,
// weight 16 + j in the high one), so plane group (n, t, h) is sub-block
// 4n + t, nibble h, and lane row g loads chunks g and 4 + g; the codebook
// lookup gives the patterns kv 2^-24 (signed, exact) and the scale is
// d 2^24 (ls - 32).
template <int T_, int NG, bool CP>
__global__ void __launch_bounds__(768) v16q6_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ x,
                                                    void *__restrict__ y, int N, int K, int nc, int segsb, int T,
                                                    int UG, Epilogue ep) {
    constexpr int DD = NG == 2 ? 1 : V16_D;  // superblocks in flight (two groups: the accumulators take the registers)
    extern __shared__ __attribute__((aligned(16))) uint8_t v16sm[];
    const int tid = (int)threadIdx.x, nthr = (int)blockDim.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (wave-uniform)
    const int tile = wave % T, ug = wave / T;
    // SwiGLU pair: waves of tiles TH..T-1 stream the same rows of ep.W2
    const int TH = ep.W2 ? T >> 1 : T;
    const bool second = tile >= TH;  // (wave-uniform)
    const int trow = second ? tile - TH : tile;
    const uint8_t *Wt = second ? reinterpret_cast<const uint8_t *>(ep.W2) : W;
    const int r = lane & 15, g = lane >> 4;
    const RowSplit split((N + 15) >> 4, (int)blockIdx.x, (int)gridDim.x);
    const int r0 = 16 * split.r0, r1 = min(16 * split.r1, N);
    const int row = r0 + 16 * trow + r;
    const bool tile_ok = r0 + 16 * trow < r1;  // (wave-uniform)
    const int S = K >> 8;
    static_assert(T_ == Q6_K || T_ == IQ4_XS, "Q6_K and IQ4_XS");
    constexpr int SBB = T_ == Q6_K ? 210 : 136;
    const uint8_t *wrow = Wt + (size_t)min(row, r1 - 1) * (size_t)(S * SBB);
    uint8_t *planes = v16sm;
    // CP (one group, fewer than 16 columns): compact planes of nc columns;
    // the lanes of columns nc..15 read a zero vector after them (written
    // here, ordered by the first segment's barrier).  At 16 columns the
    // plane offsets are compile-time constants (immediate LDS offsets).
    uint8_t *zero16 = planes + (size_t)segsb * 512 * nc;
    if (CP && tid == 0) *reinterpret_cast<uint4 *>(zero16) = make_uint4(0u, 0u, 0u, 0u);
    v16_f4 acc[NG];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) acc[cg] = v16_f4{0.f, 0.f, 0.f, 0.f};

    for (int sb0 = 0; sb0 < S; sb0 += segsb) {
        const int nsb = min(segsb, S - sb0);
        const int b0 = ug * nsb / UG, b1 = (ug + 1) * nsb / UG;
        const bool busy = tile_ok && b0 < b1;  // (wave-uniform)
        const uint8_t *wseg = wrow + SBB * sb0;
        // superblocks are 2-byte (Q6_K) or 8-byte (IQ4_XS) aligned: unaligned 16-byte loads
        auto load = [&](V16Q6Sb &d, int sbl) {
            const uint8_t *p = wseg + SBB * min(sbl, b1 - 1);
            if constexpr (T_ == Q6_K) {
                d.ql0 = *reinterpret_cast<const uint4 *>(p + 16 * g);
                d.ql1 = *reinterpret_cast<const uint4 *>(p + 64 + 16 * g);
                d.qh = *reinterpret_cast<const uint4 *>(p + 128 + 16 * g);
                d.sc = *reinterpret_cast<const uint4 *>(p + 192);
                d.d = *reinterpret_cast<const uint16_t *>(p + 208);
            } else {  // d | scales_h << 16, scales_l, qs
                const uint2 h = *reinterpret_cast<const uint2 *>(p);
                d.d = h.x;
                d.sc.x = h.y;
                d.ql0 = *reinterpret_cast<const uint4 *>(p + 8 + 16 * g);
                d.ql1 = *reinterpret_cast<const uint4 *>(p + 72 + 16 * g);
            }
        };
        V16Q6Sb buf[DD];
        if (busy)
#pragma unroll
            for (int k = 0; k < DD; ++k) load(buf[k], b0 + k);
        if (sb0 > 0) __syncthreads();  // every wave is done with the previous segment's planes
        v16q6_stage<NG>(x, nc, sb0, nsb, planes, tid, nthr);
        __syncthreads();
        if (!busy) continue;
        for (int i0 = b0; i0 < b1; i0 += DD) {
#pragma unroll
            for (int kk = 0; kk < DD; ++kk) {
                const int sbl = i0 + kk;
                const V16Q6Sb sb = buf[kk];
                load(buf[kk], sbl + DD);
                if (sbl < b1) {  // (wave-uniform)
                    // dword g of ql chunk 4n + 2(t % 2) + h and of qh chunk 2n + h
                    // (IQ4_XS: dword g of qs chunk 4n + t)
                    const uint4 L0 = v16_xpose(sb.ql0), L1 = v16_xpose(sb.ql1);
                    const uint4 HQ = T_ == Q6_K ? v16_xpose(sb.qh) : make_uint4(0u, 0u, 0u, 0u);
                    const uint32_t ql[8] = {L0.x, L0.y, L0.z, L0.w, L1.x, L1.y, L1.z, L1.w};
                    const uint32_t qh[4] = {HQ.x, HQ.y, HQ.z, HQ.w};
                    const float d = f16_lo(sb.d);
                    const uint32_t scw[4] = {sb.sc.x, sb.sc.y, sb.sc.z, sb.sc.w};
#pragma unroll
                    for (int n = 0; n < 2; ++n)
#pragma unroll
                        for (int qt = 0; qt < 4; ++qt) {
                            uint4 xv[NG];
#pragma unroll
                            for (int cg = 0; cg < NG; ++cg)
                                xv[cg] = *reinterpret_cast<const uint4 *>(
                                    CP ? (r < nc ? planes + (size_t)sbl * 512 * nc + (((n * 4 + qt) * 4 + g) * nc + r) * 16
                                                 : zero16)
                                       : planes + ((size_t)sbl * NG + cg) * V16Q6_SB + ((n * 4 + qt) * 64 + lane) * 16);
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                uint32_t p0, p1;
                                float f;
                                if constexpr (T_ == IQ4_XS) {
                                    const int ib = 4 * n + qt;
                                    iq4_pairs(h ? ql[ib] >> 4 : ql[ib], p0, p1);
                                    const uint32_t lo4 = __builtin_amdgcn_ubfe(sb.sc.x, 4u * ib, 4u);
                                    const uint32_t hi2 = __builtin_amdgcn_ubfe(sb.d, 16u + 2u * ib, 2u);
                                    f = d * 0x1p24f * (float)((int)(lo4 | hi2 << 4) - 32);
                                } else {
                                const uint32_t QL = ql[4 * n + 2 * (qt & 1) + h], QH = qh[2 * n + h];
                                if (qt < 2) {  // low nibbles, s = 1
                                    p0 = (QL & 0x000f000fu) | (((QH >> (2 * qt)) << 4) & 0x00300030u);
                                    p1 = ((QL >> 8) & 0x000f000fu) | (((QH >> (2 * qt + 8)) << 4) & 0x00300030u);
                                    p0 = padd(p0, Q6_OFF_LO);
                                    p1 = padd(p1, Q6_OFF_LO);
                                } else {  // high nibbles in place, s = 16
                                    p0 = (QL & 0x00f000f0u) | (((QH >> (2 * qt)) << 8) & 0x03000300u);
                                    p1 = ((QL >> 8) & 0x00f000f0u) | (((QH >> (2 * qt + 8)) << 8) & 0x03000300u);
                                    p0 = padd(p0, Q6_OFF_HI);
                                    p1 = padd(p1, Q6_OFF_HI);
                                }
                                const int si = 8 * n + 2 * qt + h;  // scale of the group
                                const int scv = (int)(int8_t)(uint8_t)(scw[si >> 2] >> (8 * (si & 3)));
                                f = d * (float)scv * (qt < 2 ? 0x1p24f : 0x1p20f);
                                }
#pragma unroll
                                for (int cg = 0; cg < NG; ++cg) {
                                    const v16_f4 D = mfma16(h ? xv[cg].z : xv[cg].x, h ? xv[cg].w : xv[cg].y, p0, p1,
                                                            v16_f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                                    for (int e = 0; e < 4; ++e) acc[cg][e] = __builtin_fmaf(f, D[e], acc[cg][e]);
                                }
                            }
                        }
                }
            }
        }
    }
    // the residual of the lane's outputs, read before the shares are added
    // (res may be y itself: each element is read and written by one lane)
    float rv[NG][4];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * cg + 4 * g + e;
            rv[cg][e] = ep.res && ug == 0 && !second && tile_ok && row < r1 && c < nc ? ep.res[(size_t)row * nc + c] : 0.f;
        }
    // the shares of each tile, added in share order
    __syncthreads();
    float4 *part = reinterpret_cast<float4 *>(v16sm);
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) part[cg * nthr + tid] = make_float4(acc[cg][0], acc[cg][1], acc[cg][2], acc[cg][3]);
    __syncthreads();
    if (ug == 0 && !second && tile_ok && row < r1) {
#pragma unroll
        for (int cg = 0; cg < NG; ++cg) {
            float o[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < UG; ++s) {
                const float4 v = part[cg * nthr + (s * T + tile) * 64 + lane];
                o[0] += v.x;
                o[1] += v.y;
                o[2] += v.z;
                o[3] += v.w;
                if (ep.W2) {  // the same rows of W2: tile + TH
                    const float4 w = part[cg * nthr + (s * T + tile + TH) * 64 + lane];
                    u[0] += w.x;
                    u[1] += w.y;
                    u[2] += w.z;
                    u[3] += w.w;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * cg + 4 * g + e;
                float v = o[e];
                if (ep.W2) v = silu(v) * (u[e]);
                if (ep.res) v += rv[cg][e];
                if (c < nc) store_y(y, ep.f16, (size_t)row * nc + c, v);
            }
        }
    }
}

template <int T_, int NG, bool CP>
static hipError_t launch_v16q6g(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc,
                              const Epilogue &ep, hipStream_t st) {
    const int cus = device_cus();
    const int64_t tiles = (N + 15) / 16;
    const int tmax = ep.W2 ? 6 : 8;  // (the pair streams each tile twice)
    const int64_t G = std::max<int64_t>(std::min<int64_t>(cus, tiles), (tiles + tmax - 1) / tmax);
    const int T = (int)((tiles + G - 1) / G) * (ep.W2 ? 2 : 1);
    // shares per tile: one group of columns runs faster with two shares at
    // 2-3 tiles (more superblocks per wave between the segment barriers)
    const int UG = T <= 1 ? 4 : T <= 3 ? (NG == 1 ? 2 : 4) : T <= 6 ? 2 : 1;
    const int threads = 64 * T * UG;
    const int64_t S = K / 256;
    // bytes per superblock: compact 512 per column (then a zero vector),
    // else 8 KB per group of 16 columns
    const int64_t sbb = CP ? 512 * nc : NG * V16Q6_SB, extra = CP ? 16 : 0;
    const int64_t smax = (V16_PLANES - extra) / sbb;  // superblocks per segment at most
    const int64_t nseg = (S + smax - 1) / smax;
    const int segsb = (int)((S + nseg - 1) / nseg);
    const size_t lds = std::max<size_t>((size_t)(segsb * sbb + extra), (size_t)threads * 16 * NG);
    if (T < 1 || T > 12 || threads > 768 || lds > 160 * 1024) return hipErrorInvalidValue;
    const hipError_t e = lds_opt_in<v16q6_kernel<T_, NG, CP>>(160 * 1024);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((v16q6_kernel<T_, NG, CP>), dim3((unsigned)G), dim3(threads), lds, st, (const uint8_t *)W,
                       (const uint16_t *)x, y, (int)N, (int)K, nc, segsb, T, UG, ep);
    return hipGetLastError();
}

// 5-16 columns: one group; 17-32: two
template <int T_>
static inline hipError_t launch_v16q6(const void *W, const void *x, void *y, int64_t N, int64_t K, int nc,
                                      const Epilogue &ep, hipStream_t st) {
    if (nc > 16) return launch_v16q6g<T_, 2, false>(W, x, y, N, K, nc, ep, st);
    return nc < 16 ? launch_v16q6g<T_, 1, true>(W, x, y, N, K, nc, ep, st)
                   : launch_v16q6g<T_, 1, false>(W, x, y, N, K, nc, ep, st);
}

}  // namespace qk
