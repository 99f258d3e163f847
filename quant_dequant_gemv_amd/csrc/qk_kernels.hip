// qk_kernels.hip -- gfx950 kernels of the k-quant GEMV and their launchers.
//
// gemv1_kernel : y = dequant(W) @ x for one column, the decode GEMV of the T4
//                dossier's "Mixed-Quant GEMV" prompt (section SPEC).  Every
//                weight byte is read from HBM once, with 16-byte loads
//                (HARD CONSTRAINTS: 128-bit loads); quants are unpacked in
//                registers and dotted with x by v_dot2_f32_f16 into fp32
//                accumulators (design-doc prompt, PHYSICS & CONTRACT: fp32
//                accumulation; fp16x2 is fine for the GEMV).  x is not
//                quantised.
// dequant_kernel: the same unit loads and unpacking, writing fp32 weights --
//                the bit-exact check path.
//
// Shifted form.  For a Q4_K/Q5_K sub-block j of 32 weights (KShift in
// qk_format.h), with a = d*sc_j, b = dmin*m_j and an integer c_j near b/a,
//     sum_i w_i x_i = a * sum_i (q_i - c_j) x_i  +  (a*c_j - b) * sum_i x_i ,
// and for a Q6_K group g of 16 weights
//     sum_i w_i x_i = d*sc_g * sum_i (q_i - 32) x_i ;
// q - c is one packed fp16 add per pair of weights, every product is exact,
// and no term exceeds a few times its weight's share of sum |w x|, so the
// fp32 sums cannot cancel.  The sub-block sums of x are formed once per lane
// (x stays in registers), so the per-weight work is the quant unpack, half a
// packed add and half a dot2.
#include "qk_format.h"
#include "qk_epilogue.h"
#include "qk_launch.h"

#include <algorithm>
#include <mutex>

namespace qk {

constexpr int WG = 256;  // threads per workgroup

// ---------------------------------------------------------------------------
// x held in registers.  A lane works on one fixed 64-weight unit column u of
// K for every row it visits, so it loads the 64 x values of that unit once,
// as 32 dwords of fp16 pairs in the order the quant patterns produce:
//   Q4_K/Q5_K: xr[2i], xr[2i+1]      = pairs A, B of qs word i, low sub-block
//              xr[16+2i], xr[17+2i]  = the same for the high sub-block
//              (pair A = weights (4i, 4i+2), pair B = (4i+1, 4i+3))
//   Q6_K:      xr[8t+2i], xr[8t+2i+1] = pairs A, B of word i of quarter t
// plus, for Q4_K/Q5_K, the fp32 sums of x per sub-block, xsum[0..1] (fixed
// summation order; Q6_K needs none: its -32 is taken on the patterns).
// ---------------------------------------------------------------------------
template <int T>
struct XReg {
    uint32_t xr[32];
    float xsum[2];
};

// a from the lane that the DPP control names (a full-rate VALU move)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float a) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), CTRL, 0xf, 0xf, false));
}

constexpr uint32_t ONES_F16X2 = 0x3c003c00u;  // the fp16 pair (1, 1)

// Eight consecutive halves (one 16-byte vector, two groups of four) -> the
// four pair dwords of pattern order (per group: (0, 2), then (1, 3)); returns
// their sum (fp32, fixed order: one pair after the other).
__device__ __forceinline__ float x_pairs8(const uint4 &v, uint32_t *o) {
    o[0] = (v.x & 0xffffu) | (v.y << 16);
    o[1] = (v.x >> 16) | (v.y & 0xffff0000u);
    o[2] = (v.z & 0xffffu) | (v.w << 16);
    o[3] = (v.z >> 16) | (v.w & 0xffff0000u);
    return dot2(v.w, ONES_F16X2, dot2(v.z, ONES_F16X2, dot2(v.y, ONES_F16X2, dot2(v.x, ONES_F16X2, 0.f))));
}

// Sixteen consecutive halves (two 16-byte vectors) -> 8 pair dwords + fp32 sum.
__device__ __forceinline__ float x_pairs16(const uint4 &v0, const uint4 &v1, uint32_t *o) {
    return x_pairs8(v0, o) + x_pairs8(v1, o + 4);
}

// x of one segment is staged in LDS ready for the dot: every 64-weight unit
// takes 144 bytes, its 32 pair dwords (16-byte chunk c of the segment, i.e.
// halves 8c .. 8c+7, as the four pair dwords of x_pairs8 at 144*(c/8) +
// 16*(c%8)) and then the fp32 sums of its two 32-weight sub-blocks (times
// 2^-24, the unit of the partial sums) at 144*(c/8) + 128.  The 16-byte pad
// also puts the eight 16-byte reads of the lanes of a wave (each of its own
// unit) on distinct banks.
constexpr int XSTRIDE = 144;

__device__ __forceinline__ uint4 x_chunk(const uint8_t *xl, int c) {
    return *reinterpret_cast<const uint4 *>(xl + XSTRIDE * (c >> 3) + 16 * (c & 7));
}

// Stage x[64*s0 .. 64*(s0+ns)) into LDS: coalesced 16-byte global reads, four
// per thread per round, issued together, each chunk turned into its pair
// dwords and sum by the thread that read it.  The four chunks of a
// sub-block are consecutive, and chunk b + tid + k*nthr (b, nthr multiples
// of 4) has the residue of tid mod 4: they sit in one quad of lanes, whose
// DPP sum (pairs, then the two pairs) every lane of the quad holds.
// Indices past the segment are clamped for the reads (every lane takes part
// in the DPP sums) and write nothing.  between() runs once, after the first
// chunks' loads are issued and before they are waited for (the caller's
// weight loads then queue behind them).
struct NoLoads {
    __device__ void operator()() const {}
};
template <class Between = NoLoads>
__device__ __forceinline__ void stage_x(uint8_t *xl, const uint16_t *__restrict__ x, int s0, int ns, int tid,
                                        int nthr, const Between &between = Between()) {
    const uint4 *xg = reinterpret_cast<const uint4 *>(x) + (size_t)s0 * 8;
    const int nch = ns * 8;
    for (int b = 0; b < nch; b += 4 * nthr) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = xg[min(b + tid + k * nthr, nch - 1)];
        if (b == 0) between();  // after the first chunks' loads, before their wait
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = b + tid + k * nthr;
            uint32_t o[4];
            float sum = x_pairs8(v[k], o);
            sum += dpp_f32<0xb1>(sum);  // quad_perm [1,0,3,2]
            sum += dpp_f32<0x4e>(sum);  // quad_perm [2,3,0,1]
            if (c < nch) {
                uint8_t *unit = xl + XSTRIDE * (c >> 3);
                *reinterpret_cast<uint4 *>(unit + 16 * (c & 7)) = make_uint4(o[0], o[1], o[2], o[3]);
                if ((c & 3) == 0) reinterpret_cast<float *>(unit + 128)[(c >> 2) & 1] = sum * 0x1p-24f;
            }
        }
    }
}

// Q6_K: the lane's x straight from global memory (unit u of the row).  A
// Q6_K segment's x is up to 3.4x larger per weight byte than Q4_K's, and with
// one unit in flight per lane the copy's barrier delays the first weights:
// the direct loads measured faster for it.
__device__ __forceinline__ void load_x_q6(XReg<Q6_K> &X, const uint16_t *__restrict__ x, int u) {
    const uint4 *xv = reinterpret_cast<const uint4 *>(x);  // 8 halves per vector
    const int s = u >> 2, n = (u >> 1) & 1, b = u & 1;
    uint4 v[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k = 256 * s + 128 * n + 32 * t + 16 * b;  // first weight of quarter t
        v[2 * t] = xv[k >> 3];
        v[2 * t + 1] = xv[(k >> 3) + 1];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) (void)x_pairs16(v[2 * t], v[2 * t + 1], X.xr + 8 * t);
}

// The lane's x (Q4_K/Q5_K) from the staged copy; ul is the unit index within
// the segment.
template <int T>
__device__ __forceinline__ void load_x(XReg<T> &X, const uint8_t *xl, int ul) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint4 v = x_chunk(xl, 8 * ul + j);
        X.xr[4 * j] = v.x;
        X.xr[4 * j + 1] = v.y;
        X.xr[4 * j + 2] = v.z;
        X.xr[4 * j + 3] = v.w;
    }
    const float2 sums = *reinterpret_cast<const float2 *>(xl + XSTRIDE * ul + 128);
    X.xsum[0] = sums.x;
    X.xsum[1] = sums.y;
}

// Q6_K: sum over quarter t of sc_t * sum (q - 32) x, the -32 taken on the
// patterns (every product exact, no cancellation between two sums).
template <int L>
__device__ __forceinline__ float unit_dot_q6(const Unit<Q6_K> &U, int q, const XReg<Q6_K> &X) {
    float R[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t p[8];
        U.patterns(i, q, p);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t off = t < 2 ? Q6_OFF_LO : Q6_OFF_HI;
            R[t] = dot2(padd(p[2 * t], off), X.xr[8 * t + 2 * i], R[t]);
            R[t] = dot2(padd(p[2 * t + 1], off), X.xr[8 * t + 2 * i + 1], R[t]);
        }
    }
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float k = t < 2 ? 0x1p24f : 0x1p20f;  // patterns hold s*(q-32)*2^-24, s = 1 or 16
        acc = __builtin_fmaf((float)U.template scale<L>(t, q), R[t] * k, acc);
    }
    return f16_lo(U.d) * acc;
}

// Dot of one unit with the register-held x of the same unit column.
// IQ4_XS: d*(ls - 32) * sum kv x per sub-block, kv*2^-24 on the patterns
// (signed, exact) and d*2^24 from the unit: no min term, nothing to cancel.
// Word i of the low sub-block holds x pairs i (low nibbles) and 4 + i (high);
// word 4 + i of the high sub-block pairs 8 + i and 12 + i.
__device__ __forceinline__ float unit_dot_iq4(const Unit<IQ4_XS> &U, int q, const XReg<IQ4_XS> &X) {
    float aL = 0.f, aH = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t pl[4], ph[4];
        U.patterns(i, q, pl);
        U.patterns(i + 4, q, ph);
        aL = dot2(pl[0], X.xr[2 * i], aL);
        aH = dot2(ph[0], X.xr[2 * (i + 8)], aH);
        aL = dot2(pl[1], X.xr[2 * i + 1], aL);
        aH = dot2(ph[1], X.xr[2 * (i + 8) + 1], aH);
        aL = dot2(pl[2], X.xr[2 * (i + 4)], aL);
        aH = dot2(ph[2], X.xr[2 * (i + 12)], aH);
        aL = dot2(pl[3], X.xr[2 * (i + 4) + 1], aL);
        aH = dot2(ph[3], X.xr[2 * (i + 12) + 1], aH);
    }
    const float d = U.d24();
    return __builtin_fmaf(d * (float)U.scale(q, 0), aL, d * (float)U.scale(q, 1) * aH);
}

template <int T, int L>
__device__ __forceinline__ float unit_dot(const Unit<T> &U, int q, const KScaleSel &sel, const XReg<T> &X) {
    if constexpr (T == IQ4_XS) {
        return unit_dot_iq4(U, q, X);
    } else if constexpr (T == Q6_K) {
        return unit_dot_q6<L>(U, q, X);
    } else {
        // The shifted form of each sub-block (KShift).  Units of 2^-48: the
        // 6-bit sc / m read as fp16 bit patterns are sc*2^-24 / m*2^-24, the
        // patterns hold s*(q - c)*2^-24 (s = 1 low, 16 high sub-block) and the
        // x sums are held times 2^-24.
        constexpr int QMAX = T == Q4_K ? 15 : 31;
        const uint4 h = U.header();
        const KScales s = k_scales(h, sel);
        const float d = f16_lo(h.x), dmin = f16_hi(h.x);
        auto pat = [](uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)v); };
        const KShift kL = k_shift<QMAX, 1>(d, dmin, pat(s.sc_lo), pat(s.m_lo));
        const KShift kH = k_shift<QMAX, 16>(d, dmin, pat(s.sc_hi), pat(s.m_hi));
        uint32_t p[4];
        U.patterns(0, q, p);
        float aL = dot2(padd(p[0], kL.neg), X.xr[0], 0.f), aH = dot2(padd(p[2], kH.neg), X.xr[16], 0.f);
        aL = dot2(padd(p[1], kL.neg), X.xr[1], aL);
        aH = dot2(padd(p[3], kH.neg), X.xr[17], aH);
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            U.patterns(i, q, p);
            aL = dot2(padd(p[0], kL.neg), X.xr[2 * i], aL);
            aL = dot2(padd(p[1], kL.neg), X.xr[2 * i + 1], aL);
            aH = dot2(padd(p[2], kH.neg), X.xr[16 + 2 * i], aH);
            aH = dot2(padd(p[3], kH.neg), X.xr[17 + 2 * i], aH);
        }
        // aL = 2^-24 sum (q-c) x, aH = 2^-20 sum (q-c) x
        float acc = kL.e * X.xsum[0];
        acc = __builtin_fmaf(kH.e, X.xsum[1], acc);
        acc = __builtin_fmaf(kL.a, aL, acc);
        return __builtin_fmaf(kH.a * 0x1p-4f, aH, acc);
    }
}


// ---------------------------------------------------------------------------
// One column, x-stationary and row-balanced.
//
// Workgroup b owns a contiguous run of floor(N/G) or ceil(N/G) rows (G =
// gridDim.x; RowSplit), so every workgroup streams the same number of bytes
// to within one row.  K is
// walked in segments of at most `useg` units.  Inside a segment lane
// t < P*useg owns unit column uc = t % useg and row phase ph = t / useg: it
// holds x of that unit in registers and visits rows r0+ph, r0+ph+P, ... ; a
// wave reads up to 16 consecutive superblocks of one row per load.
//
// The rows of a lane are taken RL at a time, and the body for RL rows is
// straight-line code with a ring of D units in flight.  There is no branch
// in it: row offsets past the workgroup's last row are clamped to it, and
// every lane (also a lane past the last row, or a tail lane of the last wave)
// writes its partial sum to a slot of its own, which the final reduction
// reads only for real rows -- so the compiler knows exactly how many loads
// are in flight and waits for one unit at a time: the math on the first rows
// overlaps the arrival of the later ones.  At the end every row's partials
// are added in a fixed order.
// ---------------------------------------------------------------------------
// Workgroup blk of nblk (nthr threads, a multiple of 64) takes the rows
// RowSplit(N, blk, nblk) gives it.  PAIR (the SwiGLU epilogue): the workgroup
// streams those rows of W and then of ep.W2 as 2R rows of one schedule, and
// row r's output combines the sums of rows r and R + r.  EPI: the store
// applies ep's residual / fp16 options (else it is the plain fp32 store).
// Hook: called once by every thread after the first round's weight loads are
// issued and before x or the residual is read (the chain kernel waits there
// for the previous step; a no-op elsewhere).  With a real hook every type
// issues its first round before reading x.
struct NoHook {
    __device__ void operator()() const {}
};

// __syncthreads() calls of one body, the hook's own excepted (waves of the
// workgroup that sit out a body execute as many to keep the barriers in step).
__host__ __device__ constexpr int body_syncs(int T, int U, int useg) {
    return T == Q6_K ? 1 : 2 * ((U + useg - 1) / useg);
}

template <int T, int L, int RL, int D, bool NT, bool PAIR, bool EPI, class Hook = NoHook>
__device__ __forceinline__ void gemv1_body(const uint8_t *__restrict__ W, const uint16_t *__restrict__ x,
                                           void *y, int N, int K, int useg, int P, int blk, int nblk,
                                           int nthr, const Epilogue &ep, const Hook &hook = Hook(), int fc = 0,
                                           int fcap = 0) {
    extern __shared__ __attribute__((aligned(16))) float part[];  // partial sums, slot rows of useg floats
    constexpr int DD = D < RL ? D : RL;  // units in flight
    const int tid = (int)threadIdx.x;
    const RowSplit split(N, blk, nblk, fc, fcap);
    const int r0 = split.r0, r1 = split.r1;
    const int R = r1 - r0;
    const int RV = PAIR ? 2 * R : R;  // rows of the schedule
    const int U = K >> 6;
    const size_t row_bytes = (size_t)layout_row_bytes(T, L, K);
    const int ph = small_div(tid, useg), uc = tid - ph * useg;
    const bool lane_ok = ph < P;
    const int ph_c = lane_ok ? ph : 0;
    const int rows_lane = small_div(RV + P - 1, P);  // same schedule for every lane
    // Q4_K issues weight loads of a segment's first round before staging its
    // x (the early ring: see below), except where a unit live across the
    // staging would spill under the 128-register bound: rounds of four rows,
    // and the epilogue and pair variants on PLANAR rows.  Q5_K (no gain),
    // Q6_K (x read per lane) and IQ4_XS keep the plain order.
    constexpr bool CHAIN = !__is_same(Hook, NoHook);
    constexpr bool PRE = CHAIN || (T == Q4_K && RL != 4 && (L == GGUF || (!EPI && !PAIR)));
    // Partial sums: the lane of phase ph (tail lanes ph >= P included) writes
    // its i-th row to slot row i*PT + ph, PT = phases incl. the tail, so every
    // lane owns a distinct slot and no write needs a guard.  Row r of the
    // workgroup is slot row (r / P) * PT + r % P.
    const int PT = small_div(nthr + useg - 1, useg);
    const int slot0 = ph * useg + uc, slot_step = PT * useg;
    uint8_t *xl = reinterpret_cast<uint8_t *>(part + rows_lane * PT * useg);  // the segment's x
    // residuals for the store: the final reduction gives row group g = tid/16
    // rows g, g + NG, g + 2NG, ... (NG = nthr/16); lane j of the group reads
    // the residual of its j-th row now, and the storing lane fetches it with
    // a cross-lane read at the end
    float resp = 0.f;
    auto read_res = [&]() {
        if constexpr (EPI) {
            const int rj = (tid >> 4) + (tid & 15) * (nthr >> 4);
            if (ep.res && rj < R) resp = ep.res[r0 + rj];
        }
    };
    if constexpr (!PRE) {
        hook();
        read_res();
    }

    for (int s0 = 0; s0 < U; s0 += useg) {
        const int ns = min(useg, U - s0);
        const bool col_ok = lane_ok && uc < ns;
        const int u = s0 + min(uc, ns - 4 + (uc & 3));  // clamped, same q
        const int q = u & 3;
        const KScaleSel sel(q);
        const UnitAddr<T, L> ua(K >> 8, u);
        // lane rows past the workgroup's last row re-read the last row.
        // (64-bit row pointers: loads addressed as a uniform base plus a
        // 32-bit lane offset measured 10-30% slower)
        auto load_row = [&](Unit<T> &dst, int i) {
            if constexpr (PAIR) {
                const int v = min(ph_c + P * i, RV - 1);
                const uint8_t *base = v < R ? W + (size_t)(r0 + v) * row_bytes
                                            : reinterpret_cast<const uint8_t *>(ep.W2) +
                                                  (size_t)(r0 + v - R) * row_bytes;
                dst.template load<NT, L>(base, ua);
            } else {
                const int row = min(r0 + ph_c + P * i, r1 - 1);
                dst.template load<NT, L>(W + (size_t)row * row_bytes, ua);
            }
        };
        // the round of RL rows from row i0 of the lane: a straight line with
        // a ring of DD units in flight, the first DD already issued
        auto run_round = [&](Unit<T> *buf, const XReg<T> &X, int i0) {
#pragma unroll
            for (int p = 0; p < RL; ++p) {
                const float v = unit_dot<T, L>(buf[p % DD], q, sel, X);
                if (p + DD < RL) load_row(buf[p % DD], i0 + p + DD);
                // the round's rows past rows_lane (RL need not divide it) have
                // no slot: the partial-sum region ends there
                if (i0 + p < rows_lane) {
                    float *slot = part + slot0 + (i0 + p) * slot_step;
                    if (s0 == 0) *slot = v;
                    else *slot += col_ok ? v : 0.f;  // a short last segment: lanes past it add nothing
                }
            }
        };
        XReg<T> X;
        if constexpr (PRE) {
            // the first round's ring is issued before x is staged (the
            // copy's global reads come after it but are waited for alone:
            // loads retire in order, and the ring is older)
            Unit<T> buf[DD];
            if (T != Q6_K && s0 > 0) __syncthreads();  // every lane holds the previous segment's x in registers
            // Before the copy the chain issues its whole first ring (its wait
            // for the previous step comes next); a single launch issues the
            // first unit only -- the smaller opening burst of the whole grid
            // brings every wave's first unit in sooner -- and the rest of the
            // ring after the copy's loads (GGUF rows) or after its wait
            // (PLANAR rows), as measured fastest.
            constexpr int EARLY = CHAIN ? DD : 1;
#pragma unroll
            for (int p = 0; p < EARLY; ++p) load_row(buf[p], p);
            auto rest = [&]() {
#pragma unroll
                for (int p = EARLY; p < DD; ++p) load_row(buf[p], p);
            };
            if (s0 == 0) {
                hook();
                read_res();
            }
            if constexpr (T == Q6_K) {
                load_x_q6(X, x, u);
            } else if constexpr (L == GGUF) {
                stage_x(xl, x, s0, ns, tid, nthr, rest);
                __syncthreads();
                load_x<T>(X, xl, u - s0);
            } else {
                stage_x(xl, x, s0, ns, tid, nthr);
                rest();
                __syncthreads();
                load_x<T>(X, xl, u - s0);
            }
            for (int i0 = 0; i0 < rows_lane; i0 += RL) {
                if (i0 > 0)
#pragma unroll
                    for (int p = 0; p < DD; ++p) load_row(buf[p], i0 + p);
                run_round(buf, X, i0);
            }
        } else {
            if constexpr (T == Q6_K) {
                load_x_q6(X, x, u);
            } else {
                if (s0 > 0) __syncthreads();  // every lane holds the previous segment's x in registers
                stage_x(xl, x, s0, ns, tid, nthr);
                __syncthreads();
                load_x<T>(X, xl, u - s0);
            }
            for (int i0 = 0; i0 < rows_lane; i0 += RL) {
                Unit<T> buf[DD];
#pragma unroll
                for (int p = 0; p < DD; ++p) load_row(buf[p], i0 + p);
                run_round(buf, X, i0);
            }
        }
    }
    __syncthreads();
    // y[row] = sum of its partials in a fixed order: 16 lanes per row, each
    // adding float4 groups c, c+16, ... (useg is a multiple of 4), then a
    // butterfly over the 16 lanes.  Every lane runs the same number of rounds
    // so the shuffles see whole groups.
    const int c4 = min(useg, U) >> 2;
    const int j = tid & 15;
    // v / P = umulhi(2v, ceil(2^31 / P)) for v < 2^20 (the partial sums in
    // LDS bound the rows far lower) and P <= 1024: the multiplier exceeds
    // 2^31 / P by less than 1, so the product exceeds 2^32 v / P by less than
    // 2^21, short of the next multiple of 2^32 (at least 2^32 / P >= 2^22
    // away).  ceil(2^32 / P) itself would not fit 32 bits for P = 1.
    const uint32_t inv_p2 = (0x80000000u + (uint32_t)P - 1u) / (uint32_t)P;
    constexpr float oscale = T == Q6_K || T == IQ4_XS ? 1.f : 0x1p48f;
    // the sum of schedule row v (valid or not, every lane of the 16 takes part)
    // as two steps: `issue` reads the lane's float4 groups c = j, j + 16, ...
    // (at most NRD of them; groups past c4 read as zero, which leaves every
    // sum unchanged: it starts at +0), `fold` adds them in that order and sums
    // over the 16-lane row with DPP (no LDS round trips): pairs, quads, the
    // two quads of each half-row, the two half-rows
    constexpr int NRD = T == Q6_K ? 5 : 2;
    auto issue = [&](int v, bool ok, float4 (&w)[NRD]) {
        const int vi = (int)__umulhi(2u * (uint32_t)v, inv_p2);
        const int sr = ok ? vi * PT + (v - vi * P) : 0;
        const float4 *pr = reinterpret_cast<const float4 *>(part + (size_t)sr * useg);
#pragma unroll
        for (int k = 0; k < NRD; ++k) w[k] = j + 16 * k < c4 ? pr[j + 16 * k] : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto fold = [&](float a, const float4 (&w)[NRD], int n) {
#pragma unroll
        for (int k = 0; k < NRD; ++k)
            if (k < n) a += (w[k].x + w[k].y) + (w[k].z + w[k].w);
        a += dpp_f32<0xb1>(a);   // quad_perm [1,0,3,2]
        a += dpp_f32<0x4e>(a);   // quad_perm [2,3,0,1]
        a += dpp_f32<0x141>(a);  // row_half_mirror
        a += dpp_f32<0x140>(a);  // row_mirror
        return a * oscale;
    };
    // the general form: any number of groups per lane, read and added in turn
    auto row_sum = [&](int v, bool ok) {
        const int vi = (int)__umulhi(2u * (uint32_t)v, inv_p2);
        const int sr = ok ? vi * PT + (v - vi * P) : 0;
        const float4 *pr = reinterpret_cast<const float4 *>(part + (size_t)sr * useg);
        float a = 0.f;
#pragma unroll 4
        for (int c = j; c < c4; c += 16) {
            const float4 w = pr[c];
            a += (w.x + w.y) + (w.z + w.w);
        }
        const float4 none[NRD] = {};
        return fold(a, none, 0);
    };
    // the store of schedule row rr (pass: the lane's round of rows so far)
    auto store = [&](int rr, int pass, float v) {
        const bool rok = rr < R;
        float rv = 0.f;
        if constexpr (EPI)  // (all 16 lanes take part in the cross-lane read)
            if (pass < 16) rv = __shfl(resp, (tid & 63 & ~15) + pass);
        if (rok && j == 0) {
            if constexpr (EPI) {
                if (ep.res) v += pass < 16 ? rv : ep.res[r0 + rr];
                store_y(y, ep.f16, (size_t)(r0 + rr), v);
            } else {
                reinterpret_cast<float *>(y)[r0 + rr] = v;
            }
        }
    };
    const int rpp = nthr >> 4;  // rows per round of the 16-lane groups
    // at most two rounds: every LDS read of a lane's rows is issued before
    // the first sum, one wait instead of one per group and round
    auto rounds = [&](auto np) {
        constexpr int NP = decltype(np)::value, NS = PAIR ? 2 : 1;
        float4 w[NP][NS][NRD];
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int g = (tid >> 4) + pass * rpp;
            issue(g, g < R, w[pass][0]);
            if constexpr (PAIR) issue(R + g, g < R, w[pass][NS - 1]);
        }
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            float v = fold(0.f, w[pass][0], NRD);
            if constexpr (PAIR) v = silu(v) * fold(0.f, w[pass][NS - 1], NRD);
            store((tid >> 4) + pass * rpp, pass, v);
        }
    };
    if (c4 <= 16 * NRD && R <= rpp) {
        rounds(std::integral_constant<int, 1>());
    } else if (c4 <= 16 * NRD && R <= 2 * rpp) {
        rounds(std::integral_constant<int, 2>());
    } else {
        int pass = 0;
        for (int rr = tid >> 4; rr - (tid >> 4) < R; rr += rpp, ++pass) {
            const bool rok = rr < R;
            float v = row_sum(rr, rok);
            if constexpr (PAIR) v = silu(v) * row_sum(R + rr, rok);
            store(rr, pass, v);
        }
    }
}

// Thread bound of a one-column kernel: 1024 (128 VGPRs), except where a
// round needs more registers: Q5_K rounds of 3 or 4 rows take at most 512
// threads (256 VGPRs), Q6_K rounds with a ring of units at most 768.  (More
// registers than a round needs are not free: given 256 VGPRs the scheduler
// hoists the x reads of Q4_K one-row rounds, measured 10% slower at
// 1024 x 5120.)
template <int T, int RL, int D>
constexpr int gemv1_bound() {
    return T == Q5_K && RL > 2 ? 512 : T == Q6_K && D > 1 ? 768 : 1024;
}

template <int T, int L, int RL, int D, bool NT, bool PAIR, bool EPI>
__global__ void __launch_bounds__((gemv1_bound<T, RL, D>())) gemv1_kernel(const uint8_t *__restrict__ W,
                                                      const uint16_t *__restrict__ x, void *y, int N, int K,
                                                      int useg, int P, int fc, int fcap, const Epilogue ep) {
    gemv1_body<T, L, RL, D, NT, PAIR, EPI>(W, x, y, N, K, useg, P, (int)blockIdx.x, (int)gridDim.x,
                                           (int)blockDim.x, ep, NoHook(), fc, fcap);
}

// ---------------------------------------------------------------------------
// Batched one-column GEMVs: independent (W, x, y) entries in one launch.
// Entry i owns workgroups [first[i], first[i+1]) and runs the one-column
// body with the geometry its own launch would take -- except that a run of
// adjacent entries of one type and K reading the same x (q, k and v of a
// layer) takes the geometry of a single launch of all their rows, each entry
// with its share of the workgroups: small tensors then get a few workgroups
// of the same size as the large one's instead of hundreds of tiny ones that
// hold the CUs' slots (measured: q+k+v of an attention layer 14.8 -> 12 us,
// PLANAR rows 15.8 -> 10.7 us).  A row's arithmetic depends only on K (the
// segment length), so every y is bit-identical to that of a single call.
// Entries travel in the kernel arguments (no device memory).  A workgroup
// with more threads than its entry needs retires the surplus waves at once
// (a retired wave does not hold up the barrier).
// ---------------------------------------------------------------------------
enum BodyCode {
    B_Q4_1, B_Q4_2, B_Q4_4, B_Q4_6, B_Q4_8, B_Q4_12, B_Q5_1, B_Q5_2, B_Q6_1, B_Q6_2,
    B_IQ4_1, B_IQ4_2, B_IQ4_4, B_IQ4_6, B_IQ4_8, B_IQ4_12, B_COUNT
};
// code + B_COUNT: the same body on the PLANAR layout

struct BatchItem {
    const uint8_t *W;
    const uint16_t *x;
    float *y;
    int N, K, useg, P, threads, code;
    int fc, fcap;  // RowSplit's front loading over the entry's workgroups (fc = 0: even)
};
struct BatchArgs {
    int count;
    int first[MAX_BATCH + 1];
    BatchItem it[MAX_BATCH];
};

__global__ void __launch_bounds__(1024) gemv1_batch_kernel(const BatchArgs a) {
    int i = 0;
    while (i + 1 < a.count && (int)blockIdx.x >= a.first[i + 1]) ++i;
    const BatchItem &e = a.it[i];
    if ((int)threadIdx.x >= e.threads) return;
    const int blk = (int)blockIdx.x - a.first[i], nblk = a.first[i + 1] - a.first[i];
    const Epilogue plain{nullptr, nullptr, 0};
#define QK_BODY(T, RL, D) \
    gemv1_body<T, GGUF, RL, D, false, false, false>(e.W, e.x, e.y, e.N, e.K, e.useg, e.P, blk, nblk, e.threads, \
                                                    plain, NoHook(), e.fc, e.fcap)
#define QK_BODYP(T, RL, D) \
    gemv1_body<T, PLANAR, RL, D, true, false, false>(e.W, e.x, e.y, e.N, e.K, e.useg, e.P, blk, nblk, e.threads, \
                                                      plain, NoHook(), e.fc, e.fcap)
    switch (e.code) {
    case B_Q4_1: QK_BODY(Q4_K, 1, 1); break;
    case B_Q4_2: QK_BODY(Q4_K, 2, 2); break;
    case B_Q4_4: QK_BODY(Q4_K, 4, 2); break;
    case B_Q4_6: QK_BODY(Q4_K, 6, 2); break;
    case B_Q4_8: QK_BODY(Q4_K, 8, 2); break;
    case B_Q4_12: QK_BODY(Q4_K, 12, 2); break;
    case B_Q5_1: QK_BODY(Q5_K, 1, 1); break;
    case B_Q5_2: QK_BODY(Q5_K, 2, 2); break;
    case B_Q6_1: QK_BODY(Q6_K, 1, 1); break;
    case B_Q6_2: QK_BODY(Q6_K, 2, 2); break;
    case B_IQ4_1: QK_BODY(IQ4_XS, 1, 1); break;
    case B_IQ4_2: QK_BODY(IQ4_XS, 2, 2); break;
    case B_IQ4_4: QK_BODY(IQ4_XS, 4, 2); break;
    case B_IQ4_6: QK_BODY(IQ4_XS, 6, 2); break;
    case B_IQ4_8: QK_BODY(IQ4_XS, 8, 2); break;
    case B_IQ4_12: QK_BODY(IQ4_XS, 12, 2); break;
    case B_COUNT + B_Q4_1: QK_BODYP(Q4_K, 1, 1); break;
    case B_COUNT + B_Q4_2: QK_BODYP(Q4_K, 2, 2); break;
    case B_COUNT + B_Q4_4: QK_BODYP(Q4_K, 4, 2); break;
    case B_COUNT + B_Q4_6: QK_BODYP(Q4_K, 6, 2); break;
    case B_COUNT + B_Q4_8: QK_BODYP(Q4_K, 8, 2); break;
    case B_COUNT + B_Q4_12: QK_BODYP(Q4_K, 12, 2); break;
    case B_COUNT + B_Q5_1: QK_BODYP(Q5_K, 1, 1); break;
    case B_COUNT + B_Q5_2: QK_BODYP(Q5_K, 2, 2); break;
    case B_COUNT + B_Q6_1: QK_BODYP(Q6_K, 1, 1); break;
    case B_COUNT + B_Q6_2: QK_BODYP(Q6_K, 2, 2); break;
    default: break;
    }
#undef QK_BODYP
#undef QK_BODY
}

// ---------------------------------------------------------------------------
// Dequantisation, one 64-weight unit per thread, through the same unit loads
// and pattern decoders as the GEMV.  Q4_K/Q5_K: w = (d*sc)*q - dmin*m (both
// products exact in fp32, one rounding); Q6_K: w = d * (sc*(q-32)) (exact);
// IQ4_XS: w = d*(ls-32)*kv (exact).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pat_lo(uint32_t p, int shift) { return (p & 0xffffu) >> shift; }
__device__ __forceinline__ uint32_t pat_hi(uint32_t p, int shift) { return (p >> 16) >> shift; }

template <int T, int L>
__global__ void __launch_bounds__(WG) dequant_kernel(const uint8_t *__restrict__ W, float *__restrict__ out,
                                                     int64_t N, int K) {
    const int64_t unit = (int64_t)blockIdx.x * WG + threadIdx.x;
    const int upr = K >> 6;
    if (unit >= N * upr) return;
    const int64_t row = unit / upr;
    const int u = (int)(unit - row * upr);
    const int s = u >> 2, q = u & 3;
    float *o = out + (size_t)row * (size_t)K + 256 * s;
    Unit<T> U;
    U.template load<false, L>(W + (size_t)row * (size_t)layout_row_bytes(T, L, K), UnitAddr<T, L>(K >> 8, u));
    if constexpr (T == IQ4_XS) {
        // d*2^24*(ls - 32) exact (17 significant bits), times kv*2^-24 from
        // the pattern: at most 24 significant bits, exact
        const float d = U.d24();
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const float f = d * (float)U.scale(q, hi);
            float *ob = o + 64 * q + 32 * hi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t p[4];
                U.patterns(4 * hi + i, q, p);
                *reinterpret_cast<float4 *>(ob + 4 * i) =
                    make_float4(f * f16_lo(p[0]), f * f16_lo(p[1]), f * f16_hi(p[0]), f * f16_hi(p[1]));
                *reinterpret_cast<float4 *>(ob + 16 + 4 * i) =
                    make_float4(f * f16_lo(p[2]), f * f16_lo(p[3]), f * f16_hi(p[2]), f * f16_hi(p[3]));
            }
        }
    } else if constexpr (T == Q6_K) {
        const float d = f16_lo(U.d);
        const int kb = 128 * (q >> 1) + 16 * (q & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t p[8];
            U.patterns(i, q, p);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int sh = t < 2 ? 0 : 4;
                const int sc = U.template scale<L>(t, q);
                const uint32_t pa = p[2 * t], pb = p[2 * t + 1];
                float4 w;
                w.x = d * (float)(sc * ((int)pat_lo(pa, sh) - 32));
                w.y = d * (float)(sc * ((int)pat_lo(pb, sh) - 32));
                w.z = d * (float)(sc * ((int)pat_hi(pa, sh) - 32));
                w.w = d * (float)(sc * ((int)pat_hi(pb, sh) - 32));
                *reinterpret_cast<float4 *>(o + kb + 32 * t + 4 * i) = w;
            }
        }
    } else {
        const uint4 h = U.header();
        const KScales s4 = k_scales(h, KScaleSel(q));
        const float d = f16_lo(h.x), dmin = f16_hi(h.x);
        const float dl = d * (float)s4.sc_lo, dh = d * (float)s4.sc_hi;
        const float ml = dmin * (float)s4.m_lo, mh = dmin * (float)s4.m_hi;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t p[4];
            U.patterns(i, q, p);
            float4 lo, hi;
            lo.x = dl * (float)pat_lo(p[0], 0) - ml;
            lo.y = dl * (float)pat_lo(p[1], 0) - ml;
            lo.z = dl * (float)pat_hi(p[0], 0) - ml;
            lo.w = dl * (float)pat_hi(p[1], 0) - ml;
            hi.x = dh * (float)pat_lo(p[2], 4) - mh;
            hi.y = dh * (float)pat_lo(p[3], 4) - mh;
            hi.z = dh * (float)pat_hi(p[2], 4) - mh;
            hi.w = dh * (float)pat_hi(p[3], 4) - mh;
            *reinterpret_cast<float4 *>(o + 64 * q + 4 * i) = lo;
            *reinterpret_cast<float4 *>(o + 64 * q + 32 + 4 * i) = hi;
        }
    }
}

// ---------------------------------------------------------------------------
// GGUF -> PLANAR repack, one superblock per thread: the same bytes moved to
// the planes (qk_format.h); the Q6_K row padding is written as zeros.
// ---------------------------------------------------------------------------
template <int T>
__global__ void __launch_bounds__(WG) repack_kernel(const uint8_t *__restrict__ W, uint8_t *__restrict__ Wp,
                                                    int64_t N, int K) {
    constexpr int BB = Fmt<T>::bytes;
    const int S = K >> 8;
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i >= N * S) return;
    const int64_t row = i / S;
    const int s = (int)(i - row * S);
    const uint8_t *sb = W + ((size_t)row * S + s) * BB;
    const size_t prow = (size_t)layout_row_bytes(T, PLANAR, K);
    uint8_t *rp = Wp + (size_t)row * prow;
    auto cp16 = [](uint8_t *dst, const uint8_t *src) {
        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    };
    if constexpr (T == Q6_K) {
        // scales[16] at 192 and d at 208; superblocks are only 2-byte aligned
        uint8_t sc[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) sc[k] = sb[192 + k];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const UnitAddr<Q6_K, GGUF> g(0, q);
            const UnitAddr<Q6_K, PLANAR> o(S, 4 * s + q);
            cp16(rp + o.a, sb + g.a);
            cp16(rp + o.b, sb + g.b);
            cp16(rp + o.c, sb + g.c);
            const int n = q >> 1, b = q & 1;
            uint32_t v = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) v |= (uint32_t)sc[8 * n + 2 * t + b] << (8 * t);
            *reinterpret_cast<uint32_t *>(rp + o.sc) = v;
        }
        *reinterpret_cast<uint16_t *>(rp + UnitAddr<Q6_K, PLANAR>(S, 4 * s).d) =
            *reinterpret_cast<const uint16_t *>(sb + 208);
        if (s == S - 1)
            for (size_t k = (size_t)210 * S; k < prow; ++k) rp[k] = 0;
    } else {
        const UnitAddr<T, PLANAR> o0(S, 4 * s);
        cp16(rp + o0.h, sb);
        if constexpr (T == Q5_K) {
            cp16(rp + o0.qh0, sb + 16);
            cp16(rp + o0.qh1, sb + 32);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const UnitAddr<T, GGUF> g(0, q);
            const UnitAddr<T, PLANAR> o(S, 4 * s + q);
            cp16(rp + o.a, sb + g.a);
            cp16(rp + o.b, sb + g.b);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers.  The type argument carries the PLANAR_FLAG bit of the C ABI.
// ---------------------------------------------------------------------------
constexpr int LDS_PART = 128 * 1024;  // LDS budget of one workgroup: partial sums and the x copy
constexpr int LDS_MAX = 160 * 1024;   // gfx950: the most one workgroup may take

// Launch geometry of the ncols = 1 kernel.
struct Geo { int G, threads, useg, P, RL, fc = 0, fcap = 0; };  // fc, fcap: RowSplit's front loading

static int cu_count() { return device_cus(); }

// Rows per straight-line round that each type is compiled for.  Q6_K units
// are the largest (58 B of loads per lane): on GGUF rows one unit in flight
// per lane streams them fastest (two-row rounds with a ring measured 10-30%
// slower); PLANAR rows take the same phases in two-row rounds with two units
// in flight when the launch has at most ring_threads threads (5% faster at
// 5120 x 17408; see geometry).  Q5_K units hold 20 dwords: rounds of 3 or 4 rows
// need the 256 VGPRs that the single-launch kernel's 512-thread bound leaves
// (measured: 5120 x 6144 in one round of 4 beats two rounds of 2 by 5%);
// the merged-launch kernel (1024-thread bound) runs Q5_K in rounds of 2.
// Q4_K rounds go up to 12 rows.
template <int T> struct RowRounds;
template <> struct RowRounds<Q4_K> { static constexpr int n = 6, rl[n] = {1, 2, 4, 6, 8, 12}, max_threads = 512; };
// IQ4_XS: 4-bit quants in units of 10 dwords, rounds as for Q4_K
template <> struct RowRounds<IQ4_XS> { static constexpr int n = 6, rl[n] = {1, 2, 4, 6, 8, 12}, max_threads = 512; };
template <> struct RowRounds<Q5_K> { static constexpr int n = 4, rl[n] = {1, 2, 3, 4}, max_threads = 512; };
template <> struct RowRounds<Q6_K> { static constexpr int n = 1, rl[n] = {1}, max_threads = 1024, ring_threads = 768; };
static_assert(RowRounds<Q6_K>::ring_threads == gemv1_bound<Q6_K, 2, 2>(), "gemv1_kernel's bound for Q6_K rings");
static_assert(RowRounds<Q5_K>::max_threads <= gemv1_bound<Q5_K, 4, 2>(), "gemv1_kernel's bound for Q5_K rounds");

// LDS of one workgroup: ceil(R / P) slot rows per phase, tail phase included
// (mult = 2: the paired rows of the SwiGLU epilogue).
static size_t part_lds(int64_t N, const Geo &g, int mult = 1) {
    const int64_t R = mult * std::max<int64_t>((N + g.G - 1) / g.G, g.fcap), rows_lane = (R + g.P - 1) / g.P;
    const int64_t PT = (g.threads + g.useg - 1) / g.useg;
    return (size_t)(rows_lane * PT * g.useg) * 4 + (size_t)g.useg * XSTRIDE;  // partial sums + x copy (Q4_K/Q5_K)
}

// Rows are split evenly over G workgroups (one per CU unless the partial
// sums would not fit in LDS).  Within a workgroup P row phases of useg lanes
// each take every P-th row, RL rows per straight-line round.  P and RL are
// chosen to waste the fewest row slots (P * rounds * RL - R), then for the
// most lanes.  mult = 2: each workgroup streams its rows of two tensors.
// Q4_K: several small workgroups of four waves (P = 256 / useg row phases)
// per CU hide latency better than one large one, measured on the projection
// shapes at K = 5120: the fewest per CU (two to four) that keep a lane's
// rows within one round of at most 8 (whose ring the kernel issues before
// staging x), when a lane still gets 4..12 rows (fewer do not amortise the
// workgroup's x staging and reduction).
template <int T, int L>
static bool small_workgroups(int64_t N, int cus, int mult, Geo &g) {
    if constexpr (T != Q4_K && T != IQ4_XS) {
        return false;
    } else {
        using RR = RowRounds<T>;
        const int p4 = 256 / g.useg;
        if (p4 < 1) return false;
        // the fewest workgroups per CU (two to four) that leave a lane at most
        // eight rows: one round of RL <= 8
        int64_t G = 0, R = 0, rows = 0;
        for (int k = 2; k <= 4; ++k) {
            G = std::min<int64_t>(N, (int64_t)cus * mult * k);
            R = mult * ((N + G - 1) / G);
            rows = (R + p4 - 1) / p4;
            if (rows <= 8) break;
        }
        if (rows < 4 || rows > RR::rl[RR::n - 1]) return false;
        g.G = (int)G;
        g.P = p4;
        for (int k = 0; k < RR::n; ++k)
            if (RR::rl[k] >= rows) { g.RL = RR::rl[k]; break; }
        g.threads = (p4 * g.useg + 63) / 64 * 64;
        // several rounds of one workgroup per CU in one straight-line round:
        // front-load them (RowSplit)
        const int64_t rounds = G % cus == 0 ? G / cus : 0, fcap = (int64_t)p4 * g.RL / mult;
        if (rounds >= 2 && (G - cus) * fcap <= N && rows <= g.RL) {
            g.fc = cus;
            g.fcap = (int)fcap;
        }
        return part_lds(N, g, mult) <= (size_t)LDS_PART;
    }
}

template <int T, int L = GGUF>
static Geo geometry(int64_t N, int64_t K, int cus, int mult = 1) {
    using RR = RowRounds<T>;
    Geo g;
    const int64_t U = K / 64;
    g.useg = (int)(U < 512 ? U : 512);
    const int pmax = RR::max_threads / g.useg > 0 ? RR::max_threads / g.useg : 1;
    if (small_workgroups<T, L>(N, cus, mult, g)) return g;
    // one workgroup per CU and tensor streamed (mult = 2: both halves of the
    // pair have their own CU's worth of rows, as two launches would)
    for (int64_t G = std::min<int64_t>(N, (int64_t)cus * mult);; G *= 2) {
        if (G > N) G = N;
        g.G = (int)G;
        const int64_t R = mult * ((N + G - 1) / G);
        auto plan = [&](int p, int &rl) {  // row slots of p phases, and the round length
            const int64_t rows = (R + p - 1) / p;
            rl = RR::rl[RR::n - 1];
            for (int k = 0; k < RR::n; ++k)
                if (RR::rl[k] >= rows) { rl = RR::rl[k]; break; }
            return (int64_t)p * ((rows + rl - 1) / rl) * rl;
        };
        // with at least pmax rows, at least half the phases (the fewest
        // slots alone could pick one phase of a handful of lanes per CU)
        const int plo = R >= pmax ? (pmax + 1) / 2 : 1;
        int64_t best = INT64_MAX;
        for (int p = plo; p <= pmax; ++p) {
            int rl;
            best = std::min(best, plan(p, rl));
        }
        // the most phases among the fewest slots
        g.P = plo;
        g.RL = 1;
        for (int p = plo; p <= pmax; ++p) {
            int rl;
            if (plan(p, rl) <= best) { g.P = p; g.RL = rl; }
        }
        g.threads = (g.P * g.useg + 63) / 64 * 64;
        // Q6_K on PLANAR rows: the same phases in two-row rounds, two units
        // in flight per lane (the kernel's bound for a ring is ring_threads;
        // an odd row count re-reads the last row once)
        if constexpr (T == Q6_K && L == PLANAR)
            if (g.threads <= RR::ring_threads && (R + g.P - 1) / g.P >= 2) g.RL = 2;
        if (G == N || part_lds(N, g, mult) <= (size_t)LDS_PART) break;  // the partial sums fit in LDS
    }
    return g;
}


// Dynamic LDS above the default 64 KB needs the kernel's opt-in (a failed
// opt-in shows as the launch's error).
template <auto Kernel>
static void allow_lds() {
    (void)lds_opt_in<Kernel>(LDS_MAX);
}

template <int T, int L, int RL, int D, bool NT, bool PAIR>
static hipError_t launch1(const void *W, const void *x, void *y, int64_t N, int64_t K, Geo geo,
                          const Epilogue &ep, hipStream_t st) {
    const size_t lds = part_lds(N, geo, PAIR ? 2 : 1);
    // plain launches run a body without the epilogue's store options
    if (!PAIR && !ep.res && !ep.f16) {
        allow_lds<gemv1_kernel<T, L, RL, D, NT, false, false>>();
        hipLaunchKernelGGL((gemv1_kernel<T, L, RL, D, NT, false, false>), dim3(geo.G), dim3(geo.threads), lds, st,
                           (const uint8_t *)W, (const uint16_t *)x, y, (int)N, (int)K, geo.useg, geo.P, geo.fc,
                           geo.fcap, ep);
    } else {
        allow_lds<gemv1_kernel<T, L, RL, D, NT, PAIR, true>>();
        hipLaunchKernelGGL((gemv1_kernel<T, L, RL, D, NT, PAIR, true>), dim3(geo.G), dim3(geo.threads), lds, st,
                           (const uint8_t *)W, (const uint16_t *)x, y, (int)N, (int)K, geo.useg, geo.P, geo.fc,
                           geo.fcap, ep);
    }
    return hipGetLastError();
}

// Units in flight per lane (the ring of a straight-line round): one for
// one-row rounds, otherwise two (three spill under the 128-register bound and
// measured 20-40% slower).
constexpr int RING = 2;
template <int T, int L, bool PAIR>
static hipError_t gemv1_dispatch(const void *W, const void *x, void *y, int64_t N, int64_t K,
                                 const Epilogue &ep, hipStream_t st) {
    const Geo geo = geometry<T, L>(N, K, cu_count(), PAIR ? 2 : 1);
    // PLANAR rows stream with non-temporal loads (measured faster there; no
    // change on GGUF rows)
    constexpr bool NT = L == PLANAR;
    switch (geo.RL) {
    case 1: return launch1<T, L, 1, 1, NT, PAIR>(W, x, y, N, K, geo, ep, st);
    case 2: if constexpr (T != Q6_K || L == PLANAR) return launch1<T, L, 2, RING, NT, PAIR>(W, x, y, N, K, geo, ep, st); break;
    case 3: if constexpr (T == Q5_K) return launch1<T, L, 3, RING, NT, PAIR>(W, x, y, N, K, geo, ep, st); break;
    case 4: if constexpr (T != Q6_K) return launch1<T, L, 4, RING, NT, PAIR>(W, x, y, N, K, geo, ep, st); break;
    case 6: if constexpr (T == Q4_K || T == IQ4_XS) return launch1<T, L, 6, RING, NT, PAIR>(W, x, y, N, K, geo, ep, st); break;
    case 8: if constexpr (T == Q4_K || T == IQ4_XS) return launch1<T, L, 8, RING, NT, PAIR>(W, x, y, N, K, geo, ep, st); break;
    case 12: if constexpr (T == Q4_K || T == IQ4_XS) return launch1<T, L, 12, RING, NT, PAIR>(W, x, y, N, K, geo, ep, st); break;
    default: break;
    }
    return hipErrorInvalidValue;
}

template <int T, int L>
static hipError_t gemv1_pair(const void *W, const void *x, void *y, int64_t N, int64_t K, const Epilogue &ep,
                             hipStream_t st) {
    return ep.W2 ? gemv1_dispatch<T, L, true>(W, x, y, N, K, ep, st)
                 : gemv1_dispatch<T, L, false>(W, x, y, N, K, ep, st);
}

hipError_t launch_gemv1(int type, const void *W, const void *x, void *y, int64_t N, int64_t K,
                        const Epilogue &ep, hipStream_t st) {
    switch (type) {
    case Q4_K: return gemv1_pair<Q4_K, GGUF>(W, x, y, N, K, ep, st);
    case Q5_K: return gemv1_pair<Q5_K, GGUF>(W, x, y, N, K, ep, st);
    case Q6_K: return gemv1_pair<Q6_K, GGUF>(W, x, y, N, K, ep, st);
    case IQ4_XS: return gemv1_pair<IQ4_XS, GGUF>(W, x, y, N, K, ep, st);
    case Q4_K | PLANAR_FLAG: return gemv1_pair<Q4_K, PLANAR>(W, x, y, N, K, ep, st);
    case Q5_K | PLANAR_FLAG: return gemv1_pair<Q5_K, PLANAR>(W, x, y, N, K, ep, st);
    case Q6_K | PLANAR_FLAG: return gemv1_pair<Q6_K, PLANAR>(W, x, y, N, K, ep, st);
    default: return hipErrorInvalidValue;
    }
}

static Geo geometry_front(int type, int64_t N, int64_t K, int cus) {
    const bool planar = (type & PLANAR_FLAG) != 0;
    switch (type & ~PLANAR_FLAG) {
    case Q4_K: return planar ? geometry<Q4_K, PLANAR>(N, K, cus) : geometry<Q4_K, GGUF>(N, K, cus);
    case Q5_K: return geometry<Q5_K>(N, K, cus);
    case IQ4_XS: return geometry<IQ4_XS>(N, K, cus);
    default: return planar ? geometry<Q6_K, PLANAR>(N, K, cus) : geometry<Q6_K, GGUF>(N, K, cus);
    }
}

// (the merged launch splits an entry's rows evenly unless it front-loads a
// run itself)
static Geo geometry_of(int type, int64_t N, int64_t K, int cus) {
    const bool planar = (type & PLANAR_FLAG) != 0;
    Geo g;
    switch (type & ~PLANAR_FLAG) {
    case Q4_K: g = planar ? geometry<Q4_K, PLANAR>(N, K, cus) : geometry<Q4_K, GGUF>(N, K, cus); break;
    case Q5_K: g = geometry<Q5_K>(N, K, cus); break;
    case IQ4_XS: g = geometry<IQ4_XS>(N, K, cus); break;
    default: g = planar ? geometry<Q6_K, PLANAR>(N, K, cus) : geometry<Q6_K, GGUF>(N, K, cus); break;
    }
    g.fc = g.fcap = 0;
    return g;
}

static int body_code_gguf(int type, int rl);

static int body_code(int type_flags, int rl) {
    const int type = type_flags & ~PLANAR_FLAG, plane = (type_flags & PLANAR_FLAG) ? B_COUNT : 0;
    if (plane && type == IQ4_XS) return -1;  // GGUF rows only
    const int c = body_code_gguf(type, rl);
    return c < 0 ? -1 : c + plane;
}

static int body_code_gguf(int type, int rl) {
    if (type == Q4_K) {
        switch (rl) {
        case 1: return B_Q4_1;
        case 2: return B_Q4_2;
        case 4: return B_Q4_4;
        case 6: return B_Q4_6;
        case 8: return B_Q4_8;
        case 12: return B_Q4_12;
        default: return -1;
        }
    }
    // (rounds of 3 or 4 Q5_K rows need more registers than the merged kernel
    // has: two-row rounds instead, the same arithmetic in a different order
    // of loads)
    if (type == Q5_K) return rl == 1 ? B_Q5_1 : (rl >= 2 && rl <= 4) ? B_Q5_2 : -1;
    if (type == Q6_K) return rl == 1 ? B_Q6_1 : rl == 2 ? B_Q6_2 : -1;
    if (type == IQ4_XS) {
        switch (rl) {
        case 1: return B_IQ4_1;
        case 2: return B_IQ4_2;
        case 4: return B_IQ4_4;
        case 6: return B_IQ4_6;
        case 8: return B_IQ4_8;
        case 12: return B_IQ4_12;
        default: return -1;
        }
    }
    return -1;
}

hipError_t launch_gemv_batch(const BatchEntry *in, int count, hipStream_t st) {
    if (count < 1 || count > MAX_BATCH) return hipErrorInvalidValue;
    BatchArgs a{};
    a.count = count;
    a.first[0] = 0;
    size_t lds = 4;
    int threads = 64;
    int64_t total = 0;
    const int cus = cu_count();
    // entries [i0, i1) with geometry g (joint: each entry's share of g.G
    // workgroups; else each entry's own launch geometry); false if a share
    // would need more LDS than a workgroup's budget
    auto place = [&](int i0, int i1, bool joint, const Geo &g, int64_t rows) {
        int64_t done = 0, given = 0;  // rows and workgroups of the run's earlier entries
        int64_t t = total;
        size_t l = lds;
        int th = threads;
        // Front loading (RowSplit) for a run that starts at a dispatch round
        // and takes several rounds of small workgroups: the first entry's
        // rows fill every round but the last at fcap rows per workgroup, and
        // its remaining rows and the later entries share the last round.
        const Geo gf = geometry_front(in[i0].type, rows, in[i0].K, cus);
        const int64_t front = gf.fc ? (int64_t)gf.G - cus : 0;
        const bool fl = joint && front > 0 && total % cus == 0 && gf.G == g.G && gf.RL == g.RL &&
                        in[i0].N >= front * gf.fcap;
        const int64_t last_rows = rows - front * gf.fcap;  // rows of the run's last round
        for (int i = i0; i < i1; ++i) {
            const BatchEntry &e = in[i];
            Geo gi = joint ? g : geometry_of(e.type, e.N, e.K, cus);
            if (fl) {
                // entry i's last-round workgroups in proportion to its last-round rows
                const int64_t lr = i == i0 ? e.N - front * gf.fcap : e.N;
                done += lr;
                const int64_t upto = last_rows > 0 ? (int64_t)cus * done / last_rows : 0;
                int64_t nl = std::min<int64_t>(upto - given, lr);
                if (lr > 0) nl = std::max<int64_t>(nl, 1);
                given += nl;
                if (nl * gf.fcap < lr) return false;  // (cannot happen: the last round fits)
                gi.G = (int)((i == i0 ? front : 0) + nl);
                gi.fc = (int)nl;
                gi.fcap = gf.fcap;
                if (gi.G < 1 || part_lds(e.N, gi) > (size_t)LDS_PART) return false;
            } else if (joint) {
                // workgroups in proportion to the rows (cumulative rounding:
                // the run's total is the joint launch's), at least one each
                done += e.N;
                const int64_t upto = (int64_t)g.G * done / rows;
                gi.G = (int)std::max<int64_t>(1, std::min<int64_t>(upto - given, e.N));
                given += gi.G;
                if (part_lds(e.N, gi) > (size_t)LDS_PART) return false;
            }
            const int code = body_code(e.type, gi.RL);
            if (code < 0) return false;
            a.it[i] = BatchItem{(const uint8_t *)e.W, (const uint16_t *)e.x, (float *)e.y, (int)e.N, (int)e.K,
                                gi.useg, gi.P, gi.threads, code, gi.fc, gi.fcap};
            t += gi.G;
            if (t > INT32_MAX) return false;
            a.first[i + 1] = (int)t;
            l = std::max(l, part_lds(e.N, gi));
            th = std::max(th, gi.threads);
        }
        total = t;
        lds = l;
        threads = th;
        return true;
    };
    for (int i0 = 0; i0 < count;) {
        // the run [i0, i1) of adjacent entries that share type, K and x
        int i1 = i0 + 1;
        int64_t rows = in[i0].N;
        while (i1 < count && in[i1].type == in[i0].type && in[i1].K == in[i0].K && in[i1].x == in[i0].x) {
            rows += in[i1].N;
            ++i1;
        }
        const Geo g = geometry_of(in[i0].type, rows, in[i0].K, cus);
        // (a single entry placed jointly takes the run's geometry: its own)
        if (!place(i0, i1, true, g, rows) && !place(i0, i1, false, g, rows))
            return hipErrorInvalidValue;
        i0 = i1;
    }
    allow_lds<gemv1_batch_kernel>();
    hipLaunchKernelGGL(gemv1_batch_kernel, dim3((unsigned)total), dim3(threads), lds, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Chain: steps of one-column GEMVs in one persistent launch.  Step s+1 may
// read what step s wrote (its x or residual may be an earlier y), so every
// workgroup arrives at a barrier after its stores of step s and waits for
// all arrivals before it reads x of step s+1 -- but it issues the first
// round of step s+1's weight loads before waiting (weights never depend on
// earlier steps), so the previous step's tail and this step's first memory
// latency overlap instead of adding up launch after launch.
//
// One workgroup per CU (a cooperative launch: the runtime checks that the
// whole grid is resident, so the barriers cannot wait on an unscheduled
// workgroup).  Each step's entries share the grid in proportion to their
// weight bytes and run the one-column body with the geometry that share
// gives; a row's arithmetic depends only on K, so every y is bit-identical to
// what qk_gemv / qk_gemv_ex / qk_gemv_swiglu write.
//
// Synchronisation words (caller memory, or the library's own array): [0]
// error flags, [1] unused, [2 + k] arrivals at the barrier after step k.  A
// small kernel zeroes them before each launch.  Waits are bounded by a
// wall-clock limit: a workgroup that times out sets CHAIN_TIMEOUT and every
// workgroup stops at its next wait (the outputs are then incomplete, and the
// flag tells the caller so).
// ---------------------------------------------------------------------------
constexpr uint32_t CHAIN_MAGIC = 0x31484351u;  // "QCH1"
constexpr uint32_t CHAIN_TIMEOUT = 1u;

struct ChainHdr {
    uint32_t magic, nsteps, nentries, G;
    int32_t threads, cus;
    uint32_t lds, entries_off;
};
struct ChainStepD { int32_t e0, e1; };
struct ChainEntryD {
    const uint8_t *W;
    const void *W2;
    const uint16_t *x;
    void *y;
    const float *res;
    int32_t N, K, useg, P, threads, code, first, last, f16, pad;
};
constexpr int CHAIN_PAIR = 32;  // code + CHAIN_PAIR: the SwiGLU pair body
static_assert(2 * B_COUNT <= CHAIN_PAIR, "chain body codes");
// dynamic LDS of the chain kernel: the most a workgroup may take, less the
// kernel's static word
constexpr int CHAIN_LDS_MAX = LDS_MAX - 64;

__global__ void __launch_bounds__(256) chain_reset_kernel(uint32_t *sync, int words) {
    for (int i = (int)threadIdx.x; i < words; i += (int)blockDim.x) sync[i] = 0u;
}

// Every wave's stores of the step are complete before the workgroup
// barrier; one thread then makes them visible device-wide (one L2 write-back
// per workgroup, not one per wave) and counts the arrival.
__device__ __forceinline__ void chain_arrive(uint32_t *sync, int k) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(&sync[2 + k], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Wait until all G workgroups arrived after step k (every thread calls it
// once).  Returns false when the chain is abandoned (this workgroup timed
// out, or another one did).
__device__ __forceinline__ bool chain_wait(uint32_t *sync, int k, uint32_t G, uint64_t limit, uint32_t *s_ok) {
    if (threadIdx.x == 0) {
        uint32_t ok = 1;
        const uint64_t t0 = wall_clock64();
        while (__hip_atomic_load(&sync[2 + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < G) {
            if (__hip_atomic_load(&sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                ok = 0;
                break;
            }
            if (wall_clock64() - t0 > limit) {
                __hip_atomic_fetch_or(&sync[0], CHAIN_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
        // the earlier steps' stores, before any read of the workgroup (one
        // invalidation of this CU's caches serves every wave)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_ok = ok;
    }
    __syncthreads();
    return *s_ok != 0u;
}

// A pointer read from memory is generic to the compiler (flat loads, which
// also count against the LDS counter); these all point to device memory.
template <class P>
__device__ __forceinline__ P *global_ptr(P *p) {
    return (P *)(__attribute__((address_space(1))) P *)(uintptr_t)p;
}

// The wait of a chain step (every thread of the workgroup calls it once);
// its verdict goes to the workgroup's shared word.
struct ChainHook {
    uint32_t *sync, *s_ok;
    uint64_t limit;
    int k;  // the barrier after step k, or -1: nothing to wait for
    uint32_t G;
    __device__ void operator()() const {
        if (k >= 0) (void)chain_wait(sync, k, G, limit, s_ok);
    }
};

// One body of the chain (inlined: compiled as functions of their own, the
// bodies get the 64-register budget of a device function and spill).
template <int T, int L, int RL, int D, bool PAIR>
__device__ __forceinline__ void chain_run(const ChainEntryD &e, int blk, int nblk, ChainHook hook) {
    const Epilogue ep{global_ptr(e.W2), global_ptr(e.res), e.f16};
    gemv1_body<T, L, RL, D, L == PLANAR, PAIR, true, ChainHook>(global_ptr(e.W), global_ptr(e.x), global_ptr(e.y),
                                                                 e.N, e.K, e.useg, e.P, blk, nblk, e.threads, ep,
                                                                 hook);
}

__device__ __forceinline__ void chain_body(const ChainEntryD &e, int blk, int nblk, const ChainHook &hook) {
#define QK_CB(CODE, T, L, RL, D, PAIR) \
    case CODE: chain_run<T, L, RL, D, PAIR>(e, blk, nblk, hook); break;
    switch (e.code) {
        QK_CB(B_Q4_1, Q4_K, GGUF, 1, 1, false)
        QK_CB(B_Q4_2, Q4_K, GGUF, 2, 2, false)
        QK_CB(B_Q4_4, Q4_K, GGUF, 4, 2, false)
        QK_CB(B_Q4_6, Q4_K, GGUF, 6, 2, false)
        QK_CB(B_Q4_8, Q4_K, GGUF, 8, 2, false)
        QK_CB(B_Q4_12, Q4_K, GGUF, 12, 2, false)
        QK_CB(B_Q5_1, Q5_K, GGUF, 1, 1, false)
        QK_CB(B_Q5_2, Q5_K, GGUF, 2, 2, false)
        QK_CB(B_Q6_1, Q6_K, GGUF, 1, 1, false)
        QK_CB(B_COUNT + B_Q4_1, Q4_K, PLANAR, 1, 1, false)
        QK_CB(B_COUNT + B_Q4_2, Q4_K, PLANAR, 2, 2, false)
        QK_CB(B_COUNT + B_Q4_4, Q4_K, PLANAR, 4, 2, false)
        QK_CB(B_COUNT + B_Q4_6, Q4_K, PLANAR, 6, 2, false)
        QK_CB(B_COUNT + B_Q4_8, Q4_K, PLANAR, 8, 2, false)
        QK_CB(B_COUNT + B_Q4_12, Q4_K, PLANAR, 12, 2, false)
        QK_CB(B_COUNT + B_Q5_1, Q5_K, PLANAR, 1, 1, false)
        QK_CB(B_COUNT + B_Q5_2, Q5_K, PLANAR, 2, 2, false)
        QK_CB(B_COUNT + B_Q6_1, Q6_K, PLANAR, 1, 1, false)
        QK_CB(B_COUNT + B_Q6_2, Q6_K, PLANAR, 2, 2, false)
        QK_CB(CHAIN_PAIR + B_Q4_1, Q4_K, GGUF, 1, 1, true)
        QK_CB(CHAIN_PAIR + B_Q4_2, Q4_K, GGUF, 2, 2, true)
        QK_CB(CHAIN_PAIR + B_Q4_4, Q4_K, GGUF, 4, 2, true)
        QK_CB(CHAIN_PAIR + B_Q4_6, Q4_K, GGUF, 6, 2, true)
        QK_CB(CHAIN_PAIR + B_Q4_8, Q4_K, GGUF, 8, 2, true)
        QK_CB(CHAIN_PAIR + B_Q4_12, Q4_K, GGUF, 12, 2, true)
        QK_CB(CHAIN_PAIR + B_COUNT + B_Q4_1, Q4_K, PLANAR, 1, 1, true)
        QK_CB(CHAIN_PAIR + B_COUNT + B_Q4_2, Q4_K, PLANAR, 2, 2, true)
        QK_CB(CHAIN_PAIR + B_COUNT + B_Q4_4, Q4_K, PLANAR, 4, 2, true)
        QK_CB(CHAIN_PAIR + B_COUNT + B_Q4_6, Q4_K, PLANAR, 6, 2, true)
        QK_CB(CHAIN_PAIR + B_COUNT + B_Q4_8, Q4_K, PLANAR, 8, 2, true)
        QK_CB(CHAIN_PAIR + B_COUNT + B_Q4_12, Q4_K, PLANAR, 12, 2, true)
    default: break;
    }
#undef QK_CB
}

__device__ __forceinline__ int chain_code_type(int code) {
    const int c = (code & (CHAIN_PAIR - 1)) % B_COUNT;
    return c <= B_Q4_12 ? Q4_K : c <= B_Q5_2 ? Q5_K : c <= B_Q6_2 ? Q6_K : IQ4_XS;
}

__global__ void __launch_bounds__(1024) gemv1_chain_kernel(const uint8_t *__restrict__ plan, uint32_t *sync,
                                                           uint64_t limit) {
    __shared__ uint32_t s_ok;
    const ChainHdr h = *reinterpret_cast<const ChainHdr *>(plan);
    const ChainStepD *steps = reinterpret_cast<const ChainStepD *>(plan + sizeof(ChainHdr));
    const ChainEntryD *ents = reinterpret_cast<const ChainEntryD *>(plan + h.entries_off);
    const int blk = (int)blockIdx.x;
    if (threadIdx.x == 0) s_ok = 1u;
    for (int s = 0; s < (int)h.nsteps; ++s) {
        if (s > 0) chain_arrive(sync, s - 1);
        const ChainHook hook{sync, &s_ok, limit, s - 1, h.G};
        const ChainStepD st = steps[s];
        int i = st.e0;
        while (i < st.e1 && !(blk >= ents[i].first && blk < ents[i].last)) ++i;
        if (i < st.e1) {
            const ChainEntryD e = ents[i];
            if ((int)threadIdx.x < e.threads) {
                chain_body(e, blk - e.first, e.last - e.first, hook);
            } else {  // waves this body does not use keep the barriers in step
                hook();
                const int n = body_syncs(chain_code_type(e.code), e.K >> 6, e.useg);
                for (int k = 0; k < n; ++k) __syncthreads();
            }
        } else {
            hook();
        }
        if (s > 0 && s_ok == 0u) return;  // the same word for every wave, read after the wait's barrier
    }
}

// Chain geometry: one workgroup per CU in the whole launch, so an entry's
// share g.G of the grid is given; P phases and RL rows per round are chosen
// as in geometry() for the round lengths the chain's bodies are compiled for
// and at most 1024 threads.
// One workgroup per CU of at most 1024 threads (measured: two of 512 or
// three of 320 per CU were no faster, and three did not all fit at once).
constexpr int CHAIN_PER_CU = 1;
constexpr int CHAIN_THREADS = 1024;

template <int T, int L>
static Geo chain_geo(int64_t N, int64_t K, int G, int mult) {
    static constexpr int q4[] = {1, 2, 4, 6, 8, 12}, q5[] = {1, 2}, q6[] = {1}, q6p[] = {1, 2};
    const int *rl = T == Q4_K ? q4 : T == Q5_K ? q5 : (L == PLANAR ? q6p : q6);
    const int nrl = T == Q4_K ? 6 : T == Q5_K ? 2 : (L == PLANAR ? 2 : 1);
    Geo g;
    const int64_t U = K / 64;
    g.useg = (int)(U < 512 ? U : 512);
    g.G = G;
    const int pmax = std::max(1, CHAIN_THREADS / g.useg);
    const int64_t R = mult * ((N + G - 1) / G);
    auto plan = [&](int p, int &r) {
        const int64_t rows = (R + p - 1) / p;
        r = rl[nrl - 1];
        for (int k = 0; k < nrl; ++k)
            if (rl[k] >= rows) { r = rl[k]; break; }
        return (int64_t)p * ((rows + r - 1) / r) * r;
    };
    const int plo = R >= pmax ? (pmax + 1) / 2 : 1;
    int64_t best = INT64_MAX;
    for (int p = plo; p <= pmax; ++p) {
        int r;
        best = std::min(best, plan(p, r));
    }
    g.P = plo;
    g.RL = 1;
    for (int p = plo; p <= pmax; ++p) {
        int r;
        if (plan(p, r) <= best) { g.P = p; g.RL = r; }
    }
    g.threads = (g.P * g.useg + 63) / 64 * 64;
    return g;
}

static Geo chain_geo_of(int type, int64_t N, int64_t K, int G, int mult) {
    const bool planar = (type & PLANAR_FLAG) != 0;
    switch (type & ~PLANAR_FLAG) {
    case Q4_K: return planar ? chain_geo<Q4_K, PLANAR>(N, K, G, mult) : chain_geo<Q4_K, GGUF>(N, K, G, mult);
    case Q5_K: return planar ? chain_geo<Q5_K, PLANAR>(N, K, G, mult) : chain_geo<Q5_K, GGUF>(N, K, G, mult);
    default: return planar ? chain_geo<Q6_K, PLANAR>(N, K, G, mult) : chain_geo<Q6_K, GGUF>(N, K, G, mult);
    }
}

static size_t align16(size_t v) { return (v + 15) / 16 * 16; }

int64_t chain_plan_bytes(int nsteps, int nentries) {
    if (nsteps < 1 || nentries < nsteps) return -1;
    return (int64_t)(align16(sizeof(ChainHdr) + sizeof(ChainStepD) * (size_t)nsteps) +
                     sizeof(ChainEntryD) * (size_t)nentries);
}

hipError_t chain_plan(const ChainEntryIn *in, int nentries, const int *step_sizes, int nsteps, void *plan,
                      int64_t bytes) {
    const int64_t need = chain_plan_bytes(nsteps, nentries);
    if (need < 0 || bytes < need) return hipErrorInvalidValue;
    uint8_t *out = static_cast<uint8_t *>(plan);
    ChainHdr h{};
    h.magic = CHAIN_MAGIC;
    h.nsteps = (uint32_t)nsteps;
    h.nentries = (uint32_t)nentries;
    h.cus = device_cus();
    h.G = (uint32_t)(h.cus * CHAIN_PER_CU);
    h.entries_off = (uint32_t)align16(sizeof(ChainHdr) + sizeof(ChainStepD) * (size_t)nsteps);
    ChainStepD *steps = reinterpret_cast<ChainStepD *>(out + sizeof(ChainHdr));
    ChainEntryD *ents = reinterpret_cast<ChainEntryD *>(out + h.entries_off);
    int threads = 64;
    size_t lds = 16;
    int e0 = 0;
    for (int s = 0; s < nsteps; ++s) {
        const int n = step_sizes[s];
        if (n < 1 || n > MAX_BATCH || e0 + n > nentries) return hipErrorInvalidValue;
        steps[s] = ChainStepD{e0, e0 + n};
        // the grid shared in proportion to weight bytes (cumulative
        // rounding), at least one workgroup and at most one per schedule row
        double total = 0.0;
        for (int i = e0; i < e0 + n; ++i) total += (in[i].W2 ? 2.0 : 1.0) * (double)in[i].N * (double)in[i].row_bytes;
        double done = 0.0;
        int given = 0;
        for (int i = e0; i < e0 + n; ++i) {
            const ChainEntryIn &e = in[i];
            const int mult = e.W2 ? 2 : 1;
            done += mult * (double)e.N * (double)e.row_bytes;
            int upto = (int)(h.G * (done / total) + 0.5);
            if (i == e0 + n - 1) upto = (int)h.G;
            int share = std::max(1, upto - given);
            share = (int)std::min<int64_t>(share, e.N);
            if (given + share > (int)h.G) return hipErrorInvalidValue;  // more entries than workgroups
            Geo g = chain_geo_of(e.type, e.N, e.K, share, mult);
            const int base = body_code(e.type, g.RL);
            // the chain compiles bodies for the k-quants only (SwiGLU pairs: Q4_K)
            if (base < 0 || (e.type & ~PLANAR_FLAG) == IQ4_XS || (e.W2 && (e.type & ~PLANAR_FLAG) != Q4_K))
                return hipErrorInvalidValue;
            const size_t l = part_lds(e.N, g, mult);
            if (l > (size_t)CHAIN_LDS_MAX) return hipErrorInvalidValue;
            lds = std::max(lds, l);
            threads = std::max(threads, g.threads);
            ChainEntryD d{};
            d.W = static_cast<const uint8_t *>(e.W);
            d.W2 = e.W2;
            d.x = static_cast<const uint16_t *>(e.x);
            d.y = e.y;
            d.res = static_cast<const float *>(e.res);
            d.N = (int32_t)e.N;
            d.K = (int32_t)e.K;
            d.useg = g.useg;
            d.P = g.P;
            d.threads = g.threads;
            d.code = base + (e.W2 ? CHAIN_PAIR : 0);
            d.first = given;
            d.last = given + share;
            d.f16 = e.f16;
            ents[i] = d;
            given += share;
        }
        e0 += n;
    }
    if (e0 != nentries) return hipErrorInvalidValue;
    h.threads = threads;
    h.lds = (uint32_t)lds;
    *reinterpret_cast<ChainHdr *>(out) = h;
    return hipSuccess;
}

int chain_steps(const void *plan_host) {
    const ChainHdr *h = static_cast<const ChainHdr *>(plan_host);
    return h->magic == CHAIN_MAGIC ? (int)h->nsteps : -1;
}

static uint64_t wall_ticks_per_us() {
    static std::atomic<uint64_t> cache[MAX_DEVICES];
    const int dev = current_device();
    uint64_t v = cache[dev].load(std::memory_order_relaxed);
    if (v) return v;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
    v = std::max<uint64_t>(1, (uint64_t)khz / 1000);
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

static thread_local const char *g_chain_stage = "";
const char *chain_stage() { return g_chain_stage; }

hipError_t launch_chain(const void *plan_host, const void *plan_dev, uint32_t *sync, int64_t sync_words,
                        int64_t timeout_us, hipStream_t st) {
    const ChainHdr &h = *static_cast<const ChainHdr *>(plan_host);
    g_chain_stage = "plan";
    if (h.magic != CHAIN_MAGIC || h.cus != device_cus() || sync_words < (int64_t)h.nsteps + 2)
        return hipErrorInvalidValue;
    g_chain_stage = "LDS opt-in";
    hipError_t e = lds_opt_in<gemv1_chain_kernel>(CHAIN_LDS_MAX);
    if (e != hipSuccess) return e;
    g_chain_stage = "occupancy";
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemv1_chain_kernel, h.threads, h.lds);
    if (e != hipSuccess) return e;
    if ((int64_t)per_cu * h.cus < (int64_t)h.G) return hipErrorCooperativeLaunchTooLarge;
    g_chain_stage = "workspace clear";
    hipLaunchKernelGGL(chain_reset_kernel, dim3(1), dim3(256), 0, st, sync, (int)(h.nsteps + 2));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    g_chain_stage = "cooperative launch";
    const uint8_t *p = static_cast<const uint8_t *>(plan_dev);
    uint64_t limit = (uint64_t)(timeout_us > 0 ? timeout_us : 2000000) * wall_ticks_per_us();
    void *args[] = {&p, &sync, &limit};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(gemv1_chain_kernel), dim3(h.G), dim3(h.threads),
                                   args, h.lds, st);
    if (e == hipSuccess) g_chain_stage = "";
    return e;
}

// ---------------------------------------------------------------------------
// The chain without a caller workspace: its barrier counters live in a
// file-scope device array, one copy per GPU, kept until the process ends.
// Host code never passes the array's name to a kernel (in host code it is a
// stand-in, not a device address): it takes the device address once per
// device with hipGetSymbolAddress and uses that.  Every call on one GPU
// shares the array, so calls that overlap on one GPU race; each run clears
// the words it uses (a kernel, not a memset) before its chain starts.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t scratch[CHAIN_SCRATCH_WORDS];

__global__ void __launch_bounds__(64) chain_status_kernel(const uint32_t *sync, uint32_t *status) {
    if (threadIdx.x == 0) *status = sync[0];
}

static hipError_t chain_scratch(uint32_t **out) {
    static std::atomic<uint32_t *> addr[MAX_DEVICES];
    static std::mutex mu;
    const int dev = current_device();
    uint32_t *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *a = nullptr;
            const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!a) return hipErrorInvalidSymbol;
            p = static_cast<uint32_t *>(a);
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_chain_noalloc(const void *plan_host, const void *plan_dev, void *status, int64_t timeout_us,
                                hipStream_t st) {
    uint32_t *sync = nullptr;
    g_chain_stage = "scratch address";
    hipError_t e = chain_scratch(&sync);
    if (e != hipSuccess) return e;
    e = launch_chain(plan_host, plan_dev, sync, CHAIN_SCRATCH_WORDS, timeout_us, st);
    if (e != hipSuccess || !status) return e;
    g_chain_stage = "status copy";
    hipLaunchKernelGGL(chain_status_kernel, dim3(1), dim3(64), 0, st, (const uint32_t *)sync, (uint32_t *)status);
    e = hipGetLastError();
    if (e == hipSuccess) g_chain_stage = "";
    return e;
}

template <int T, int L>
static hipError_t launch_deq(const void *W, void *out, int64_t N, int64_t K, hipStream_t st) {
    const int64_t units = N * (K / 64);
    const unsigned grid = (unsigned)((units + WG - 1) / WG);
    hipLaunchKernelGGL((dequant_kernel<T, L>), dim3(grid), dim3(WG), 0, st, (const uint8_t *)W, (float *)out, N,
                       (int)K);
    return hipGetLastError();
}

hipError_t launch_dequant(int type, const void *W, void *out, int64_t N, int64_t K, hipStream_t st) {
    switch (type) {
    case Q4_K: return launch_deq<Q4_K, GGUF>(W, out, N, K, st);
    case Q5_K: return launch_deq<Q5_K, GGUF>(W, out, N, K, st);
    case Q6_K: return launch_deq<Q6_K, GGUF>(W, out, N, K, st);
    case IQ4_XS: return launch_deq<IQ4_XS, GGUF>(W, out, N, K, st);
    case Q4_K | PLANAR_FLAG: return launch_deq<Q4_K, PLANAR>(W, out, N, K, st);
    case Q5_K | PLANAR_FLAG: return launch_deq<Q5_K, PLANAR>(W, out, N, K, st);
    case Q6_K | PLANAR_FLAG: return launch_deq<Q6_K, PLANAR>(W, out, N, K, st);
    default: return hipErrorInvalidValue;
    }
}

template <int T>
static hipError_t launch_rp(const void *W, void *Wp, int64_t N, int64_t K, hipStream_t st) {
    const int64_t sbs = N * (K / 256);
    const unsigned grid = (unsigned)((sbs + WG - 1) / WG);
    hipLaunchKernelGGL((repack_kernel<T>), dim3(grid), dim3(WG), 0, st, (const uint8_t *)W, (uint8_t *)Wp, N, (int)K);
    return hipGetLastError();
}

hipError_t launch_repack(int type, const void *W, void *Wp, int64_t N, int64_t K, hipStream_t st) {
    switch (type) {
    case Q4_K: return launch_rp<Q4_K>(W, Wp, N, K, st);
    case Q5_K: return launch_rp<Q5_K>(W, Wp, N, K, st);
    case Q6_K: return launch_rp<Q6_K>(W, Wp, N, K, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qk
