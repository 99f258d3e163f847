// qk_format.h -- gfx950 device-side decoding of GGML k-quant superblocks.
//
// Formats (GGML k-quant layout, the reference named by the T4 dossier's
// "Mixed-Quant GEMV" prompt, section SPEC; the Q4_K struct and formula are in
// its design-doc prompt, section QUANTIZATION MIX):
//   Q4_K 144 B: d f16 @0, dmin f16 @2, scales[12] @4, qs[128] @16
//   Q5_K 176 B: d @0, dmin @2, scales[12] @4, qh[32] @16, qs[128] @48
//   Q6_K 210 B: ql[128] @0, qh[64] @128, scales[16] int8 @192, d f16 @208
//   IQ4_XS 136 B: d f16 @0, scales_h u16 @2, scales_l[4] @4, qs[128] @8
//            (GGML's block_iq4_xs; the same prompt's SPEC names IQ4_XS beside
//            Q4_K under the type flag, GGML's dequantisation as the reference)
//
// Work unit.  A superblock is split into 4 "units" of 64 weights, one per
// lane; the unit index q = 0..3 is a per-lane constant in every kernel.
//   Q4_K/Q5_K unit q : sub-blocks 2q (low nibbles of qs[32q..32q+31]) and
//                      2q+1 (high nibbles), i.e. weights 64q .. 64q+63.
//   Q6_K unit q=2n+b : half n, rows l = 16b..16b+15 of all four quarters t,
//                      i.e. weights 128n + 32t + 16b + (0..15), t = 0..3.
//   IQ4_XS unit q    : sub-blocks 2q (qs[32q..32q+15]) and 2q+1 (the next 16
//                      bytes); byte l of a sub-block holds its weights l (low
//                      nibble) and l+16 (high nibble): weights 64q .. 64q+63.
//
// Quant "patterns".  Quants are turned into packed fp16 pairs without any
// conversion instruction: a 16-bit pattern p < 2048 read as an fp16 is
// exactly p * 2^-24 (subnormal for p < 1024, smallest exponent above).  Masks
// pick the quant bits in place, so a pattern holds s*q for a power of two s
// (s = 1 for bits 0..3, s = 16 for bits 4..7 of a byte); 1/s and 2^24 are
// folded into the per-sub-block scale.  From one 32-bit word w of quant
// bytes (l, l+1, l+2, l+3):
//   pair A = weights (l, l+2)   from bytes 0 and 2 of w
//   pair B = weights (l+1, l+3) from bytes 1 and 3 (w >> 8)
// so x is kept with each group of four halves reordered to (0, 2, 1, 3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

enum : int { Q4_K = 12, Q5_K = 13, Q6_K = 14, IQ4_XS = 23 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int T> struct Fmt;
template <> struct Fmt<Q4_K> { static constexpr int bytes = 144; static constexpr int group = 32; };
template <> struct Fmt<Q5_K> { static constexpr int bytes = 176; static constexpr int group = 32; };
template <> struct Fmt<Q6_K> { static constexpr int bytes = 210; static constexpr int group = 16; };
template <> struct Fmt<IQ4_XS> { static constexpr int bytes = 136; static constexpr int group = 32; };

// ---------------------------------------------------------------------------
// Row layouts.  GGUF: a row is K/256 superblocks back to back, as in the file.
// PLANAR: the same bytes of a row regrouped into planes, so that the pieces
// the 64 lanes of a wave read for 64 consecutive units are consecutive in
// memory (whole 1 KB per load instruction instead of 16-byte pieces at the
// superblock stride).  S = K/256 superblocks, U = 4S units, unit u = 4s + q:
//   Q4_K: H[S][16] (d, dmin, scales)  A[U][16] = qs[32q..32q+15] of unit u
//         B[U][16] = qs[32q+16..32q+31]                         = 144 S bytes
//   Q5_K: H[S][16]  QH0[S][16] = qh[0..15]  QH1[S][16] = qh[16..31]
//         A[U][16]  B[U][16] (qs halves as for Q4_K)             = 176 S bytes
//   Q6_K: A[U][16] = ql[64n+16b..]  B[U][16] = ql[64n+32+16b..]
//         C[U][16] = qh[32n+16b..]  SC[U][4] = scales[8n+2t+b], t = 0..3
//         D[S][2] = d                       (q = 2n+b)          = 210 S bytes,
//         row padded to a multiple of 16 bytes.
// ---------------------------------------------------------------------------
enum : int { GGUF = 0, PLANAR = 1 };

__host__ __device__ constexpr int64_t layout_row_bytes(int T, int L, int64_t K) {
    const int64_t S = K / 256;
    const int64_t b = S * (T == Q4_K ? 144 : T == Q5_K ? 176 : T == IQ4_XS ? 136 : 210);
    return (L == PLANAR && T == Q6_K) ? (b + 15) / 16 * 16 : b;
}

// Byte offsets, within a row, of the pieces unit u reads (S superblocks per row).
template <int T, int L> struct UnitAddr;
template <> struct UnitAddr<Q4_K, GGUF> {
    uint32_t h, a, b;
    __host__ __device__ UnitAddr(int /*S*/, int u) : h(144u * (u >> 2)), a(h + 16u + 32u * (u & 3)), b(a + 16u) {}
};
template <> struct UnitAddr<Q4_K, PLANAR> {
    uint32_t h, a, b;
    __host__ __device__ UnitAddr(int S, int u) : h(16u * (u >> 2)), a(16u * S + 16u * u), b(80u * S + 16u * u) {}
};
template <> struct UnitAddr<Q5_K, GGUF> {
    uint32_t h, qh0, qh1, a, b;
    __host__ __device__ UnitAddr(int /*S*/, int u)
        : h(176u * (u >> 2)), qh0(h + 16u), qh1(h + 32u), a(h + 48u + 32u * (u & 3)), b(a + 16u) {}
};
template <> struct UnitAddr<Q5_K, PLANAR> {
    uint32_t h, qh0, qh1, a, b;
    __host__ __device__ UnitAddr(int S, int u)
        : h(16u * (u >> 2)), qh0(16u * S + h), qh1(32u * S + h), a(48u * S + 16u * u), b(112u * S + 16u * u) {}
};
template <> struct UnitAddr<Q6_K, GGUF> {
    uint32_t a, b, c, sc, d;
    __host__ __device__ UnitAddr(int /*S*/, int u) {
        const uint32_t sb = 210u * (u >> 2), n = (u >> 1) & 1, bb = u & 1;
        a = sb + 64u * n + 16u * bb;
        b = a + 32u;
        c = sb + 128u + 32u * n + 16u * bb;
        sc = sb + 192u + 8u * n;
        d = sb + 208u;
    }
};
template <> struct UnitAddr<IQ4_XS, GGUF> {
    uint32_t h, a, b;
    __host__ __device__ UnitAddr(int /*S*/, int u) : h(136u * (u >> 2)), a(h + 8u + 32u * (u & 3)), b(a + 16u) {}
};
template <> struct UnitAddr<Q6_K, PLANAR> {
    uint32_t a, b, c, sc, d;
    __host__ __device__ UnitAddr(int S, int u)
        : a(16u * u), b(64u * S + 16u * u), c(128u * S + 16u * u), sc(192u * S + 4u * u), d(208u * S + 2u * (u >> 2)) {}
};

// floor(a / b) for 0 <= a < 2^21 and b >= 1 in three instructions: with
// rcp's error of at most one ulp the product is within (a + 1/2) / b * 2^-22
// < 1/(4b) of (a + 1/2) / b, whose distance to the integers is at least 1/(2b).
// (The compiler's integer division is a long scalar sequence that every wave
// runs before its first weight load.)
__device__ __forceinline__ int small_div(int a, int b) {
    return (int)(((float)a + 0.5f) * __builtin_amdgcn_rcpf((float)b));
}

// Rows [r0, r1) of workgroup blk of nblk: N rows split as evenly as possible,
// the first N % nblk workgroups taking one row more.  A row's arithmetic does
// not depend on its workgroup.
//
// Front-loaded (fc > 0): the workgroups are dispatched in rounds of fc, one
// per CU, and a CU's memory requests are served oldest workgroup first, so
// the last round's weights arrive last.  The workgroups of every round but
// the last take fcap rows each (a full straight-line round), the last round
// the rest, split evenly: the launch's tail is shorter.  The launcher checks
// nblk % fc == 0 and (nblk - fc) * fcap <= N.
struct RowSplit {
    int r0, r1;
    __device__ RowSplit(int N, int blk, int nblk, int fc = 0, int fcap = 0) {
        int base = 0;
        if (fc > 0) {
            const int front = nblk - fc;
            if (blk < front) {
                r0 = blk * fcap;
                r1 = r0 + fcap;
                return;
            }
            base = front * fcap;
            N -= base;
            blk -= front;
            nblk = fc;
        }
        const int q = (int)((uint32_t)N / (uint32_t)nblk), r = N - q * nblk;
        r0 = base + blk * q + min(blk, r);
        r1 = r0 + q + (blk < r ? 1 : 0);
    }
};

// fp32 += a.lo*b.lo + a.hi*b.hi with fp16 operands (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_4x4x4_16b_f16: 16 independent 4x4x4 blocks per wave; block b is
// lanes 4b..4b+3, lane 4b+j supplies row j of A (a0, a1) and column j of B
// (b0, b1) and receives D[0..3][j] += sum_k A[i][k] B[k][j].
__device__ __forceinline__ f32x4 mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
    const half4_t a = __builtin_bit_cast(half4_t, make_uint2(a0, a1));
    const half4_t b = __builtin_bit_cast(half4_t, make_uint2(b0, b1));
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0);
}

// Packed fp16 add (v_pk_add_f16).  On quant patterns (multiples of 2^-24
// below 2^-14) every sum is exact: the fp16 denormals are kept.
__device__ __forceinline__ uint32_t padd(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) + __builtin_bit_cast(half2_t, b));
}

// ---------------------------------------------------------------------------
// Shifted form of a Q4_K/Q5_K sub-block.  With a = d*sc and b = dmin*m,
//     sum_i w_i x_i = a * sum_i (q_i - c) x_i + e * sum_i x_i,   e = a*c - b,
// for any integer c.  Taking c = clamp(rint(b / a), 0, QMAX) gives, for every
// quant value q of the sub-block, |a|*|q - c| + |e| <= 3 |a*q - b|: no term of
// the sum is larger than three times its weight's share of sum_i |w_i x_i|,
// so the fp32 rounding of the sums stays a small multiple of 2^-24 times that
// (the plain factored form a*sum q x - b*sum x can cancel: a sub-block whose
// weights are all zero, d*sc*q = dmin*m, leaves rounding noise where the
// exact answer is 0).  q - c is formed per weight on the fp16 patterns, so
// every product stays exact; e is one fp32 fma (one rounding, the same value
// the dequantised weight of quant c takes).  Units: a = d*sc*2^-24, e times
// 2^-24, as the patterns; c is an exact small integer in fp32.
// ---------------------------------------------------------------------------
struct KShift {
    float a, e;      // d*sc*2^-24, (a*c - dmin*m*2^-24) rounded once
    uint32_t neg;    // the fp16 pair (-s*c*2^-24, -s*c*2^-24) to add to patterns holding s*q
};

template <int QMAX, int S>
__device__ __forceinline__ KShift k_shift(float d, float dmin, float sc_p, float m_p) {
    KShift k;
    // exact products (11 x 6 significant bits), written as fmas with a zero
    // addend so that both factors stay fp16 operands (v_fma_mix_f32)
    k.a = __builtin_fmaf(d, sc_p, 0.f);
    const float b = __builtin_fmaf(dmin, m_p, 0.f);
    // a = 0 gives b * inf (inf or NaN): fmaxf takes 0 for NaN, the clamp
    // handles inf; with a = 0 the quant sum is multiplied by 0 anyway
    const float c = fminf(fmaxf(rintf(b * __builtin_amdgcn_rcpf(k.a)), 0.f), (float)QMAX);
    k.e = __builtin_fmaf(k.a, c, -b);
    const float nc = c * (-(float)S * 0x1p-24f);  // exact, a fp16 denormal
    k.neg = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(nc, nc));
    return k;
}

// Q6_K: w = d*sc*(q - 32); the patterns of quarters 0-1 hold q*2^-24, those
// of quarters 2-3 16q*2^-24, so q - 32 is one packed add of these constants.
constexpr uint32_t Q6_OFF_LO = 0x80208020u;  // fp16 pair (-32*2^-24, -32*2^-24)
constexpr uint32_t Q6_OFF_HI = 0x82008200u;  // fp16 pair (-512*2^-24, -512*2^-24)

__device__ __forceinline__ float f16_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Weight loads.  NT selects the nontemporal (streaming) form: every weight
// byte is read once per call, so there is nothing to keep in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint8_t *p) {
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4 *>(p);
    }
}
template <bool NT>
__device__ __forceinline__ uint2 ld8(const uint8_t *p) {
    if constexpr (NT) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        return make_uint2(v.x, v.y);
    } else {
        return *reinterpret_cast<const uint2 *>(p);
    }
}
template <bool NT>
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    else return *reinterpret_cast<const uint32_t *>(p);
}
template <bool NT>
__device__ __forceinline__ uint32_t ld2(const uint8_t *p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
    else return *reinterpret_cast<const uint16_t *>(p);
}

// The loads of a unit leave together: the scheduler may not sink any of them
// into the arithmetic that follows (under register pressure it otherwise
// spreads them out and serialises their memory latencies: Q6_K 5120 x 17408
// measured 25.4 us without this barrier, 18.7 us with it).
__device__ __forceinline__ void issue_together() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Q4_K / Q5_K 6-bit scales and mins of the unit's two sub-blocks (2q, 2q+1).
// scales[12] as three words S0 = bytes 0..3, S1 = 4..7, S2 = 8..11:
//   j < 4 : sc_j = byte j of S0 & 63,  m_j = byte j of S1 & 63
//   j >= 4: sc_j = nibble lo of byte j-4 of S2 | (bits 6..7 of byte j-4 of S0) << 4
//           m_j  = nibble hi of byte j-4 of S2 | (bits 6..7 of byte j-4 of S1) << 4
// Both sub-blocks of a unit sit in adjacent bytes, so one per-lane shift and
// a per-lane set of masks covers all four units without branching.
// ---------------------------------------------------------------------------
struct KScaleSel {
    // per-lane bit offsets / widths: for q < 2 the fields are 6-bit bytes of
    // S0 (sc) and S1 (m); for q >= 2 a nibble of S2 plus 2 bits of S0 / S1.
    uint32_t o, wn, o2, w2, sl;
    __device__ explicit KScaleSel(int q) {
        const bool hi = q >= 2;
        o = 16u * (uint32_t)(q & 1);  // bit offset of byte j (j = 2q or 2q-4) in its word
        wn = hi ? 4u : 0u;            // nibble width taken from S2 (0: none)
        o2 = o + (hi ? 6u : 0u);      // offset of the bits taken from S0 / S1
        w2 = hi ? 2u : 6u;
        sl = hi ? 4u : 0u;            // where those bits land
    }
};

struct KScales { uint32_t sc_lo, sc_hi, m_lo, m_hi; };

__device__ __forceinline__ uint32_t bfe(uint32_t v, uint32_t off, uint32_t w) {
    return __builtin_amdgcn_ubfe(v, off, w);
}

__device__ __forceinline__ KScales k_scales(const uint4 &hdr, const KScaleSel &s) {
    const uint32_t S0 = hdr.y, S1 = hdr.z, S2 = hdr.w;
    KScales r;
    r.sc_lo = bfe(S2, s.o, s.wn) | (bfe(S0, s.o2, s.w2) << s.sl);
    r.sc_hi = bfe(S2, s.o + 8, s.wn) | (bfe(S0, s.o2 + 8, s.w2) << s.sl);
    r.m_lo = bfe(S2, s.o + 4, s.wn) | (bfe(S1, s.o2, s.w2) << s.sl);
    r.m_hi = bfe(S2, s.o + 12, s.wn) | (bfe(S1, s.o2 + 8, s.w2) << s.sl);
    return r;
}

// ---------------------------------------------------------------------------
// Raw registers of one unit and its pattern decoder.
// ---------------------------------------------------------------------------
template <int T> struct Unit;

// Q4_K: the 16-byte header and the unit's 32 bytes of qs.  The four lanes of
// a superblock load the same header (one cache line, served once).
// Patterns of qs word i (l = 4i):
//   p[0] = low-sub-block pair A  (s = 1)    p[1] = low pair B  (s = 1)
//   p[2] = high-sub-block pair A (s = 16)   p[3] = high pair B (s = 16)
template <> struct Unit<Q4_K> {
    uint4 h, a, b;
    // row: the row's first byte.  On GGUF rows the second half of the
    // quants follows the first (b = a + 16): addressed as an immediate offset
    // of the first half's pointer, one 64-bit address less per unit.
    template <bool NT, int L>
    __device__ __forceinline__ void load(const uint8_t *row, const UnitAddr<Q4_K, L> &o) {
        const uint8_t *pa = row + o.a;
        h = ld16<NT>(row + o.h);
        a = ld16<NT>(pa);
        b = ld16<NT>(L == GGUF ? pa + 16 : row + o.b);
        issue_together();
    }
    __device__ __forceinline__ uint4 header() const { return h; }
    __device__ __forceinline__ uint32_t qword(int i) const { return i < 4 ? word(a, i) : word(b, i - 4); }
    __device__ __forceinline__ void patterns(int i, int /*q*/, uint32_t p[4]) const {
        const uint32_t w = qword(i), t = w >> 8;
        p[0] = w & 0x000f000fu;
        p[1] = t & 0x000f000fu;
        p[2] = w & 0x00f000f0u;
        p[3] = t & 0x00f000f0u;
    }
};

// Q5_K: as Q4_K plus the high-bit plane qh[32]; bit j of qh[l] is bit 4 of the
// quant of weight 32j + l.  For unit q the two bits of interest of each qh
// byte are bits 2q (low sub-block) and 2q+1 (high sub-block).
template <> struct Unit<Q5_K> {
    uint4 h, qh0, qh1, a, b;
    template <bool NT, int L>
    // (GGUF rows: qh0 / qh1 at 16 / 32 bytes past the header, b = a + 16,
    // as immediate offsets)
    __device__ __forceinline__ void load(const uint8_t *row, const UnitAddr<Q5_K, L> &o) {
        const uint8_t *ph = row + o.h, *pa = row + o.a;
        h = ld16<NT>(ph);
        qh0 = ld16<NT>(L == GGUF ? ph + 16 : row + o.qh0);
        qh1 = ld16<NT>(L == GGUF ? ph + 32 : row + o.qh1);
        a = ld16<NT>(pa);
        b = ld16<NT>(L == GGUF ? pa + 16 : row + o.b);
        issue_together();
    }
    __device__ __forceinline__ uint4 header() const { return h; }
    __device__ __forceinline__ uint32_t qword(int i) const { return i < 4 ? word(a, i) : word(b, i - 4); }
    __device__ __forceinline__ uint32_t hword(int i) const { return i < 4 ? word(qh0, i) : word(qh1, i - 4); }
    __device__ __forceinline__ void patterns(int i, int q, uint32_t p[4]) const {
        const uint32_t w = qword(i), t = w >> 8;
        const uint32_t H = hword(i) >> (2 * q);  // bit 0 / bit 1 of each byte: low / high sub-block
        p[0] = (w & 0x000f000fu) | ((H << 4) & 0x00100010u);
        p[1] = (t & 0x000f000fu) | ((H >> 4) & 0x00100010u);
        p[2] = (w & 0x00f000f0u) | ((H << 7) & 0x01000100u);
        p[3] = (t & 0x00f000f0u) | ((H >> 1) & 0x01000100u);
    }
};

// Q6_K unit q = 2n + b.  A = ql[64n + 16b ..] (quarters 0 low / 2 high nibble),
// B = ql[64n + 32 + 16b ..] (quarters 1 / 3), C = qh[32n + 16b ..] (2 bits per
// quarter: bits 2t..2t+1).  Superblocks are 2-byte aligned only; these are
// unaligned 16-byte loads, which the HSA unaligned access mode allows.
// Patterns of word i (rows l = 16b + 4i ..):
//   p[2t] = quarter t pair A, p[2t+1] = quarter t pair B;  s = 1 for t < 2, 16 for t >= 2.
template <> struct Unit<Q6_K> {
    uint4 a, b, c;
    uint2 sc;      // GGUF: scales[8n .. 8n+7];  PLANAR: .x = this unit's 4 scales, quarter order
    uint32_t d;    // fp16 d in the low half
    template <bool NT, int L>
    // (GGUF rows: b = a + 32 as an immediate offset)
    __device__ __forceinline__ void load(const uint8_t *row, const UnitAddr<Q6_K, L> &o) {
        const uint8_t *pa = row + o.a;
        a = ld16<NT>(pa);
        b = ld16<NT>(L == GGUF ? pa + 32 : row + o.b);
        c = ld16<NT>(row + o.c);
        if constexpr (L == PLANAR) sc = make_uint2(ld4<NT>(row + o.sc), 0u);
        else sc = ld8<NT>(row + o.sc);
        d = ld2<NT>(row + o.d);
        issue_together();
    }
    __device__ __forceinline__ void patterns(int i, int /*q*/, uint32_t p[8]) const {
        const uint32_t A = word(a, i), B = word(b, i), C = word(c, i);
        const uint32_t c4 = C << 4, c2 = C << 2;
        const uint32_t A8 = A >> 8, B8 = B >> 8, c4b = C >> 4, c2b = C >> 6;
        p[0] = (A & 0x000f000fu) | (c4 & 0x00300030u);
        p[1] = (A8 & 0x000f000fu) | (c4b & 0x00300030u);
        p[2] = (B & 0x000f000fu) | (c2 & 0x00300030u);
        p[3] = (B8 & 0x000f000fu) | (c2b & 0x00300030u);
        p[4] = (A & 0x00f000f0u) | (c4 & 0x03000300u);
        p[5] = (A8 & 0x00f000f0u) | (c4b & 0x03000300u);
        p[6] = (B & 0x00f000f0u) | (c2 & 0x03000300u);
        p[7] = (B8 & 0x00f000f0u) | (c2b & 0x03000300u);
    }
    // signed scale of quarter t for this unit (b = q & 1): scales[8n + 2t + b]
    template <int L = GGUF>
    __device__ __forceinline__ int scale(int t, int q) const {
        if constexpr (L == PLANAR) return (int)(int8_t)(uint8_t)(sc.x >> (8 * t));
        const int idx = 2 * t + (q & 1);
        const uint32_t wv = idx < 4 ? sc.x : sc.y;
        return (int)(int8_t)(uint8_t)(wv >> (8 * (idx & 3)));
    }
};

// ---------------------------------------------------------------------------
// IQ4_XS.  A 4-bit index selects one of 16 signed integers kv (GGML's
// non-linear IQ4_NL codebook, below); sub-block ib's weights are
// d * (ls_ib - 32) * kv with the 6-bit scale ls_ib = nibble (ib & 1) of
// scales_l[ib / 2] | bits 2ib..2ib+1 of scales_h << 4.  The codebook is
// increasing: indices 0..7 are its negative entries, 8..15 its positive ones,
// so bit 3 of an index is the sign and its low 3 bits pick a magnitude from
// one of two 8-entry tables.  Patterns are the fp16 values kv * 2^-24 (a
// sign bit over |kv| <= 127: exact subnormals, so every product with an
// fp16 x is exact), built with byte permutes (v_perm_b32 picks each result
// byte from 8 source bytes by a selector byte 0..7), four indices at a time.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr uint32_t bytes4(int b0, int b1, int b2, int b3) {
    return (uint32_t)b0 | (uint32_t)b1 << 8 | (uint32_t)b2 << 16 | (uint32_t)b3 << 24;
}
// |kv| of indices 0..3, 4..7 (kv < 0) and 8..11, 12..15 (kv > 0)
constexpr uint32_t IQ4_MAG0 = bytes4(127, 104, 83, 65), IQ4_MAG1 = bytes4(49, 35, 22, 10);
constexpr uint32_t IQ4_MAG2 = bytes4(1, 13, 25, 38), IQ4_MAG3 = bytes4(53, 69, 89, 113);

// v: four indices in bits 0..3 of its bytes (higher bits ignored), those of
// weights (l, l+1, l+2, l+3).  pa = the pattern pair of weights (l, l+2),
// pb = (l+1, l+3), as the other types' pairs A and B.
__device__ __forceinline__ void iq4_pairs(uint32_t v, uint32_t &pa, uint32_t &pb) {
    const uint32_t s7 = v & 0x07070707u;
    const uint32_t neg = __builtin_amdgcn_perm(IQ4_MAG1, IQ4_MAG0, s7);
    const uint32_t pos = __builtin_amdgcn_perm(IQ4_MAG3, IQ4_MAG2, s7);
    const uint32_t sel = ((v >> 1) & 0x04040404u) | 0x03020100u;  // byte k: k, or 4 + k if index >= 8
    const uint32_t mag = __builtin_amdgcn_perm(pos, neg, sel);
    const uint32_t sgn = __builtin_amdgcn_perm(0u, 0x80808080u, sel);  // 0x80 where index < 8
    pa = __builtin_amdgcn_perm(sgn, mag, 0x06020400u);  // |kv0|, sign0, |kv2|, sign2
    pb = __builtin_amdgcn_perm(sgn, mag, 0x07030501u);
}

// The 8-byte header and the unit's 32 bytes of qs (superblocks are 8-byte
// aligned only: unaligned 16-byte loads, as for Q6_K).  Patterns of qs word
// i (bytes l = 4(i & 3) .. of sub-block 2q + (i >> 2)):
//   p[0], p[1] = pairs A, B of the low nibbles (weights l ..)
//   p[2], p[3] = pairs A, B of the high nibbles (weights l + 16 ..)
template <> struct Unit<IQ4_XS> {
    uint2 h;  // .x = d | scales_h << 16, .y = scales_l[0..3]
    uint4 a, b;
    template <bool NT, int L>
    // (b = a + 16 as an immediate offset)
    __device__ __forceinline__ void load(const uint8_t *row, const UnitAddr<IQ4_XS, L> &o) {
        const uint8_t *pa = row + o.a;
        h = ld8<NT>(row + o.h);
        a = ld16<NT>(pa);
        b = ld16<NT>(pa + 16);
        issue_together();
    }
    __device__ __forceinline__ uint32_t qword(int i) const { return i < 4 ? word(a, i) : word(b, i - 4); }
    __device__ __forceinline__ void patterns(int i, int /*q*/, uint32_t p[4]) const {
        const uint32_t w = qword(i);
        iq4_pairs(w, p[0], p[1]);
        iq4_pairs(w >> 4, p[2], p[3]);
    }
    // ls - 32 of sub-block 2q + hi (hi = 0, 1)
    __device__ __forceinline__ int scale(int q, int hi) const {
        const uint32_t lo4 = __builtin_amdgcn_ubfe(h.y, 8u * q + 4u * hi, 4u);
        const uint32_t hi2 = __builtin_amdgcn_ubfe(h.x, 16u + 4u * q + 2u * hi, 2u);
        return (int)(lo4 | hi2 << 4) - 32;
    }
    // d * 2^24 (exact: the patterns carry 2^-24)
    __device__ __forceinline__ float d24() const { return f16_lo(h.x) * 0x1p24f; }
};

}  // namespace qk
