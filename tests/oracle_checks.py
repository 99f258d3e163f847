"""Pins of the CPU oracle against facts that do not come from the oracle.

Each check takes an ``oracle.Oracle`` handle and raises AssertionError on a
mismatch.  ``test_oracle_pins.py`` runs them on the real oracle; the mutation
test runs them on deliberately broken builds of the oracle source to show that
a plausible mistake (a dropped term, a wrong sign, a wrong index or shift, a
transposed operand) fails at least one of them.

What each check pins against:
* fp16 widening            -- numpy's float16 -> float32 conversion, all 65536 inputs;
* scale/min packing        -- single-field and random round trips through the
                              test-side packer (``kquant_pack``);
* quant planes             -- every value at every position, via the packer;
* bit structure            -- each quant bit moves exactly one weight by 2^b;
* worked examples          -- hand-packed bytes and closed forms in tests/golden
                              (E4 also fixes the IQ4_XS codebook the oracle uses);
* rounding                 -- exact integer arithmetic, rounded once to fp32 (RNE);
* Q5_K / Q4_K invariant    -- Q5_K with qh = 0 equals Q4_K of the same fields;
* GEMV                     -- integer-weight special case against numpy matmul,
                              the min-term-only closed form, and the dot of the
                              dequantised matrix against numpy matmul;
* tolerance plumbing       -- the acceptance bound accepts/rejects as stated.
"""
from __future__ import annotations

import glob
import os

import numpy as np

import kquant_pack as kp

Q4_K, Q5_K, Q6_K, IQ4_XS = kp.Q4_K, kp.Q5_K, kp.Q6_K, kp.IQ4_XS
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ONE, ZERO = kp.half_bits(1.0), 0


def _same_f32(a, b):
    """Bitwise equality of float32 arrays with -0 == +0."""
    a = np.asarray(a, dtype=np.float32) + np.float32(0.0)
    b = np.asarray(b, dtype=np.float32) + np.float32(0.0)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------- fields

def check_half_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.half_to_float(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN set differs"
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32)), "fp16 widening differs"


def check_scale_min_single_field(o):
    for which in ("sc", "m"):
        for j in range(8):
            for v in range(64):
                sc, m = [0] * 8, [0] * 8
                (sc if which == "sc" else m)[j] = v
                s = kp.pack_k_scales(sc, m)
                for jj in range(8):
                    assert o.k_scale_min(s, jj) == (sc[jj], m[jj]), (which, j, v, jj)


def check_scale_min_random(o, n=500, seed=11):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        sc, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        s = kp.pack_k_scales(sc, m)
        for j in range(8):
            assert o.k_scale_min(s, j) == (sc[j], m[j])


def _unit_block(qtype):
    """A block whose dequantised weights equal the raw quant (Q6_K: quant - 32;
    IQ4_XS: the codebook value of the index)."""
    if qtype == Q6_K:
        return kp.make_q6_block(ONE, [1] * 16, [0] * 256)
    if qtype == IQ4_XS:
        return kp.make_iq4xs_block(ONE, [33] * 8, [0] * 256)
    return kp.make_k_block(qtype, ONE, ZERO, [1] * 8, [0] * 8, [0] * 256)


def check_quant_planes(o, qtype):
    """Every quant value at every position, in one batched dequant call.
    IQ4_XS (d = 1, factor ls - 32 = 1): the weight is the codebook value of
    the index, here taken from the oracle's codebook reader (the positions are
    what this pins; the codebook itself is pinned by the worked example)."""
    levels = {Q4_K: 16, Q5_K: 32, Q6_K: 64, IQ4_XS: 16}[qtype]
    base = _unit_block(qtype)
    rows, exp = [], []
    off = -32.0 if qtype == Q6_K else 0.0
    val = (lambda v: float(o.iq4nl_value(v))) if qtype == IQ4_XS else (lambda v: v + off)
    for i in range(256):
        for v in range(1, levels):
            b = base.copy()
            kp.put_quant(qtype, b, i, v)
            rows.append(b)
            e = np.full(256, val(0), dtype=np.float32)
            e[i] = val(v)
            exp.append(e)
    got = o.dequant(qtype, np.stack(rows), 256)
    assert _same_f32(got, np.stack(exp)), f"quant plane mismatch for type {qtype}"
    # the single-weight reader agrees with the batched dequant on a sample
    for r in range(0, len(rows), 97):
        i = r // (levels - 1)
        assert o.quant(qtype, rows[r], i) == (r % (levels - 1)) + 1


def check_bit_structure(o, qtype):
    """Each bit of the quant planes moves exactly one weight, by a power of two,
    and the map bit -> (weight, power) is one-to-one onto weights x q-bits."""
    base = _unit_block(qtype)
    lo, hi = kp.quant_region(qtype)
    rows = []
    for byte in range(lo, hi):
        for bit in range(8):
            b = base.copy()
            b[byte] ^= np.uint8(1 << bit)
            rows.append(b)
    w0 = o.dequant(qtype, base[None, :], 256)[0]
    got = o.dequant(qtype, np.stack(rows), 256)
    seen = set()
    nbits = {Q4_K: 4, Q5_K: 5, Q6_K: 6}[qtype]
    for r in range(got.shape[0]):
        diff = np.nonzero(got[r] != w0)[0]
        assert diff.size == 1, f"bit {r} changes {diff.size} weights"
        i = int(diff[0])
        delta = float(got[r][i] - w0[i])
        p = int(round(np.log2(delta)))
        assert delta == 2.0 ** p and 0 <= p < nbits, (r, delta)
        seen.add((i, p))
    assert len(seen) == 256 * nbits


def check_iq4xs_bit_structure(o):
    """Each bit of the index plane changes exactly one weight, to the codebook
    value of the index with that bit flipped; bit -> (weight, index bit) is
    one-to-one onto weights x 4 bits."""
    rng = np.random.default_rng(13)
    idx = rng.integers(0, 16, 256)
    base = kp.make_iq4xs_block(ONE, [33] * 8, idx)
    lo, hi = kp.quant_region(IQ4_XS)
    rows, flips = [], []
    for byte in range(lo, hi):
        for bit in range(8):
            b = base.copy()
            b[byte] ^= np.uint8(1 << bit)
            rows.append(b)
    w0 = o.dequant(IQ4_XS, base[None, :], 256)[0]
    got = o.dequant(IQ4_XS, np.stack(rows), 256)
    seen = set()
    for r in range(got.shape[0]):
        diff = np.nonzero(got[r] != w0)[0]
        assert diff.size == 1, f"bit {r} changes {diff.size} weights"
        i = int(diff[0])
        matches = [p for p in range(4) if got[r][i] == np.float32(o.iq4nl_value(int(idx[i]) ^ (1 << p)))]
        assert len(matches) == 1, (r, i)
        seen.add((i, matches[0]))
    assert len(seen) == 256 * 4


def check_iq4xs_scale_single_field(o):
    """Every 6-bit scale value alone at every sub-block, through the packer:
    the reader returns it there and 0 elsewhere, and the weights of that
    sub-block (d = 1, index 8 whose codebook value the worked example fixes at
    1) come out as ls - 32."""
    idx = [8] * 256
    for ib in range(8):
        for v in range(64):
            ls = [0] * 8
            ls[ib] = v
            b = kp.make_iq4xs_block(ONE, ls, idx)
            for jj in range(8):
                assert o.iq4xs_scale(b, jj) == ls[jj], (ib, v, jj)
            w = o.dequant(IQ4_XS, b[None, :], 256)[0]
            exp = np.repeat(np.array(ls, dtype=np.float32) - 32, 32) * np.float32(o.iq4nl_value(8))
            assert _same_f32(w, exp), (ib, v)


def check_iq4xs_exact(o, nblocks=32, seed=14):
    """w = d * (ls - 32) * kv evaluated in exact integers (d over every fp16
    class, both signs; every scale; every index) equals the fp32 result: the
    product never rounds."""
    rng = np.random.default_rng(seed)
    kv = [o.iq4nl_value(v) for v in range(16)]
    blocks, exp = [], []
    for _ in range(nblocks):
        d_bits = int(rng.integers(0, 0x7C00)) | (int(rng.integers(0, 2)) << 15)
        ls, idx = rng.integers(0, 64, 8), rng.integers(0, 16, 256)
        blocks.append(kp.make_iq4xs_block(d_bits, ls, idx))
        Md, Ed = _f16_parts(d_bits)
        exp.append([float(Md * (int(ls[i // 32]) - 32) * kv[int(idx[i])]) * 2.0 ** Ed for i in range(256)])
    got = o.dequant(IQ4_XS, np.stack(blocks), 256)
    assert _same_f32(got, np.array(exp, dtype=np.float32))


def check_q6k_scale_index(o):
    q = [32 + 1] * 256          # q - 32 == 1 everywhere
    sc = list(range(-8, 8))     # distinct per 16-weight group
    b = kp.make_q6_block(ONE, sc, q)
    w = o.dequant(Q6_K, b[None, :], 256)[0]
    assert np.array_equal(w, np.repeat(np.array(sc, dtype=np.float32), 16))
    for i in range(0, 256, 7):
        assert o.q6k_scale(b, i) == sc[i // 16]


# ---------------------------------------------------------------- formula

def _closed_form(form, i):
    if form == "e1":
        return (i // 32 + 1) * (i % 16) - 1.0
    if form == "e2":
        j = i // 32
        return (8 * j + 7) * (i % 32) - (63 - 8 * j) / 4.0
    if form == "e3":
        return 2.0 ** -4 * (i // 16 - 8) * (i % 64 - 32)
    if form == "e4":
        f = (-4, -3, -2, -1, 1, 2, 3, 4)[i // 32]
        return 2.0 ** -3 * f * E4_CODEBOOK[i % 16]
    raise ValueError(form)


# The codebook as the worked example E4 states it (tests/golden/iq4xs_e4.txt,
# restated from GGML's IQ4_NL / IQ4_XS format; no GGML build is available
# here to compare with, so the values are a reading, not a pin against GGML).
E4_CODEBOOK = (-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113)


def _example_fields(form):
    """The hand-chosen fields of each worked example, packed by the test packer."""
    if form == "e1":
        return kp.make_k_block(Q4_K, kp.half_bits(1.0), kp.half_bits(0.5),
                               [j + 1 for j in range(8)], [2] * 8, [i % 16 for i in range(256)])
    if form == "e2":
        return kp.make_k_block(Q5_K, kp.half_bits(1.0), kp.half_bits(0.25),
                               [8 * j + 7 for j in range(8)], [63 - 8 * j for j in range(8)],
                               [i % 32 for i in range(256)])
    if form == "e3":
        return kp.make_q6_block(kp.half_bits(2.0 ** -4), [s - 8 for s in range(16)],
                                [i % 64 for i in range(256)])
    if form == "e4":
        return kp.make_iq4xs_block(kp.half_bits(2.0 ** -3), [28, 29, 30, 31, 33, 34, 35, 36],
                                   [i % 16 for i in range(256)])
    raise ValueError(form)


def check_worked_examples(o):
    files = sorted(glob.glob(os.path.join(GOLDEN, "*_e*.txt")))
    assert len(files) >= 4
    for path in files:
        qt, form, block, values = kp.load_golden(path)
        assert block.size == kp.BLOCK_BYTES[qt]
        assert np.array_equal(_example_fields(form), block), f"{path}: packer disagrees with hand bytes"
        w = o.dequant(qt, block[None, :], 256)[0]
        exp = np.array([_closed_form(form, i) for i in range(256)], dtype=np.float32)
        assert _same_f32(w, exp), f"{path}: closed form differs"
        for i, v in values.items():
            assert w[i] == np.float32(v), (path, i, w[i], v)


def _f16_parts(bits):
    """fp16 bits -> (signed integer mantissa, exponent): value = M * 2^E exactly."""
    s, e, m = (bits >> 15) & 1, (bits >> 10) & 0x1F, bits & 0x3FF
    assert e != 31
    M, E = (m, -24) if e == 0 else (1024 + m, e - 25)
    return (-M if s else M), E


def _round_f32(num: int, exp: int) -> float:
    """Round num * 2^exp to the nearest float32, ties to even (normal range)."""
    if num == 0:
        return 0.0
    sign = -1 if num < 0 else 1
    a = abs(num)
    L = a.bit_length()
    if L > 24:
        sh = L - 24
        q, r = a >> sh, a & ((1 << sh) - 1)
        half = 1 << (sh - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
        a, exp = q, exp + sh
    return float(np.float32(sign * a * 2.0 ** exp))


def check_exact_rounding(o, nblocks=48, seed=5):
    """w = d*(sc*q) - dmin*m evaluated exactly in integers, rounded once to fp32."""
    rng = np.random.default_rng(seed)
    rounded = 0
    for qt in (Q4_K, Q5_K):
        blocks, exp = [], []
        for _ in range(nblocks):
            # d, dmin over every finite fp16 magnitude, subnormals included, both signs
            d_bits = int(rng.integers(0, 0x7C00)) | (int(rng.integers(0, 2)) << 15)
            m_bits = int(rng.integers(0, 0x7C00)) | (int(rng.integers(0, 2)) << 15)
            sc, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
            q = rng.integers(0, 16 if qt == Q4_K else 32, 256)
            blocks.append(kp.make_k_block(qt, d_bits, m_bits, sc, m, q))
            (Md, Ed), (Mm, Em) = _f16_parts(d_bits), _f16_parts(m_bits)
            e0 = min(Ed, Em)
            vals = []
            for i in range(256):
                j = i // 32
                num = Md * int(sc[j]) * int(q[i]) * 2 ** (Ed - e0) - Mm * int(m[j]) * 2 ** (Em - e0)
                vals.append(_round_f32(num, e0))
                a = abs(num)
                if a and (a >> ((a & -a).bit_length() - 1)).bit_length() > 24:
                    rounded += 1  # the exact value is not an fp32: the subtraction rounds
            exp.append(vals)
        got = o.dequant(qt, np.stack(blocks), 256)
        assert _same_f32(got, np.array(exp, dtype=np.float32)), f"rounding differs for type {qt}"
    assert rounded > 100, "the sample never exercised a rounding subtraction"


def check_q6k_exact(o, nblocks=32, seed=6):
    rng = np.random.default_rng(seed)
    blocks, exp = [], []
    for _ in range(nblocks):
        d_bits = int(rng.integers(0, 0x7C00)) | (int(rng.integers(0, 2)) << 15)
        sc = rng.integers(-128, 128, 16)
        q = rng.integers(0, 64, 256)
        blocks.append(kp.make_q6_block(d_bits, sc, q))
        Md, Ed = _f16_parts(d_bits)
        exp.append([float(Md * int(sc[i // 16]) * (int(q[i]) - 32)) * 2.0 ** Ed for i in range(256)])
    got = o.dequant(Q6_K, np.stack(blocks), 256)
    assert _same_f32(got, np.array(exp, dtype=np.float32))


def check_q5_q4_invariant(o, n=64, seed=7):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        d, dm = int(rng.integers(0x0400, 0x7C00)), int(rng.integers(0x0400, 0x7C00))
        sc, m, q = rng.integers(0, 64, 8), rng.integers(0, 64, 8), rng.integers(0, 16, 256)
        b4 = kp.make_k_block(Q4_K, d, dm, sc, m, q)
        b5 = kp.make_k_block(Q5_K, d, dm, sc, m, q)
        assert _same_f32(o.dequant(Q4_K, b4[None], 256), o.dequant(Q5_K, b5[None], 256))


# ---------------------------------------------------------------- GEMV

def check_gemv_integer_textbook(o, seed=8):
    """d = 1, dmin = 0, sc = 1: W is an integer matrix; y must match numpy's matmul."""
    rng = np.random.default_rng(seed)
    N, K, nc = 37, 768, 3
    for qt in (Q4_K, Q5_K, Q6_K, IQ4_XS):
        levels = {Q4_K: 16, Q5_K: 32, Q6_K: 64, IQ4_XS: 16}[qt]
        q = rng.integers(0, levels, (N, K))
        rows = []
        for n in range(N):
            blocks = []
            for s in range(K // 256):
                qq = q[n, 256 * s:256 * s + 256]
                if qt == Q6_K:
                    blocks.append(kp.make_q6_block(ONE, [1] * 16, qq))
                elif qt == IQ4_XS:
                    blocks.append(kp.make_iq4xs_block(ONE, [33] * 8, qq))
                else:
                    blocks.append(kp.make_k_block(qt, ONE, ZERO, [1] * 8, [0] * 8, qq))
            rows.append(np.concatenate(blocks))
        W = np.stack(rows)
        x = rng.standard_normal((K, nc)).astype(np.float16)
        if qt == IQ4_XS:
            Wi = np.array(E4_CODEBOOK, dtype=np.float64)[q]
        else:
            Wi = q.astype(np.float64) - (32.0 if qt == Q6_K else 0.0)
        yref = Wi @ x.astype(np.float64)
        Sref = np.abs(Wi) @ np.abs(x.astype(np.float64))
        y, S = o.gemv(qt, W, x, K)
        assert y.shape == (N, nc)
        assert np.all(np.abs(y - yref) <= 1e-12 * Sref), f"type {qt}"
        assert np.allclose(S, Sref, rtol=1e-12, atol=0)


def check_gemv_min_term(o, seed=9):
    """All quants zero: y = -sum_j dmin*m_j*sum_{i in j} x_i (closed form)."""
    rng = np.random.default_rng(seed)
    K = 512
    for qt in (Q4_K, Q5_K):
        N = 5
        rows, yref = [], np.zeros((N, 2))
        x = rng.standard_normal((K, 2)).astype(np.float16)
        xs = x.astype(np.float64).reshape(K // 32, 32, 2).sum(axis=1)  # per sub-block sums
        for n in range(N):
            blocks = []
            for s in range(K // 256):
                dmin = float(2.0 ** rng.integers(-10, -2))
                m = rng.integers(0, 64, 8)
                blocks.append(kp.make_k_block(qt, kp.half_bits(0.75), kp.half_bits(dmin),
                                              rng.integers(0, 64, 8), m, [0] * 256))
                for j in range(8):
                    yref[n] -= dmin * m[j] * xs[8 * s + j]
            rows.append(np.concatenate(blocks))
        y, S = o.gemv(qt, np.stack(rows), x, K)
        assert np.all(np.abs(y - yref) <= 1e-12 * S), f"type {qt}"


def check_gemv_dot_of_dequant(o, synth, seed=10):
    """y equals numpy's f64 matmul of the dequantised matrix, for ncols 1 and 5."""
    for qt in (Q4_K, Q5_K, Q6_K, IQ4_XS):
        N, K = 29, 1024
        W = synth.superblocks(qt, N, K, seed)
        w = o.dequant(qt, W, K).astype(np.float64)
        for nc in (1, 5):
            x = synth.activations(K, nc, seed)
            y, S = o.gemv(qt, W, x, K)
            yref = w @ x.astype(np.float64)
            Sref = np.abs(w) @ np.abs(x.astype(np.float64))
            assert np.all(np.abs(y - yref) <= 1e-12 * Sref), f"type {qt} ncols {nc}"
            assert np.allclose(S, Sref, rtol=1e-12)


def check_tolerance_plumbing(within):
    rng = np.random.default_rng(12)
    yref = rng.standard_normal(1000)
    S = np.abs(yref) * 3 + 1.0
    sign = np.where(rng.random(1000) < 0.5, -1.0, 1.0)
    assert within(yref + sign * 0.5e-4 * S, yref, S).all()
    assert not within(yref + sign * 2e-4 * S, yref, S).any()
    z = np.zeros(4)
    assert within(z, z, z).all() and not within(z + 1e-30, z, z).any()


ALL_CHECKS = [
    check_half_exhaustive,
    check_scale_min_single_field,
    check_scale_min_random,
    lambda o: check_quant_planes(o, Q4_K),
    lambda o: check_quant_planes(o, Q5_K),
    lambda o: check_quant_planes(o, Q6_K),
    lambda o: check_quant_planes(o, IQ4_XS),
    check_iq4xs_bit_structure,
    check_iq4xs_scale_single_field,
    check_iq4xs_exact,
    lambda o: check_bit_structure(o, Q4_K),
    lambda o: check_bit_structure(o, Q5_K),
    lambda o: check_bit_structure(o, Q6_K),
    check_q6k_scale_index,
    check_worked_examples,
    check_exact_rounding,
    check_q6k_exact,
    check_q5_q4_invariant,
    check_gemv_integer_textbook,
    check_gemv_min_term,
]
