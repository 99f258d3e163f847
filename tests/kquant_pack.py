"""Test-side superblock PACKERS: field values -> bytes.

These write the GGML k-quant layout in the packing direction (the oracle only
ever reads it), one field at a time, so a round trip through the oracle's
readers checks both against the layout tables independently.

Layout (GGML k-quant, the reference named by the "Mixed-Quant GEMV" prompt of
the T4 dossier, section SPEC; the Q4_K struct itself is in the dossier's design
prompt, section QUANTIZATION MIX):

* Q4_K 144 B: d fp16 @0, dmin fp16 @2, scales[12] @4, qs[128] @16
* Q5_K 176 B: d @0, dmin @2, scales[12] @4, qh[32] @16, qs[128] @48
* Q6_K 210 B: ql[128] @0, qh[64] @128, scales[16] int8 @192, d fp16 @208
* IQ4_XS 136 B: d fp16 @0, scales_h u16 @2, scales_l[4] @4, qs[128] @8 (GGML's
  block_iq4_xs: the kernel prompt's SPEC asks for IQ4_XS beside Q4_K/Q5_K and
  names GGML's dequantisation as the reference)
"""
from __future__ import annotations

import numpy as np

Q4_K, Q5_K, Q6_K, IQ4_XS = 12, 13, 14, 23
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210, IQ4_XS: 136}
QS_OFFSET = {Q4_K: 16, Q5_K: 48}


def pack_k_scales(sc, m) -> np.ndarray:
    """12-byte scales field from eight 6-bit scales and eight 6-bit mins.

    sc_0..3 / m_0..3 go to the low 6 bits of bytes 0..3 / 4..7; sc_4..7 / m_4..7
    are split: low nibble into bytes 8..11 (sc low half, m high half), bits 4..5
    into the top two bits of bytes 0..3 (sc) / 4..7 (m)."""
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    assert len(sc) == 8 and len(m) == 8 and all(0 <= v < 64 for v in sc + m)
    out = [0] * 12
    for j in range(4):
        out[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        out[j + 4] = m[j] | ((m[j + 4] >> 4) << 6)
        out[j + 8] = (sc[j + 4] & 0xF) | ((m[j + 4] & 0xF) << 4)
    return np.array(out, dtype=np.uint8)


def put_quant(qtype: int, block: np.ndarray, i: int, v: int) -> None:
    """OR quant value v of weight i into a block whose quant planes start at zero."""
    l = i % 32
    if qtype in (Q4_K, Q5_K):
        assert 0 <= v < (16 if qtype == Q4_K else 32)
        c, h, j = i // 64, (i // 32) % 2, i // 32
        qs = QS_OFFSET[qtype]
        block[qs + 32 * c + l] |= (v & 0xF) << (4 * h)
        if qtype == Q5_K:
            block[16 + l] |= (v >> 4) << j
    elif qtype == Q6_K:
        assert 0 <= v < 64
        n, t = i // 128, (i % 128) // 32
        block[64 * n + 32 * (t % 2) + l] |= (v & 0xF) << (4 * (t // 2))
        block[128 + 32 * n + l] |= (v >> 4) << (2 * t)
    elif qtype == IQ4_XS:
        # sub-block ib = i // 32: its first 16 weights in the low nibbles of
        # qs[16 ib ..], the next 16 in the high nibbles of the same bytes
        assert 0 <= v < 16
        block[8 + 16 * (i // 32) + l % 16] |= v << (4 * (l // 16))
    else:
        raise ValueError(qtype)


def half_bits(value: float) -> int:
    return int(np.array(value, dtype=np.float16).view(np.uint16))


def make_k_block(qtype: int, d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    """Q4_K or Q5_K superblock from its fields (d, dmin as fp16 bit patterns)."""
    b = np.zeros(BLOCK_BYTES[qtype], dtype=np.uint8)
    b[0], b[1] = d_bits & 0xFF, d_bits >> 8
    b[2], b[3] = dmin_bits & 0xFF, dmin_bits >> 8
    b[4:16] = pack_k_scales(sc, m)
    for i in range(256):
        put_quant(qtype, b, i, int(q[i]))
    return b


def make_q6_block(d_bits: int, scales, q) -> np.ndarray:
    """Q6_K superblock from its fields (q before the -32 offset)."""
    b = np.zeros(210, dtype=np.uint8)
    for i in range(256):
        put_quant(Q6_K, b, i, int(q[i]))
    b[192:208] = np.asarray(scales, dtype=np.int8).view(np.uint8)
    b[208], b[209] = d_bits & 0xFF, d_bits >> 8
    return b


def make_iq4xs_block(d_bits: int, ls, idx) -> np.ndarray:
    """IQ4_XS superblock from d (fp16 bits), eight 6-bit sub-block scales ls
    (the weight factor is ls - 32) and 256 4-bit codebook indices.  Low nibble
    of ls_ib into scales_l[ib // 2] (low half for even ib), its top 2 bits into
    bits 2 ib, 2 ib + 1 of the little-endian scales_h."""
    ls = [int(v) for v in ls]
    assert len(ls) == 8 and all(0 <= v < 64 for v in ls)
    b = np.zeros(136, dtype=np.uint8)
    b[0], b[1] = d_bits & 0xFF, d_bits >> 8
    h = 0
    for ib, v in enumerate(ls):
        b[4 + ib // 2] |= (v & 0xF) << (4 * (ib % 2))
        h |= (v >> 4) << (2 * ib)
    b[2], b[3] = h & 0xFF, h >> 8
    for i in range(256):
        put_quant(IQ4_XS, b, i, int(idx[i]))
    return b


def quant_region(qtype: int):
    """(start, end) byte range of all quant bits of a superblock."""
    return {Q4_K: (16, 144), Q5_K: (16, 176), Q6_K: (0, 192), IQ4_XS: (8, 136)}[qtype]


def load_golden(path: str):
    """Parse a tests/golden/*.txt worked example: (type, form, bytes, {i: value})."""
    qt = form = None
    hexbytes: list[int] = []
    values: dict[int, float] = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "type":
            qt = {"Q4_K": Q4_K, "Q5_K": Q5_K, "Q6_K": Q6_K, "IQ4_XS": IQ4_XS}[rest.strip()]
        elif key == "form":
            form = rest.strip()
        elif key == "hex":
            hexbytes += [int(t, 16) for t in rest.split()]
        elif key == "value":
            i, v = rest.split()
            values[int(i)] = float(v)
    return qt, form, np.array(hexbytes, dtype=np.uint8), values
