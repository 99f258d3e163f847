"""Seeded synthetic inputs for the k-quant GEMV: superblock bytes and fp16 x.

This module is shared by the tests, the benchmark and the smoke check; it holds
none of the method's arithmetic (no unpacking, no dequantisation, no dot).  It
only knows where the fp16 ``d``/``dmin`` headers and the Q6_K int8 scales sit
in each superblock, so it can overwrite them with values from the stated
distributions.

Recipe (the real GGUF weights of the pages are not available; these stand in
for them at the same shapes):

* every byte of every superblock is drawn uniform over 0..255, which makes every
  6-bit scale/min, every 4/5/6-bit quant and every high-bit plane uniform over
  its full range (each field is a bijection of its bits);
* ``d`` and ``dmin`` are then overwritten with ``fp16(2**u)``, ``u ~ U[-12, -6)``
  (log-uniform in [2^-12, 2^-6]); Q6_K has ``d`` only;
* Q6_K ``scales[16]`` are overwritten with int8 values uniform over -32..31;
* IQ4_XS keeps its random 6-bit sub-block scales and 4-bit codebook indices
  (uniform over their ranges) and gets ``d`` as above;
* x is ``fp16(N(0, 1))`` of shape ``[K, ncols]`` (row-major).

Streams: weights of a tensor come from ``default_rng([seed, 0])`` and x from
``default_rng([seed, 1, ncols])`` (numpy PCG64 seeded through SeedSequence),
so a weight tensor does not change when x is redrawn for another column count.
"""
from __future__ import annotations

import numpy as np

Q4_K, Q5_K, Q6_K, IQ4_XS = 12, 13, 14, 23
TYPE_NAMES = {Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K", IQ4_XS: "IQ4_XS"}
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210, IQ4_XS: 136}
QK = 256

# Byte offsets of the fp16 scale headers and of the Q6_K int8 scales.
_D_OFFSET = {Q4_K: 0, Q5_K: 0, Q6_K: 208, IQ4_XS: 0}
_DMIN_OFFSET = {Q4_K: 2, Q5_K: 2}
_Q6_SCALES = (192, 208)


def row_bytes(qtype: int, K: int) -> int:
    return (K // QK) * BLOCK_BYTES[qtype]


def log_uniform_fp16(rng: np.random.Generator, n: int, lo: float = -12.0, hi: float = -6.0) -> np.ndarray:
    """n fp16 values 2**u, u ~ U[lo, hi), as uint16 bit patterns."""
    return np.exp2(rng.uniform(lo, hi, size=n)).astype(np.float16).view(np.uint16)


def superblocks(qtype: int, N: int, K: int, seed: int) -> np.ndarray:
    """uint8 [N, row_bytes] of random superblocks (row-major W[N][K/256])."""
    if qtype not in BLOCK_BYTES:
        raise ValueError(f"unknown k-quant type {qtype}")
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    bb = BLOCK_BYTES[qtype]
    nsb = N * (K // QK)
    rng = np.random.default_rng([seed, 0])
    raw = np.frombuffer(rng.bytes(nsb * bb), dtype=np.uint8).copy().reshape(nsb, bb)
    d = log_uniform_fp16(rng, nsb)
    o = _D_OFFSET[qtype]
    raw[:, o:o + 2] = d.view(np.uint8).reshape(nsb, 2)
    if qtype in _DMIN_OFFSET:
        dmin = log_uniform_fp16(rng, nsb)
        o = _DMIN_OFFSET[qtype]
        raw[:, o:o + 2] = dmin.view(np.uint8).reshape(nsb, 2)
    elif qtype == Q6_K:
        a, b = _Q6_SCALES
        raw[:, a:b] = rng.integers(-32, 32, size=(nsb, b - a), dtype=np.int8).view(np.uint8)
    return raw.reshape(N, (K // QK) * bb)


def activations(K: int, ncols: int, seed: int) -> np.ndarray:
    """fp16 [K, ncols], N(0, 1)."""
    rng = np.random.default_rng([seed, 1, ncols])
    return rng.standard_normal((K, ncols)).astype(np.float16)


# ---------------------------------------------------------------------------
# The workloads: the shapes of a 64-layer hybrid Gated-DeltaNet / GQA decoder
# at hidden size 5120 and FFN size 17408 (GGUF arch qwen35).
# ---------------------------------------------------------------------------

HIDDEN, FFN = 5120, 17408

#: the small correctness case: Q4_K, N=1024, K=5120
SMALL = dict(qtype=Q4_K, N=1024, K=5120, seed=0)

#: Q4_K projections at K=5120: fused DeltaNet QKV, attention Q, FFN gate/up
Q4K_PROJECTIONS = [
    dict(name="attn_qkv", qtype=Q4_K, N=10240, K=5120, seed=1),
    dict(name="attn_q", qtype=Q4_K, N=12288, K=5120, seed=2),
    dict(name="ffn_up", qtype=Q4_K, N=17408, K=5120, seed=3),
]

#: mixed types: Q6_K FFN down and Q5_K output projection
MIXED = [
    dict(name="ffn_down", qtype=Q6_K, N=5120, K=17408, seed=4),
    dict(name="ssm_out", qtype=Q5_K, N=5120, K=6144, seed=5),
]

#: few-column verify: Q4_K 17408 x 5120 against x[K, ncols]
VERIFY = dict(qtype=Q4_K, N=17408, K=5120, seed=6, ncols=(1, 2, 4, 8))

N_LAYERS = 64


def is_attention_layer(layer: int) -> bool:
    """Full GQA attention every 4th layer (3, 7, ..., 63); DeltaNet otherwise."""
    return layer % 4 == 3


def decode_stream(n_layers: int = N_LAYERS):
    """The per-token GEMV list of the decoder, in execution order.

    Each entry: dict(layer, name, qtype, N, K, seed) with seed
    1000 + 16*layer + t, t the position within the layer."""
    out = []
    for layer in range(n_layers):
        if is_attention_layer(layer):
            mix = [("attn_q", Q4_K, 12288, HIDDEN), ("attn_k", Q4_K, 1024, HIDDEN),
                   ("attn_v", Q4_K, 1024, HIDDEN), ("attn_output", Q5_K, HIDDEN, 6144)]
        else:
            mix = [("attn_qkv", Q4_K, 10240, HIDDEN), ("ssm_alpha", Q6_K, 48, HIDDEN),
                   ("ssm_beta", Q6_K, 48, HIDDEN), ("ssm_out", Q5_K, HIDDEN, 6144)]
        mix += [("ffn_gate", Q4_K, FFN, HIDDEN), ("ffn_up", Q4_K, FFN, HIDDEN),
                ("ffn_down", Q6_K, HIDDEN, FFN)]
        for t, (name, qt, n, k) in enumerate(mix):
            out.append(dict(layer=layer, name=name, qtype=qt, N=n, K=k, seed=1000 + 16 * layer + t))
    return out


# Projections of one layer that read the same activations (the layer input,
# the mixer output, the FFN input, the FFN hidden state) and so may share one
# launch; entries of a group are adjacent in decode_stream order.
X_GROUP = {"attn_qkv": "in", "ssm_alpha": "in", "ssm_beta": "in", "attn_q": "in", "attn_k": "in", "attn_v": "in",
           "ssm_out": "mix", "attn_output": "mix", "ffn_gate": "ffn_in", "ffn_up": "ffn_in", "ffn_down": "ffn_mid"}


def decode_groups(entries):
    """Index lists of the adjacent entries that share a layer and an input."""
    groups = []
    for i, e in enumerate(entries):
        key = (e["layer"], X_GROUP[e["name"]])
        if groups and groups[-1][0] == key:
            groups[-1][1].append(i)
        else:
            groups.append((key, [i]))
    return [idx for _, idx in groups]


def weight_bytes(entries) -> int:
    return sum(e["N"] * row_bytes(e["qtype"], e["K"]) for e in entries)
