"""Test-side PLANAR packer, written from the layout description in
include/qkgemv.h (QK_PLANAR): the same bytes of each GGUF row regrouped into
planes.  Independent of the HIP path; used to check qk_repack byte for byte."""
from __future__ import annotations

import numpy as np

Q4_K, Q5_K, Q6_K = 12, 13, 14
BLOCK = {Q4_K: 144, Q5_K: 176, Q6_K: 210}


def planar_row_bytes(qt: int, K: int) -> int:
    b = (K // 256) * BLOCK[qt]
    return -(-b // 16) * 16 if qt == Q6_K else b


def pack_row(qt: int, row: np.ndarray, K: int) -> np.ndarray:
    """One GGUF row (uint8, S superblocks) -> one PLANAR row."""
    S = K // 256
    sb = row.reshape(S, BLOCK[qt])
    planes = []
    if qt in (Q4_K, Q5_K):
        qs0 = 16 if qt == Q4_K else 48
        planes.append(sb[:, 0:16])                          # H
        if qt == Q5_K:
            planes.append(sb[:, 16:32])                     # QH0
            planes.append(sb[:, 32:48])                     # QH1
        qs = sb[:, qs0:qs0 + 128].reshape(S, 4, 32)         # unit q: qs[32q .. 32q+31]
        planes.append(qs[:, :, :16].reshape(4 * S, 16))     # A
        planes.append(qs[:, :, 16:].reshape(4 * S, 16))     # B
    else:
        A, B, C, SC = [], [], [], []
        for q in range(4):
            n, b = q >> 1, q & 1
            A.append(sb[:, 64 * n + 16 * b:64 * n + 16 * b + 16])
            B.append(sb[:, 64 * n + 32 + 16 * b:64 * n + 48 + 16 * b])
            C.append(sb[:, 128 + 32 * n + 16 * b:128 + 32 * n + 16 * b + 16])
            SC.append(sb[:, [192 + 8 * n + 2 * t + b for t in range(4)]])
        unit = lambda parts: np.stack(parts, axis=1).reshape(4 * S, -1)  # unit u = 4s + q
        planes += [unit(A), unit(B), unit(C), unit(SC), sb[:, 208:210]]
    out = np.concatenate([p.reshape(-1) for p in planes])
    pad = planar_row_bytes(qt, K) - out.size
    return np.concatenate([out, np.zeros(pad, np.uint8)]) if pad else out


def pack(qt: int, W: np.ndarray, K: int) -> np.ndarray:
    """GGUF tensor (N rows, any shape of uint8 with N leading) -> PLANAR bytes [N][row]."""
    rows = W.reshape(W.shape[0], -1)
    return np.stack([pack_row(qt, r, K) for r in rows])
