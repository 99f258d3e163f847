"""Helpers for the GPU parity tests (device copies, oracle comparisons)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    torch = None
    HAVE_GPU = False

needs_gpu = pytest.mark.skipif(not HAVE_GPU, reason="no GPU visible")


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_gemv(qt, W: np.ndarray, x: np.ndarray, N: int, K: int):
    from quant_dequant_gemv_amd import binding
    Wd = dev(W.reshape(-1))
    xd = dev(x)
    y = binding.gemv(qt, Wd, xd, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_dequant(qt, W: np.ndarray, N: int, K: int):
    from quant_dequant_gemv_amd import binding
    out = binding.dequant(qt, dev(W.reshape(-1)), N, K)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_row_bound(y_gpu, y_ref, S, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(y_ref.shape)
    ok = oracle.within_row_bound(y_gpu, y_ref, S)
    if not ok.all():
        err = np.abs(y_gpu - y_ref) / np.where(S > 0, S, 1.0)
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside 1e-4*S; worst at {i}: "
                             f"gpu={y_gpu[i]!r} ref={y_ref[i]!r} S={S[i]!r} rel={err[i]:.3e}")
    return float((np.abs(y_gpu - y_ref) / np.where(S > 0, S, 1.0)).max())


def same_f32(a, b) -> bool:
    a = np.asarray(a, dtype=np.float32) + np.float32(0.0)
    b = np.asarray(b, dtype=np.float32) + np.float32(0.0)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))
