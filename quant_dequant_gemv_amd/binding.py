"""ctypes binding of libqkgemv.so (declared in include/qkgemv.h).

Argument marshalling only: every step of the GEMV runs in the library's HIP
kernels.  The raw entry points keep the C names and take integer device
addresses; ``gemv`` / ``dequant`` accept torch tensors and pass their data
pointers and the current HIP stream.  If the library is not built, every call
raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqkgemv.so")

Q4_K, Q5_K, Q6_K = 12, 13, 14
QK_OK, QK_EINVAL_TYPE, QK_EINVAL_SHAPE, QK_EINVAL_PTR, QK_ELAUNCH, QK_EINVAL_FLAGS = 0, -1, -2, -3, -4, -5
MAX_NCOLS = 32
MAX_BATCH = 16
PLANAR = 0x100  # QK_PLANAR: layout flag OR'ed into a type
Y_F16 = 0x1  # QK_Y_F16: epilogue flag, y stored as fp16

EXPORTS = ("qk_gemv", "qk_gemv_ex", "qk_gemv_swiglu", "qk_gemv_batch", "qk_dequant", "qk_repack",
           "qk_block_bytes", "qk_row_bytes", "qk_strerror", "qk_version")


class qk_gemv_item(ctypes.Structure):
    """struct qk_gemv_item of include/qkgemv.h."""
    _fields_ = [("type", ctypes.c_int), ("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class QKError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {qk_strerror(code)} (code {code})")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libqkgemv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run quant_dequant_gemv_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    P, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.qk_gemv.argtypes = [c_int, P, P, P, i64, i64, c_int, P]
    lib.qk_gemv.restype = c_int
    lib.qk_gemv_ex.argtypes = [c_int, P, P, P, i64, i64, c_int, P, c_int, P]
    lib.qk_gemv_ex.restype = c_int
    lib.qk_gemv_swiglu.argtypes = [c_int, P, P, P, P, i64, i64, c_int, c_int, P]
    lib.qk_gemv_swiglu.restype = c_int
    lib.qk_gemv_batch.argtypes = [ctypes.POINTER(qk_gemv_item), c_int, P]
    lib.qk_gemv_batch.restype = c_int
    lib.qk_dequant.argtypes = [c_int, P, P, i64, i64, P]
    lib.qk_dequant.restype = c_int
    lib.qk_repack.argtypes = [c_int, P, P, i64, i64, P]
    lib.qk_repack.restype = c_int
    lib.qk_block_bytes.argtypes = [c_int]
    lib.qk_block_bytes.restype = c_int
    lib.qk_row_bytes.argtypes = [c_int, i64]
    lib.qk_row_bytes.restype = i64
    lib.qk_strerror.argtypes = [c_int]
    lib.qk_strerror.restype = ctypes.c_char_p
    lib.qk_version.argtypes = []
    lib.qk_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------- raw C names

def qk_gemv(qtype: int, W: int, x: int, y: int, N: int, K: int, ncols: int, stream: int = 0) -> int:
    return load_library().qk_gemv(qtype, W, x, y, N, K, ncols, stream)


def qk_gemv_ex(qtype: int, W: int, x: int, y: int, N: int, K: int, ncols: int, residual, flags: int,
               stream: int = 0) -> int:
    return load_library().qk_gemv_ex(qtype, W, x, y, N, K, ncols, residual, flags, stream)


def qk_gemv_swiglu(qtype: int, Wg: int, Wu: int, x: int, y: int, N: int, K: int, ncols: int, flags: int,
                   stream: int = 0) -> int:
    return load_library().qk_gemv_swiglu(qtype, Wg, Wu, x, y, N, K, ncols, flags, stream)


def qk_gemv_batch(items, stream: int = 0) -> int:
    """items: sequence of (type, W, x, y, N, K) with integer device addresses."""
    arr = (qk_gemv_item * max(1, len(items)))(*[qk_gemv_item(*it) for it in items])
    return load_library().qk_gemv_batch(arr, len(items), stream)


def qk_dequant(qtype: int, W: int, out: int, N: int, K: int, stream: int = 0) -> int:
    return load_library().qk_dequant(qtype, W, out, N, K, stream)


def qk_repack(qtype: int, W: int, Wp: int, N: int, K: int, stream: int = 0) -> int:
    return load_library().qk_repack(qtype, W, Wp, N, K, stream)


def qk_block_bytes(qtype: int) -> int:
    return load_library().qk_block_bytes(qtype)


def qk_row_bytes(qtype: int, K: int) -> int:
    return load_library().qk_row_bytes(qtype, K)


def qk_strerror(code: int) -> str:
    return load_library().qk_strerror(code).decode()


def qk_version() -> str:
    return load_library().qk_version().decode()


# ---------------------------------------------------------------- torch helpers

def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def gemv(qtype: int, W, x, N: int, K: int, out=None, stream=None):
    """y = dequant(W) @ x on the GPU.  W: uint8 device tensor of N rows of
    superblocks; x: float16 device tensor [K] or [K, ncols]; returns float32
    [N, ncols] (or writes ``out``)."""
    import torch
    ncols = 1 if x.dim() == 1 else int(x.shape[1])
    if out is None:
        out = torch.empty((N, ncols), dtype=torch.float32, device=x.device)
    if x.dtype != torch.float16 or out.dtype != torch.float32 or W.dtype != torch.uint8:
        raise TypeError("W must be uint8, x float16, out float32")
    if not (W.is_contiguous() and x.is_contiguous() and out.is_contiguous()):
        raise ValueError("tensors must be contiguous")
    rc = qk_gemv(qtype, W.data_ptr(), x.data_ptr(), out.data_ptr(), N, K, ncols, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_gemv")
    return out


def _check_out(x, out, f16, N, ncols):
    import torch
    dt = torch.float16 if f16 else torch.float32
    if out is None:
        out = torch.empty((N, ncols), dtype=dt, device=x.device)
    if out.dtype != dt or not out.is_contiguous() or out.numel() != N * ncols:
        raise ValueError(f"out must be a contiguous {dt} tensor of N*ncols elements")
    return out


def gemv_ex(qtype: int, W, x, N: int, K: int, residual=None, f16: bool = False, out=None, stream=None):
    """y = residual + dequant(W) @ x, stored as float32 (or float16 with f16).
    residual: None or a float32 device tensor of N*ncols elements (may be
    ``out`` itself for an in-place update of a float32 y)."""
    import torch
    ncols = 1 if x.dim() == 1 else int(x.shape[1])
    if x.dtype != torch.float16 or W.dtype != torch.uint8 or not (W.is_contiguous() and x.is_contiguous()):
        raise TypeError("W must be contiguous uint8, x contiguous float16")
    out = _check_out(x, out, f16, N, ncols)
    rp = 0
    if residual is not None:
        if residual.dtype != torch.float32 or not residual.is_contiguous() or residual.numel() != N * ncols:
            raise ValueError("residual must be a contiguous float32 tensor of N*ncols elements")
        rp = residual.data_ptr()
    rc = qk_gemv_ex(qtype, W.data_ptr(), x.data_ptr(), out.data_ptr(), N, K, ncols, rp or None,
                    Y_F16 if f16 else 0, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_gemv_ex")
    return out


def gemv_swiglu(qtype: int, Wg, Wu, x, N: int, K: int, f16: bool = False, out=None, stream=None):
    """y = silu(dequant(Wg) @ x) * (dequant(Wu) @ x) in one launch."""
    import torch
    ncols = 1 if x.dim() == 1 else int(x.shape[1])
    for W in (Wg, Wu):
        if W.dtype != torch.uint8 or not W.is_contiguous():
            raise TypeError("Wg and Wu must be contiguous uint8")
    if x.dtype != torch.float16 or not x.is_contiguous():
        raise TypeError("x must be contiguous float16")
    out = _check_out(x, out, f16, N, ncols)
    rc = qk_gemv_swiglu(qtype, Wg.data_ptr(), Wu.data_ptr(), x.data_ptr(), out.data_ptr(), N, K, ncols,
                        Y_F16 if f16 else 0, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_gemv_swiglu")
    return out


def gemv_batch(entries, stream=None):
    """Independent one-column GEMVs in one launch.  entries: sequence of
    (qtype, W, x, N, K) or (qtype, W, x, N, K, out) with torch device tensors
    (W uint8, x float16 [K], out float32 [N]); returns the list of outputs."""
    import torch
    items, outs = [], []
    for e in entries:
        qtype, W, x, N, K = e[:5]
        out = e[5] if len(e) > 5 else torch.empty(N, dtype=torch.float32, device=x.device)
        if x.dtype != torch.float16 or out.dtype != torch.float32 or W.dtype != torch.uint8:
            raise TypeError("W must be uint8, x float16, out float32")
        if not (W.is_contiguous() and x.is_contiguous() and out.is_contiguous()):
            raise ValueError("tensors must be contiguous")
        items.append((qtype, W.data_ptr(), x.data_ptr(), out.data_ptr(), N, K))
        outs.append(out)
    rc = qk_gemv_batch(items, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_gemv_batch")
    return outs


def dequant(qtype: int, W, N: int, K: int, out=None, stream=None):
    """fp32 [N, K] dequantised weights on the GPU."""
    import torch
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=W.device)
    rc = qk_dequant(qtype, W.data_ptr(), out.data_ptr(), N, K, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_dequant")
    return out


def repack(qtype: int, W, N: int, K: int, out=None, stream=None):
    """GGUF rows -> PLANAR rows on the GPU; returns the uint8 device tensor to
    pass with type ``qtype | PLANAR``."""
    import torch
    nbytes = N * qk_row_bytes(qtype | PLANAR, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    rc = qk_repack(qtype, W.data_ptr(), out.data_ptr(), N, K, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_repack")
    return out
