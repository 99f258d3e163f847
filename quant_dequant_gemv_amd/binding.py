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

Q4_K, Q5_K, Q6_K, IQ4_XS = 12, 13, 14, 23
QK_OK, QK_EINVAL_TYPE, QK_EINVAL_SHAPE, QK_EINVAL_PTR, QK_ELAUNCH, QK_EINVAL_FLAGS = 0, -1, -2, -3, -4, -5
MAX_NCOLS = 32
MAX_BATCH = 16
PLANAR = 0x100  # QK_PLANAR: layout flag OR'ed into a type
Y_F16 = 0x1  # QK_Y_F16: epilogue flag, y stored as fp16

EXPORTS = ("qk_gemv", "qk_gemv_ex", "qk_gemv_swiglu", "qk_gemv_batch", "qk_dequant", "qk_repack",
           "qk_block_bytes", "qk_row_bytes", "qk_strerror", "qk_version",
           "qk_chain_plan_bytes", "qk_chain_plan", "qk_chain_workspace_bytes", "qk_gemv_chain",
           "qk_gemv_chain_noalloc")
CHAIN_TIMEOUT = 0x1  # QK_CHAIN_TIMEOUT: bit of the chain workspace's first word
CHAIN_NOALLOC_MAX_STEPS = 4094  # QK_CHAIN_NOALLOC_MAX_STEPS


class qk_gemv_item(ctypes.Structure):
    """struct qk_gemv_item of include/qkgemv.h."""
    _fields_ = [("type", ctypes.c_int), ("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class qk_chain_entry(ctypes.Structure):
    """struct qk_chain_entry of include/qkgemv.h."""
    _fields_ = [("type", ctypes.c_int), ("flags", ctypes.c_int), ("W", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("residual", ctypes.c_void_p),
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
    lib.qk_chain_plan_bytes.argtypes = [c_int, c_int]
    lib.qk_chain_plan_bytes.restype = i64
    lib.qk_chain_plan.argtypes = [ctypes.POINTER(qk_chain_entry), c_int, ctypes.POINTER(c_int), c_int, P, i64]
    lib.qk_chain_plan.restype = c_int
    lib.qk_chain_workspace_bytes.argtypes = [c_int]
    lib.qk_chain_workspace_bytes.restype = i64
    lib.qk_gemv_chain.argtypes = [P, P, P, i64, i64, P]
    lib.qk_gemv_chain.restype = c_int
    lib.qk_gemv_chain_noalloc.argtypes = [P, P, P, i64, P]
    lib.qk_gemv_chain_noalloc.restype = c_int
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


def qk_chain_plan_bytes(nsteps: int, nentries: int) -> int:
    return load_library().qk_chain_plan_bytes(nsteps, nentries)


def qk_chain_plan(entries, step_sizes, plan) -> int:
    """entries: sequence of qk_chain_entry (or tuples of its fields);
    step_sizes: ints; plan: a writable host buffer (numpy uint8 array)."""
    arr = (qk_chain_entry * max(1, len(entries)))(*[e if isinstance(e, qk_chain_entry) else qk_chain_entry(*e)
                                                     for e in entries])
    sizes = (ctypes.c_int * max(1, len(step_sizes)))(*step_sizes)
    return load_library().qk_chain_plan(arr, len(entries), sizes, len(step_sizes),
                                        ctypes.c_void_p(plan.ctypes.data), int(plan.nbytes))


def qk_chain_workspace_bytes(nsteps: int) -> int:
    return load_library().qk_chain_workspace_bytes(nsteps)


def qk_gemv_chain(plan, plan_dev: int, workspace: int, workspace_bytes: int, timeout_us: int = 0,
                  stream: int = 0) -> int:
    """plan: the host plan (numpy uint8 array)."""
    return load_library().qk_gemv_chain(ctypes.c_void_p(plan.ctypes.data), plan_dev, workspace, workspace_bytes,
                                        timeout_us, stream)


def qk_gemv_chain_noalloc(plan, plan_dev: int, status: int = 0, timeout_us: int = 0, stream: int = 0) -> int:
    """plan: the host plan (numpy uint8 array); status: 0 or a device word."""
    return load_library().qk_gemv_chain_noalloc(ctypes.c_void_p(plan.ctypes.data), plan_dev, status, timeout_us,
                                                stream)


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
# The C ABI cannot see buffer lengths, so these helpers check every tensor
# before anything is enqueued: dtype, contiguity, size against N, K and ncols,
# and that all of them sit on one CUDA device.  (A wrong size or a host tensor
# passed on would make a kernel read or write out of bounds.)  Type and shape
# arguments themselves are checked by the library, which returns its error
# code before launching anything.

def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, name, dtype, numel=None, min_numel=None):
    """Check one tensor argument (sizes before the device, so the checks run
    without a GPU too)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, has {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must have at least {min_numel} elements, has {t.numel()}")


def _same_cuda_device(**tensors):
    devs = {t.device for t in tensors.values() if t is not None}
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA (HIP) device tensor, is on {t.device}")
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(str(d) for d in devs)}")


def _weights(qtype, W, N, K, name="W"):
    """W: uint8, at least N rows of qk_row_bytes(qtype, K) bytes (skipped when
    the library would reject the type or shape itself)."""
    import torch
    rb = qk_row_bytes(qtype, K) if isinstance(qtype, int) else -1
    _need(W, name, torch.uint8, min_numel=N * rb if (rb > 0 and N >= 1) else None)


def _activations(x, K):
    """x: float16 [K'] or [K', ncols] with K' >= K (the kernels read the first
    K rows: a longer buffer is a valid input); returns ncols."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch tensor")
    if x.dim() not in (1, 2) or x.shape[0] < K:
        raise ValueError(f"x must have shape [K] or [K, ncols] with at least K = {K} rows, got {tuple(x.shape)}")
    ncols = 1 if x.dim() == 1 else int(x.shape[1])
    _need(x, "x", torch.float16, min_numel=K * ncols)
    return ncols


def gemv(qtype: int, W, x, N: int, K: int, out=None, stream=None):
    """y = dequant(W) @ x on the GPU.  W: uint8 device tensor of N rows of
    superblocks; x: float16 device tensor [K] or [K, ncols]; returns float32
    [N, ncols] (or writes ``out``, N*ncols float32 elements)."""
    import torch
    _weights(qtype, W, N, K)
    ncols = _activations(x, K)
    if out is None:
        out = torch.empty((max(N, 0), ncols), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, numel=N * ncols)
    _same_cuda_device(W=W, x=x, out=out)
    rc = qk_gemv(qtype, W.data_ptr(), x.data_ptr(), out.data_ptr(), N, K, ncols, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_gemv")
    return out


def _check_out(x, out, f16, N, ncols):
    import torch
    dt = torch.float16 if f16 else torch.float32
    if out is None:
        out = torch.empty((max(N, 0), ncols), dtype=dt, device=x.device)
    _need(out, "out", dt, numel=N * ncols)
    return out


def gemv_ex(qtype: int, W, x, N: int, K: int, residual=None, f16: bool = False, out=None, stream=None):
    """y = residual + dequant(W) @ x, stored as float32 (or float16 with f16).
    residual: None or a float32 device tensor of N*ncols elements (may be
    ``out`` itself for an in-place update of a float32 y)."""
    import torch
    _weights(qtype, W, N, K)
    ncols = _activations(x, K)
    out = _check_out(x, out, f16, N, ncols)
    if residual is not None:
        _need(residual, "residual", torch.float32, numel=N * ncols)
    _same_cuda_device(W=W, x=x, out=out, residual=residual)
    rp = residual.data_ptr() if residual is not None else None
    rc = qk_gemv_ex(qtype, W.data_ptr(), x.data_ptr(), out.data_ptr(), N, K, ncols, rp,
                    Y_F16 if f16 else 0, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_gemv_ex")
    return out


def gemv_swiglu(qtype: int, Wg, Wu, x, N: int, K: int, f16: bool = False, out=None, stream=None):
    """y = silu(dequant(Wg) @ x) * (dequant(Wu) @ x) in one launch."""
    _weights(qtype, Wg, N, K, "Wg")
    _weights(qtype, Wu, N, K, "Wu")
    ncols = _activations(x, K)
    out = _check_out(x, out, f16, N, ncols)
    _same_cuda_device(Wg=Wg, Wu=Wu, x=x, out=out)
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
    for i, e in enumerate(entries):
        qtype, W, x, N, K = e[:5]
        _weights(qtype, W, N, K, f"entries[{i}].W")
        if _activations(x, K) != 1:
            raise ValueError(f"entries[{i}].x must be one column")
        out = e[5] if len(e) > 5 else torch.empty(max(N, 0), dtype=torch.float32, device=x.device)
        _need(out, f"entries[{i}].out", torch.float32, numel=N)
        items.append((qtype, W, x, out, N, K))
        outs.append(out)
    tensors = {}
    for i, (_, W, x, out, _, _) in enumerate(items):
        tensors.update({f"entries[{i}].W": W, f"entries[{i}].x": x, f"entries[{i}].out": out})
    if tensors:
        _same_cuda_device(**tensors)
    items = [(qt, W.data_ptr(), x.data_ptr(), out.data_ptr(), N, K) for qt, W, x, out, N, K in items]
    rc = qk_gemv_batch(items, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_gemv_batch")
    return outs


def dequant(qtype: int, W, N: int, K: int, out=None, stream=None):
    """fp32 [N, K] dequantised weights on the GPU (``out``: N*K float32)."""
    import torch
    _weights(qtype, W, N, K)
    if out is None:
        out = torch.empty((max(N, 0), max(K, 0)), dtype=torch.float32, device=W.device)
    _need(out, "out", torch.float32, numel=N * K)
    _same_cuda_device(W=W, out=out)
    rc = qk_dequant(qtype, W.data_ptr(), out.data_ptr(), N, K, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_dequant")
    return out


def repack(qtype: int, W, N: int, K: int, out=None, stream=None):
    """GGUF rows -> PLANAR rows on the GPU; returns the uint8 device tensor to
    pass with type ``qtype | PLANAR`` (``out``: at least
    N * qk_row_bytes(qtype | PLANAR, K) bytes)."""
    import torch
    _weights(qtype, W, N, K)
    prb = qk_row_bytes(qtype | PLANAR, K) if isinstance(qtype, int) and not (qtype & PLANAR) else -1
    nbytes = N * prb if (prb > 0 and N >= 1) else 0
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=W.device)
    _need(out, "out", torch.uint8, min_numel=nbytes or None)
    _same_cuda_device(W=W, out=out)
    rc = qk_repack(qtype, W.data_ptr(), out.data_ptr(), N, K, _stream_handle(stream))
    if rc != QK_OK:
        raise QKError(rc, "qk_repack")
    return out


class Chain:
    """A planned chain of one-column GEMV steps (qk_chain_plan / qk_gemv_chain).

    steps: list of steps; each step a list of dicts with keys qtype, W, x, y,
    N, K and optionally W2 (SwiGLU up tensor), residual (fp32, may be y) and
    f16 (y stored as fp16).  Every tensor is checked like the other helpers
    check theirs; the plan is uploaded once and the workspace allocated here,
    so run() enqueues the chain and nothing else."""

    def __init__(self, steps):
        import numpy as np
        import torch
        entries, sizes, keep = [], [], []
        for s, step in enumerate(steps):
            if not step:
                raise ValueError(f"step {s} is empty")
            sizes.append(len(step))
            for i, e in enumerate(step):
                qt, W, x, y, N, K = e["qtype"], e["W"], e["x"], e["y"], e["N"], e["K"]
                f16 = bool(e.get("f16", False))
                where = f"steps[{s}][{i}]"
                _weights(qt, W, N, K, where + ".W")
                if e.get("W2") is not None:
                    _weights(qt, e["W2"], N, K, where + ".W2")
                if _activations(x, K) != 1:
                    raise ValueError(f"{where}.x must be one column")
                _need(y, where + ".y", torch.float16 if f16 else torch.float32, numel=N)
                res = e.get("residual")
                if res is not None:
                    _need(res, where + ".residual", torch.float32, numel=N)
                _same_cuda_device(W=W, W2=e.get("W2"), x=x, y=y, residual=res)
                entries.append(qk_chain_entry(qt, Y_F16 if f16 else 0, W.data_ptr(),
                                              e["W2"].data_ptr() if e.get("W2") is not None else None,
                                              x.data_ptr(), y.data_ptr(), res.data_ptr() if res is not None else None,
                                              N, K))
                keep.append(e)
        nbytes = qk_chain_plan_bytes(len(sizes), len(entries))
        if nbytes < 0:
            raise ValueError("bad chain size")
        self.plan = np.zeros(nbytes, dtype=np.uint8)
        rc = qk_chain_plan(entries, sizes, self.plan)
        if rc != QK_OK:
            raise QKError(rc, "qk_chain_plan")
        dev = entries and steps[0][0]["W"].device
        self.plan_dev = torch.from_numpy(self.plan).to(dev)
        self.ws_bytes = qk_chain_workspace_bytes(len(sizes))
        self.workspace = torch.zeros(self.ws_bytes // 4, dtype=torch.int32, device=dev)
        self.nsteps = len(sizes)
        self._keep = keep

    def run(self, stream=None, timeout_us: int = 0):
        rc = qk_gemv_chain(self.plan, self.plan_dev.data_ptr(), self.workspace.data_ptr(), self.ws_bytes,
                           timeout_us, _stream_handle(stream))
        if rc != QK_OK:
            raise QKError(rc, "qk_gemv_chain")

    def status(self) -> int:
        """The workspace's flag word (synchronises): 0, or CHAIN_TIMEOUT."""
        return int(self.workspace[0].item())
