"""MI355X-native mixed k-quant GEMV: y = dequant(W[N, K]) @ x[K, ncols].

The compute path is the C-ABI library ``libqkgemv.so`` (hand-written HIP
kernels for gfx950, declared in ``include/qkgemv.h``).  ``binding`` is a thin
ctypes layer over it with the same function names; PyTorch supplies device
memory and streams only.  ``synth`` generates seeded synthetic superblocks.

The binding is imported lazily so that ``synth`` can be used on machines
without a GPU; calling any compute entry point without the built library
raises instead of falling back to anything else.
"""
from __future__ import annotations

Q4_K, Q5_K, Q6_K = 12, 13, 14

_BINDING_NAMES = {
    "qk_gemv", "qk_dequant", "qk_block_bytes", "qk_row_bytes", "qk_strerror", "qk_version",
    "gemv", "dequant", "load_library", "QKError", "LIB_PATH",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
