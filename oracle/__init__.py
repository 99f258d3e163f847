"""CPU oracle for the k-quant dequantisation and GEMV -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import, call or link it, and it imports nothing from them.

The arithmetic lives in ``qk_oracle.c`` (plain scalar C, built with
``-ffp-contract=off``); this module only builds and marshals.  What it computes,
and from which passage of the pages, is written at the top of that file:

* ``dequant``  -- fp32 weights, ``w = d*(sc*q) - dmin*m`` (Q4_K/Q5_K),
  ``w = d*sc*(q-32)`` (Q6_K) or ``w = d*(ls-32)*kv[idx]`` (IQ4_XS), one
  rounding at most;
* ``gemv``     -- the f64 reference ``y = sum_k w*x`` in ascending k, plus
  ``S = sum_k |w*x|`` for the per-row tolerance;
* ``half_to_float``, ``k_scale_min``, ``quant``, ``q6k_scale``,
  ``iq4xs_scale``, ``iq4nl_value`` -- the field readers, exposed so the tests
  can pin each one on its own;
* ``silu``, ``gemv_residual``, ``swiglu`` -- the fused epilogues, in f64 numpy
  on top of ``gemv``; ``residual_bound`` / ``swiglu_bound``, the tolerances
  that the row bound 1e-4 * sum|w*x| implies for them, and ``within``, the
  acceptance test (with the fp16 overflow rule).

Every function is pinned by ``tests/test_oracle_pins.py`` or
``tests/test_oracle_epilogue.py``; none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q4_K, Q5_K, Q6_K, IQ4_XS = 12, 13, 14, 23

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qk_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared", "-pthread"]


def compile_oracle(src: str = SOURCE, out: str = LIB_PATH, extra_flags=()) -> str:
    """gcc-compile an oracle source into a shared library (always recompiles)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, *extra_flags, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    return compile_oracle()


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """ctypes handle on one build of qk_oracle.c."""

    def __init__(self, path: str = LIB_PATH):
        lib = ctypes.CDLL(path)
        P, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "oracle_block_bytes": ([c_int], c_int),
            "oracle_half_to_float": ([ctypes.c_uint16], ctypes.c_float),
            "oracle_half_to_float_n": ([P, P, i64], None),
            "oracle_k_scale_min": ([P, c_int, P, P], None),
            "oracle_quant": ([c_int, P, c_int], c_int),
            "oracle_q6k_scale": ([P, c_int], c_int),
            "oracle_iq4xs_scale": ([P, c_int], c_int),
            "oracle_iq4nl_value": ([c_int], c_int),
            "oracle_dequant": ([c_int, P, i64, i64, P, c_int], c_int),
            "oracle_gemv": ([c_int, P, P, i64, i64, c_int, P, P, c_int], c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes, f.restype = args, res
        self.lib = lib
        self.path = path

    def block_bytes(self, qtype: int) -> int:
        return self.lib.oracle_block_bytes(int(qtype))

    def half_to_float(self, bits) -> np.ndarray:
        """Widen uint16 fp16 bit patterns to float32 (exact)."""
        b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
        out = np.empty(b.shape, dtype=np.float32)
        self.lib.oracle_half_to_float_n(_ptr(b), _ptr(out), b.size)
        return out

    def k_scale_min(self, scales12, j: int):
        """(sc, m) of sub-block j from the 12-byte Q4_K/Q5_K scales field."""
        s = np.ascontiguousarray(np.asarray(scales12, dtype=np.uint8))
        if s.size != 12:
            raise ValueError("scales field is 12 bytes")
        sc, m = ctypes.c_int(), ctypes.c_int()
        self.lib.oracle_k_scale_min(_ptr(s), int(j), ctypes.byref(sc), ctypes.byref(m))
        return sc.value, m.value

    def quant(self, qtype: int, block, i: int) -> int:
        """Integer quant of weight i in one superblock (Q6_K: before the -32)."""
        b = np.ascontiguousarray(np.asarray(block, dtype=np.uint8))
        return self.lib.oracle_quant(int(qtype), _ptr(b), int(i))

    def q6k_scale(self, block, i: int) -> int:
        b = np.ascontiguousarray(np.asarray(block, dtype=np.uint8))
        return self.lib.oracle_q6k_scale(_ptr(b), int(i))

    def iq4xs_scale(self, block, ib: int) -> int:
        """6-bit scale ls of sub-block ib of an IQ4_XS superblock (the weight
        factor is ls - 32)."""
        b = np.ascontiguousarray(np.asarray(block, dtype=np.uint8))
        return self.lib.oracle_iq4xs_scale(_ptr(b), int(ib))

    def iq4nl_value(self, idx: int) -> int:
        """Codebook value of a 4-bit IQ4_XS index."""
        return self.lib.oracle_iq4nl_value(int(idx))

    def _rows(self, W, qtype: int, K: int) -> np.ndarray:
        bb = self.block_bytes(qtype)
        if bb < 0:
            raise ValueError(f"unknown k-quant type {qtype}")
        if K % 256:
            raise ValueError("K must be a multiple of 256")
        W = np.ascontiguousarray(np.asarray(W, dtype=np.uint8))
        return W.reshape(-1, (K // 256) * bb)

    def dequant(self, qtype: int, W, K: int, nthreads: int | None = None) -> np.ndarray:
        """fp32 [N, K] dequantised weights of the superblock rows in W."""
        Wr = self._rows(W, qtype, K)
        N = Wr.shape[0]
        out = np.empty((N, K), dtype=np.float32)
        rc = self.lib.oracle_dequant(int(qtype), _ptr(Wr), N, K, _ptr(out),
                                     nthreads or default_threads())
        if rc:
            raise RuntimeError(f"oracle_dequant failed: {rc}")
        return out

    def gemv(self, qtype: int, W, x, K: int, nthreads: int | None = None):
        """(y, S), both f64 [N, ncols].  x is fp16 [K] or [K, ncols]."""
        Wr = self._rows(W, qtype, K)
        N = Wr.shape[0]
        x = np.asarray(x)
        if x.dtype != np.float16:
            raise TypeError("x must be float16")
        x2 = np.ascontiguousarray(x.reshape(K, -1))
        ncols = x2.shape[1]
        y = np.empty((N, ncols), dtype=np.float64)
        S = np.empty((N, ncols), dtype=np.float64)
        rc = self.lib.oracle_gemv(int(qtype), _ptr(Wr), _ptr(x2.view(np.uint16)), N, K, ncols,
                                  _ptr(y), _ptr(S), nthreads or default_threads())
        if rc:
            raise RuntimeError(f"oracle_gemv failed: {rc}")
        return y, S


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from this directory (compiled on first use if absent or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def block_bytes(qtype):
    return load().block_bytes(qtype)


def half_to_float(bits):
    return load().half_to_float(bits)


def k_scale_min(scales12, j):
    return load().k_scale_min(scales12, j)


def quant(qtype, block, i):
    return load().quant(qtype, block, i)


def q6k_scale(block, i):
    return load().q6k_scale(block, i)


def iq4xs_scale(block, ib):
    return load().iq4xs_scale(block, ib)


def iq4nl_value(idx):
    return load().iq4nl_value(idx)


def dequant(qtype, W, K, nthreads=None):
    return load().dequant(qtype, W, K, nthreads)


def gemv(qtype, W, x, K, nthreads=None):
    return load().gemv(qtype, W, x, K, nthreads)


def within_row_bound(y_test, y_ref, S, rel: float = 1e-4) -> np.ndarray:
    """Acceptance of a GEMV result: |y_test - y_ref| <= rel * S, elementwise.

    Where S == 0 every product is zero, so y_test must be exactly zero."""
    y_test = np.asarray(y_test, dtype=np.float64)
    err = np.abs(y_test - np.asarray(y_ref, dtype=np.float64))
    return err <= rel * np.asarray(S, dtype=np.float64)


# ---------------------------------------------------------------- epilogues
# The B70 plan ("Qwen3.6 27B Single-B70 Maximum-Speed Requirements And
# Execution Plan", "Phase 3: Maximum Useful Fusion") fuses into the weight
# streaming pass a residual add after the output projections (family 1) and
# the SiLU gate times the up projection (family 3).  Their definitions, in
# f64 on the f64 GEMV above:

def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)) in f64 (-0 for z -> -inf)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gemv_residual(qtype, W, x, K, residual, nthreads=None):
    """(y, S): y = residual + dequant(W) @ x in f64, S = sum_k |w*x| as in gemv."""
    y, S = gemv(qtype, W, x, K, nthreads)
    r = np.asarray(residual, dtype=np.float64).reshape(y.shape)
    return y + r, S


def swiglu(qtype, Wg, Wu, x, K, nthreads=None):
    """(y, g, Sg, u, Su): y = silu(g) * u with g = dequant(Wg) @ x and
    u = dequant(Wu) @ x, all f64."""
    g, Sg = gemv(qtype, Wg, x, K, nthreads)
    u, Su = gemv(qtype, Wu, x, K, nthreads)
    return silu(g) * u, g, Sg, u, Su


# Largest |silu'(z)| over the reals: silu'(z) = s(z) (1 + z (1 - s(z))),
# s = sigmoid; its maximum is about 1.0998 (near z = 2.4).
SILU_SLOPE = 1.1


def _f16_rounding(y_ref, err):
    """Half an fp16 ulp of a value within err of y_ref, plus half the
    smallest subnormal."""
    return 2.0 ** -11 * (np.abs(y_ref) + err) + 2.0 ** -25


# Round to nearest even takes an fp32 value to fp16 infinity from
# 65504 + half an ulp (16) on: |v| >= 65520.
F16_OVERFLOW = 65520.0


def within(y_test, y_ref, tol, f16=False) -> np.ndarray:
    """Acceptance of an epilogue result: |y_test - y_ref| <= tol elementwise;
    for an fp16 y also the infinity of y_ref's sign wherever a value within
    tol of y_ref would round past the fp16 range."""
    y = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        ok = np.abs(y - y_ref) <= tol
    if f16:
        ok |= np.isinf(y) & (np.sign(y) == np.sign(y_ref)) & (np.abs(y_ref) + tol >= F16_OVERFLOW)
    return ok


def residual_bound(y_ref, S, f16=False, rel=1e-4):
    """Tolerance of y = residual + W x: the GEMV's rel*S, the fp32 rounding of
    the add (2^-24 |y|, with |y| <= |y_ref| + rel*S), and with f16 the fp16
    rounding of the stored value."""
    y_ref = np.abs(np.asarray(y_ref, dtype=np.float64))
    e = rel * np.asarray(S, dtype=np.float64)
    e = e + 2.0 ** -24 * (y_ref + e)
    return e + _f16_rounding(y_ref, e) if f16 else e


def swiglu_bound(y_ref, g, Sg, u, Su, f16=False, rel=1e-4):
    """Tolerance of y = silu(g) * u when g and u are each within rel*S of
    their exact values: with eg, eu those errors and |silu'| <= SILU_SLOPE,
    |silu(g+eg)(u+eu) - silu(g)u| <= SILU_SLOPE |eg| (|u| + |eu|) + |silu(g)| |eu|;
    plus 2^-20 |y| for the fp32 evaluation (expf, the add, the quotient, the
    product: a few ulps) and with f16 the fp16 rounding."""
    eg = rel * np.asarray(Sg, dtype=np.float64)
    eu = rel * np.asarray(Su, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    u = np.abs(np.asarray(u, dtype=np.float64))
    y_ref = np.abs(np.asarray(y_ref, dtype=np.float64))
    e = SILU_SLOPE * eg * (u + eu) + np.abs(silu(g)) * eu
    e = e + 2.0 ** -20 * (y_ref + e)
    return e + _f16_rounding(y_ref, e) if f16 else e
