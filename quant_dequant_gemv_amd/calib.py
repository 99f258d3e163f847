"""ctypes handle on libqkcalib.so, the plain-read reference kernels that the
benchmark (read ceilings) and the traffic counters (byte calibration) use.
Not part of the GEMV library."""
import ctypes

_lib = None


def load():
    global _lib
    if _lib is None:
        from quant_dequant_gemv_amd import build as qb
        lib = ctypes.CDLL(qb.CALIB_LIB)
        for name in ("qk_stream_read", "qk_stream_read_plain"):
            f = getattr(lib, name)
            f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                          ctypes.c_void_p]
            f.restype = ctypes.c_int
        _lib = lib
    return _lib
