"""Build libqkgemv.so (the GEMV library) and libqkcalib.so (the benchmark's
streaming-read reference) in-tree with hipcc for gfx950; always recompiles.
The library's sources compile in parallel, then link once."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqkgemv.so")
SOURCES = ["qk_api.hip", "qk_kernels.hip", "qk_verify.hip", "qk_verify_q4k.hip", "qk_verify_q5k.hip",
           "qk_verify_q6k.hip", "qk_verify_iq4xs.hip"]
CALIB_LIB = os.path.join(HERE, "libqkcalib.so")
CALIB_SOURCES = ["qk_stream_read.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed: {what}")


def _link(lib: str, sources, verbose: bool) -> str:
    objs = [lib + "." + os.path.splitext(src)[0] + ".o" for src in sources]
    with ThreadPoolExecutor(max_workers=len(sources)) as pool:
        list(pool.map(lambda so: _run([hipcc(), *HIPCC_FLAGS, "-c", "-o", so[1], os.path.join(CSRC, so[0])],
                                      verbose, so[0]), zip(sources, objs)))
    tmp = lib + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs], verbose, os.path.basename(lib))
    for o in objs:
        os.remove(o)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _link(CALIB_LIB, CALIB_SOURCES, verbose)
    return _link(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
