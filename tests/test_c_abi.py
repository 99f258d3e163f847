"""CPU-only: include/qkgemv.h is a valid C99 and C++ header, and a C program
built against it links libqkgemv.so and gets the documented results from the
calls that need no GPU (tests/c_abi_check.c)."""
import os
import shutil
import subprocess

import pytest

from quant_dequant_gemv_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(binding.LIB_PATH)

pytestmark = [pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                 reason="libqkgemv.so not built (run __graft_entry__.build())"),
              pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")]


def test_c_program_links_and_checks(tmp_path):
    exe = tmp_path / "c_abi_check"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INC,
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", str(exe), "-L", LIBDIR, "-lqkgemv",
                    "-Wl,-rpath," + LIBDIR], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks held" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no C++ compiler")
def test_header_compiles_as_cpp(tmp_path):
    src = tmp_path / "h.cpp"
    src.write_text('#include "qkgemv.h"\nint main() { return qk_block_bytes(QK_Q4_K) == 144 ? 0 : 1; }\n')
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Werror", "-fsyntax-only", "-I", INC, str(src)], check=True)
