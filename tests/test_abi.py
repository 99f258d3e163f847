"""CPU-only: the C-ABI library loads and exports every function include/qkgemv.h
declares; host-side argument validation returns the documented codes without
launching anything (no GPU is touched by any call here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from quant_dequant_gemv_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkgemv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libqkgemv.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qk_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in binding.EXPORTS:
        assert n in names
    assert "qk_gemv" in names and "qk_dequant" in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in qkgemv.h but not exported"


def test_sizes_and_strings():
    assert binding.qk_block_bytes(binding.Q4_K) == 144
    assert binding.qk_block_bytes(binding.Q5_K) == 176
    assert binding.qk_block_bytes(binding.Q6_K) == 210
    assert binding.qk_block_bytes(7) == -1
    assert binding.qk_row_bytes(binding.Q4_K, 5120) == 20 * 144
    assert binding.qk_row_bytes(binding.Q6_K, 17408) == 68 * 210
    assert binding.qk_row_bytes(binding.Q4_K, 300) == -1
    assert binding.qk_row_bytes(99, 256) == -1
    assert "gfx950" in binding.qk_version()
    for code in (0, -1, -2, -3, -4, -99):
        assert isinstance(binding.qk_strerror(code), str) and binding.qk_strerror(code)


FAKE = 1 << 20  # a 16-byte aligned non-null address: never dereferenced, the checks fail first


@pytest.mark.parametrize("args,code", [
    ((99, FAKE, FAKE, FAKE, 4, 256, 1), binding.QK_EINVAL_TYPE),
    ((binding.Q4_K, FAKE, FAKE, FAKE, 0, 256, 1), binding.QK_EINVAL_SHAPE),
    ((binding.Q4_K, FAKE, FAKE, FAKE, 4, 255, 1), binding.QK_EINVAL_SHAPE),
    ((binding.Q4_K, FAKE, FAKE, FAKE, 4, 0, 1), binding.QK_EINVAL_SHAPE),
    ((binding.Q5_K, FAKE, FAKE, FAKE, 4, 512 + 128, 1), binding.QK_EINVAL_SHAPE),
    ((binding.Q6_K, FAKE, FAKE, FAKE, 4, 256, 0), binding.QK_EINVAL_SHAPE),
    ((binding.Q6_K, FAKE, FAKE, FAKE, 4, 256, 33), binding.QK_EINVAL_SHAPE),
    ((binding.Q4_K, 0, FAKE, FAKE, 4, 256, 1), binding.QK_EINVAL_PTR),
    ((binding.Q4_K, FAKE, 0, FAKE, 4, 256, 1), binding.QK_EINVAL_PTR),
    ((binding.Q4_K, FAKE, FAKE, 0, 4, 256, 1), binding.QK_EINVAL_PTR),
    ((binding.Q4_K, FAKE + 8, FAKE, FAKE, 4, 256, 1), binding.QK_EINVAL_PTR),
    ((binding.Q4_K, FAKE, FAKE + 2, FAKE, 4, 256, 1), binding.QK_EINVAL_PTR),
    ((binding.Q4_K, FAKE, FAKE, FAKE + 2, 4, 256, 1), binding.QK_EINVAL_PTR),
])
def test_gemv_validation_codes(args, code):
    assert binding.qk_gemv(*args, 0) == code


def test_dequant_validation_codes():
    assert binding.qk_dequant(1, FAKE, FAKE, 4, 256, 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_dequant(binding.Q4_K, FAKE, FAKE, 4, 100, 0) == binding.QK_EINVAL_SHAPE
    assert binding.qk_dequant(binding.Q4_K, 0, FAKE, 4, 256, 0) == binding.QK_EINVAL_PTR
    assert binding.qk_dequant(binding.Q4_K, FAKE, FAKE + 1, 4, 256, 0) == binding.QK_EINVAL_PTR


def test_python_wrappers_raise_not_fallback():
    with pytest.raises(binding.QKError) as e:
        err = binding.qk_gemv(99, FAKE, FAKE, FAKE, 4, 256, 1, 0)
        raise binding.QKError(err, "qk_gemv")
    assert e.value.code == binding.QK_EINVAL_TYPE


def test_batch_item_layout_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct qk_gemv_item \{(.*?)\} qk_gemv_item;", text, flags=re.S).group(1)
    fields = re.findall(r"(\w+);", body)
    assert fields == [f for f, _ in binding.qk_gemv_item._fields_]
    assert ctypes.sizeof(binding.qk_gemv_item) == 48
    assert binding.MAX_BATCH == int(re.search(r"#define QK_MAX_BATCH (\d+)", text).group(1))


def test_batch_validation_codes():
    good = (binding.Q4_K, FAKE, FAKE, FAKE, 4, 256)
    assert binding.qk_gemv_batch([], 0) == binding.QK_EINVAL_SHAPE
    assert binding.qk_gemv_batch([good] * (binding.MAX_BATCH + 1), 0) == binding.QK_EINVAL_SHAPE
    assert binding.load_library().qk_gemv_batch(None, 1, None) == binding.QK_EINVAL_SHAPE
    assert binding.qk_gemv_batch([good, (99, FAKE, FAKE, FAKE, 4, 256)], 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_gemv_batch([good, (binding.Q6_K, FAKE, FAKE, FAKE, 4, 300)], 0) == binding.QK_EINVAL_SHAPE
    assert binding.qk_gemv_batch([(binding.Q5_K, FAKE, FAKE + 2, FAKE, 4, 256), good], 0) == binding.QK_EINVAL_PTR
    assert binding.qk_gemv_batch([good, (binding.Q4_K, FAKE, FAKE, 0, 4, 256)], 0) == binding.QK_EINVAL_PTR


def test_planar_row_bytes_and_flag_validation():
    P = binding.PLANAR
    assert binding.qk_row_bytes(binding.Q4_K | P, 5120) == 20 * 144
    assert binding.qk_row_bytes(binding.Q5_K | P, 6144) == 24 * 176
    assert binding.qk_row_bytes(binding.Q6_K | P, 17408) == 14288  # 68 * 210 rounded up to 16
    assert binding.qk_row_bytes(binding.Q6_K | P, 2048) == 8 * 210 == 1680
    assert binding.qk_row_bytes(binding.Q4_K | 0x200, 5120) == -1
    assert binding.qk_gemv(binding.Q4_K | P, FAKE, FAKE, FAKE, 4, 256, 2, 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_gemv(binding.Q4_K | 0x200, FAKE, FAKE, FAKE, 4, 256, 1, 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_dequant(binding.Q5_K | P, FAKE, FAKE, 4, 300, 0) == binding.QK_EINVAL_SHAPE
    assert binding.qk_gemv_batch([(binding.Q6_K | P, FAKE, FAKE, FAKE + 2, 4, 256)], 0) == binding.QK_EINVAL_PTR


def test_iq4xs_type_codes():
    """IQ4_XS (GGUF id 23, 136-byte superblocks) is a type of its own for the
    GEMV, verify, epilogue, batch and dequant calls; it has no PLANAR layout,
    no repack and no chain entries."""
    IQ, P = binding.IQ4_XS, binding.PLANAR
    assert binding.qk_block_bytes(IQ) == 136
    assert binding.qk_row_bytes(IQ, 5120) == 20 * 136
    assert binding.qk_row_bytes(IQ | P, 5120) == -1
    assert binding.qk_gemv(IQ | P, FAKE, FAKE, FAKE, 4, 256, 1, 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_dequant(IQ | P, FAKE, 4 * FAKE, 4, 256, 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_gemv_batch([(IQ | P, FAKE, FAKE, 4 * FAKE, 4, 256)], 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_repack(IQ, FAKE, 4 * FAKE, 4, 256, 0) == binding.QK_EINVAL_TYPE
    # the argument checks before any launch apply as for the k-quants
    assert binding.qk_gemv(IQ, FAKE, FAKE, FAKE, 4, 300, 1, 0) == binding.QK_EINVAL_SHAPE
    assert binding.qk_gemv(IQ, FAKE + 8, FAKE, 4 * FAKE, 4, 256, 1, 0) == binding.QK_EINVAL_PTR
    e = binding.qk_chain_entry(IQ, 0, FAKE, None, FAKE, 4 * FAKE, None, 4, 256)
    plan = np.zeros(binding.qk_chain_plan_bytes(1, 1), dtype=np.uint8)
    assert binding.qk_chain_plan([e], [1], plan) == binding.QK_EINVAL_TYPE


def test_repack_validation_codes():
    P = binding.PLANAR
    assert binding.qk_repack(binding.Q4_K | P, FAKE, 4 * FAKE, 4, 256, 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_repack(99, FAKE, 4 * FAKE, 4, 256, 0) == binding.QK_EINVAL_TYPE
    assert binding.qk_repack(binding.Q4_K, FAKE, 4 * FAKE, 4, 300, 0) == binding.QK_EINVAL_SHAPE
    assert binding.qk_repack(binding.Q4_K, FAKE + 8, 4 * FAKE, 4, 256, 0) == binding.QK_EINVAL_PTR
    assert binding.qk_repack(binding.Q4_K, FAKE, 4 * FAKE + 4, 4, 256, 0) == binding.QK_EINVAL_PTR
    assert binding.qk_repack(binding.Q6_K, FAKE, FAKE + 16 * 210, 32, 256, 0) == binding.QK_EINVAL_PTR  # overlap


def test_epilogue_validation_codes():
    """qk_gemv_ex / qk_gemv_swiglu: shape and type checks as qk_gemv, then the
    flags, then the pointers (the residual may be y only for an fp32 y)."""
    Q4, Q6 = binding.Q4_K, binding.Q6_K
    F16 = binding.Y_F16
    ex = binding.qk_gemv_ex
    sw = binding.qk_gemv_swiglu
    assert ex(99, FAKE, FAKE, FAKE, 4, 256, 1, None, 0, 0) == binding.QK_EINVAL_TYPE
    assert ex(Q4, FAKE, FAKE, FAKE, 4, 300, 1, None, 0, 0) == binding.QK_EINVAL_SHAPE
    assert ex(Q4, FAKE, FAKE, FAKE, 4, 256, 33, None, 0, 0) == binding.QK_EINVAL_SHAPE
    assert ex(Q4, FAKE, FAKE, FAKE, 4, 256, 1, None, 2, 0) == binding.QK_EINVAL_FLAGS
    assert ex(Q4, FAKE, FAKE, FAKE, 4, 256, 1, None, F16 | 4, 0) == binding.QK_EINVAL_FLAGS
    assert ex(Q4, 0, FAKE, FAKE, 4, 256, 1, None, 0, 0) == binding.QK_EINVAL_PTR
    assert ex(Q4, FAKE, FAKE + 8, FAKE, 4, 256, 1, None, 0, 0) == binding.QK_EINVAL_PTR
    assert ex(Q4, FAKE, FAKE, FAKE + 2, 4, 256, 1, None, 0, 0) == binding.QK_EINVAL_PTR  # fp32 y, 2-aligned
    assert ex(Q4, FAKE, FAKE, FAKE + 1, 4, 256, 1, None, F16, 0) == binding.QK_EINVAL_PTR  # fp16 y, odd
    assert ex(Q4, FAKE, FAKE, FAKE, 4, 256, 1, FAKE + 2, 0, 0) == binding.QK_EINVAL_PTR  # residual alignment
    # residual overlapping y: allowed only as y itself with an fp32 y
    assert ex(Q4, FAKE, FAKE, FAKE, 4, 256, 2, FAKE + 4, 0, 0) == binding.QK_EINVAL_PTR
    assert ex(Q4, FAKE, FAKE, FAKE, 4, 256, 2, FAKE, F16, 0) == binding.QK_EINVAL_PTR
    assert ex(Q4, FAKE, FAKE, FAKE + 32, 4, 256, 2, FAKE + 16, F16, 0) == binding.QK_EINVAL_PTR
    assert binding.qk_gemv_ex(Q4 | binding.PLANAR, FAKE, FAKE, FAKE, 4, 256, 2, None, 0, 0) == \
        binding.QK_EINVAL_TYPE
    assert sw(99, FAKE, FAKE, FAKE, FAKE, 4, 256, 1, 0, 0) == binding.QK_EINVAL_TYPE
    assert sw(Q6, FAKE, FAKE, FAKE, FAKE, 0, 256, 1, 0, 0) == binding.QK_EINVAL_SHAPE
    assert sw(Q6, FAKE, FAKE, FAKE, FAKE, 4, 256, 1, 8, 0) == binding.QK_EINVAL_FLAGS
    assert sw(Q6, FAKE, 0, FAKE, FAKE, 4, 256, 1, 0, 0) == binding.QK_EINVAL_PTR
    assert sw(Q6, FAKE, FAKE + 4, FAKE, FAKE, 4, 256, 1, 0, 0) == binding.QK_EINVAL_PTR
    assert sw(Q6, FAKE, FAKE, FAKE, FAKE + 1, 4, 256, 1, F16, 0) == binding.QK_EINVAL_PTR
    for code in (binding.QK_EINVAL_FLAGS,):
        assert "flag" in binding.qk_strerror(code)
