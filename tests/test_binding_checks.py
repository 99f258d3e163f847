"""CPU-only: the torch helpers of the binding reject wrong dtypes, sizes and
devices before anything reaches the library, and the C ABI rejects outputs
that overlap inputs (fake aligned addresses: the checks fail before any
launch, nothing is dereferenced)."""
import os

import pytest
import torch

from quant_dequant_gemv_amd import binding

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libqkgemv.so not built (run __graft_entry__.build())")

Q4, Q5, Q6 = binding.Q4_K, binding.Q5_K, binding.Q6_K
P = binding.PLANAR
N, K = 8, 512
RB = 2 * 144  # Q4_K row bytes at K = 512


def cpu(n, dtype):
    return torch.zeros(n, dtype=dtype)


def test_gemv_sizes_and_dtypes():
    W, x = cpu(N * RB, torch.uint8), cpu(K, torch.float16)
    with pytest.raises(ValueError, match="at least"):
        binding.gemv(Q4, cpu(N * RB - 1, torch.uint8), x, N, K)  # W one byte short
    with pytest.raises(ValueError, match="at least K"):
        binding.gemv(Q4, W, cpu(K - 8, torch.float16), N, K)  # x short
    with pytest.raises(ValueError, match="shape"):
        binding.gemv(Q4, W, torch.zeros((2, K, 1), dtype=torch.float16), N, K)
    with pytest.raises(TypeError):
        binding.gemv(Q4, W.to(torch.int8), x, N, K)
    with pytest.raises(TypeError):
        binding.gemv(Q4, W, x.float(), N, K)
    with pytest.raises(ValueError, match="contiguous"):
        binding.gemv(Q4, W, torch.zeros((K, 2), dtype=torch.float16).t().contiguous().t(), N, K)
    with pytest.raises(ValueError, match="elements"):
        binding.gemv(Q4, W, x, N, K, out=cpu(N + 1, torch.float32))  # out of the wrong size
    with pytest.raises(TypeError):
        binding.gemv(Q4, W, x, N, K, out=cpu(N, torch.float16))
    # Q6_K rows are larger: the same buffer is too short for them
    with pytest.raises(ValueError, match="at least"):
        binding.gemv(Q6, W, x, N, K)
    # PLANAR Q6_K rows are padded to 16 bytes
    with pytest.raises(ValueError, match="at least"):
        binding.gemv(Q6 | P, cpu(N * 2 * 210, torch.uint8), x, N, K)


def test_every_helper_needs_device_tensors():
    """Correct sizes on host tensors: refused as not on the GPU, before the library is called."""
    W, x = cpu(N * RB, torch.uint8), cpu(K, torch.float16)
    with pytest.raises(ValueError, match="CUDA"):
        binding.gemv(Q4, W, x, N, K, out=cpu(N, torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        binding.gemv_ex(Q4, W, x, N, K, residual=cpu(N, torch.float32), out=cpu(N, torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        binding.gemv_swiglu(Q4, W, W, x, N, K, out=cpu(N, torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        binding.gemv_batch([(Q4, W, x, N, K, cpu(N, torch.float32))])
    with pytest.raises(ValueError, match="CUDA"):
        binding.dequant(Q4, W, N, K, out=cpu(N * K, torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        binding.repack(Q4, W, N, K, out=cpu(N * RB, torch.uint8))


def test_epilogue_batch_dequant_repack_sizes():
    W, x = cpu(N * RB, torch.uint8), cpu(K, torch.float16)
    with pytest.raises(ValueError, match="residual"):
        binding.gemv_ex(Q4, W, x, N, K, residual=cpu(N - 1, torch.float32), out=cpu(N, torch.float32))
    with pytest.raises(TypeError):
        binding.gemv_ex(Q4, W, x, N, K, residual=cpu(N, torch.float16), out=cpu(N, torch.float32))
    with pytest.raises(ValueError, match="out"):
        binding.gemv_ex(Q4, W, x, N, K, f16=True, out=cpu(N - 1, torch.float16))
    with pytest.raises(ValueError, match="Wu"):
        binding.gemv_swiglu(Q4, W, cpu(N * RB - 16, torch.uint8), x, N, K, out=cpu(N, torch.float32))
    with pytest.raises(ValueError, match=r"entries\[1\]"):
        binding.gemv_batch([(Q4, W, x, N, K, cpu(N, torch.float32)),
                            (Q4, cpu(RB, torch.uint8), x, N, K, cpu(N, torch.float32))])
    with pytest.raises(ValueError, match="one column"):
        binding.gemv_batch([(Q4, W, torch.zeros((K, 2), dtype=torch.float16), N, K)])
    with pytest.raises(ValueError, match="elements"):
        binding.dequant(Q4, W, N, K, out=cpu(N * K - 1, torch.float32))
    with pytest.raises(ValueError, match="at least"):
        binding.repack(Q6, cpu(N * 2 * 210, torch.uint8), N, K, out=cpu(N * 2 * 210, torch.uint8))  # padded rows


FAKE = 1 << 24  # aligned, never dereferenced


def test_c_abi_rejects_outputs_over_inputs():
    code = binding.QK_EINVAL_PTR
    W, x = FAKE, 8 * FAKE
    wbytes = N * RB
    # y inside W, y over x, y == x
    assert binding.qk_gemv(Q4, W, x, W + wbytes - 16, N, K, 1, 0) == code
    assert binding.qk_gemv(Q4, W, x, x + 2 * K - 4, N, K, 1, 0) == code
    assert binding.qk_gemv(Q4, W, x, x, N, K, 1, 0) == code
    # multi-column x extent: K * ncols halves
    assert binding.qk_gemv(Q4, W, x, x + 2 * K * 3 - 16, N, K, 4, 0) == code
    assert binding.qk_gemv_ex(Q4, W, x, W, N, K, 1, None, binding.Y_F16, 0) == code
    # SwiGLU: y over the up tensor
    assert binding.qk_gemv_swiglu(Q4, W, 4 * FAKE, x, 4 * FAKE + 64, N, K, 1, 0, 0) == code
    # dequant: out over W
    assert binding.qk_dequant(Q4, W, W + 32, N, K, 0) == code
    # batch: an entry's y over another entry's x, W or y
    a = (Q4, W, x, 16 * FAKE, N, K)
    assert binding.qk_gemv_batch([a, (Q4, 2 * FAKE, 3 * FAKE, x + 16, N, K)], 0) == code
    assert binding.qk_gemv_batch([a, (Q4, 2 * FAKE, 3 * FAKE, W + 64, N, K)], 0) == code
    assert binding.qk_gemv_batch([a, (Q4, 2 * FAKE, 3 * FAKE, 16 * FAKE + 4 * N - 4, N, K)], 0) == code
    assert binding.qk_gemv_batch([a, (Q4, 2 * FAKE, 3 * FAKE, 16 * FAKE, N, K)], 0) == code
    assert "overlaps" in binding.qk_strerror(code)
