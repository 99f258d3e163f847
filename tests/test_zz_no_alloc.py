"""GPU tests of qk_gemv_chain_noalloc through the C ABI: the chain with its
barrier counters in the library's own per-GPU array instead of a caller
workspace.

* on two calls in a row, the second with a smaller chain, every output is
  bit-identical to what qk_gemv_chain (the same plan, a caller workspace)
  writes, and the status word it copies out is 0;
* a run whose waits are forced to expire from the host (a 1 us limit) leaves
  QK_CHAIN_TIMEOUT in the status word, and the next call, which shares the
  array, starts clean and is whole;
* the largest chain it takes (QK_CHAIN_NOALLOC_MAX_STEPS steps) runs and
  matches; one step more, a null plan_dev or a misaligned status word are
  rejected before anything is launched;
* repeated calls leave the device's free memory unchanged.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, needs_gpu
from quant_dequant_gemv_amd import binding, synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6 = synth.Q4_K, synth.Q5_K, synth.Q6_K


def _bits(t):
    a = t.cpu().numpy().reshape(-1)
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


def _chain(seed, n, k, repeat=1):
    """A chain with dependencies: fp16 y of one step is the next step's x, two
    steps add into one residual stream.  n, k scale the shapes."""
    rng = np.random.default_rng(seed)
    W = lambda qt, N, K, s: dev(synth.superblocks(qt, N, K, seed + s).reshape(-1))
    t = dict(x0=dev(synth.activations(k, 1, seed).reshape(-1)),
             h0=rng.standard_normal(k).astype(np.float32))
    t["h"] = dev(t["h0"].copy())
    t["a16"] = torch.empty(n, dtype=torch.float16, device="cuda")
    t["b"] = torch.empty(96, dtype=torch.float32, device="cuda")
    t["g16"] = torch.empty(2 * n, dtype=torch.float16, device="cuda")
    Wa, Wb, Wc = W(Q4, n, k, 1), W(Q6, 96, k, 2), W(Q5, k, n, 3)
    Wg, Wu, Wd = W(Q4, 2 * n, k, 4), W(Q4, 2 * n, k, 5), W(Q6, k, 2 * n, 6)
    t["keep"] = (Wa, Wb, Wc, Wg, Wu, Wd)
    steps = [
        [dict(qtype=Q4, W=Wa, x=t["x0"], y=t["a16"], N=n, K=k, f16=True),
         dict(qtype=Q6, W=Wb, x=t["x0"], y=t["b"], N=96, K=k)],
        [dict(qtype=Q5, W=Wc, x=t["a16"], y=t["h"], residual=t["h"], N=k, K=n)],
        [dict(qtype=Q4, W=Wg, W2=Wu, x=t["x0"], y=t["g16"], N=2 * n, K=k, f16=True)],
        [dict(qtype=Q6, W=Wd, x=t["g16"], y=t["h"], residual=t["h"], N=k, K=2 * n)],
    ] * repeat
    return t, binding.Chain(steps)


def _outputs(t):
    torch.cuda.synchronize()
    return {k: _bits(t[k]) for k in ("a16", "b", "h", "g16")}


def _reset(t):
    t["h"].copy_(torch.from_numpy(t["h0"]))
    for k in ("a16", "b", "g16"):
        t[k].zero_()


def _noalloc(ch, status, timeout_us=0):
    return binding.qk_gemv_chain_noalloc(ch.plan, ch.plan_dev.data_ptr(), status.data_ptr(), timeout_us,
                                         torch.cuda.current_stream().cuda_stream)


def _check_same_as_workspace_run(t, ch, status):
    _reset(t)
    ch.run()
    ref = _outputs(t)
    assert ch.status() == 0
    _reset(t)
    status.fill_(-1)
    assert _noalloc(ch, status) == binding.QK_OK
    got = _outputs(t)
    assert int(status.item()) == 0
    for k in ref:
        assert np.array_equal(got[k], ref[k]), f"noalloc output {k} differs from qk_gemv_chain's"


def test_noalloc_matches_workspace_chain_twice_second_smaller():
    status = torch.empty(1, dtype=torch.int32, device="cuda")
    big, chb = _chain(11, 1536, 2048)
    small, chs = _chain(12, 256, 512)
    _check_same_as_workspace_run(big, chb, status)
    _check_same_as_workspace_run(small, chs, status)


def test_noalloc_timeout_flag_then_clean_run():
    status = torch.empty(1, dtype=torch.int32, device="cuda")
    t, ch = _chain(13, 512, 1024, repeat=5)  # 20 steps: 19 barriers
    assert _noalloc(ch, status, timeout_us=1) == binding.QK_OK
    torch.cuda.synchronize()  # every workgroup left the kernel
    assert int(status.item()) & binding.CHAIN_TIMEOUT
    small, chs = _chain(14, 256, 512)
    _check_same_as_workspace_run(small, chs, status)


def test_noalloc_calls_leave_device_memory_unchanged():
    """After a first call (module loading and the per-device address of the
    counter array), further calls take no device memory: the free memory the
    driver reports (hipMemGetInfo) is the same before and after 20 calls."""
    status = torch.empty(1, dtype=torch.int32, device="cuda")
    t, ch = _chain(15, 512, 1024)
    assert _noalloc(ch, status) == binding.QK_OK
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(20):
        assert _noalloc(ch, status) == binding.QK_OK
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    assert int(status.item()) == 0


def test_noalloc_step_limit_and_bad_pointers():
    n = binding.CHAIN_NOALLOC_MAX_STEPS
    W = dev(synth.superblocks(Q4, 64, 256, 21).reshape(-1))
    x = dev(synth.activations(256, 1, 21).reshape(-1))
    ys = [torch.empty(64, dtype=torch.float32, device="cuda") for _ in range(2)]
    step = lambda s: [dict(qtype=Q4, W=W, x=x, y=ys[s % 2], N=64, K=256)]
    status = torch.empty(2, dtype=torch.int32, device="cuda")
    over = binding.Chain([step(s) for s in range(n + 1)])
    assert _noalloc(over, status) == binding.QK_EINVAL_SHAPE
    top = binding.Chain([step(s) for s in range(n)])
    top.run()
    torch.cuda.synchronize()
    assert top.status() == 0
    ref = [y.clone() for y in ys]
    for y in ys:
        y.zero_()
    status.fill_(-1)
    assert _noalloc(top, status) == binding.QK_OK
    torch.cuda.synchronize()
    assert int(status[0].item()) == 0
    for y, r in zip(ys, ref):
        assert np.array_equal(_bits(y), _bits(r))
    stream = torch.cuda.current_stream().cuda_stream
    assert binding.qk_gemv_chain_noalloc(top.plan, 0, 0, 0, stream) == binding.QK_EINVAL_PTR
    assert binding.qk_gemv_chain_noalloc(top.plan, top.plan_dev.data_ptr(), status.data_ptr() + 2, 0,
                                         stream) == binding.QK_EINVAL_PTR
