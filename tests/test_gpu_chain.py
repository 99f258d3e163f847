"""GPU tests of the chain entry point (qk_chain_plan / qk_gemv_chain) through
the C ABI: a chain of dependent one-column steps in one persistent launch.

* every y is bit-identical to the same GEMV run as a single qk_gemv_ex /
  qk_gemv_swiglu call, including steps whose x or residual is what an earlier
  step of the same chain wrote (the barrier between steps orders them);
* every y is within the row bound of the CPU oracle on the inputs it saw;
* repeated runs give the same bits (the workspace is cleared per run);
* the bounded wait: forced to expire from the host (a 1 us limit), it sets
  the flag in the workspace and every workgroup leaves the kernel normally;
  the next run with the default limit is whole again.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_row_bound, dev, needs_gpu
from quant_dequant_gemv_amd import binding, synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6 = synth.Q4_K, synth.Q5_K, synth.Q6_K
P = binding.PLANAR


def _W(qt, N, K, seed):
    host = synth.superblocks(qt, N, K, seed)
    return host, dev(host.reshape(-1))


def _build(seed=0):
    """A token-like chain with real dependencies between its steps."""
    rng = np.random.default_rng(seed)
    t = {}
    t["x0"] = dev(synth.activations(512, 1, seed).reshape(-1))
    t["h0"] = rng.standard_normal(512).astype(np.float32)
    t["h"] = dev(t["h0"].copy())
    t["W0h"], t["W0"] = _W(Q4, 768, 512, seed + 1)     # step 0: "qkv" -> fp16, read by step 1
    t["W1h"], t["W1"] = _W(Q6, 48, 512, seed + 2)      # step 0: "alpha"
    t["W2h"], t["W2"] = _W(Q5, 512, 768, seed + 3)     # step 1: "out" += into h, x = step 0's fp16 y
    t["Wgh"], t["Wg"] = _W(Q4, 1024, 512, seed + 4)    # step 2: gate/up SwiGLU -> fp16
    t["Wuh"], t["Wu"] = _W(Q4, 1024, 512, seed + 5)
    t["W4h"], t["W4"] = _W(Q6, 512, 1024, seed + 6)    # step 3: "down" += into h, x = step 2's fp16 y
    t["W5h"], W5 = _W(Q4, 256, 512, seed + 7)           # step 4: PLANAR rows
    t["W5p"] = binding.repack(Q4, W5, 256, 512)
    t["a16"] = torch.empty(768, dtype=torch.float16, device="cuda")
    t["b"] = torch.empty(48, dtype=torch.float32, device="cuda")
    t["g16"] = torch.empty(1024, dtype=torch.float16, device="cuda")
    t["f"] = torch.empty(256, dtype=torch.float32, device="cuda")
    steps = [
        [dict(qtype=Q4, W=t["W0"], x=t["x0"], y=t["a16"], N=768, K=512, f16=True),
         dict(qtype=Q6, W=t["W1"], x=t["x0"], y=t["b"], N=48, K=512)],
        [dict(qtype=Q5, W=t["W2"], x=t["a16"], y=t["h"], residual=t["h"], N=512, K=768)],
        [dict(qtype=Q4, W=t["Wg"], W2=t["Wu"], x=t["x0"], y=t["g16"], N=1024, K=512, f16=True)],
        [dict(qtype=Q6, W=t["W4"], x=t["g16"], y=t["h"], residual=t["h"], N=512, K=1024)],
        [dict(qtype=Q4 | P, W=t["W5p"], x=t["x0"], y=t["f"], N=256, K=512)],
    ]
    return t, steps


def _sequential(t):
    """The same GEMVs as single calls, in the same order."""
    h = dev(t["h0"].copy())
    a16 = binding.gemv_ex(Q4, t["W0"], t["x0"], 768, 512, f16=True)
    b = binding.gemv(Q6, t["W1"], t["x0"], 48, 512)
    binding.gemv_ex(Q5, t["W2"], a16, 512, 768, residual=h, out=h)
    g16 = binding.gemv_swiglu(Q4, t["Wg"], t["Wu"], t["x0"], 1024, 512, f16=True)
    binding.gemv_ex(Q6, t["W4"], g16, 512, 1024, residual=h, out=h)
    f = binding.gemv(Q4 | P, t["W5p"], t["x0"], 256, 512)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().reshape(-1) for k, v in dict(a16=a16, b=b, h=h, g16=g16, f=f).items()}


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


def test_chain_bit_identical_to_single_calls_and_within_bound():
    t, steps = _build(0)
    ch = binding.Chain(steps)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    got = {k: t[k].cpu().numpy().reshape(-1) for k in ("a16", "b", "h", "g16", "f")}
    ref = _sequential(t)
    for k in got:
        assert np.array_equal(_bits(got[k]), _bits(ref[k])), f"chain output {k} differs from the single calls"
    # against the oracle, on the inputs each step saw (the fp16 outputs of
    # earlier steps included)
    x0 = t["x0"].cpu().numpy()
    y, S = oracle.gemv(Q6, t["W1h"], x0, 512)
    assert_row_bound(got["b"], y, S, "alpha")
    y, S = oracle.gemv(Q4, t["W5h"], x0, 512)
    assert_row_bound(got["f"], y, S, "planar step")
    h, S1 = oracle.gemv_residual(Q5, t["W2h"], got["a16"], 768, t["h0"])
    y, S2 = oracle.gemv(Q6, t["W4h"], got["g16"], 1024)
    # two adds into h, each rounded once in fp32
    tol = oracle.residual_bound(h[:, 0] + y[:, 0], S1[:, 0] + S2[:, 0]) + 2.0 ** -24 * np.abs(h[:, 0])
    assert oracle.within(got["h"], h[:, 0] + y[:, 0], tol).all(), "residual stream"


def test_chain_repeat_and_long_chain():
    rng = np.random.default_rng(3)
    x = dev(synth.activations(512, 1, 3).reshape(-1))
    Ws, ys, steps = [], [], []
    for s in range(40):  # 40 steps, each two small GEMVs of different types
        qa = (Q4, Q5, Q6)[s % 3]
        Wa = dev(synth.superblocks(qa, 96 + 8 * (s % 5), 512, 100 + s).reshape(-1))
        Wb = dev(synth.superblocks(Q4, 40, 512, 200 + s).reshape(-1))
        ya = torch.empty(96 + 8 * (s % 5), dtype=torch.float32, device="cuda")
        yb = torch.empty(40, dtype=torch.float32, device="cuda")
        Ws.append((qa, Wa, Wb))
        ys.append((ya, yb))
        steps.append([dict(qtype=qa, W=Wa, x=x, y=ya, N=ya.numel(), K=512),
                      dict(qtype=Q4, W=Wb, x=x, y=yb, N=40, K=512)])
    ch = binding.Chain(steps)
    ch.run()
    torch.cuda.synchronize()
    first = [(a.cpu().numpy().copy(), b.cpu().numpy().copy()) for a, b in ys]
    for a, b in ys:
        a.zero_()
        b.zero_()
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    for (a, b), (fa, fb), (qa, Wa, Wb) in zip(ys, first, Ws):
        assert np.array_equal(_bits(a.cpu().numpy()), _bits(fa)) and np.array_equal(_bits(b.cpu().numpy()), _bits(fb))
        ref = binding.gemv(qa, Wa, x, a.numel(), 512).cpu().numpy().reshape(-1)
        assert np.array_equal(_bits(fa), _bits(ref))


def test_chain_bounded_wait_gives_up_visibly():
    t, steps = _build(5)
    ch = binding.Chain(steps * 4)  # 20 steps: 19 barriers
    ch.run(timeout_us=1)
    torch.cuda.synchronize()  # every workgroup left the kernel
    assert ch.status() & binding.CHAIN_TIMEOUT
    # a normal run afterwards: the flag cleared, every step whole
    t2, steps2 = _build(5)
    ch2 = binding.Chain(steps2)
    ch2.run()
    torch.cuda.synchronize()
    assert ch2.status() == 0
    ref = _sequential(t2)
    assert np.array_equal(_bits(t2["f"].cpu().numpy().reshape(-1)), _bits(ref["f"]))


def test_chain_rejects_bad_plans():
    t, steps = _build(1)
    bad = [list(s) for s in steps]
    bad[0] = bad[0] + [dict(qtype=Q4, W=t["W0"], x=t["a16"], y=t["b"], N=48, K=512)]  # x written by the same step
    with pytest.raises(binding.QKError) as e:
        binding.Chain(bad)
    assert e.value.code == binding.QK_EINVAL_PTR
    with pytest.raises(binding.QKError) as e:  # SwiGLU pairs are Q4_K only
        binding.Chain([[dict(qtype=Q6, W=t["W1"], W2=t["W1"], x=t["x0"], y=t["b"], N=48, K=512)]])
    assert e.value.code == binding.QK_EINVAL_TYPE
