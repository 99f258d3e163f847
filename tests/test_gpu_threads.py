"""Calls from several host threads at once, each thread on a stream of its own:
every output bit-identical to the same call made alone.  The library keeps
host state per device (compute-unit counts, the kernels' LDS opt-in) in
atomics, and a result depends only on its inputs, not on the stream or on
other calls in flight."""
import threading

import pytest

from gpu_util import dev, needs_gpu, torch
from quant_dequant_gemv_amd import binding, synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6 = synth.Q4_K, synth.Q5_K, synth.Q6_K

# (type, N, K, ncols): one-column and verify launches of every type, and a
# PLANAR tensor
CASES = [(Q4, 1024, 5120, 1), (Q5, 129, 6144, 1), (Q6, 96, 17408, 1), (Q4, 300, 5120, 4), (Q6, 77, 2048, 8),
         (Q4 | binding.PLANAR, 640, 5120, 1)]
THREADS, ROUNDS = 4, 8


def test_concurrent_calls_match_single_calls():
    data = []
    for i, (qt, N, K, nc) in enumerate(CASES):
        base = qt & ~binding.PLANAR
        W = dev(synth.superblocks(base, N, K, 900 + i).reshape(-1))
        if qt & binding.PLANAR:
            W = binding.repack(base, W, N, K)
        x = dev(synth.activations(K, nc, 900 + i))
        if nc == 1:
            x = x.reshape(-1)
        ref = binding.gemv(qt, W, x, N, K)
        data.append((qt, W, x, N, K, ref))
    torch.cuda.synchronize()

    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            outs = [[torch.empty_like(d[5]) for d in data] for _ in range(ROUNDS)]
            for r in range(ROUNDS):
                for (qt, W, x, N, K, _), y in zip(data, outs[r]):
                    binding.gemv(qt, W, x, N, K, out=y, stream=s)
            s.synchronize()
            for r in range(ROUNDS):
                for (qt, _, _, N, K, ref), y in zip(data, outs[r]):
                    if not torch.equal(y, ref):
                        errors.append(f"thread {t} round {r}: type {qt:#x} {N}x{K} differs")
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:5]
