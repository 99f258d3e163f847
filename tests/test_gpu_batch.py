"""GPU parity of qk_gemv_batch (independent one-column GEMVs in one launch)
through the C ABI: every output bit-identical to the single-call qk_gemv on
the same entry, and within the 1e-4 row bound of the CPU oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_row_bound, dev, needs_gpu, torch
from quant_dequant_gemv_amd import binding, synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6, IQ4 = synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.IQ4_XS


def _make(entries):
    """entries: (qtype, N, K, seed, x_key); entries with the same x_key share x."""
    xs, host, out = {}, [], []
    for qt, N, K, seed, xk in entries:
        W = synth.superblocks(qt, N, K, seed)
        if xk not in xs:
            xs[xk] = synth.activations(K, 1, seed)
        host.append((qt, W, xs[xk], N, K))
        out.append((qt, dev(W.reshape(-1)), dev(xs[xk]).reshape(-1), N, K))
    return host, out


def _single(e):
    qt, Wd, xd, N, K = e
    y = binding.gemv(qt, Wd, xd, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(-1)


def _check(entries):
    host, devs = _make(entries)
    ys = binding.gemv_batch(devs)
    torch.cuda.synchronize()
    for i, ((qt, W, x, N, K), y) in enumerate(zip(host, ys)):
        yb = y.cpu().numpy()
        ys1 = _single(devs[i])
        assert np.array_equal(yb.view(np.uint32), ys1.view(np.uint32)), f"entry {i}: batch != single call"
        y_ref, S = oracle.gemv(qt, W, x, K)
        assert_row_bound(yb, y_ref, S, f"entry {i} type {qt} {N}x{K}")


def test_batch_shared_x_mixed_types():
    # a DeltaNet layer's first group: fused qkv (Q4_K) with alpha and beta (Q6_K), one x
    _check([(Q4, 10240, 5120, 1000, "h"), (Q6, 48, 5120, 1001, "h"), (Q6, 48, 5120, 1002, "h")])


def test_batch_gate_up():
    _check([(Q4, 17408, 5120, 1005, "h"), (Q4, 17408, 5120, 1006, "h")])


def test_batch_distinct_shapes_all_rows():
    _check([(Q5, 300, 6144, 7, "a"), (Q6, 200, 17408, 8, "b"), (Q4, 1000, 5120, 9, "c"), (Q4, 1, 256, 10, "d"),
            (Q6, 5, 512, 11, "e"), (Q5, 777, 1280, 12, "f")])


def test_batch_iq4xs_entries():
    # IQ4_XS beside the k-quants: a stacked run of two IQ4_XS entries sharing
    # x (one joint geometry), an IQ4_XS entry at rounds of 12 rows, and
    # k-quant entries around them
    _check([(IQ4, 4096, 5120, 30, "h"), (IQ4, 1024, 5120, 31, "h"), (Q4, 512, 5120, 32, "h"),
            (IQ4, 38000, 5120, 33, "g"), (Q6, 96, 1024, 34, "k"), (IQ4, 7, 256, 35, "m")])


def test_batch_sixteen_entries_shared_weights():
    host, devs = _make([(Q4, 129, 2048, 20, "a")])
    qt, Wd, xd, N, K = devs[0]
    xs = [synth.activations(K, 1, 100 + i) for i in range(binding.MAX_BATCH)]
    entries = [(qt, Wd, dev(x).reshape(-1), N, K) for x in xs]
    ys = binding.gemv_batch(entries)
    torch.cuda.synchronize()
    W = host[0][1]
    for i, (x, y) in enumerate(zip(xs, ys)):
        y_ref, S = oracle.gemv(qt, W, x, K)
        assert_row_bound(y.cpu().numpy(), y_ref, S, f"entry {i}")
        assert np.array_equal(y.cpu().numpy().view(np.uint32), _single(entries[i]).view(np.uint32))


def test_large_partial_sum_lds():
    # 34 rows x 512 unit columns per workgroup: 68 KB of partial sums, above the default 64 KB
    _check([(Q4, 8500, 32768, 30, "a"), (Q6, 64, 512, 31, "b")])


def test_batch_several_k_segments():
    # K = 65792: segments of 512, 512 and 4 units; a run sharing x and one entry on its own
    _check([(Q4, 300, 65792, 32, "a"), (Q4, 45, 65792, 33, "a"), (Q6, 64, 65792, 34, "b"),
            (Q5, 100, 33024, 35, "c")])


def test_batch_single_phase_entries():
    # entries whose launch has one row phase and several rows per workgroup
    _check([(Q4, 1000, 17408, 21, "a"), (Q5, 600, 17408, 22, "a"), (Q6, 300, 5120, 23, "b")])


# Adjacent entries of one type and K that read the same x are stacked into one
# row range (up to four tensors per stack) with the geometry of a single launch
# of all their rows; every output must still equal its single call bit for bit.
def test_batch_stacked_attention_qkv():
    # an attention layer's q, k and v (Q4_K 12288 / 1024 / 1024 x 5120), one x
    _check([(Q4, 12288, 5120, 1010, "h"), (Q4, 1024, 5120, 1011, "h"), (Q4, 1024, 5120, 1012, "h")])


def test_batch_stacked_runs_all_rows():
    # six Q4_K tensors on one x: a stack of four, then one of two (every row);
    # then Q5_K and Q6_K runs on another x, a repeated tensor, and a Q4_K entry
    # after a type change (not stacked with the first run)
    _check([(Q4, 300, 5120, 40, "a"), (Q4, 7, 5120, 41, "a"), (Q4, 1, 5120, 42, "a"), (Q4, 129, 5120, 43, "a"),
            (Q4, 64, 5120, 44, "a"), (Q4, 500, 5120, 45, "a"),
            (Q5, 250, 6144, 46, "b"), (Q5, 33, 6144, 47, "b"), (Q6, 48, 6144, 48, "b"), (Q6, 48, 6144, 48, "b"),
            (Q4, 90, 5120, 49, "a")])


# Front-loaded stacks: a stack that takes several dispatch rounds of small
# workgroups and starts at a round boundary lets its first tensor fill every
# round but the last at a full straight-line round of rows; the first
# tensor's remaining rows and the later tensors share the last round.  q+k+v
# (12288 rows fill two rounds exactly), 13000 + 1024 + 1024 (712 rows of the
# first tensor left for the last round), a single-tensor run first, and a
# stack after it (which starts mid-round: an even split).
def test_batch_front_loaded_stacks_all_rows():
    _check([(Q4, 13000, 5120, 1020, "h"), (Q4, 1024, 5120, 1021, "h"), (Q4, 1024, 5120, 1022, "h")])
    _check([(Q4, 10240, 5120, 1023, "a"), (Q4, 12288, 5120, 1024, "b"), (Q4, 1024, 5120, 1025, "b"),
            (Q4, 1024, 5120, 1026, "b")])


def test_batch_front_loaded_planar():
    # PLANAR q+k+v, front-loaded as GGUF rows are
    P = binding.PLANAR
    x = synth.activations(5120, 1, 70)
    xd = dev(x).reshape(-1)
    host, entries = [], []
    for N, seed in [(12288, 71), (1024, 72), (1024, 73)]:
        W = synth.superblocks(Q4, N, 5120, seed)
        host.append((W, N))
        entries.append((Q4 | P, binding.repack(Q4, dev(W.reshape(-1)), N, 5120), xd, N, 5120))
    ys = binding.gemv_batch(entries)
    torch.cuda.synchronize()
    for (W, N), e, y in zip(host, entries, ys):
        yb = y.cpu().numpy()
        assert np.array_equal(yb.view(np.uint32), _single(e).view(np.uint32)), f"planar {N} rows"
        y_ref, S = oracle.gemv(Q4, W, x, 5120)
        assert_row_bound(yb, y_ref, S, f"planar {N} rows")


def test_batch_same_x_pointer_other_k_not_stacked():
    # one x buffer read with K = 5120 and, by the next entry, with K = 2560
    # (its first half): equal type and x pointer but another K -- no stack
    W1 = synth.superblocks(Q4, 400, 5120, 50)
    W2 = synth.superblocks(Q4, 300, 2560, 51)
    x = synth.activations(5120, 1, 50)
    xd = dev(x).reshape(-1)
    entries = [(Q4, dev(W1.reshape(-1)), xd, 400, 5120), (Q4, dev(W2.reshape(-1)), xd, 300, 2560)]
    ys = binding.gemv_batch(entries)
    torch.cuda.synchronize()
    for e, y, W, K in zip(entries, ys, (W1, W2), (5120, 2560)):
        yb = y.cpu().numpy()
        assert np.array_equal(yb.view(np.uint32), _single(e).view(np.uint32))
        y_ref, S = oracle.gemv(Q4, W, np.ascontiguousarray(x[:K]), K)
        assert_row_bound(yb, y_ref, S, f"K={K}")


def test_batch_stacked_planar():
    # PLANAR rows stack like GGUF rows: q/k/v-like Q4_K and a Q6_K pair, one x
    P = binding.PLANAR
    x = synth.activations(5120, 1, 60)
    xd = dev(x).reshape(-1)
    host, entries = [], []
    for qt, N, seed in [(Q4, 2000, 61), (Q4, 130, 62), (Q4, 130, 63), (Q6, 48, 64), (Q6, 48, 65)]:
        W = synth.superblocks(qt, N, 5120, seed)
        Wp = binding.repack(qt, dev(W.reshape(-1)), N, 5120)
        host.append((qt, W, N))
        entries.append((qt | P, Wp, xd, N, 5120))
    ys = binding.gemv_batch(entries)
    torch.cuda.synchronize()
    for (qt, W, N), e, y in zip(host, entries, ys):
        yb = y.cpu().numpy()
        assert np.array_equal(yb.view(np.uint32), _single(e).view(np.uint32)), f"planar type {qt} {N} rows"
        y_ref, S = oracle.gemv(qt, W, x, 5120)
        assert_row_bound(yb, y_ref, S, f"planar type {qt} {N} rows")
