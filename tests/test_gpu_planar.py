"""GPU parity of the PLANAR row layout (qk_repack, QK_PLANAR) through the C
ABI: the repack matches the test-side packer byte for byte; dequantising the
repacked tensor is bit-exact against the oracle's GGUF dequantisation; the
GEMV on it is within the oracle's row bound and bit-identical to the GEMV on
the GGUF tensor (same units, same geometry, same summation order)."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_row_bound, dev, gpu_gemv, needs_gpu, same_f32, torch
from kquant_planar import pack
from quant_dequant_gemv_amd import binding, synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6 = synth.Q4_K, synth.Q5_K, synth.Q6_K
TYPES = [Q4, Q5, Q6]
NAMES = {Q4: "Q4_K", Q5: "Q5_K", Q6: "Q6_K"}
P = binding.PLANAR
# K = 2048 (8 superblocks: Q6_K rows need no pad), 1280 and 17408 (Q6_K rows padded)
# (37 x 33024: two K segments of the one-column kernel, the second of 4 units)
SHAPES = [(1, 256), (5, 1280), (47, 2048), (130, 5120), (37, 17408), (3000, 5120), (37, 33024)]


def _repacked(qt, W, N, K):
    Wp = binding.repack(qt, dev(W.reshape(-1)), N, K)
    torch.cuda.synchronize()
    return Wp


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SHAPES)
def test_repack_matches_packer(qt, N, K):
    W = synth.superblocks(qt, N, K, 40 + N)
    Wp = _repacked(qt, W, N, K).cpu().numpy().reshape(N, -1)
    assert np.array_equal(Wp, pack(qt, W, K))


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SHAPES[:5])
def test_planar_dequant_bit_exact(qt, N, K):
    W = synth.superblocks(qt, N, K, 50 + N)
    Wp = _repacked(qt, W, N, K)
    out = binding.dequant(qt | P, Wp, N, K)
    torch.cuda.synchronize()
    assert same_f32(out.cpu().numpy(), oracle.dequant(qt, W, K))


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SHAPES)
def test_planar_gemv_bound_and_identical_to_gguf(qt, N, K):
    W = synth.superblocks(qt, N, K, 60 + N)
    x = synth.activations(K, 1, 60 + N)
    Wp = _repacked(qt, W, N, K)
    xd = dev(x).reshape(-1)
    yp = binding.gemv(qt | P, Wp, xd, N, K).cpu().numpy().reshape(-1)
    yg = gpu_gemv(qt, W, x, N, K).reshape(-1)
    assert np.array_equal(yp.view(np.uint32), yg.view(np.uint32)), "planar != GGUF"
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(yp, y_ref, S, f"{NAMES[qt]} planar {N}x{K}")


@pytest.mark.parametrize("case", synth.Q4K_PROJECTIONS + synth.MIXED, ids=lambda c: c["name"])
def test_planar_full_shapes_all_rows(case):
    qt, N, K = case["qtype"], case["N"], case["K"]
    W = synth.superblocks(qt, N, K, case["seed"])
    x = synth.activations(K, 1, case["seed"])
    Wp = _repacked(qt, W, N, K)
    y = binding.gemv(qt | P, Wp, dev(x).reshape(-1), N, K).cpu().numpy().reshape(-1)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{case['name']} planar")
    w = binding.dequant(qt | P, Wp, N, K).cpu().numpy()
    assert same_f32(w, oracle.dequant(qt, W, K)), f"{case['name']} planar dequant"


def test_planar_batch_mixed_layouts():
    ents, host = [], []
    for qt, N, K, seed, planar in [(Q4, 1000, 5120, 1, True), (Q6, 48, 5120, 2, True), (Q5, 300, 6144, 3, False),
                                   (Q6, 200, 17408, 4, True), (Q4, 77, 2048, 5, False)]:
        W = synth.superblocks(qt, N, K, seed)
        x = synth.activations(K, 1, seed)
        Wd = _repacked(qt, W, N, K) if planar else dev(W.reshape(-1))
        ents.append((qt | (P if planar else 0), Wd, dev(x).reshape(-1), N, K))
        host.append((qt, W, x, N, K))
    ys = binding.gemv_batch(ents)
    torch.cuda.synchronize()
    for (qt, W, x, N, K), e, y in zip(host, ents, ys):
        y1 = binding.gemv(*e).cpu().numpy().reshape(-1)
        yb = y.cpu().numpy()
        assert np.array_equal(yb.view(np.uint32), y1.view(np.uint32))
        y_ref, S = oracle.gemv(qt, W, x, K)
        assert_row_bound(yb, y_ref, S, f"batch type {e[0]:#x}")


# Q6_K launches on PLANAR rows with at most 768 threads run two-row rounds
# with two units in flight.  Odd rows per lane leave the last round half used
# (3400x17408: 2 phases of 7 rows; 2300x11008: 3 phases of 3; 2600x8192: one
# phase of 11); 4000x5120 has 8 phases of 2 rows; 5120x17408 is the FFN down
# projection.  Every row is checked against the oracle and must equal the
# GGUF launch bit for bit (the summation order depends only on the segment
# length).
@pytest.mark.parametrize("N,K", [(3400, 17408), (2300, 11008), (2600, 8192), (4000, 5120), (5120, 17408)])
def test_planar_q6k_two_row_rounds(N, K):
    W = synth.superblocks(Q6, N, K, 70 + N)
    x = synth.activations(K, 1, 70 + N)
    Wp = _repacked(Q6, W, N, K)
    yp = binding.gemv(Q6 | P, Wp, dev(x).reshape(-1), N, K).cpu().numpy().reshape(-1)
    yg = gpu_gemv(Q6, W, x, N, K).reshape(-1)
    assert np.array_equal(yp.view(np.uint32), yg.view(np.uint32)), "planar != GGUF"
    y_ref, S = oracle.gemv(Q6, W, x, K)
    assert_row_bound(yp, y_ref, S, f"Q6_K planar {N}x{K}")


def test_planar_q6k_two_row_rounds_merged_and_pair():
    """The same rounds inside the merged launch (bit-identical to single calls)
    and in the SwiGLU pair (1700 x 17408: 2 phases of 4 paired rows;
    bit-identical to GGUF rows and within the oracle's bound)."""
    ents, host = [], []
    for qt, N, K, seed in [(Q6, 3400, 17408, 11), (Q6, 48, 5120, 12), (Q4, 1000, 5120, 13)]:
        W = synth.superblocks(qt, N, K, seed)
        x = synth.activations(K, 1, seed)
        ents.append((qt | P, _repacked(qt, W, N, K), dev(x).reshape(-1), N, K))
        host.append((qt, W, x, N, K))
    ys = binding.gemv_batch(ents)
    torch.cuda.synchronize()
    for (qt, W, x, N, K), e, y in zip(host, ents, ys):
        y1 = binding.gemv(*e).cpu().numpy().reshape(-1)
        yb = y.cpu().numpy()
        assert np.array_equal(yb.view(np.uint32), y1.view(np.uint32)), f"merged != single {N}x{K}"
        y_ref, S = oracle.gemv(qt, W, x, K)
        assert_row_bound(yb, y_ref, S, f"merged type {e[0]:#x} {N}x{K}")

    N, K = 1700, 17408
    Wg, Wu = synth.superblocks(Q6, N, K, 14), synth.superblocks(Q6, N, K, 15)
    x = synth.activations(K, 1, 14)
    Wgd, Wud, xd = dev(Wg.reshape(-1)), dev(Wu.reshape(-1)), dev(x).reshape(-1)
    a = binding.gemv_swiglu(Q6, Wgd, Wud, xd, N, K)
    b = binding.gemv_swiglu(Q6 | P, binding.repack(Q6, Wgd, N, K), binding.repack(Q6, Wud, N, K), xd, N, K)
    torch.cuda.synchronize()
    a, b = a.cpu().numpy().reshape(-1), b.cpu().numpy().reshape(-1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "planar pair != GGUF pair"
    y_ref, g, Sg, u, Su = oracle.swiglu(Q6, Wg, Wu, x, K)
    y_ref = y_ref.reshape(-1)
    tol = oracle.swiglu_bound(y_ref, g.reshape(-1), Sg.reshape(-1), u.reshape(-1), Su.reshape(-1))
    assert oracle.within(b, y_ref, tol, False).all(), "Q6_K planar SwiGLU pair outside the oracle's bound"
