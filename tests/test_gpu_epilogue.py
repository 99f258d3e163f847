"""GPU parity of the fused epilogues through the C ABI (qk_gemv_ex,
qk_gemv_swiglu): residual add (separate and in place), fp16 y, and the SwiGLU
pair (silu(Wg x) * (Wu x) in one launch), for the one-column kernel and the
verify form, against the oracle's f64 definitions within the tolerances the
row bound implies (oracle.residual_bound, oracle.swiglu_bound).  fp16 y is
also the round-to-nearest-even of the same launch's fp32 y, bit for bit."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, needs_gpu, torch
from quant_dequant_gemv_amd import binding, synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6, IQ4 = synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.IQ4_XS
TYPES = [Q4, Q5, Q6, IQ4]
NAMES = {Q4: "Q4_K", Q5: "Q5_K", Q6: "Q6_K", IQ4: "IQ4_XS"}
# ragged rows, a partial 16-unit step, a long K (several x segments)
# (29 x 33024: two K segments of the one-column kernel, the second of 4 units)
SHAPES = [(1, 256), (37, 1280), (130, 5120), (300, 6144), (61, 17408), (29, 33024)]


def _assert_within(y, y_ref, tol, what, f16=False):
    y = np.asarray(y, dtype=np.float64).reshape(y_ref.shape)
    bad = ~oracle.within(y, y_ref, tol, f16)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, 1.0, 0.0)), y.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the bound; worst at {i}: "
                             f"gpu={y[i]!r} ref={y_ref[i]!r} tol={tol[i]!r}")


def _residual(N, ncols, seed):
    return (np.random.default_rng([seed, 7]).standard_normal((N, ncols)) * 4).astype(np.float32)


# 12 / 16 / 17 / 32 columns: the tile kernels, one and two groups of 16
# columns (the residual read before the shares are added)
@pytest.mark.parametrize("ncols", [1, 2, 5, 8, 12, 16, 17, 32])
@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SHAPES)
def test_residual_and_f16(qt, N, K, ncols):
    W = synth.superblocks(qt, N, K, 500 + N)
    x = synth.activations(K, ncols, 500 + N)
    r = _residual(N, ncols, N)
    Wd, xd, rd = dev(W.reshape(-1)), dev(x), dev(r)
    y32 = binding.gemv_ex(qt, Wd, xd, N, K, residual=rd)
    y16 = binding.gemv_ex(qt, Wd, xd, N, K, residual=rd, f16=True)
    yin = rd.clone()  # in place: y += W x
    binding.gemv_ex(qt, Wd, xd, N, K, residual=yin, out=yin)
    torch.cuda.synchronize()
    y32, y16, yin = y32.cpu().numpy(), y16.cpu().numpy(), yin.cpu().numpy().reshape(N, ncols)
    y_ref, S = oracle.gemv_residual(qt, W, x, K, r)
    what = f"{NAMES[qt]} N={N} K={K} ncols={ncols}"
    _assert_within(y32, y_ref, oracle.residual_bound(y_ref, S), what + " fp32")
    _assert_within(y16, y_ref, oracle.residual_bound(y_ref, S, f16=True), what + " fp16", f16=True)
    with np.errstate(over="ignore"):  # values past the fp16 range round to infinity on both sides
        rne = y32.astype(np.float16)
    assert np.array_equal(y16.view(np.uint16), rne.view(np.uint16)), what + " fp16 = RNE(fp32)"
    assert np.array_equal(yin.view(np.uint32), y32.view(np.uint32)), what + " in place"


@pytest.mark.parametrize("ncols", [1, 3, 8])
@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_ex_without_epilogue_is_qk_gemv(qt, ncols):
    N, K = 257, 5120
    W = synth.superblocks(qt, N, K, 61)
    x = synth.activations(K, ncols, 61)
    Wd, xd = dev(W.reshape(-1)), dev(x)
    a = binding.gemv(qt, Wd, xd, N, K)
    b = binding.gemv_ex(qt, Wd, xd, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("ncols", [1, 2, 4, 5, 8, 9, 16, 24])
@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SHAPES)
def test_swiglu(qt, N, K, ncols):
    Wg = synth.superblocks(qt, N, K, 600 + N)
    Wu = synth.superblocks(qt, N, K, 700 + N)
    x = synth.activations(K, ncols, 600 + N)
    Wgd, Wud, xd = dev(Wg.reshape(-1)), dev(Wu.reshape(-1)), dev(x)
    y32 = binding.gemv_swiglu(qt, Wgd, Wud, xd, N, K)
    y16 = binding.gemv_swiglu(qt, Wgd, Wud, xd, N, K, f16=True)
    torch.cuda.synchronize()
    y32, y16 = y32.cpu().numpy(), y16.cpu().numpy()
    y_ref, g, Sg, u, Su = oracle.swiglu(qt, Wg, Wu, x, K)
    what = f"{NAMES[qt]} N={N} K={K} ncols={ncols}"
    _assert_within(y32, y_ref, oracle.swiglu_bound(y_ref, g, Sg, u, Su), what + " fp32")
    _assert_within(y16, y_ref, oracle.swiglu_bound(y_ref, g, Sg, u, Su, f16=True), what + " fp16", f16=True)
    with np.errstate(over="ignore"):  # values past the fp16 range round to infinity on both sides
        rne = y32.astype(np.float16)
    assert np.array_equal(y16.view(np.uint16), rne.view(np.uint16)), what + " fp16 = RNE(fp32)"
    assert np.isfinite(y32).all()  # (fp16 may overflow: its infinities are checked above)


@pytest.mark.parametrize("ncols", [1, 4])
@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_swiglu_same_tensor_and_planar(qt, ncols):
    """Wg == Wu is allowed (y = silu(g) * g); PLANAR rows give the same bits
    as GGUF rows at ncols = 1 (the k-quants: IQ4_XS has no PLANAR layout)."""
    N, K = 211, 5120
    W = synth.superblocks(qt, N, K, 81)
    x = synth.activations(K, ncols, 81)
    Wd, xd = dev(W.reshape(-1)), dev(x)
    y = binding.gemv_swiglu(qt, Wd, Wd, xd, N, K)
    torch.cuda.synchronize()
    y_ref, g, Sg, u, Su = oracle.swiglu(qt, W, W, x, K)
    _assert_within(y.cpu().numpy(), y_ref, oracle.swiglu_bound(y_ref, g, Sg, u, Su), f"{NAMES[qt]} same tensor")
    if ncols == 1 and qt != IQ4:
        Wp = binding.repack(qt, Wd, N, K)
        W2 = synth.superblocks(qt, N, K, 82)
        W2d = dev(W2.reshape(-1))
        W2p = binding.repack(qt, W2d, N, K)
        a = binding.gemv_swiglu(qt, Wd, W2d, xd, N, K)
        b = binding.gemv_swiglu(qt | binding.PLANAR, Wp, W2p, xd, N, K)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("ncols", [1, 2, 8])
def test_swiglu_ffn_shape_all_rows(ncols):
    """The FFN gate/up pair at its real shape (Q4_K 17408 x 5120), every row."""
    N, K = 17408, 5120
    Wg = synth.superblocks(Q4, N, K, 2)
    Wu = synth.superblocks(Q4, N, K, 3)
    x = synth.activations(K, ncols, 2)
    y = binding.gemv_swiglu(Q4, dev(Wg.reshape(-1)), dev(Wu.reshape(-1)), dev(x), N, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, g, Sg, u, Su = oracle.swiglu(Q4, Wg, Wu, x, K)
    _assert_within(y, y_ref, oracle.swiglu_bound(y_ref, g, Sg, u, Su), f"ffn gate/up ncols={ncols}")


def test_residual_down_shape_all_rows():
    """FFN down (Q6_K 5120 x 17408) with its residual, in place, every row."""
    N, K = 5120, 17408
    W = synth.superblocks(Q6, N, K, 4)
    x = synth.activations(K, 1, 4)
    r = _residual(N, 1, 4)
    y = dev(r.copy())
    binding.gemv_ex(Q6, dev(W.reshape(-1)), dev(x), N, K, residual=y, out=y)
    torch.cuda.synchronize()
    y = y.cpu().numpy().reshape(N, 1)
    y_ref, S = oracle.gemv_residual(Q6, W, x, K, r)
    _assert_within(y, y_ref, oracle.residual_bound(y_ref, S), "ffn down + residual")


@pytest.mark.parametrize("planar", [False, True], ids=["GGUF", "PLANAR"])
def test_front_loaded_epilogues_all_rows(planar):
    """Front-loaded row splits with empty workgroups in the last dispatch
    round: the SwiGLU pair at 9220 x 5120 (252 of the last round's workgroups
    have no rows) and the residual added in place at 18440 x 5120 (248).
    Every row."""
    K = 5120
    Ng, Nr = 9220, 18440
    Wg, Wu = synth.superblocks(Q4, Ng, K, 31), synth.superblocks(Q4, Ng, K, 32)
    Wr = synth.superblocks(Q4, Nr, K, 33)
    x = synth.activations(K, 1, 31)
    r = _residual(Nr, 1, 33)
    Wgd, Wud, Wrd, xd = dev(Wg.reshape(-1)), dev(Wu.reshape(-1)), dev(Wr.reshape(-1)), dev(x)
    t = Q4
    if planar:
        Wgd, Wud = binding.repack(Q4, Wgd, Ng, K), binding.repack(Q4, Wud, Ng, K)
        Wrd = binding.repack(Q4, Wrd, Nr, K)
        t = Q4 | binding.PLANAR
    ys = binding.gemv_swiglu(t, Wgd, Wud, xd, Ng, K)
    yr = dev(r.copy())
    binding.gemv_ex(t, Wrd, xd, Nr, K, residual=yr, out=yr)
    torch.cuda.synchronize()
    y_ref, g, Sg, u, Su = oracle.swiglu(Q4, Wg, Wu, x, K)
    _assert_within(ys.cpu().numpy(), y_ref, oracle.swiglu_bound(y_ref, g, Sg, u, Su), f"swiglu {Ng}x{K}")
    y_ref, S = oracle.gemv_residual(Q4, Wr, x, K, r)
    _assert_within(yr.cpu().numpy().reshape(Nr, 1), y_ref, oracle.residual_bound(y_ref, S), f"residual {Nr}x{K}")


@pytest.mark.parametrize("qt,N,K", [(Q4, 17408, 5120), (Q4, 200000, 256), (Q5, 120000, 512)],
                         ids=["rows68_per_wg", "rows782_per_wg", "Q5_rows469_per_wg"])
def test_residual_many_rows_per_workgroup(qt, N, K):
    """Each 16-lane row group of the final reduction stores several rows (3,
    and more than 16, whose residuals are read late): every pass must add its
    own row's residual.  Every row."""
    W = synth.superblocks(qt, N, K, 90)
    x = synth.activations(K, 1, 90)
    r = _residual(N, 1, 90)
    y = binding.gemv_ex(qt, dev(W.reshape(-1)), dev(x), N, K, residual=dev(r))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, S = oracle.gemv_residual(qt, W, x, K, r)
    _assert_within(y, y_ref, oracle.residual_bound(y_ref, S), f"{NAMES[qt]} {N}x{K} residual")
