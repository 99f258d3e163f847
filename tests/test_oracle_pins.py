"""CPU-only: the oracle pinned against facts that are not the oracle (see oracle_checks)."""
import numpy as np
import pytest

import oracle
import oracle_checks as oc
from quant_dequant_gemv_amd import synth


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: getattr(f, "__name__", "check"))
def test_pin(orc, check):
    check(orc)


def test_gemv_dot_of_dequant(orc):
    oc.check_gemv_dot_of_dequant(orc, synth)


def test_tolerance_plumbing():
    oc.check_tolerance_plumbing(oracle.within_row_bound)


def test_threads_deterministic(orc):
    W = synth.superblocks(synth.Q4_K, 64, 2048, 3)
    x = synth.activations(2048, 2, 3)
    y1, S1 = orc.gemv(synth.Q4_K, W, x, 2048, nthreads=1)
    y8, S8 = orc.gemv(synth.Q4_K, W, x, 2048, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(S1, S8)


def test_bad_arguments(orc):
    with pytest.raises(ValueError):
        orc.dequant(99, np.zeros(144, np.uint8), 256)
    with pytest.raises(ValueError):
        orc.gemv(synth.Q4_K, np.zeros(144, np.uint8), np.zeros(100, np.float16), 100)
    assert orc.block_bytes(99) == -1


def test_generator_distribution(orc):
    """The synthetic superblocks have the stated field distributions."""
    W = synth.superblocks(synth.Q4_K, 64, 5120, 0).reshape(-1, 144)
    d = orc.half_to_float(W[:, 0:2].copy().view(np.uint16).ravel())
    dmin = orc.half_to_float(W[:, 2:4].copy().view(np.uint16).ravel())
    for v in (d, dmin):
        assert v.min() >= 2.0 ** -12 and v.max() <= 2.0 ** -6
        assert abs(np.log2(v).mean() + 9.0) < 0.1  # log-uniform on [-12, -6]
    counts = np.zeros(64)
    for blk in W[:400]:
        for j in range(8):
            sc, m = orc.k_scale_min(blk[4:16], j)
            counts[sc] += 1
            counts[m] += 1
    expected = counts.sum() / 64
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 120  # 63 degrees of freedom; p ~ 1e-5 at 120
    W6 = synth.superblocks(synth.Q6_K, 16, 17408, 4).reshape(-1, 210)
    sc6 = W6[:, 192:208].view(np.int8)
    assert sc6.min() == -32 and sc6.max() == 31
    x = synth.activations(5120, 1, 0)
    assert x.dtype == np.float16 and abs(float(x.astype(np.float64).std()) - 1.0) < 0.05


def test_generator_seeded():
    a = synth.superblocks(synth.Q5_K, 8, 512, 42)
    b = synth.superblocks(synth.Q5_K, 8, 512, 42)
    c = synth.superblocks(synth.Q5_K, 8, 512, 43)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (8, 2 * 176)


def test_decode_stream_shapes():
    st = synth.decode_stream()
    assert len(st) == 64 * 7
    att = [e for e in st if e["name"] == "attn_q"]
    assert [e["layer"] for e in att] == list(range(3, 64, 4))
    assert synth.weight_bytes(st) == 14_576_209_920
