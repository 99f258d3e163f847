"""GPU parity of the few-column verify form (ncols 2..8, matrix cores) against
the CPU oracle, through the C ABI: per-(row, column) 1e-4 bound, exact one-hot
columns, determinism, and the full verify shape, every row."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_row_bound, gpu_gemv, needs_gpu, same_f32
from quant_dequant_gemv_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6, IQ4 = synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.IQ4_XS
TYPES = [Q4, Q5, Q6, IQ4]
NAMES = {Q4: "Q4_K", Q5: "Q5_K", Q6: "Q6_K", IQ4: "IQ4_XS"}

# ragged rows (not a multiple of 4), K with a partial 16-unit step, the real K
# values, and K = 29184 so that the x planes need several tiles at ncols = 8
SHAPES = [(1, 256), (5, 512), (47, 1280), (130, 5120), (61, 6144), (37, 17408), (9, 29184)]


@pytest.mark.parametrize("ncols", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SHAPES)
def test_verify_row_bound(qt, N, K, ncols):
    W = synth.superblocks(qt, N, K, 300 + N)
    x = synth.activations(K, ncols, 300 + N)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert y.shape == (N, ncols)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} N={N} K={K} ncols={ncols}")


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_verify_one_hot_columns_exact(qt):
    """x[:, c] = e_{k_c}: column c of y must be column k_c of W, bit-exact."""
    N, K, ncols = 53, 1024, 8
    W = synth.superblocks(qt, N, K, 17)
    w = oracle.dequant(qt, W, K)
    ks = [0, 1, 2, 3, 63, 200, 511, 1023]
    x = np.zeros((K, ncols), dtype=np.float16)
    for c, k in enumerate(ks):
        x[k, c] = 1.0
    y = gpu_gemv(qt, W, x, N, K)
    for c, k in enumerate(ks):
        assert same_f32(y[:, c], w[:, k]), f"{NAMES[qt]} column {c} (k={k})"


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_verify_deterministic_and_matches_single_column(qt):
    N, K = 200, 5120
    W = synth.superblocks(qt, N, K, 21)
    x = synth.activations(K, 4, 21)
    y1 = gpu_gemv(qt, W, x, N, K)
    y2 = gpu_gemv(qt, W, x, N, K)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    y_ref, S = oracle.gemv(qt, W, x, K)
    for c in range(4):  # each column also agrees with the one-column kernel within the bound
        yc = gpu_gemv(qt, W, np.ascontiguousarray(x[:, c:c + 1]), N, K)
        assert_row_bound(yc, y_ref[:, c:c + 1], S[:, c:c + 1], f"column {c} one-column")


@pytest.mark.parametrize("ncols", [2, 4, 8])
def test_verify_full_shape_all_rows(ncols):
    c = synth.VERIFY
    N, K = c["N"], c["K"]
    W = synth.superblocks(c["qtype"], N, K, c["seed"])
    x = synth.activations(K, ncols, c["seed"])
    y = gpu_gemv(c["qtype"], W, x, N, K)
    y_ref, S = oracle.gemv(c["qtype"], W, x, K)
    assert_row_bound(y, y_ref, S, f"verify {N}x{K} ncols={ncols}")


@pytest.mark.parametrize("ncols", [2, 4, 8])
def test_verify_iq4xs_ffn_shape_all_rows(ncols):
    N, K = 17408, 5120
    W = synth.superblocks(IQ4, N, K, 1003)
    x = synth.activations(K, ncols, 1003)
    y = gpu_gemv(IQ4, W, x, N, K)
    y_ref, S = oracle.gemv(IQ4, W, x, K)
    assert_row_bound(y, y_ref, S, f"IQ4_XS {N}x{K} ncols={ncols}")


@pytest.mark.parametrize("case", synth.MIXED, ids=lambda c: c["name"])
def test_verify_mixed_shapes_all_rows(case):
    N, K, qt = case["N"], case["K"], case["qtype"]
    W = synth.superblocks(qt, N, K, case["seed"])
    x = synth.activations(K, 4, case["seed"])
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{case['name']} ncols=4")


# Row counts at which each workgroup's quads (4 rows) per lane take straight-
# line rounds of every length 1..8 (the launch picks the length from the rows
# per workgroup and the phases), for one and two column blocks.  Plain Q4_K
# launches of two blocks also take workgroups above 512 threads in rounds of
# 1..3 quads (8254, 16395, 25608 x 256 and the FFN shape at 6 columns).
ROUND_CASES = [(1, 256, 2), (12328, 256, 2), (14365, 256, 2), (27654, 256, 2), (24647, 256, 2),
               (10291, 5120, 2), (6217, 5120, 2), (14365, 5120, 2),
               (8254, 256, 8), (14365, 256, 8), (18439, 256, 8), (24647, 256, 8), (35899, 256, 8),
               (6217, 5120, 8), (7187, 5120, 8), (27680, 256, 8), (16395, 256, 8), (25608, 256, 8),
               (17408, 5120, 6)]


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K,ncols", ROUND_CASES)
def test_verify_round_lengths_all_rows(qt, N, K, ncols):
    """Every row of shapes that reach every round length, including rounds
    that run past the lane's last quad."""
    W = synth.superblocks(qt, N, K, 900 + N)
    x = synth.activations(K, ncols, 900 + N)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} N={N} K={K} ncols={ncols}")
    assert np.isfinite(y).all()


# Wider verification on the 16x16x16 tiles: 9-16 columns in one group of 16
# (the unused columns of the tile zero), 17-32 in two groups; K = 17408 takes
# several segments of x planes (Q6_K / IQ4_XS: four), N = 5 and 37 leave
# short tiles and idle waves.
@pytest.mark.parametrize("ncols", [9, 12, 13, 16, 17, 24, 25, 32])
@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", [(5, 512), (130, 5120), (37, 17408)])
def test_verify_wide_row_bound(qt, N, K, ncols):
    W = synth.superblocks(qt, N, K, 1300 + N)
    x = synth.activations(K, ncols, 1300 + N)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert y.shape == (N, ncols)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} N={N} K={K} ncols={ncols}")


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_verify_wide_one_hot_columns_exact(qt):
    """Column c of x = e_{k_c}: column c of y is column k_c of W, bit-exact,
    in every column group."""
    N, K, ncols = 53, 1024, 17
    W = synth.superblocks(qt, N, K, 19)
    w = oracle.dequant(qt, W, K)
    ks = [0, 1, 2, 3, 63, 64, 127, 200, 255, 256, 511, 512, 700, 768, 1000, 1022, 1023]
    x = np.zeros((K, ncols), dtype=np.float16)
    for c, k in enumerate(ks):
        x[k, c] = 1.0
    y = gpu_gemv(qt, W, x, N, K)
    for c, k in enumerate(ks):
        assert same_f32(y[:, c], w[:, k]), f"{NAMES[qt]} column {c} (k={k})"


@pytest.mark.parametrize("ncols", [16, 17])
@pytest.mark.parametrize("case", [synth.VERIFY] + list(synth.MIXED), ids=lambda c: c.get("name", "q4k_17408x5120"))
def test_verify_wide_full_shape_all_rows(case, ncols):
    """Every row at the verify shape and the mixed-type shapes (Q6_K FFN
    down: four segments of x planes on the tiles; Q5_K output projection)."""
    c = case
    N, K = c["N"], c["K"]
    W = synth.superblocks(c["qtype"], N, K, c["seed"])
    x = synth.activations(K, ncols, c["seed"])
    y = gpu_gemv(c["qtype"], W, x, N, K)
    y_ref, S = oracle.gemv(c["qtype"], W, x, K)
    assert_row_bound(y, y_ref, S, f"verify {N}x{K} ncols={ncols}")
