"""CPU: the test-side PLANAR packer keeps every byte of a row exactly once
(a permutation plus zero padding), and moves the pieces a unit reads to the
positions the layout names."""
import numpy as np
import pytest

from kquant_planar import BLOCK, Q4_K, Q5_K, Q6_K, pack, planar_row_bytes
from quant_dequant_gemv_amd import synth


@pytest.mark.parametrize("qt", [Q4_K, Q5_K, Q6_K])
@pytest.mark.parametrize("K", [256, 1280, 5120, 17408])
def test_planar_is_a_byte_permutation(qt, K):
    W = synth.superblocks(qt, 3, K, 9)
    P = pack(qt, W, K)
    n = (K // 256) * BLOCK[qt]
    assert P.shape == (3, planar_row_bytes(qt, K))
    for r in range(3):
        assert np.array_equal(np.sort(P[r, :n]), np.sort(W[r].reshape(-1)))
        assert not P[r, n:].any()
    if qt != Q6_K:
        assert P.shape[1] == n


def test_planar_positions_by_hand():
    K = 512  # two superblocks, eight units
    for qt in (Q4_K, Q5_K, Q6_K):
        W = synth.superblocks(qt, 1, K, 4).reshape(2, BLOCK[qt])
        P = pack(qt, W.reshape(1, -1), K)[0]
        S, U = 2, 8
        if qt == Q4_K:
            assert np.array_equal(P[16:32], W[1, 0:16])                      # header of superblock 1
            u = 6                                                            # superblock 1, q = 2
            assert np.array_equal(P[16 * S + 16 * u:16 * S + 16 * u + 16], W[1, 16 + 64:16 + 80])
            assert np.array_equal(P[16 * S + 16 * U + 16 * u:][:16], W[1, 16 + 80:16 + 96])
        elif qt == Q5_K:
            assert np.array_equal(P[16 * S + 16:16 * S + 32], W[1, 16:32])  # QH0 of superblock 1
            assert np.array_equal(P[32 * S:32 * S + 16], W[0, 32:48])       # QH1 of superblock 0
            u = 3
            assert np.array_equal(P[48 * S + 16 * u:][:16], W[0, 48 + 96:48 + 112])
        else:
            u = 7                                                            # superblock 1, n = 1, b = 1
            assert np.array_equal(P[16 * u:16 * u + 16], W[1, 64 + 16:64 + 32])
            assert np.array_equal(P[16 * U + 16 * u:][:16], W[1, 64 + 48:64 + 64])
            assert np.array_equal(P[32 * U + 16 * u:][:16], W[1, 128 + 48:128 + 64])
            assert list(P[48 * U + 4 * u:48 * U + 4 * u + 4]) == [W[1, 192 + 8 + 2 * t + 1] for t in range(4)]
            assert np.array_equal(P[52 * U + 2:52 * U + 4], W[1, 208:210])
