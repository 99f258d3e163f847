"""CPU-only: the oracle's fused-epilogue definitions (silu, residual add,
SwiGLU) and their tolerances, pinned against closed forms, scipy's logistic
function, exact integer cases, and simulated fp32 evaluations; plus plausible
mistakes in them, each shown to fail a pin."""
import math

import numpy as np
import pytest
from scipy.special import expit

import kquant_pack as kp
import oracle

Q4_K, Q5_K, Q6_K = kp.Q4_K, kp.Q5_K, kp.Q6_K
ONE, ZERO = kp.half_bits(1.0), 0


def integer_tensor(qt, q):
    """Superblock rows whose dequantised weights are the integers q (Q6_K: q - 32):
    d = 1, dmin = 0, every scale 1."""
    N, K = q.shape
    rows = []
    for n in range(N):
        blocks = []
        for s in range(K // 256):
            qq = q[n, 256 * s:256 * s + 256]
            if qt == Q6_K:
                blocks.append(kp.make_q6_block(ONE, [1] * 16, qq))
            else:
                blocks.append(kp.make_k_block(qt, ONE, ZERO, [1] * 8, [0] * 8, qq))
        rows.append(np.concatenate(blocks))
    return np.stack(rows)


# ---------------------------------------------------------------- silu

def check_silu(silu):
    assert silu(0.0) == 0.0
    l3 = math.log(3.0)  # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert abs(silu(l3) - 0.75 * l3) <= 1e-15 * l3
    assert abs(silu(-l3) + 0.25 * l3) <= 1e-15 * l3
    z = np.linspace(-40.0, 40.0, 8001)
    # silu(z) - silu(-z) = z * (sigmoid(z) + sigmoid(-z)) = z
    assert np.allclose(silu(z) - silu(-z), z, rtol=1e-14, atol=1e-14)
    assert np.allclose(silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert silu(800.0) == 800.0
    big_neg = silu(-800.0)
    assert big_neg == 0.0 and not np.isnan(big_neg)


def test_silu_pins():
    check_silu(oracle.silu)


def test_silu_slope_bound():
    """SILU_SLOPE bounds |silu'| = |s (1 + z (1 - s))| on a dense grid."""
    z = np.linspace(-60.0, 60.0, 1200001)
    s = expit(z)
    assert np.abs(s * (1 + z * (1 - s))).max() <= oracle.SILU_SLOPE


# ---------------------------------------------------------------- residual

def check_residual(gemv_residual):
    rng = np.random.default_rng(31)
    N, K, nc = 9, 512, 3
    q = rng.integers(0, 16, (N, K))
    W = integer_tensor(Q4_K, q)
    # small-integer x and residual: every sum is an exact integer in f64
    x = rng.integers(-3, 4, (K, nc)).astype(np.float16)
    r = rng.integers(-1000, 1000, (N, nc)).astype(np.float32)
    exact = q.astype(np.int64) @ x.astype(np.int64) + r.astype(np.int64)
    y, S = gemv_residual(Q4_K, W, x, K, r)
    assert np.array_equal(y, exact.astype(np.float64))
    # x = 0: y is the residual
    y0, S0 = gemv_residual(Q4_K, W, np.zeros((K, nc), np.float16), K, r)
    assert np.array_equal(y0, r.astype(np.float64)) and not S0.any()


def test_residual_pins():
    check_residual(oracle.gemv_residual)


# ---------------------------------------------------------------- swiglu

def check_swiglu(swiglu):
    rng = np.random.default_rng(32)
    N, K, nc = 11, 768, 2
    for qt in (Q4_K, Q6_K):
        levels = 16 if qt == Q4_K else 64
        qg, qu = rng.integers(0, levels, (N, K)), rng.integers(0, levels, (N, K))
        Wg, Wu = integer_tensor(qt, qg), integer_tensor(qt, qu)
        x = (rng.standard_normal((K, nc)) / 64).astype(np.float16)
        off = 32.0 if qt == Q6_K else 0.0
        g = (qg - off) @ x.astype(np.float64)
        u = (qu - off) @ x.astype(np.float64)
        y, g_o, Sg, u_o, Su = swiglu(qt, Wg, Wu, x, K)
        assert np.allclose(g_o, g, rtol=1e-12, atol=1e-12) and np.allclose(u_o, u, rtol=1e-12, atol=1e-12)
        ref = g * expit(g) * u
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12), f"type {qt}"
        assert np.allclose(Sg, np.abs(qg - off) @ np.abs(x.astype(np.float64)), rtol=1e-12)


def test_swiglu_pins():
    check_swiglu(oracle.swiglu)


# ---------------------------------------------------------------- bounds

def _f32(v):
    return np.asarray(v, dtype=np.float32)


def test_residual_bound_accepts_simulated_fp32_and_rejects_twice_the_error():
    rng = np.random.default_rng(33)
    n = 20000
    y = rng.standard_normal(n) * 10
    S = np.abs(y) * 5 + rng.random(n) * 50
    r = rng.standard_normal(n).astype(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    dot = _f32(y + sign * 0.999e-4 * S)  # a GEMV result at the edge of its bound
    for f16 in (False, True):
        out = _f32(dot + r)  # the fp32 add
        if f16:
            out = out.astype(np.float16)
        err = np.abs(out.astype(np.float64) - (y + r))
        assert (err <= oracle.residual_bound(y + r, S, f16)).all()
    assert not (np.abs(2.2e-4 * S) <= oracle.residual_bound(y + r, S)).any()


def test_swiglu_bound_accepts_simulated_fp32_and_rejects_twice_the_error():
    rng = np.random.default_rng(34)
    n = 20000
    g = rng.standard_normal(n) * 4
    u = rng.standard_normal(n) * 4
    Sg = np.abs(g) * 5 + rng.random(n) * 20
    Su = np.abs(u) * 5 + rng.random(n) * 20
    s1 = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    s2 = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    g32, u32 = _f32(g + s1 * 0.999e-4 * Sg), _f32(u + s2 * 0.999e-4 * Su)
    y_ref = oracle.silu(g) * u
    with np.errstate(over="ignore"):
        sil32 = g32 / (np.float32(1) + np.exp(-g32))
    for f16 in (False, True):
        out = _f32(sil32 * u32)
        if f16:
            out = out.astype(np.float16)
        err = np.abs(out.astype(np.float64) - y_ref)
        assert (err <= oracle.swiglu_bound(y_ref, g, Sg, u, Su, f16)).all()
    # Where silu' is ~1 (g >> 0) and both errors push y the same way, twice
    # the GEMV error on both inputs must fall outside the bound everywhere.
    gp = 6.0 + np.abs(g)
    Sgp = np.abs(gp) * 5 + rng.random(n) * 20
    su = np.sign(u)
    y_p = oracle.silu(gp) * u
    # dy = silu'(g) u dg + silu(g) du: dg > 0 and du of u's sign add up
    g2, u2 = gp + 2.2e-4 * Sgp, u + su * 2.2e-4 * Su
    err2 = np.abs(oracle.silu(g2) * u2 - y_p)
    assert (err2 > oracle.swiglu_bound(y_p, gp, Sgp, u, Su)).all()


# ---------------------------------------------------------------- mutants

MUTANT_SILU = {
    "sign of the exponent": lambda z: np.asarray(z, np.float64) / (1.0 + np.exp(np.asarray(z, np.float64))),
    "sigmoid only": lambda z: expit(np.asarray(z, np.float64)),
    "dropped 1": lambda z: np.asarray(z, np.float64) / np.exp(-np.asarray(z, np.float64)),
}


@pytest.mark.parametrize("name", list(MUTANT_SILU))
def test_silu_mutants_fail_a_pin(name):
    with np.errstate(over="ignore", invalid="ignore"):
        with pytest.raises(AssertionError):
            check_silu(MUTANT_SILU[name])


def test_epilogue_mutants_fail_a_pin():
    def swapped(qt, Wg, Wu, x, K):  # gate and up exchanged
        y, g, Sg, u, Su = oracle.swiglu(qt, Wu, Wg, x, K)
        return y, u, Su, g, Sg

    def no_gate(qt, Wg, Wu, x, K):  # g * u without the sigmoid
        y, g, Sg, u, Su = oracle.swiglu(qt, Wg, Wu, x, K)
        return g * u, g, Sg, u, Su

    for m in (swapped, no_gate):
        with pytest.raises(AssertionError):
            check_swiglu(m)

    def minus_residual(qt, W, x, K, r):
        y, S = oracle.gemv(qt, W, x, K)
        return y - np.asarray(r, np.float64).reshape(y.shape), S

    with pytest.raises(AssertionError):
        check_residual(minus_residual)


def test_within_fp16_overflow_rule():
    tol = oracle.residual_bound(np.array([70000.0, 70000.0, 100.0, 65519.0, -90000.0, 65000.0]),
                                np.zeros(6), f16=True)
    y_ref = np.array([70000.0, 70000.0, 100.0, 65519.0, -90000.0, 65000.0])
    y = np.array([np.inf, -np.inf, np.inf, 65504.0, -np.inf, np.inf])
    ok = oracle.within(y, y_ref, tol, f16=True)
    assert ok.tolist() == [True, False, False, True, True, False]
    # without the fp16 rule an infinity is never accepted
    assert oracle.within(y, y_ref, tol).tolist() == [False, False, False, True, False, False]
    # RNE of fp32 values at the edge, as numpy rounds them
    edge = np.array([65519.996, 65520.0], dtype=np.float32)
    with np.errstate(over="ignore"):
        e16 = edge.astype(np.float16)
    assert np.isfinite(e16[0]) and np.isinf(e16[1])
