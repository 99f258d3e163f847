"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

* qk_dequant is bit-exact (-0 == +0) on every format and shape;
* qk_gemv (ncols = 1) is within |y - y_ref| <= 1e-4 * sum|w*x| per row, at
  small ragged sizes (several tiles) and on every row of every workload
  shape, in the launch configuration the benchmark uses; dequantisation is
  bit-exact on whole tensors of every workload shape;
* exactness pins: one-hot x returns a dequantised column bit-exactly, scaling
  x by a power of two scales y exactly, and repeated calls are bitwise equal.
"""
import numpy as np
import pytest

import oracle
from gpu_util import assert_row_bound, dev, gpu_dequant, gpu_gemv, needs_gpu, same_f32, torch
from kquant_pack import load_golden
from quant_dequant_gemv_amd import binding, synth

pytestmark = [pytest.mark.gpu, needs_gpu]

Q4, Q5, Q6, IQ4 = synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.IQ4_XS
TYPES = [Q4, Q5, Q6, IQ4]
NAMES = {Q4: "Q4_K", Q5: "Q5_K", Q6: "Q6_K", IQ4: "IQ4_XS"}

# (N, K): tiny, ragged row counts, several superblocks, the real K values, and
# K beyond one segment of the one-column kernel (512 units = 32768 weights):
# 33024 runs segments of 512 and 4 units, 65792 of 512, 512 and 4 (the short
# last segment leaves most lanes without a unit).
SMALL_SHAPES = [(1, 256), (47, 512), (48, 5120), (1023, 768), (129, 6144), (96, 17408), (40, 29184),
                (37, 33024), (20, 65792)]


def _case(qt, N, K, seed):
    return synth.superblocks(qt, N, K, seed), synth.activations(K, 1, seed)


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SMALL_SHAPES)
def test_dequant_bit_exact(qt, N, K):
    W, _ = _case(qt, N, K, 100 + N)
    assert same_f32(gpu_dequant(qt, W, N, K), oracle.dequant(qt, W, K))


def test_dequant_worked_examples():
    import glob, os
    here = os.path.join(os.path.dirname(__file__), "golden")
    paths = sorted(glob.glob(os.path.join(here, "q*_e*.txt")) + glob.glob(os.path.join(here, "iq*_e*.txt")))
    assert any("iq4xs" in p for p in paths)
    for path in paths:
        qt, form, block, values = load_golden(path)
        w = gpu_dequant(qt, block[None, :], 1, 256)[0]
        assert same_f32(w, oracle.dequant(qt, block[None, :], 256)[0]), path
        for i, v in values.items():
            assert w[i] == np.float32(v), (path, i)


def test_dequant_full_small_config():
    c = synth.SMALL
    W = synth.superblocks(c["qtype"], c["N"], c["K"], c["seed"])
    assert same_f32(gpu_dequant(c["qtype"], W, c["N"], c["K"]), oracle.dequant(c["qtype"], W, c["K"]))


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K", SMALL_SHAPES)
def test_gemv_row_bound(qt, N, K):
    W, x = _case(qt, N, K, 200 + N)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} N={N} K={K}")


def test_gemv_small_config_all_rows():
    c = synth.SMALL
    W = synth.superblocks(c["qtype"], c["N"], c["K"], c["seed"])
    x = synth.activations(c["K"], 1, c["seed"])
    y = gpu_gemv(c["qtype"], W, x, c["N"], c["K"])
    y_ref, S = oracle.gemv(c["qtype"], W, x, c["K"])
    worst = assert_row_bound(y, y_ref, S, "Q4_K 1024x5120")
    assert worst < 1e-5  # the factored fp32 form is far inside the bound


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_gemv_one_hot_is_a_column(qt):
    N, K = 77, 1024
    W = synth.superblocks(qt, N, K, 7)
    w = oracle.dequant(qt, W, K)
    for k in (0, 1, 2, 3, 5, 31, 32, 63, 64, 100, 255, 256, 511, 700, K - 1):
        x = np.zeros((K, 1), dtype=np.float16)
        x[k, 0] = 1.0
        y = gpu_gemv(qt, W, x, N, K)[:, 0]
        assert same_f32(y, w[:, k]), f"{NAMES[qt]} column {k}"


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_gemv_power_of_two_and_determinism(qt):
    N, K = 300, 5120
    W, x = _case(qt, N, K, 9)
    y1 = gpu_gemv(qt, W, x, N, K)
    y2 = gpu_gemv(qt, W, x, N, K)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    y4 = gpu_gemv(qt, W, (x.astype(np.float32) * 4).astype(np.float16), N, K)
    assert np.array_equal(y4, y1 * 4), "power-of-two scaling not exact"


@pytest.mark.parametrize("qt", TYPES, ids=lambda t: NAMES[t])
def test_gemv_subnormal_x(qt):
    N, K = 64, 2048
    W = synth.superblocks(qt, N, K, 11)
    x = (synth.activations(K, 1, 11).astype(np.float32) * 2.0 ** -18).astype(np.float16)
    assert (np.abs(x) < 2.0 ** -14).mean() > 0.5  # mostly fp16 subnormals
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} subnormal x")


# Every distinct GEMV shape of the workloads: the small case, the Q4_K
# projections, the Q6_K / Q5_K pair, and the remaining shapes of the decode
# token (attention k/v 1024 x 5120, DeltaNet alpha/beta 48 x 5120), each with
# its own seed.  Checked on every row (the oracle takes tens of ms per tensor).
FULL_SHAPES = [dict(synth.SMALL, name="small")] + synth.Q4K_PROJECTIONS + synth.MIXED + [
    dict(name="attn_k", qtype=Q4, N=1024, K=5120, seed=1001),
    dict(name="ssm_alpha", qtype=Q6, N=48, K=5120, seed=1002),
    dict(name="iq4xs_ffn_up", qtype=IQ4, N=17408, K=5120, seed=1003),
    dict(name="iq4xs_ffn_down", qtype=IQ4, N=5120, K=17408, seed=1004)]


# one GPU's share of an 8-way row split of the large projections (N / 8 rows)
SHARD_SHAPES = [dict(name="shard8_attn_qkv", qtype=Q4, N=1280, K=5120, seed=1101),
                dict(name="shard8_ffn_up", qtype=Q4, N=2176, K=5120, seed=1103),
                dict(name="shard8_ffn_down", qtype=Q6, N=640, K=17408, seed=1104),
                dict(name="shard8_ssm_out", qtype=Q5, N=640, K=6144, seed=1105)]


@pytest.mark.parametrize("case", FULL_SHAPES + SHARD_SHAPES, ids=lambda c: c["name"])
def test_gemv_full_shapes_all_rows(case):
    qt, N, K, seed = case["qtype"], case["N"], case["K"], case["seed"]
    W = synth.superblocks(qt, N, K, seed)
    x = synth.activations(K, 1, seed)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} {N}x{K} all rows")


@pytest.mark.parametrize("case", FULL_SHAPES, ids=lambda c: c["name"])
def test_dequant_full_shapes_bit_exact(case):
    qt, N, K, seed = case["qtype"], case["N"], case["K"], case["seed"]
    W = synth.superblocks(qt, N, K, seed)
    assert same_f32(gpu_dequant(qt, W, N, K), oracle.dequant(qt, W, K)), f"{NAMES[qt]} {N}x{K}"


@pytest.mark.parametrize("name,qt,N,K", [("ssm_alpha", Q6, 48, 5120), ("attn_k", Q4, 1024, 5120)])
def test_gemv_stream_small_shapes(name, qt, N, K):
    W, x = _case(qt, N, K, 1000 + N)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, name)


# At K = 5120 these row counts give every lane (Q4_K) 2 rows (one workgroup
# per CU), 4, 6, 8 and 9 rows in rounds of 4, 6, 8 and 12 (two to four small
# workgroups per CU; the 4-, 8- and 12-row rounds issue their first weights
# before x is staged, the 6-row rounds after), and three rounds of 12 (one
# workgroup per CU, the later rounds' rings issued in the loop); Q5_K one
# round of two rows and three rounds of four; Q6_K one-row rounds over twelve
# row phases, one and three rows per lane.  N is not a multiple of the
# workgroup count, so workgroups differ by one row.  Every row is checked.
@pytest.mark.parametrize("qt,N", [(Q4, 3000), (Q4, 6000), (Q4, 9000), (Q4, 17000), (Q4, 25600), (Q4, 38000),
                                  (Q5, 3000), (Q5, 9000), (Q6, 3000), (Q6, 9000),
                                  (IQ4, 3000), (IQ4, 6000), (IQ4, 9000), (IQ4, 17000), (IQ4, 38000)],
                         ids=lambda v: NAMES.get(v, str(v)))
def test_gemv_row_rounds_all_rows(qt, N):
    K = 5120
    W, x = _case(qt, N, K, 500 + N)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} {N}x{K}")


# Front-loaded row splits: a launch of two to four small workgroups per CU
# gives every dispatch round but the last a full straight-line round of rows
# and the last round the rest.  At K = 5120: 9220 and 13830 rows (two and
# three workgroups per CU), 18440 (four per CU; the last round has 8 rows, so
# 248 of its workgroups have none), 24576 (four full rounds).  Every row is
# checked, on GGUF and PLANAR rows.
# (IQ4_XS has no PLANAR layout: GGUF rows only)
@pytest.mark.parametrize("qt,N,planar",
                         [(q, n, p) for q, n in [(Q4, 9220), (Q4, 13830), (Q4, 18440), (Q4, 24576), (IQ4, 18440)]
                          for p in ((False, True) if q != IQ4 else (False,))],
                         ids=lambda v: {True: "PLANAR", False: "GGUF"}[v] if isinstance(v, bool) else NAMES.get(v, str(v)))
def test_gemv_front_loaded_rounds_all_rows(qt, N, planar):
    K = 5120
    W, x = _case(qt, N, K, 600 + N)
    Wd, t = dev(W.reshape(-1)), qt
    if planar:
        Wd, t = binding.repack(qt, Wd, N, K), qt | binding.PLANAR
    y = binding.gemv(t, Wd, dev(x), N, K)
    torch.cuda.synchronize()
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y.cpu().numpy(), y_ref, S, f"{NAMES[qt]} {N}x{K} planar={planar}")


# K > 16384 leaves room for one row phase of useg = K/64 lanes (Q4_K/Q5_K:
# 512 threads at most), and useg = 272 is not a multiple of 64, so the last
# wave holds a second, partial phase: P = 1 with two slot rows per schedule
# row.  Several rows per workgroup (N > 256) then exercise the slot-row
# mapping of the reduction at P = 1.  Q6_K (up to 1024 threads) takes P = 1
# at K = 17408 when five rows per workgroup fit one phase best (N = 1200).
# Every row is checked.
@pytest.mark.parametrize("qt,N,K", [(Q4, 1000, 17408), (Q5, 600, 17408), (Q4, 300, 16640), (Q6, 1200, 17408),
                                    (IQ4, 1000, 17408)],
                         ids=lambda v: NAMES.get(v, str(v)))
def test_gemv_single_phase_several_rows(qt, N, K):
    W, x = _case(qt, N, K, 800 + N)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y, y_ref, S, f"{NAMES[qt]} {N}x{K}")


# Large extents, every row: a million rows of K = 256 (the launch grows its
# workgroup count until the partial sums fit LDS), 2^18 rows of K = 512, and
# K = 2^20 (32 segments of the one-column kernel; some 200 of the verify
# kernel at 8 columns).
@pytest.mark.parametrize("qt,N,K,ncols", [(Q4, 1 << 20, 256, 1), (Q6, 1 << 18, 512, 1), (Q5, 16, 1 << 20, 1),
                                          (Q4, 16, 1 << 20, 8), (Q6, 24, 1 << 20, 3), (IQ4, 1 << 19, 256, 1),
                                          (IQ4, 16, 1 << 20, 5)],
                         ids=lambda v: NAMES.get(v, str(v)))
def test_gemv_large_extents_all_rows(qt, N, K, ncols):
    W = synth.superblocks(qt, N, K, 1200 + ncols)
    x = synth.activations(K, ncols, 1200 + ncols)
    y = gpu_gemv(qt, W, x, N, K)
    y_ref, S = oracle.gemv(qt, W, x, K)
    assert_row_bound(y.reshape(N, ncols), y_ref, S, f"{NAMES[qt]} {N}x{K} ncols={ncols}")
    assert np.isfinite(y).all()
