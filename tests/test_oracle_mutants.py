"""CPU-only: plausible mistakes planted in copies of the oracle source must fail a pin.

Each mutant is a one-token edit of ``oracle/qk_oracle.c`` compiled into a
temporary library; the pins of ``oracle_checks`` are run against it and at
least one must raise.  This shows the pins are not blind to the kind of slip
(dropped term, flipped sign, wrong shift or index, transposed operand) that
would otherwise let the oracle and a kernel agree on a wrong answer.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_checks as oc
from quant_dequant_gemv_amd import synth

MUTANTS = {
    "drop_min_term": ("out[i] = a - b;", "out[i] = a;"),
    "min_term_sign": ("out[i] = a - b;", "out[i] = a + b;"),
    "q5_qs_offset": ("sb + (type == ORACLE_Q4_K ? 16 : 48)", "sb + (type == ORACLE_Q4_K ? 16 : 16)"),
    "nibble_order": ("(qs[32 * c + l] >> (4 * h))", "(qs[32 * c + l] >> (4 * (1 - h)))"),
    "q5_high_bit_index": ("((qh[l] >> j) & 1) << 4", "((qh[l] >> (j ^ 1)) & 1) << 4"),
    "scale_hi_bits": ("((scales[j - 4] >> 6) << 4)", "((scales[j - 4] >> 6) << 5)"),
    "scale_min_nibble_swap": ("*sc = (scales[j + 4] & 0x0f)", "*sc = (scales[j + 4] >> 4)"),
    "d_dmin_swap": ("float d = oracle_half_to_float(rd16(sb + 0));",
                    "float d = oracle_half_to_float(rd16(sb + 2));"),
    "q6_offset": ("(q - 32)", "(q - 31)"),
    "q6_qh_shift": ("(qh[32 * n + l] >> (2 * t)) & 3", "(qh[32 * n + l] >> (2 * (t ^ 1))) & 3"),
    "q6_ql_half": ("ql[64 * n + 32 * (t % 2) + l]", "ql[64 * n + 32 * (t / 2) + l]"),
    "q6_scale_group": ("sb[192 + i / 16]", "sb[192 + i / 32]"),
    "q6_d_position": ("rd16(sb + 208)", "rd16(sb + 206)"),
    "x_transposed": ("j->xd[k * j->ncols + c]", "j->xd[c * j->K + k]"),
    "abs_dropped": ("mag += fabs(p);", "mag += p;"),
    "subnormal_scale": ("ldexpf((float)m, -24)", "ldexpf((float)m, -25)"),
    "iq4_nibble_order": ("(qs[16 * ib + (l % 16)] >> (4 * (l / 16)))", "(qs[16 * ib + (l % 16)] >> (4 * (1 - l / 16)))"),
    "iq4_qs_offset": ("const uint8_t *qs = sb + 8;", "const uint8_t *qs = sb + 4;"),
    "iq4_scale_low_nibble": ("(sb[4 + ib / 2] >> (4 * (ib % 2)))", "(sb[4 + ib / 2] >> (4 * (1 - ib % 2)))"),
    "iq4_scale_high_bits": ("(rd16(sb + 2) >> (2 * ib)) & 3", "(rd16(sb + 2) >> (2 * ib + 1)) & 3"),
    "iq4_offset": ("((ls - 32) * kv)", "((ls - 31) * kv)"),
    "iq4_codebook_index": ("iq4nl_codebook[idx]", "iq4nl_codebook[idx ^ 1]"),
    "iq4_codebook_entry": ("53,  69", "53,  68"),
    "iq4_d_position": ("oracle_half_to_float(rd16(sb));", "oracle_half_to_float(rd16(sb + 2));"),
}

CHECKS = oc.ALL_CHECKS + [lambda o: oc.check_gemv_dot_of_dequant(o, synth)]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(workdir, name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = os.path.join(str(workdir), f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(str(workdir), f"lib{name}.so")
    try:
        oracle.compile_oracle(path, lib)
    except subprocess.CalledProcessError:
        pytest.skip(f"mutant {name} does not compile with this gcc")
    o = oracle.Oracle(lib)
    failures = 0
    for check in CHECKS:
        try:
            check(o)
        except (AssertionError, RuntimeError, ValueError):
            failures += 1
            break
    assert failures, f"no pin caught mutant {name}"
