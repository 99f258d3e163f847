"""CPU-only: the SQ-counter parser maps the counter dispatches of two passes
back to the launch plan by order, averages each group and derives its ratios
(synthetic counter databases in the rocprofv3 table layout)."""
import sqlite3

import pytest

from quant_dequant_gemv_amd import sqcounters


def _db(path, names, value_of, n, with_kernels=False):
    con = sqlite3.connect(path)
    con.execute("create table pmc_events (name text, dispatch_id integer, counter_name text, counter_value real)")
    con.execute("insert into pmc_events values ('at::native::fill', 0, 'SQ_WAVES', 7.0)")
    for d in range(1, n + 1):
        for cn in names:
            # two instances per dispatch (summed by the parser)
            for _ in range(2):
                con.execute("insert into pmc_events values (?, ?, ?, ?)", ("qk::gemv1_kernel<...>", d, cn,
                                                                           value_of(cn, d) / 2))
    if with_kernels:
        con.execute("create table kernels (name text, dispatch_id integer, start integer, end integer)")
        for d in range(1, n + 1):
            con.execute("insert into kernels values (?, ?, ?, ?)", ("qk::gemv1_kernel<...>", d, 1000 * d,
                                                                   1000 * d + 10000))
    con.commit()
    con.close()


def test_parse_groups_and_ratios(tmp_path):
    groups = sqcounters.plan()
    reps = 2
    n = reps * len(groups)

    def value(cn, d):
        g = (d - 1) // reps
        return {"SQ_BUSY_CYCLES": 32 * 24000.0, "SQ_INSTS_VALU": 1024 * 6000.0, "SQ_WAVE_CYCLES": 1024 * 12000.0,
                "SQ_WAIT_INST_ANY": 1024 * 3000.0, "SQ_WAIT_ANY": 1024 * 6000.0,
                "SQ_WAVES": 100.0 * (g + 1)}.get(cn, 5.0)
    _db(tmp_path / "a.db", sqcounters.PASS_A, value, n, with_kernels=True)
    _db(tmp_path / "b.db", sqcounters.PASS_B, value, n)
    out = sqcounters.parse(str(tmp_path / "a.db"), str(tmp_path / "b.db"), reps=reps,
                           out_path=str(tmp_path / "sq.json"))
    for gi, (label, qt, N, K, _, nc) in enumerate(groups):
        r = out["groups"][label]["ratios"]
        assert r["active_cycles"] == 24000 and r["active_us_nominal"] == 10.0 and r["waves"] == 100 * (gi + 1)
        assert r["valu_issue_share"] == round(1024 * 6000 * 4 / (1024 * 24000), 3)
        assert r["waves_per_simd"] == 2.0 and r["wait_inst_share"] == 0.25 and r["wait_any_share"] == 0.5
        assert r["valu_per_lane_unit"] == round(1024 * 6000 * 64 / (N * (K // 64)), 1)
        assert r["kernel_us"] == 10.0
    md = sqcounters.markdown(out)
    for label, *_ in groups:
        assert f"`{label}`" in md
    assert "rocprofv3 --pmc SQ_WAVES" in md


def test_parse_rejects_a_short_run(tmp_path):
    _db(tmp_path / "a.db", sqcounters.PASS_A, lambda cn, d: 1.0, 3)
    _db(tmp_path / "b.db", sqcounters.PASS_B, lambda cn, d: 1.0, 3)
    with pytest.raises(RuntimeError, match="expected"):
        sqcounters.parse(str(tmp_path / "a.db"), str(tmp_path / "b.db"), out_path=str(tmp_path / "sq.json"))
