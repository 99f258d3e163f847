"""CPU-only: the texture-unit counter parser maps the one-column GEMV
dispatches back to the launch plan by order (repack launches left out),
averages each group and derives its ratios (a synthetic counter database in
the rocprofv3 table layout)."""
import sqlite3

import pytest

from quant_dequant_gemv_amd import tacounters


def _db(path, value_of, n, repacks=True):
    con = sqlite3.connect(path)
    con.execute("create table pmc_events (name text, dispatch_id integer, counter_name text, counter_value real)")
    d = 0
    for i in range(n):
        if repacks and i % 8 == 4:  # a repack launch before each PLANAR group
            d += 1
            for cn in tacounters.COUNTERS:
                con.execute("insert into pmc_events values (?, ?, ?, ?)", ("qk::repack_kernel<14>", d, cn, 1e9))
        d += 1
        for cn in tacounters.COUNTERS:
            for _ in range(2):  # two instances per dispatch (summed by the parser)
                con.execute("insert into pmc_events values (?, ?, ?, ?)",
                            ("qk::gemv1_kernel<...>", d, cn, value_of(cn, i) / 2))
    con.commit()
    con.close()


def test_parse_groups_and_ratios(tmp_path):
    groups = tacounters.plan()
    reps = 2
    n = reps * len(groups)

    def value(cn, i):
        g = i // reps
        return {"TA_TA_BUSY": 256 * 2400.0 * (g + 1), "TA_FLAT_READ_WAVEFRONTS": 1000.0,
                "TCP_TOTAL_CACHE_ACCESSES": 4000.0 * (g + 1), "TCP_TCC_READ_REQ": 500.0}.get(cn, 3.0)
    _db(tmp_path / "ta.db", value, n, repacks=False)
    out = tacounters.parse(str(tmp_path / "ta.db"), reps=reps, out_path=str(tmp_path / "ta.json"))
    for gi, (label, *_r) in enumerate(groups):
        r = out["groups"][label]["ratios"]
        assert r["ta_busy_cycles_per_cu"] == 2400 * (gi + 1) and r["ta_busy_us_nominal"] == float(gi + 1)
        assert r["l1_accesses_per_load_wavefront"] == 4.0 * (gi + 1)
        assert r["l2_reads_per_load_wavefront"] == 0.5
    md = tacounters.markdown(out)
    for label, *_r in groups:
        assert f"`{label}`" in md
    assert "rocprofv3 --pmc TA_TA_BUSY" in md


def test_parse_skips_repack_launches(tmp_path):
    reps = 2
    n = reps * len(tacounters.plan())
    _db(tmp_path / "ta.db", lambda cn, i: 10.0, n, repacks=True)
    out = tacounters.parse(str(tmp_path / "ta.db"), reps=reps, out_path=str(tmp_path / "ta.json"))
    for g in out["groups"].values():
        assert g["means"]["TA_TA_BUSY"] == 10.0


def test_parse_rejects_a_short_run(tmp_path):
    _db(tmp_path / "ta.db", lambda cn, i: 1.0, 3, repacks=False)
    with pytest.raises(RuntimeError, match="expected"):
        tacounters.parse(str(tmp_path / "ta.db"), reps=2, out_path=str(tmp_path / "ta.json"))
