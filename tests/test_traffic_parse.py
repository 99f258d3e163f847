"""CPU-only: the HBM-traffic parser maps counter dispatches back to the launch
plan by order, scales them by the 512 MiB copy, reports the scales the two
512 MiB plain reads give, and compares each group with its algorithmic bytes
(synthetic counter databases in the rocprofv3 table layout)."""
import json
import sqlite3

from quant_dequant_gemv_amd import traffic


def _db(path, counter, values, copy_kib, read_kib=(), reps=0):
    con = sqlite3.connect(path)
    con.execute("create table pmc_events (name text, dispatch_id integer, counter_name text, counter_value real)")
    did = 0
    con.execute("insert into pmc_events values (?, ?, ?, ?)", ("at::native::fill", did, counter, 3.0))
    for name, v in values:
        did += 1
        # two rows per dispatch (counter instances), summed by the parser
        con.execute("insert into pmc_events values (?, ?, ?, ?)", (name, did, counter, v / 2))
        con.execute("insert into pmc_events values (?, ?, ?, ?)", (name, did, counter, v / 2))
    con.execute("insert into pmc_events values (?, ?, ?, ?)", ("__amd_rocclr_copyBuffer", did + 1, counter, copy_kib))
    did += 2
    for (_, _, kname), kib in zip(traffic.READS, read_kib):
        for _ in range(reps):
            con.execute("insert into pmc_events values (?, ?, ?, ?)",
                        (f"void {kname}(unsigned int const*, unsigned long, unsigned int*)", did, counter, kib))
            did += 1
    con.commit()
    con.close()


def test_parse_groups_by_dispatch_order(tmp_path):
    groups = traffic.plan()
    reps = 2
    fetch, write = [], []
    for gi, (name, launches) in enumerate(groups):
        for _ in launches:
            for _ in range(reps):
                fetch.append(("qk::kernel", 1000.0 * (gi + 1)))
                write.append(("qk::kernel", 10.0 * (gi + 1)))
    _db(tmp_path / "f.db", "FETCH_SIZE", fetch, 262144.0, (262144.0, 259000.0), reps)  # reads half: scale 2
    _db(tmp_path / "w.db", "WRITE_SIZE", write, 524288.0)  # scale 1
    out = traffic.parse(str(tmp_path / "f.db"), str(tmp_path / "w.db"), reps=reps, out_path=str(tmp_path / "t.json"))
    assert json.load(open(tmp_path / "t.json")) == out
    refs = out["counters"]["fetch"]["read_refs"]
    assert refs["read_nt"]["scale"] == 2.0 and abs(refs["read_plain"]["scale"] - 524288 / 259000) < 1e-12
    for gi, (name, launches) in enumerate(groups):
        want = 1000.0 * (gi + 1) * 1024 * 2 + 10.0 * (gi + 1) * 1024
        assert out["per_launch_bytes"][name] == round(want)
        assert out["ratios"][name] == round(round(want) / out["algorithmic_bytes"][name], 4)
    step = groups[0][0]
    assert out["kernel"] == step and out["ratio_to_algorithmic"] == out["ratios"][step]
    # the step's algorithmic bytes: weights + x + y, mean of its three shapes
    from quant_dequant_gemv_amd import synth
    alg = sum(e["N"] * synth.row_bytes(e["qtype"], e["K"]) + 2 * e["K"] + 4 * e["N"]
              for e in synth.Q4K_PROJECTIONS) / len(synth.Q4K_PROJECTIONS)
    assert out["algorithmic_bytes_per_launch"] == round(alg)


def test_parse_rejects_a_short_run(tmp_path):
    _db(tmp_path / "f.db", "FETCH_SIZE", [("qk::kernel", 1.0)], 262144.0, (262144.0, 262144.0), traffic.REPS)
    _db(tmp_path / "w.db", "WRITE_SIZE", [("qk::kernel", 1.0)], 524288.0)
    try:
        traffic.parse(str(tmp_path / "f.db"), str(tmp_path / "w.db"), out_path=str(tmp_path / "t.json"))
    except RuntimeError as e:
        assert "expected" in str(e)
    else:
        raise AssertionError("a run with missing dispatches must be rejected")


def test_markdown_lists_every_group(tmp_path):
    groups = traffic.plan()
    vals = [("qk::kernel", 100.0)] * (traffic.REPS * sum(len(l) for _, l in groups))
    _db(tmp_path / "f.db", "FETCH_SIZE", vals, 262144.0, (262144.0, 262144.0), traffic.REPS)
    _db(tmp_path / "w.db", "WRITE_SIZE", vals, 524288.0)
    out = traffic.parse(str(tmp_path / "f.db"), str(tmp_path / "w.db"), out_path=str(tmp_path / "t.json"))
    md = traffic.markdown(out)
    for name, _ in groups:
        assert f"`{name}`" in md
    assert out["kernel_hash"] in md and "rocprofv3 --pmc FETCH_SIZE" in md
    assert "stream_read_kernel<false>" in md
