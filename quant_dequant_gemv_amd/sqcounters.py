"""Where the GEMV kernels spend their cycles, from rocprofv3 SQ counters.

Two counter passes (eight SQ counters each, the most one pass can hold) over
the same launch plan, run from the repository root on the GPU:

    rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU \\
        SQ_WAIT_INST_ANY SQ_INSTS_VMEM_RD SQ_INSTS_LDS GRBM_GUI_ACTIVE -d gpurun_out/sq_a -o run -- \\
        python3 -m quant_dequant_gemv_amd.sqcounters run
    rocprofv3 --pmc SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VMEM SQ_VALU_MFMA_BUSY_CYCLES \\
        SQ_INSTS_SALU SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_LDS SQ_INSTS_MFMA GRBM_GUI_ACTIVE \\
        -d gpurun_out/sq_b -o run -- python3 -m quant_dequant_gemv_amd.sqcounters run
    python3 -m quant_dequant_gemv_amd.sqcounters parse gpurun_out/sq_a/run_results.db \\
        gpurun_out/sq_b/run_results.db

`run` launches each group of plan() REPS times on distinct weight copies, one
dispatch per launch.  `parse` maps the GEMV dispatches back to the plan by
their order, averages each counter over a group's dispatches (a dispatch's
value is the sum over the counter's instances: shader engines and XCDs) and
writes profiles/sq_counters_workload_shapes.md with the raw means and a few
ratios:

* VALU instructions per lane-unit: SQ_INSTS_VALU (wave instructions) x 64 /
  (row, 64-weight unit) pairs of the launch -- the arithmetic one lane spends
  on one unit of one row;
* active cycles: SQ_BUSY_CYCLES / 32 shader engines, the cycles in which a
  shader engine holds any wave of the kernel (the dispatch's start and end
  outside them), and the same at the nominal 2.4 GHz in us;
* VALU issue share: SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x active cycles),
  the fraction of the SIMDs' cycles taken by issuing VALU instructions (a
  wave64 instruction occupies a 16-lane SIMD for 4 cycles);
* resident waves per SIMD: SQ_WAVE_CYCLES (quad-cycles) x 4 / (1024 x active
  cycles);
* wait shares: SQ_WAIT_ANY and SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES, the
  fractions of the waves' lifetime spent waiting for anything (memory
  counters included) and unable to issue the next instruction;
* MFMA busy share: SQ_VALU_MFMA_BUSY_CYCLES / (1024 x active cycles).
"""
from __future__ import annotations

import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "profiles", "sq_counters_workload_shapes.json")
MD = os.path.join(ROOT, "profiles", "sq_counters_workload_shapes.md")
REPS = 4
SIMDS = 1024  # 256 CUs x 4 SIMDs
SES = 32  # 8 XCDs x 4 shader engines
CLOCK_MHZ = 2400
PASS_A = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY",
          "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]
PASS_B = ["SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VMEM", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_SALU",
          "SQ_BUSY_CU_CYCLES", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"]
COMMANDS = f"""    rocprofv3 --pmc {' '.join(PASS_A)} -d gpurun_out/sq_a -o run -- python3 -m quant_dequant_gemv_amd.sqcounters run
    rocprofv3 --pmc {' '.join(PASS_B)} -d gpurun_out/sq_b -o run -- python3 -m quant_dequant_gemv_amd.sqcounters run
    python3 -m quant_dequant_gemv_amd.sqcounters parse gpurun_out/sq_a/run_results.db gpurun_out/sq_b/run_results.db"""


def plan():
    """[(label, qtype, N, K, seed, ncols)]: the launch groups, in order."""
    from quant_dequant_gemv_amd import synth
    Q4, Q5, Q6, IQ4 = synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.IQ4_XS
    return [("gemv1_kernel<Q4_K> 17408x5120", Q4, 17408, 5120, 3, 1),
            ("gemv1_kernel<Q4_K> 10240x5120", Q4, 10240, 5120, 1, 1),
            ("gemv1_kernel<Q6_K> 5120x17408", Q6, 5120, 17408, 4, 1),
            ("gemv1_kernel<Q5_K> 5120x6144", Q5, 5120, 6144, 5, 1),
            ("gemv1_kernel<IQ4_XS> 17408x5120", IQ4, 17408, 5120, 1003, 1),
            ("verify_kernel<Q4_K> 17408x5120 ncols 8", Q4, 17408, 5120, 6, 8),
            ("verify_kernel<Q6_K> 5120x17408 ncols 8", Q6, 5120, 17408, 4, 8),
            ("v16_kernel<Q4_K> 17408x5120 ncols 16", Q4, 17408, 5120, 6, 16),
            ("v16q6_kernel<Q6_K> 5120x17408 ncols 16", Q6, 5120, 17408, 4, 16)]


def run(reps: int = REPS) -> None:
    import torch

    from quant_dequant_gemv_amd import binding, synth
    lib = binding.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    for _, qt, N, K, seed, nc in plan():
        W = synth.superblocks(qt, N, K, seed)
        Ws = [torch.from_numpy(W.reshape(-1)).cuda() for _ in range(reps)]
        x = torch.from_numpy(synth.activations(K, nc, seed)).cuda()
        y = torch.empty(N * nc, dtype=torch.float32, device="cuda")
        for Wd in Ws:
            rc = lib.qk_gemv(qt, Wd.data_ptr(), x.data_ptr(), y.data_ptr(), N, K, nc, stream)
            if rc:
                raise binding.QKError(rc, "qk_gemv")
            torch.cuda.synchronize()
        del Ws
    print("sq counter run done", flush=True)


def _per_dispatch(db: str):
    """{counter: [value per GEMV dispatch, in dispatch order]} (values summed
    over the counter's instances)."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall()
    agg = {}
    for name, did, cn, v in rows:
        if "qk::" not in name:
            continue
        agg.setdefault(cn, {}).setdefault(did, 0.0)
        agg[cn][did] += v
    return {cn: [v for _, v in sorted(d.items())] for cn, d in agg.items()}


def _durations_us(db: str):
    """Durations (us) of the GEMV dispatches in order, if the database holds
    the kernel table (rocprofv3's `kernels` view); else None."""
    try:
        con = sqlite3.connect(db)
        rows = con.execute("select name, dispatch_id, start, end from kernels").fetchall()
    except sqlite3.Error:
        return None
    return [(e - b) * 1e-3 for n, _, b, e in sorted(rows, key=lambda r: r[1]) if "qk::" in n]


def parse(db_a: str, db_b: str, reps: int = REPS, out_path: str = OUT) -> dict:
    groups = plan()
    want = reps * len(groups)
    raw = {}
    for db, names in ((db_a, PASS_A), (db_b, PASS_B)):
        d = _per_dispatch(db)
        for cn in names:
            v = d.get(cn, [])
            if len(v) != want:
                raise RuntimeError(f"{cn}: {len(v)} GEMV dispatches (expected {want})")
            key = cn if cn != "GRBM_GUI_ACTIVE" else f"GRBM_GUI_ACTIVE/{'a' if names is PASS_A else 'b'}"
            raw[key] = v
    us = _durations_us(db_a)
    out = {"reps": reps, "groups": {}}
    for gi, (label, qt, N, K, _, nc) in enumerate(groups):
        m = {k: sum(v[gi * reps:(gi + 1) * reps]) / reps for k, v in raw.items()}
        cycles = m["SQ_BUSY_CYCLES"] / SES
        lane_units = N * (K // 64)
        ratios = {
            "active_cycles": round(cycles),
            "active_us_nominal": round(cycles / CLOCK_MHZ, 2),
            "waves": round(m["SQ_WAVES"]),
            "valu_per_lane_unit": round(m["SQ_INSTS_VALU"] * 64 / lane_units, 1),
            "valu_issue_share": round(m["SQ_INSTS_VALU"] * 4 / (SIMDS * cycles), 3),
            "waves_per_simd": round(m["SQ_WAVE_CYCLES"] * 4 / (SIMDS * cycles), 2),
            "wait_any_share": round(m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"], 3),
            "wait_inst_share": round(m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"], 3),
            "mfma_busy_share": round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cycles), 3),
            "vmem_rd_per_lane_unit": round(m["SQ_INSTS_VMEM_RD"] * 64 / lane_units, 2),
        }
        if us and len(us) == len(groups) * reps:
            ratios["kernel_us"] = round(sum(us[gi * reps:(gi + 1) * reps]) / reps, 2)  # profiled duration
        out["groups"][label] = {"ncols": nc, "means": {k: round(v, 1) for k, v in m.items()}, "ratios": ratios}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def markdown(out: dict) -> str:
    lines = ["# Where the GEMV kernels spend their cycles: rocprofv3 SQ counters at the workload shapes", "",
             "Commands (run from the repository root on one MI355X; two counter passes over the same launches):",
             "", COMMANDS, "",
             f"`sqcounters run` launches each group {out['reps']} times on distinct weight copies; every figure "
             "is the mean over a group's dispatches, each counter summed over its instances.  Definitions of the "
             "ratios are in `quant_dequant_gemv_amd/sqcounters.py`.", "",
             "| group | kernel µs (profiled) | active cycles (µs at 2.4 GHz) | waves | waves / SIMD | "
             "VALU / lane-unit | VALU issue share | waiting (any / issue) | MFMA busy share | VMEM reads / lane-unit |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for name, g in out["groups"].items():
        r = g["ratios"]
        lines.append(f"| `{name}` | {r.get('kernel_us', '')} | {r['active_cycles']} ({r['active_us_nominal']}) | "
                     f"{r['waves']} | {r['waves_per_simd']} | {r['valu_per_lane_unit']} | {r['valu_issue_share']} | "
                     f"{r['wait_any_share']} / {r['wait_inst_share']} | {r['mfma_busy_share']} | "
                     f"{r['vmem_rd_per_lane_unit']} |")
    lines += ["", "Raw means per dispatch:", "",
              "| group | " + " | ".join(next(iter(out["groups"].values()))["means"]) + " |",
              "|---|" + "---|" * len(next(iter(out["groups"].values()))["means"])]
    for name, g in out["groups"].items():
        lines.append(f"| `{name}` | " + " | ".join(f"{v:.0f}" for v in g["means"].values()) + " |")
    lines.append("")
    return "\n".join(lines)


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        sys.path.insert(0, ROOT)
        run()
    elif len(sys.argv) == 4 and sys.argv[1] == "parse":
        sys.path.insert(0, ROOT)
        res = parse(sys.argv[2], sys.argv[3])
        with open(MD, "w") as fh:
            fh.write(markdown(res))
        print(markdown(res))
    else:
        print(__doc__)
        sys.exit(2)
