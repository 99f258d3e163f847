"""The load path of the one-column kernels, from rocprofv3 texture-unit counters.

One counter pass (two TA, four TCP and one TD counter: within one pass's
limits) over Q6_K 5120 x 17408 and Q4_K 17408 x 5120, each on GGUF and on
PLANAR rows, run from the repository root on the GPU:

    rocprofv3 --pmc TA_TA_BUSY TA_FLAT_READ_WAVEFRONTS TCP_TOTAL_CACHE_ACCESSES TCP_TCC_READ_REQ \\
        TCP_PENDING_STALL_CYCLES TCP_READ_TAGCONFLICT_STALL_CYCLES TD_TC_STALL \\
        -d gpurun_out/ta -o run -- python3 -m quant_dequant_gemv_amd.tacounters run
    python3 -m quant_dequant_gemv_amd.tacounters parse gpurun_out/ta/run_results.db

`run` launches each group of plan() REPS times on distinct weight copies.
`parse` maps the GEMV dispatches back to the plan by their order, averages
each counter over a group's dispatches (a dispatch's value is the sum over
the counter's instances) and writes profiles/ta_counters_row_layouts.md:

* texture-addresser busy cycles per CU: TA_TA_BUSY / 256 CUs, and the same
  at the nominal 2.4 GHz in us -- the time one CU's address unit spends on
  the launch's vector memory instructions;
* L1 accesses per load wavefront: TCP_TOTAL_CACHE_ACCESSES /
  TA_FLAT_READ_WAVEFRONTS -- how many cache accesses one wave-wide load
  instruction turns into (16-byte lane loads that straddle lines take more);
* L2 read requests per load wavefront: TCP_TCC_READ_REQ /
  TA_FLAT_READ_WAVEFRONTS.
"""
from __future__ import annotations

import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "profiles", "ta_counters_row_layouts.json")
MD = os.path.join(ROOT, "profiles", "ta_counters_row_layouts.md")
REPS = 4
CUS = 256
CLOCK_MHZ = 2400
COUNTERS = ["TA_TA_BUSY", "TA_FLAT_READ_WAVEFRONTS", "TCP_TOTAL_CACHE_ACCESSES", "TCP_TCC_READ_REQ",
            "TCP_PENDING_STALL_CYCLES", "TCP_READ_TAGCONFLICT_STALL_CYCLES", "TD_TC_STALL"]
COMMANDS = f"""    rocprofv3 --pmc {' '.join(COUNTERS)} -d gpurun_out/ta -o run -- python3 -m quant_dequant_gemv_amd.tacounters run
    python3 -m quant_dequant_gemv_amd.tacounters parse gpurun_out/ta/run_results.db"""


def plan():
    """[(label, qtype, N, K, seed, planar)]: the launch groups, in order."""
    from quant_dequant_gemv_amd import synth
    return [("gemv1_kernel<Q6_K> 5120x17408 GGUF", synth.Q6_K, 5120, 17408, 4, False),
            ("gemv1_kernel<Q6_K> 5120x17408 PLANAR", synth.Q6_K, 5120, 17408, 4, True),
            ("gemv1_kernel<Q4_K> 17408x5120 GGUF", synth.Q4_K, 17408, 5120, 3, False),
            ("gemv1_kernel<Q4_K> 17408x5120 PLANAR", synth.Q4_K, 17408, 5120, 3, True)]


def run(reps: int = REPS) -> None:
    import torch

    from quant_dequant_gemv_amd import binding, synth
    for _, qt, N, K, seed, planar in plan():
        W = torch.from_numpy(synth.superblocks(qt, N, K, seed).reshape(-1)).cuda()
        t = qt
        if planar:
            W = binding.repack(qt, W, N, K)
            t = qt | binding.PLANAR
        Ws = [W.clone() for _ in range(reps)]
        x = torch.from_numpy(synth.activations(K, 1, seed)).cuda()
        torch.cuda.synchronize()
        for Wd in Ws:
            binding.gemv(t, Wd, x, N, K)
            torch.cuda.synchronize()
        del Ws, W
    print("ta counter run done", flush=True)


def _per_dispatch(db: str):
    """{counter: [value per one-column GEMV dispatch, in dispatch order]}
    (values summed over the counter's instances; the repack launches of the
    PLANAR groups are left out)."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall()
    agg = {}
    for name, did, cn, v in rows:
        if "gemv1_kernel" not in name:
            continue
        agg.setdefault(cn, {}).setdefault(did, 0.0)
        agg[cn][did] += v
    return {cn: [v for _, v in sorted(d.items())] for cn, d in agg.items()}


def parse(db: str, reps: int = REPS, out_path: str = OUT) -> dict:
    groups = plan()
    want = reps * len(groups)
    d = _per_dispatch(db)
    raw = {}
    for cn in COUNTERS:
        v = d.get(cn, [])
        if len(v) != want:
            raise RuntimeError(f"{cn}: {len(v)} GEMV dispatches (expected {want})")
        raw[cn] = v
    out = {"reps": reps, "groups": {}}
    for gi, (label, *_rest) in enumerate(groups):
        m = {k: sum(v[gi * reps:(gi + 1) * reps]) / reps for k, v in raw.items()}
        busy = m["TA_TA_BUSY"] / CUS
        wf = m["TA_FLAT_READ_WAVEFRONTS"]
        ratios = {
            "ta_busy_cycles_per_cu": round(busy),
            "ta_busy_us_nominal": round(busy / CLOCK_MHZ, 2),
            "l1_accesses_per_load_wavefront": round(m["TCP_TOTAL_CACHE_ACCESSES"] / wf, 1) if wf else None,
            "l2_reads_per_load_wavefront": round(m["TCP_TCC_READ_REQ"] / wf, 2) if wf else None,
        }
        out["groups"][label] = {"means": {k: round(v, 1) for k, v in m.items()}, "ratios": ratios}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def markdown(out: dict) -> str:
    lines = ["# The load path by row layout: rocprofv3 texture-unit counters", "",
             "Commands (run from the repository root on one MI355X; one counter pass):", "", COMMANDS, "",
             f"`tacounters run` launches each group {out['reps']} times on distinct weight copies; every figure is "
             "the mean over a group's dispatches, each counter summed over its instances.  Definitions are in "
             "`quant_dequant_gemv_amd/tacounters.py`.", "",
             "| group | TA busy cycles per CU (µs at 2.4 GHz) | L1 accesses per load wavefront | "
             "L2 reads per load wavefront |",
             "|---|---|---|---|"]
    for name, g in out["groups"].items():
        r = g["ratios"]
        lines.append(f"| `{name}` | {r['ta_busy_cycles_per_cu']} ({r['ta_busy_us_nominal']}) | "
                     f"{r['l1_accesses_per_load_wavefront']} | {r['l2_reads_per_load_wavefront']} |")
    lines += ["", "Raw means per dispatch:", "", "| group | " + " | ".join(COUNTERS) + " |",
              "|---|" + "---|" * len(COUNTERS)]
    for name, g in out["groups"].items():
        lines.append(f"| `{name}` | " + " | ".join(f"{g['means'][c]:.0f}" for c in COUNTERS) + " |")
    lines.append("")
    return "\n".join(lines)


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        sys.path.insert(0, ROOT)
        run()
    elif len(sys.argv) == 3 and sys.argv[1] == "parse":
        sys.path.insert(0, ROOT)
        res = parse(sys.argv[2])
        with open(MD, "w") as fh:
            fh.write(markdown(res))
        print(markdown(res))
    else:
        print(__doc__)
        sys.exit(2)
