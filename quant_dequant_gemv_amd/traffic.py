"""HBM traffic of the one-column GEMV from rocprofv3 counters.

Two steps, each a separate rocprofv3 counter pass (FETCH_SIZE, then WRITE_SIZE),
run from the repository root on the GPU:

    rocprofv3 --pmc FETCH_SIZE -d gpurun_out/traffic_fetch -o run -- python3 -m quant_dequant_gemv_amd.traffic run
    rocprofv3 --pmc WRITE_SIZE -d gpurun_out/traffic_write -o run -- python3 -m quant_dequant_gemv_amd.traffic run
    python3 -m quant_dequant_gemv_amd.traffic parse gpurun_out/traffic_fetch/run_results.db \\
        gpurun_out/traffic_write/run_results.db

`run` launches each of the three Q4_K projection shapes (N = 10240, 12288,
17408; K = 5120) a few times on distinct weight copies, directly (one dispatch
per launch), and a plain device-to-device copy of 512 MiB as the calibration:
its counters are scaled to the known 512 MiB read and 512 MiB written, and the
same factors are applied to the GEMV's counters.  `parse` writes
profiles/traffic.json (per-launch HBM bytes of the kernel, with the hash of
the kernel sources it was measured on) that bench.py reports as
roofline.traffic while the sources are unchanged.
"""
from __future__ import annotations

import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 512 * 1024 * 1024
OUT = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["quant_dequant_gemv_amd/csrc/qk_kernels.hip", "quant_dequant_gemv_amd/csrc/qk_format.h",
                  "quant_dequant_gemv_amd/csrc/qk_epilogue.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def run(reps: int = 4) -> None:
    import torch

    from quant_dequant_gemv_amd import binding, synth
    lib = binding.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    for e in synth.Q4K_PROJECTIONS:
        W = synth.superblocks(e["qtype"], e["N"], e["K"], e["seed"])
        Ws = [torch.from_numpy(W.reshape(-1)).cuda() for _ in range(reps)]
        x = torch.from_numpy(synth.activations(e["K"], 1, e["seed"])).cuda()
        y = torch.empty(e["N"], dtype=torch.float32, device="cuda")
        for Wd in Ws:
            rc = lib.qk_gemv(e["qtype"], Wd.data_ptr(), x.data_ptr(), y.data_ptr(), e["N"], e["K"], 1, stream)
            if rc:
                raise binding.QKError(rc, "qk_gemv")
            torch.cuda.synchronize()
        del Ws
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
        torch.cuda.synchronize()
    print("traffic run done", flush=True)


def _per_dispatch(db: str, counter: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall()
    agg = {}
    for name, did, cn, v in rows:
        if cn != counter:
            continue
        agg.setdefault((name, did), 0.0)
        agg[(name, did)] += v
    return agg


def parse(fetch_db: str, write_db: str) -> dict:
    from quant_dequant_gemv_amd import synth
    res = {}
    for label, db, counter in (("fetch", fetch_db, "FETCH_SIZE"), ("write", write_db, "WRITE_SIZE")):
        d = _per_dispatch(db, counter)
        gemv = [v for (n, _), v in d.items() if "gemv1_kernel<12" in n]
        copy = [v for (n, _), v in d.items() if "copy" in n.lower() and v > 0]
        if not gemv or not copy:
            raise RuntimeError(f"{counter}: missing dispatches (gemv {len(gemv)}, copy {len(copy)})")
        gemv_kib = sum(gemv) / len(gemv)  # mean over the three shapes, like achieved
        copy_kib = max(copy)  # the 512 MiB copy is the largest copy dispatch
        factor = COPY_BYTES / (copy_kib * 1024.0)
        res[label] = {"counter": counter, "gemv_kib_mean": gemv_kib, "copy_kib": copy_kib,
                      "scale": factor, "gemv_bytes": gemv_kib * 1024.0 * factor}
    step = synth.Q4K_PROJECTIONS
    alg = sum(e["N"] * synth.row_bytes(e["qtype"], e["K"]) + 2 * e["K"] + 4 * e["N"] for e in step) / len(step)
    per_launch = res["fetch"]["gemv_bytes"] + res["write"]["gemv_bytes"]
    out = {"kernel_hash": kernel_hash(), "kernel": "gemv1_kernel<Q4_K>",
           "per_launch_bytes": {"gemv1_kernel<Q4_K>": round(per_launch)},
           "algorithmic_bytes_per_launch": round(alg),
           "ratio_to_algorithmic": round(per_launch / alg, 4),
           "counters": res,
           "note": "mean over the step's three shapes' launches; scaled by a 512 MiB device copy"}
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
    return out


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        sys.path.insert(0, ROOT)
        run()
    elif len(sys.argv) == 4 and sys.argv[1] == "parse":
        sys.path.insert(0, ROOT)
        print(json.dumps(parse(sys.argv[2], sys.argv[3]), indent=1))
    else:
        print(__doc__)
        sys.exit(2)
