"""HBM traffic of the GEMV kernels from rocprofv3 counters.

Two steps, each a separate rocprofv3 counter pass (FETCH_SIZE, then WRITE_SIZE),
run from the repository root on the GPU:

    rocprofv3 --pmc FETCH_SIZE -d gpurun_out/traffic_fetch -o run -- python3 -m quant_dequant_gemv_amd.traffic run
    rocprofv3 --pmc WRITE_SIZE -d gpurun_out/traffic_write -o run -- python3 -m quant_dequant_gemv_amd.traffic run
    python3 -m quant_dequant_gemv_amd.traffic parse gpurun_out/traffic_fetch/run_results.db \\
        gpurun_out/traffic_write/run_results.db

`run` launches, a few times each on distinct weight copies and directly (one
dispatch per launch), the groups of plan(): the three Q4_K projection shapes
(N = 10240, 12288, 17408; K = 5120) -- the benchmark's step --, the Q4_K
17408 x 5120 verify form at 2, 4, 8, 16 and 17 columns, the one-column Q6_K
and Q5_K shapes and IQ4_XS 17408 x 5120; then three known reads of 512 MiB
as the calibration: a device-to-device copy (512 MiB read, 512 MiB
written), and the plain read of libqkcalib.so with non-temporal and with
ordinary loads.  The copy's factors scale the GEMV's counters; the two
reads give independent FETCH_SIZE factors as a cross-check.  `parse`
maps the dispatches back to plan() by their order and writes
profiles/traffic.json (per-launch HBM bytes of each group against its
algorithmic bytes, with the hash of the kernel sources it was measured on)
and the markdown summary beside it; bench.py reports the step's figure as
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
MD = os.path.join(ROOT, "profiles", "traffic_gemv1_verify_workload_shapes.md")
COMMANDS = """    rocprofv3 --pmc FETCH_SIZE -d gpurun_out/traffic_fetch -o run -- python3 -m quant_dequant_gemv_amd.traffic run
    rocprofv3 --pmc WRITE_SIZE -d gpurun_out/traffic_write -o run -- python3 -m quant_dequant_gemv_amd.traffic run
    python3 -m quant_dequant_gemv_amd.traffic parse gpurun_out/traffic_fetch/run_results.db gpurun_out/traffic_write/run_results.db"""
KERNEL_SOURCES = ["quant_dequant_gemv_amd/csrc/qk_kernels.hip", "quant_dequant_gemv_amd/csrc/qk_verify.h",
                  "quant_dequant_gemv_amd/csrc/qk_verify16.h", "quant_dequant_gemv_amd/csrc/qk_format.h",
                  "quant_dequant_gemv_amd/csrc/qk_epilogue.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


REPS = 4
STEP = "gemv1_kernel<Q4_K>"  # the key bench.py reads


def plan():
    """[(label, [(qtype, N, K, seed, ncols), ...])]: the launch groups, in order."""
    from quant_dequant_gemv_amd import synth
    v = synth.VERIFY
    groups = [(STEP, [(e["qtype"], e["N"], e["K"], e["seed"], 1) for e in synth.Q4K_PROJECTIONS])]
    for nc in (2, 4, 8, 16, 17):  # (9-32 columns: the 16x16x16 tile kernel)
        kern = "verify_kernel" if nc <= 8 else "v16_kernel"
        groups.append((f"{kern}<Q4_K> {v['N']}x{v['K']} ncols {nc}", [(v["qtype"], v["N"], v["K"], v["seed"], nc)]))
    for e in synth.MIXED:
        groups.append((f"gemv1_kernel<{synth.TYPE_NAMES[e['qtype']]}> {e['N']}x{e['K']}",
                       [(e["qtype"], e["N"], e["K"], e["seed"], 1)]))
    groups.append(("gemv1_kernel<IQ4_XS> 17408x5120", [(synth.IQ4_XS, 17408, 5120, 1003, 1)]))
    q6 = synth.MIXED[0]  # Q6_K FFN down: four segments of x planes on the tiles
    for nc in (16, 17):
        groups.append((f"v16q6_kernel<Q6_K> {q6['N']}x{q6['K']} ncols {nc}", [(q6["qtype"], q6["N"], q6["K"], q6["seed"], nc)]))
    groups.append(("v16q6_kernel<IQ4_XS> 17408x5120 ncols 17", [(synth.IQ4_XS, 17408, 5120, 1003, 17)]))
    return groups


READS = (("read_nt", "qk_stream_read", "stream_read_kernel<true>"),
         ("read_plain", "qk_stream_read_plain", "stream_read_kernel<false>"))


def run(reps: int = REPS) -> None:
    import torch

    from quant_dequant_gemv_amd import binding, synth
    lib = binding.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    for _, launches in plan():
        for qt, N, K, seed, nc in launches:
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
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
        torch.cuda.synchronize()
    del dst
    from quant_dequant_gemv_amd import calib
    cl = calib.load()
    out = torch.empty(1024 * 1024, dtype=torch.int32, device="cuda")
    for _, fn, _ in READS:
        for _ in range(reps):
            if getattr(cl, fn)(src.data_ptr(), COPY_BYTES, out.data_ptr(), 1024, 1024, stream):
                raise RuntimeError(fn)
            torch.cuda.synchronize()
    print("traffic run done", flush=True)


def _per_dispatch(db: str, counter: str):
    """[(dispatch_id, name, value)] of one counter, in dispatch order."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall()
    agg = {}
    for name, did, cn, v in rows:
        if cn != counter:
            continue
        agg.setdefault((did, name), 0.0)
        agg[(did, name)] += v
    return [(did, name, v) for (did, name), v in sorted(agg.items())]


def _alg_bytes(qt, N, K, nc):
    from quant_dequant_gemv_amd import synth
    return N * synth.row_bytes(qt, K) + 2 * K * nc + 4 * N * nc


def parse(fetch_db: str, write_db: str, reps: int = REPS, out_path: str = OUT) -> dict:
    groups = plan()
    res = {}
    for label, db, counter in (("fetch", fetch_db, "FETCH_SIZE"), ("write", write_db, "WRITE_SIZE")):
        d = _per_dispatch(db, counter)
        ours = [v for _, n, v in d if "qk::" in n]
        copy = [v for _, n, v in d if "copy" in n.lower() and v > 0]
        want = reps * sum(len(launches) for _, launches in groups)
        if len(ours) != want or not copy:
            raise RuntimeError(f"{counter}: {len(ours)} GEMV dispatches (expected {want}), {len(copy)} copies")
        factor = COPY_BYTES / (max(copy) * 1024.0)  # the 512 MiB copy is the largest copy dispatch
        refs = {}
        if counter == "FETCH_SIZE":  # the plain reads: independent factors for the same counter
            for key, _, kname in READS:
                v = [x for _, n, x in d if kname in n]
                if len(v) != reps:
                    raise RuntimeError(f"{counter}: {len(v)} dispatches of {kname} (expected {reps})")
                kib = sum(v) / len(v)
                refs[key] = {"kib_mean": kib, "scale": COPY_BYTES / (kib * 1024.0)}
        per_group, i = {}, 0
        for name, launches in groups:
            n = reps * len(launches)
            kib = sum(ours[i:i + n]) / n  # mean over the group's launches
            per_group[name] = {"kib_mean": kib, "bytes": kib * 1024.0 * factor}
            i += n
        res[label] = {"counter": counter, "copy_kib": max(copy), "scale": factor, "groups": per_group,
                      "read_refs": refs}
    per_launch, alg, ratio = {}, {}, {}
    for name, launches in groups:
        per_launch[name] = round(res["fetch"]["groups"][name]["bytes"] + res["write"]["groups"][name]["bytes"])
        alg[name] = round(sum(_alg_bytes(*l[:3], l[4]) for l in launches) / len(launches))
        ratio[name] = round(per_launch[name] / alg[name], 4)
    out = {"kernel_hash": kernel_hash(), "kernel": STEP,
           "per_launch_bytes": per_launch,
           "algorithmic_bytes_per_launch": alg[STEP],
           "ratio_to_algorithmic": ratio[STEP],
           "algorithmic_bytes": alg,
           "ratios": ratio,
           "counters": res,
           "note": "means over each group's launches (the step: its three shapes); counters scaled by a "
                   "512 MiB device copy, cross-checked by 512 MiB plain reads (non-temporal and ordinary loads)"}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def markdown(out: dict, reps: int = REPS) -> str:
    """The summary kept with the profiles."""
    f, w = out["counters"]["fetch"], out["counters"]["write"]
    lines = ["# HBM traffic of the GEMV kernels at the workload shapes: rocprofv3 counters", "",
             "Commands (run from the repository root on one MI355X; one counter per pass):", "", COMMANDS, "",
             f"`traffic run` launches each group below {reps} times on distinct weight copies (one dispatch per "
             "launch), then a 512 MiB device-to-device copy and two plain reads of 512 MiB.", "",
             "Calibration by the copy (known 512 MiB read, 512 MiB written):", "",
             "| counter | copy reads as | scale |", "|---|---|---|",
             f"| FETCH_SIZE | {f['copy_kib']:.1f} KiB | {f['scale']:.4f} |",
             f"| WRITE_SIZE | {w['copy_kib']:.1f} KiB | {w['scale']:.4f} |", "",
             "Cross-check of the FETCH_SIZE scale by two reads of the same 512 MiB with libqkcalib.so's plain "
             "read kernel (1024 x 1024 threads):", "",
             "| reference | FETCH_SIZE reads as | scale |", "|---|---|---|"]
    for key, _, kname in READS:
        r = f["read_refs"][key]
        lines.append(f"| `{kname}` | {r['kib_mean']:.1f} KiB | {r['scale']:.4f} |")
    lines += ["",
             "Per launch (mean over the group's dispatches; the step: its three Q4_K shapes 10240 / 12288 / "
             "17408 x 5120):", "",
             "| group | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes | algorithmic bytes (W + x + y) | ratio |",
             "|---|---|---|---|---|---|"]
    for name in out["per_launch_bytes"]:
        lines.append(f"| `{name}` | {f['groups'][name]['kib_mean']:.1f} | {w['groups'][name]['kib_mean']:.1f} | "
                     f"{out['per_launch_bytes'][name]} | {out['algorithmic_bytes'][name]} | {out['ratios'][name]:.4f} |")
    lines += ["", "A ratio near 1 means every weight byte is fetched from HBM once per launch (the verify form "
              "included, at every width: W is read once for all its columns; the ratio above 1 is what the "
              "caches did not absorb).  Kernel source hash " +
              out["kernel_hash"] +
              " (bench.py reports `roofline.traffic` from profiles/traffic.json only while the sources hash the "
              "same).", ""]
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
        print(json.dumps(res, indent=1))
    else:
        print(__doc__)
        sys.exit(2)
