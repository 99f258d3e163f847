"""Summarise a rocprofv3 kernel trace of bench.py as the markdown kept with
the profiles.

    rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_bench -o bench -- \\
        python3 -u bench.py --no-stream --no-cpu > gpurun_out/prof_bench.json
    python3 -m quant_dequant_gemv_amd.profsum gpurun_out/prof_bench/bench_kernel_trace.csv \\
        gpurun_out/prof_bench.json profiles/<name>.md --command "<the rocprofv3 command>" \\
        --stats gpurun_out/prof_bench/bench_kernel_stats.csv

Dispatches are grouped by kernel, workgroup size and grid size (one group per
tensor shape, since shapes sharing a kernel instance differ in launch
geometry).  The timed region of bench.py is the first warmup*3 + steps*3
one-column Q4_K GEMV dispatches after the warm-up ones; their mean duration
is set beside bench.py's own roofline.avg_launch_us from the same run.
"""
from __future__ import annotations

import argparse
import csv
import json
import re
import statistics


def short(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\(.*\)$", "", name)


def load(trace: str):
    rows = []
    with open(trace, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Kind", "KERNEL_DISPATCH") != "KERNEL_DISPATCH":
                continue
            rows.append(dict(name=short(r["Kernel_Name"]), dispatch=int(r["Dispatch_Id"]),
                             us=(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3,
                             wg=int(r["Workgroup_Size_X"]), grid=int(r["Grid_Size_X"]),
                             lds=int(r["LDS_Block_Size"]), vgpr=int(r["VGPR_Count"]),
                             scratch=int(r["Scratch_Size"])))
    rows.sort(key=lambda r: r["dispatch"])
    return rows


def _bench(path: str) -> dict:
    with open(path) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def stats_rows(stats_csv: str) -> list:
    """The library's rows of a rocprofv3 --stats kernel table (all dispatches
    of each kernel name in the run)."""
    out = ["| kernel (rocprofv3 --stats) | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    with open(stats_csv, newline="") as f:
        for r in csv.DictReader(f):
            name = short(r["Name"])
            if not name.startswith("qk::"):
                continue
            out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) * 1e-3:.3f} | "
                       f"{float(r['MinNs']) * 1e-3:.3f} | {float(r['MaxNs']) * 1e-3:.3f} | "
                       f"{float(r['Percentage']):.1f}% |")
    return out


def summarise(trace: str, bench_json: str, command: str, plain_json: str | None = None,
              stats_csv: str | None = None) -> str:
    rows = load(trace)
    bench = _bench(bench_json)
    total = sum(r["us"] for r in rows)
    groups = {}
    for r in rows:
        groups.setdefault((r["name"], r["wg"], r["grid"]), []).append(r)
    out = ["| kernel | threads/WG | WGs | calls | avg us | median us | min us | max us | share |",
           "|---|---|---|---|---|---|---|---|---|"]
    for (name, wg, grid), g in sorted(groups.items(), key=lambda kv: -sum(r["us"] for r in kv[1])):
        d = [r["us"] for r in g]
        out.append(f"| `{name}` | {wg} | {grid // max(wg, 1)} | {len(d)} | {statistics.mean(d):.3f} | "
                   f"{statistics.median(d):.3f} | {min(d):.3f} | {max(d):.3f} | {100 * sum(d) / total:.1f}% |")
    step = [r for r in rows if r["name"].startswith("qk::gemv1_kernel<12,")]
    per_step = 3
    w, k = int(bench["warmup"]), int(bench["steps"])
    timed = step[w * per_step:(w + k) * per_step]
    rl = bench["roofline"]
    lines = [f"Command (run from the repository root on one MI355X):", "", f"    {command}", "",
             "Every dispatch of the profiled run, grouped by kernel and launch geometry "
             "(one group per tensor shape):", ""] + out
    if timed:
        avg = statistics.mean(r["us"] for r in timed)
        achieved = rl["bytes_per_launch"] / (avg * 1e-6) / 1e9
        lines += ["", "Timed region of bench.py (its warm-up and timed graphs are the first "
                  f"{(w + k) * per_step} one-column Q4_K dispatches; the last {k * per_step} are timed):", "",
                  f"- rocprofv3 mean duration of the {len(timed)} timed dispatches: {avg:.3f} us",
                  f"- bench.py `roofline.avg_launch_us` of the same run (HIP-event span / launches): "
                  f"{rl['avg_launch_us']:.3f} us (ratio {rl['avg_launch_us'] / avg:.3f})",
                  f"- algorithmic bytes per launch {rl['bytes_per_launch']} -> {achieved:.1f} GB/s by rocprofv3, "
                  f"{rl['achieved']:.1f} GB/s by bench.py = {rl['frac']:.3f} of {rl['peak']:.0f} GB/s",
                  f"- bench.py `value` of the same run: {bench['value']} {bench['unit']}"]
        if plain_json:
            pb = _bench(plain_json)
            prl = pb["roofline"]
            lines += [f"- the same bench.py without the profiler, just before on the same GPU: "
                      f"`roofline.avg_launch_us` {prl['avg_launch_us']:.3f} us (ratio {prl['avg_launch_us'] / avg:.3f} "
                      f"to the traced kernel mean), achieved {prl['achieved']:.1f} GB/s = {prl['frac']:.3f}, "
                      f"`value` {pb['value']} {pb['unit']}.  Tracing adds time between dispatches, which "
                      f"the event span counts and the kernel durations do not."]
    if stats_csv:
        lines += ["", "The same run's rocprofv3 --stats table (averages over every dispatch of a kernel "
                  "instance in the run: warm-up, timed region and the per-shape sections below):", ""]
        lines += stats_rows(stats_csv)
    lines += ["", "Per-shape times reported by bench.py in the same run (graph of back-to-back launches of one "
              "tensor over >= 1.2 GB of copies):", ""]
    for sec in ("per_gemv", "mixed_types", "verify"):
        for r in bench.get(sec, []):
            extra = f", ncols {r['ncols']}" if "ncols" in r else ""
            lines.append(f"- {r['name']} ({r['type']} {r['N']}x{r['K']}{extra}): {r['us']} us, "
                         f"{r['weight_GBs']} GB/s")
    lines.append(f"\nKernel source hash (bench.py `kernel_hash`): {bench.get('kernel_hash')}")
    return "\n".join(lines) + "\n"


def summarise_stream(trace: str, stream_json: str, command: str, plain_json: str | None = None) -> str:
    """A trace of `bench.py --stream-only VARIANT --tokens T`: the last
    T * launches_per_token dispatches of the library's kernels are the timed
    tokens; their summed durations per token are the gap-free bound of the
    stream, beside the event span per token."""
    rows = [r for r in load(trace) if r["name"].startswith("qk::")]
    st = _bench(stream_json)
    T, L = st["tokens"], st["launches_per_token"]
    timed = rows[-T * L:]
    kern_ms = sum(r["us"] for r in timed) / T * 1e-3
    groups = {}
    for r in timed:
        groups.setdefault(r["name"], []).append(r["us"])
    lines = [f"Command (run from the repository root on one MI355X):\n\n    {command}\n",
             f"Decode stream variant `{st['variant']}`: {L} launches per token, {T} timed tokens after "
             f"{st['warm_tokens']} warm-up tokens.\n",
             "| kernel | dispatches per token | total us per token | share |", "|---|---|---|---|"]
    for name, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {len(d) / T:.0f} | {sum(d) / T:.1f} | {sum(d) / T / (kern_ms * 1e3):.1%} |")
    lines += ["",
              f"- sum of kernel durations per token (the gap-free bound): {kern_ms:.4f} ms "
              f"-> {1 / kern_ms * 1e3:.1f} tok/s",
              f"- event span per token in the same traced run: {st['token_ms']:.4f} ms "
              f"(kernels busy {kern_ms / st['token_ms']:.1%} of it)"]
    if plain_json:
        pl = _bench(plain_json)
        lines.append(f"- the same variant without the profiler, just before on the same GPU: {pl['token_ms']:.4f} ms "
                     f"per token ({pl['tok_s']:.1f} tok/s; the traced kernel durations sum to {kern_ms / pl['token_ms']:.1%} of it)")
    if "device" in st:
        lines.append(f"- device: {st['device']}")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("trace")
    ap.add_argument("bench_json")
    ap.add_argument("out")
    ap.add_argument("--command", required=True)
    ap.add_argument("--plain", help="bench.py JSON of an unprofiled run on the same GPU")
    ap.add_argument("--title", help="heading (default: by the kind of trace)")
    ap.add_argument("--stream", action="store_true", help="the trace is of bench.py --stream-only")
    ap.add_argument("--stats", help="the run's rocprofv3 --stats kernel table (CSV)")
    a = ap.parse_args()
    body = (summarise_stream(a.trace, a.bench_json, a.command, a.plain) if a.stream
            else summarise(a.trace, a.bench_json, a.command, a.plain, a.stats))
    title = a.title
    if title is None and a.stream:
        with open(a.bench_json) as f:
            variant = json.loads(f.read().strip().splitlines()[-1])["variant"]
        title = f"Decode stream, one token of the 64-layer weight stream ({variant}): rocprofv3 kernel trace"
    elif title is None:
        title = "gemv1_kernel (one column): Q4_K projection step, rocprofv3 kernel trace"
    text = f"# {title}\n\n" + body
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
