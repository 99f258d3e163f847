#!/usr/bin/env python3
"""Benchmark of the MI355X k-quant GEMV: weight GB/s, fraction of HBM peak, and
the implied tokens/s of a 64-layer decode weight stream.

One step is one pass over the Q4_K projection workload of a 27B hybrid
DeltaNet/GQA decoder at hidden size 5120: three GEMVs, N = 10240 (fused
DeltaNet QKV), 12288 (attention Q) and 17408 (FFN gate/up), K = 5120, one
column, fp16 x.  Weights are seeded synthetic superblocks (the real GGUF
weights are not available); enough distinct copies are rotated that every step
reads them from HBM, not from the 256 MB Infinity Cache.

Printed: one JSON line (rank 0).  `value` is weight bytes / wall time of the
timed steps; `roofline.achieved` is the algorithmic bytes of one launch of the
dominant kernel over its average duration, measured with HIP events on the
launch stream; `cpu_baseline` times the CPU oracle on the host.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
MIN_ROTATION_BYTES = 1.2e9  # > 4x the 256 MB Infinity Cache
METRIC = "weight GB/s and % of HBM peak per GEMV; implied tok/s for 64-layer stream"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

def kernel_hash() -> str:
    """Hash of the one-column kernel's sources (the one profiles/traffic.json records)."""
    from quant_dequant_gemv_amd import traffic
    return traffic.kernel_hash()


def algorithmic_bytes(qt, N, K, ncols=1):
    from quant_dequant_gemv_amd import synth
    return N * synth.row_bytes(qt, K) + 2 * K * ncols + 4 * N * ncols


class Launcher:
    """Direct ctypes calls of qk_gemv with pre-computed device addresses."""

    def __init__(self):
        from quant_dequant_gemv_amd import binding
        self.lib = binding.load_library()

    def gemv(self, qt, W, x, y, N, K, ncols, stream):
        rc = self.lib.qk_gemv(qt, W, x, y, N, K, ncols, stream)
        if rc != 0:
            from quant_dequant_gemv_amd import binding
            raise binding.QKError(rc, "qk_gemv")


def make_tensors(torch, entries, seed_offset=0):
    """Device weights (with rotation copies), x and y for each entry."""
    from quant_dequant_gemv_amd import synth
    out = []
    for e in entries:
        W = synth.superblocks(e["qtype"], e["N"], e["K"], e["seed"] + seed_offset)
        Wd = torch.from_numpy(W.reshape(-1)).cuda()
        x = torch.from_numpy(synth.activations(e["K"], e.get("ncols", 1), e["seed"])).cuda()
        y = torch.empty((e["N"], e.get("ncols", 1)), dtype=torch.float32, device="cuda")
        out.append(dict(e, W=[Wd], x=x, y=y, bytes=Wd.numel()))
    return out


def progress(msg):
    """One line per finished section on stderr (the JSON line stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_planar(torch, entries):
    """The same tensors repacked once into PLANAR rows (qk_repack, outside any
    timed region); bytes stay the GGUF weight bytes, the algorithmic count."""
    from quant_dequant_gemv_amd import binding, synth
    out = []
    for t in make_tensors(torch, entries):
        Wp = binding.repack(t["qtype"], t["W"][0], t["N"], t["K"])
        torch.cuda.synchronize()
        out.append(dict(t, qtype=t["qtype"] | binding.PLANAR, W=[Wp], bytes=t["N"] * synth.row_bytes(t["qtype"], t["K"])))
    return out


def add_rotation(tensors):
    total = sum(t["bytes"] for t in tensors)
    copies = max(2, int(-(-MIN_ROTATION_BYTES // total)))
    for t in tensors:
        t["W"] += [t["W"][0].clone() for _ in range(copies - 1)]
    return copies


def capture(torch, launcher, calls):
    """One HIP graph replaying `calls` = [(tensor, copy index), ...] in order."""
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for t, c in calls:
            launcher.gemv(t["qtype"], t["W"][c].data_ptr(), t["x"].data_ptr(), t["y"].data_ptr(),
                          t["N"], t["K"], t["x"].shape[1], s.cuda_stream)
    return g


# A GPU that has idled (while the host builds inputs or captures a graph)
# runs its first milliseconds of work at lower clocks: replays of one graph
# measured 14.2 -> 12.5 us per launch over the first ~6 ms.  Every timed
# region is therefore preceded by this busy-wait kernel on the same stream,
# outside the timed span.
SPIN_CYCLES = int(2e7)


def graph_span(torch, g, reps=3):
    """Median HIP-event span (s) of one replay on the current stream; each
    timed replay follows a GPU busy-wait (outside the span)."""
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    spans = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN_CYCLES)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        spans.append(a.elapsed_time(b) * 1e-3)
    return sorted(spans)[len(spans) // 2]


def per_shape(torch, launcher, tensors):
    """Average kernel duration per tensor: its own rotation of >= 1.2 GB of
    copies, one graph of back-to-back launches of that tensor alone, event
    span / launches."""
    from quant_dequant_gemv_amd import synth
    out = []
    for t in tensors:
        base = t["W"]
        t["W"] = [base[0]]
        copies = add_rotation([t])
        n = 4 * copies
        g = capture(torch, launcher, [(t, i % copies) for i in range(n)])
        us = graph_span(torch, g) / n * 1e6
        del g
        t["W"] = base
        torch.cuda.empty_cache()
        out.append({"name": t["name"], "type": synth.TYPE_NAMES[t["qtype"] & 0xff], "N": t["N"], "K": t["K"],
                    "us": round(us, 3), "weight_GBs": round(t["bytes"] / us / 1e3, 1),
                    "frac_peak": round(t["bytes"] / us / 1e3 / PEAK_HBM_GBS, 4), "rotation_copies": copies})
    return out


def ab_us(torch, launches, n, reps=3):
    """Average duration (us) per call of each launch(i, stream), i < n, each
    captured in its own graph; the graphs are replayed in turn `reps` times
    (so neither always runs first on freshly allocated memory) and each
    keeps its fastest replay."""
    graphs = []
    for launch in launches:
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                launch(i, s.cuda_stream)
        graphs.append(g)
    best = [float("inf")] * len(graphs)
    for _ in range(reps):
        for k, g in enumerate(graphs):
            best[k] = min(best[k], graph_span(torch, g, reps=1) / n * 1e6)
    del graphs
    return best


def fused_epilogues(torch):
    """The fused epilogues at the FFN shapes, each beside its unfused form on
    the same weights: gate/up as one SwiGLU launch vs the two-entry merged
    launch (no SiLU, no product), and FFN down with its residual added in
    place vs plain.  Rotation over >= 1.2 GB of weight copies."""
    import ctypes

    from quant_dequant_gemv_amd import binding, synth
    lib = binding.load_library()
    out = []
    N, K = 17408, 5120
    for nc in (1, 4):
        Wg = torch.from_numpy(synth.superblocks(synth.Q4_K, N, K, 1005).reshape(-1)).cuda()
        Wu = torch.from_numpy(synth.superblocks(synth.Q4_K, N, K, 1006).reshape(-1)).cuda()
        pair = 2 * Wg.numel()
        copies = max(2, int(-(-MIN_ROTATION_BYTES // pair)))
        Wgs = [Wg] + [Wg.clone() for _ in range(copies - 1)]
        Wus = [Wu] + [Wu.clone() for _ in range(copies - 1)]
        x = torch.from_numpy(synth.activations(K, nc, 1005)).cuda()
        y = torch.empty((N, nc), dtype=torch.float32, device="cuda")
        y2 = torch.empty((N, nc), dtype=torch.float32, device="cuda")

        def swiglu(i, st):
            rc = lib.qk_gemv_swiglu(synth.Q4_K, Wgs[i % copies].data_ptr(), Wus[i % copies].data_ptr(),
                                    x.data_ptr(), y.data_ptr(), N, K, nc, 0, st)
            if rc:
                raise binding.QKError(rc, "qk_gemv_swiglu")

        def separate(i, st):
            if nc == 1:
                items = (binding.qk_gemv_item * 2)(
                    binding.qk_gemv_item(synth.Q4_K, Wgs[i % copies].data_ptr(), x.data_ptr(), y.data_ptr(), N, K),
                    binding.qk_gemv_item(synth.Q4_K, Wus[i % copies].data_ptr(), x.data_ptr(), y2.data_ptr(), N, K))
                rc = lib.qk_gemv_batch(items, 2, st)
            else:
                rc = lib.qk_gemv(synth.Q4_K, Wgs[i % copies].data_ptr(), x.data_ptr(), y.data_ptr(), N, K, nc, st)
                rc = rc or lib.qk_gemv(synth.Q4_K, Wus[i % copies].data_ptr(), x.data_ptr(), y2.data_ptr(), N, K,
                                       nc, st)
            if rc:
                raise binding.QKError(rc, "unfused gate/up")

        t_f, t_s = ab_us(torch, [swiglu, separate], 4 * copies)
        out.append({"name": f"ffn_gate_up_swiglu_ncols{nc}", "type": "Q4_K", "N": N, "K": K, "ncols": nc,
                    "us": round(t_f, 3), "weight_GBs": round(pair / t_f / 1e3, 1),
                    "frac_peak": round(pair / t_f / 1e3 / PEAK_HBM_GBS, 4),
                    "unfused": "one qk_gemv_batch launch of both" if nc == 1 else "two qk_gemv launches",
                    "unfused_us": round(t_s, 3), "rotation_copies": copies})
        del Wgs, Wus, Wg, Wu
        torch.cuda.empty_cache()

    Nd, Kd = 5120, 17408
    W = torch.from_numpy(synth.superblocks(synth.Q6_K, Nd, Kd, 4).reshape(-1)).cuda()
    copies = max(2, int(-(-MIN_ROTATION_BYTES // W.numel())))
    Ws = [W] + [W.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.activations(Kd, 1, 4)).cuda()
    h = torch.zeros((Nd, 1), dtype=torch.float32, device="cuda")
    yp = torch.empty((Nd, 1), dtype=torch.float32, device="cuda")

    def resid(i, st):
        rc = lib.qk_gemv_ex(synth.Q6_K, Ws[i % copies].data_ptr(), x.data_ptr(), h.data_ptr(), Nd, Kd, 1,
                            ctypes.c_void_p(h.data_ptr()), 0, st)
        if rc:
            raise binding.QKError(rc, "qk_gemv_ex")

    def plain(i, st):
        rc = lib.qk_gemv(synth.Q6_K, Ws[i % copies].data_ptr(), x.data_ptr(), yp.data_ptr(), Nd, Kd, 1, st)
        if rc:
            raise binding.QKError(rc, "qk_gemv")

    t_f, t_p = ab_us(torch, [resid, plain], 4 * copies)
    out.append({"name": "ffn_down_residual_inplace", "type": "Q6_K", "N": Nd, "K": Kd, "ncols": 1,
                "us": round(t_f, 3), "weight_GBs": round(W.numel() / t_f / 1e3, 1),
                "frac_peak": round(W.numel() / t_f / 1e3 / PEAK_HBM_GBS, 4),
                "unfused": "qk_gemv without the residual", "unfused_us": round(t_p, 3),
                "rotation_copies": copies})
    del Ws, W
    torch.cuda.empty_cache()
    return out


def read_ceiling(torch, sizes):
    """The achievable-bandwidth reference: a plain 16-byte read of buffers of
    the step's sizes (libqkcalib.so: non-temporal loads, grid-stride), one
    launch per buffer, rotated over >= 1.2 GB of copies like the GEMV step and
    replayed from one graph; the fastest of three launch shapes."""
    lib = _calib_lib()
    total = sum(sizes)
    copies = max(2, int(-(-MIN_ROTATION_BYTES // total)))
    bufs = [[torch.empty(n, dtype=torch.uint8, device="cuda").fill_(c % 251) for n in sizes] for c in range(copies)]
    out = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    best = None
    for blocks, threads in ((512, 1024), (1024, 512), (2048, 256)):
        def launch(i, st, blocks=blocks, threads=threads):
            c, k = divmod(i, len(sizes))
            rc = lib.qk_stream_read(bufs[c % copies][k].data_ptr(), sizes[k], out.data_ptr(), blocks, threads, st)
            if rc != 0:
                raise RuntimeError(f"qk_stream_read failed: {rc}")
        n = 4 * copies * len(sizes)
        us = ab_us(torch, [launch], n)[0]
        if best is None or us < best[0]:
            best = (us, blocks, threads)
    us, blocks, threads = best
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "plain 16-byte read, non-temporal loads, grid-stride (libqkcalib.so)",
            "bytes_per_launch": round(total / len(sizes)), "avg_launch_us": round(us, 3),
            "GBs": round(total / len(sizes) / us / 1e3, 1), "blocks": blocks, "threads": threads,
            "rotation_copies": copies}


def _calib_lib():
    from quant_dequant_gemv_amd import calib
    return calib.load()


SUSTAINED_BYTES = 4 << 30


def sustained_read(torch, shapes=((512, 1024), (1024, 512), (2048, 256), (4096, 256))):
    """HBM's sustained streaming rate: one launch of the plain 16-byte read
    (non-temporal loads, XOR-folded) over a 4 GiB buffer -- 16x the Infinity
    Cache, so nothing is served twice, and ~0.5 ms long, so a launch's fixed
    dispatch / fill / drain cost is well under 1% of it.  Median of three
    launches per shape, each after a GPU busy-wait; the fastest shape."""
    lib = _calib_lib()
    buf = torch.empty(SUSTAINED_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
    out = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for blocks, threads in shapes:
        spans = []
        for _ in range(3):
            torch.cuda._sleep(SPIN_CYCLES)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = lib.qk_stream_read(buf.data_ptr(), SUSTAINED_BYTES, out.data_ptr(), blocks, threads,
                                    stream.cuda_stream)
            b.record(stream)
            if rc != 0:
                raise RuntimeError(f"qk_stream_read failed: {rc}")
            torch.cuda.synchronize()
            spans.append(a.elapsed_time(b) * 1e-3)
        us = sorted(spans)[1] * 1e6
        if best is None or us < best[0]:
            best = (us, blocks, threads)
    us, blocks, threads = best
    del buf
    torch.cuda.empty_cache()
    gbs = SUSTAINED_BYTES / us / 1e3
    return {"kernel": "plain 16-byte read, non-temporal loads, grid-stride (libqkcalib.so)",
            "bytes": SUSTAINED_BYTES, "us": round(us, 1), "GBs": round(gbs, 1),
            "frac_peak": round(gbs / PEAK_HBM_GBS, 4), "blocks": blocks, "threads": threads}


def cpu_baseline(entries, min_seconds=10.0):
    """The CPU oracle on the step's three GEMVs (all rows), repeated until at
    least `min_seconds` of wall time; plus one single-threaded step."""
    import oracle
    from quant_dequant_gemv_amd import synth
    data = [(e["qtype"], synth.superblocks(e["qtype"], e["N"], e["K"], e["seed"]),
             synth.activations(e["K"], 1, e["seed"]), e["K"]) for e in entries]
    threads = oracle.default_threads()
    oracle.load()
    nbytes = sum(W.size for _, W, _, _ in data)
    steps = 0
    t0 = time.perf_counter()
    while True:
        for qt, W, x, K in data:
            oracle.gemv(qt, W, x, K, nthreads=threads)
        steps += 1
        t = time.perf_counter() - t0
        if t >= min_seconds and steps >= 3:
            break
    t1 = time.perf_counter()
    for qt, W, x, K in data:
        oracle.gemv(qt, W, x, K, nthreads=1)
    one = time.perf_counter() - t1
    return {"value": round(steps * nbytes / t / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full steps (3 GEMVs, {nbytes} weight bytes each) in {t:.1f} s wall",
            "one_thread_GBs": round(nbytes / one / 1e9, 4),
            "cpu": _cpu_model(), "workloads": cpu_workloads(threads)}


def _oracle_rate(calls, min_seconds):
    """Wall seconds per pass of `calls` (oracle GEMVs), repeated until
    min_seconds (at least one pass)."""
    import oracle
    n, t0 = 0, time.perf_counter()
    while True:
        for qt, W, x, K, threads in calls:
            oracle.gemv(qt, W, x, K, nthreads=threads)
        n += 1
        t = time.perf_counter() - t0
        if t >= min_seconds:
            return t / n, n


def cpu_workloads(threads):
    """The CPU oracle on the other workloads, each a bounded sample: the small
    Q4_K 1024 x 5120 GEMV; the Q6_K / Q5_K pair; the verify shape at 1-8
    columns; and the decode token, sampled as layers 0-3 (three DeltaNet
    layers and one attention layer: 28 of the 448 GEMVs, the same mix as the
    whole 64 layers) and scaled by 16."""
    from quant_dequant_gemv_amd import synth

    def data(e, ncols=1):
        return (e["qtype"], synth.superblocks(e["qtype"], e["N"], e["K"], e["seed"]),
                synth.activations(e["K"], ncols, e["seed"]), e["K"], threads)

    out = {}
    d = data(synth.SMALL)
    sec, n = _oracle_rate([d], 1.0)
    out["small_q4k_1024x5120"] = {"ms_per_gemv": round(sec * 1e3, 3), "weight_GBs": round(d[1].size / sec / 1e9, 3),
                                  "passes": n}
    ds = [data(e) for e in synth.MIXED]
    out["mixed_types"] = []
    for e, d in zip(synth.MIXED, ds):
        sec, n = _oracle_rate([d], 1.0)
        out["mixed_types"].append({"name": e["name"], "type": synth.TYPE_NAMES[e["qtype"]], "N": e["N"], "K": e["K"],
                                   "ms_per_gemv": round(sec * 1e3, 2),
                                   "weight_GBs": round(d[1].size / sec / 1e9, 3), "passes": n})
    v = synth.VERIFY
    out["verify_q4k_17408x5120"] = []
    W = synth.superblocks(v["qtype"], v["N"], v["K"], v["seed"])
    for nc in v["ncols"]:
        d = (v["qtype"], W, synth.activations(v["K"], nc, v["seed"]), v["K"], threads)
        sec, n = _oracle_rate([d], 0.5)
        out["verify_q4k_17408x5120"].append({"ncols": nc, "ms_per_call": round(sec * 1e3, 2),
                                             "weight_GBs": round(W.size / sec / 1e9, 3), "passes": n})
    del W
    sample = [e for e in synth.decode_stream() if e["layer"] < 4]
    calls = [data(e) for e in sample]
    nbytes = sum(c[1].size for c in calls)
    sec, n = _oracle_rate(calls, 1.0)
    scale = synth.N_LAYERS / 4
    out["decode_token"] = {"s_per_token": round(sec * scale, 3), "tok_s": round(1.0 / (sec * scale), 4),
                           "weight_GBs": round(nbytes / sec / 1e9, 3),
                           "sample": f"layers 0-3 ({len(sample)} GEMVs, {nbytes} weight bytes) x {n} passes "
                                     f"in {sec * n:.2f} s, scaled by {scale:g} to the 64-layer token"}
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def traffic_for(kernel, frac_bytes):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    v = t.get("per_launch_bytes", {}).get(kernel)
    return v


def device_info(torch):
    """GPU name, architecture, CUs, memory and HIP version.  (No clock
    reading: a query after the run sees the idle clock, not the one the timed
    region ran at.)"""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "memory_GB": round(p.total_memory / 1e9, 1), "hip": torch.version.hip}


def run_stream(torch, launcher, warm=2, only=None, tokens=1):
    """448 GEMVs of one decode token, all weights resident, back to back on
    one stream: one launch per GEMV; one qk_gemv_batch launch per group of
    projections that read the same activations (256 launches); and the same
    256 launches with the epilogues fused (SwiGLU gate/up, residual adds).
    Each is timed as plain launches enqueued ahead of the GPU (behind a spin
    kernel) and as one captured graph; HIP-event spans."""
    import ctypes

    from quant_dequant_gemv_amd import binding, synth
    entries = synth.decode_stream()
    groups = synth.decode_groups(entries)
    tensors = make_tensors(torch, entries)
    for idx in groups:  # a group's projections read one activation vector
        for i in idx[1:]:
            tensors[i]["x"] = tensors[idx[0]]["x"]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    lib = binding.load_library()
    batches = []
    for idx in groups:
        arr = (binding.qk_gemv_item * len(idx))(*[
            binding.qk_gemv_item(tensors[i]["qtype"], tensors[i]["W"][0].data_ptr(), tensors[i]["x"].data_ptr(),
                                 tensors[i]["y"].data_ptr(), tensors[i]["N"], tensors[i]["K"]) for i in idx])
        batches.append((arr, len(idx)))

    # fused: gate+up as one SwiGLU launch, the mixer output and FFN down
    # projections adding into an fp32 residual stream in place, the other
    # groups merged as above -- the same launch count
    hres = torch.zeros(synth.HIDDEN, dtype=torch.float32, device="cuda")
    fused = []
    for (arr, n), idx in zip(batches, groups):
        names = [entries[i]["name"] for i in idx]
        if names == ["ffn_gate", "ffn_up"]:
            g, u = tensors[idx[0]], tensors[idx[1]]
            fused.append(("swiglu", (g["qtype"], g["W"][0].data_ptr(), u["W"][0].data_ptr(), g["x"].data_ptr(),
                                     g["y"].data_ptr(), g["N"], g["K"], 1, 0)))
        elif len(idx) == 1 and names[0] in ("ssm_out", "attn_output", "ffn_down"):
            t = tensors[idx[0]]
            fused.append(("ex", (t["qtype"], t["W"][0].data_ptr(), t["x"].data_ptr(), hres.data_ptr(), t["N"],
                                 t["K"], 1, ctypes.c_void_p(hres.data_ptr()), 0)))
        else:
            fused.append(("batch", (arr, n)))

    # the same fused stream with every tensor on PLANAR rows (each repacked
    # once here, outside the timed regions)
    planar_w = {}
    for i, t in enumerate(tensors):
        planar_w[i] = binding.repack(t["qtype"], t["W"][0], t["N"], t["K"])
    torch.cuda.synchronize()

    def wp(i):  # (type, weight address) of entry i on the rows this stream uses
        t = tensors[i]
        return (t["qtype"] | binding.PLANAR, planar_w[i].data_ptr()) if i in planar_w else \
            (t["qtype"], t["W"][0].data_ptr())

    fused_planar = []
    for (arr, n), idx in zip(batches, groups):
        names = [entries[i]["name"] for i in idx]
        if names == ["ffn_gate", "ffn_up"]:
            (tg, pg), (_, pu) = wp(idx[0]), wp(idx[1])
            g = tensors[idx[0]]
            fused_planar.append(("swiglu", (tg, pg, pu, g["x"].data_ptr(), g["y"].data_ptr(), g["N"], g["K"], 1, 0)))
        elif len(idx) == 1 and names[0] in ("ssm_out", "attn_output", "ffn_down"):
            t = tensors[idx[0]]
            tt, pw = wp(idx[0])
            fused_planar.append(("ex", (tt, pw, t["x"].data_ptr(), hres.data_ptr(), t["N"], t["K"], 1,
                                        ctypes.c_void_p(hres.data_ptr()), 0)))
        else:
            items = (binding.qk_gemv_item * len(idx))(*[
                binding.qk_gemv_item(*wp(i), tensors[i]["x"].data_ptr(), tensors[i]["y"].data_ptr(),
                                     tensors[i]["N"], tensors[i]["K"]) for i in idx])
            fused_planar.append(("batch", (items, len(idx))))

    def run_fused(plan, h):
        for kind, a in plan:
            if kind == "swiglu":
                rc = lib.qk_gemv_swiglu(*a, h)
            elif kind == "ex":
                rc = lib.qk_gemv_ex(*a, h)
            else:
                rc = lib.qk_gemv_batch(*a, h)
            if rc != 0:
                raise binding.QKError(rc, kind)

    def one_token_fused_planar(st=None):
        run_fused(fused_planar, sh if st is None else st)

    # the same fused steps as one chain launch (qk_gemv_chain): one step per
    # group, a barrier between steps, each step's first weights issued before
    # its wait
    def chain_of(use_planar):
        steps = []
        for idx in groups:
            names = [entries[i]["name"] for i in idx]
            ws = [wp(i) if use_planar else (tensors[i]["qtype"], tensors[i]["W"][0]) for i in idx]
            wt = [(q, planar_w[i] if use_planar else tensors[i]["W"][0]) for (q, _), i in zip(ws, idx)]
            if names == ["ffn_gate", "ffn_up"]:
                g = tensors[idx[0]]
                steps.append([dict(qtype=wt[0][0], W=wt[0][1], W2=wt[1][1], x=g["x"], y=g["y"], N=g["N"],
                                   K=g["K"])])
            elif len(idx) == 1 and names[0] in ("ssm_out", "attn_output", "ffn_down"):
                t = tensors[idx[0]]
                steps.append([dict(qtype=wt[0][0], W=wt[0][1], x=t["x"], y=hres, residual=hres, N=t["N"],
                                   K=t["K"])])
            else:
                steps.append([dict(qtype=q, W=w, x=tensors[i]["x"], y=tensors[i]["y"], N=tensors[i]["N"],
                                   K=tensors[i]["K"]) for (q, w), i in zip(wt, idx)])
        return binding.Chain(steps)

    chains = {"chain": chain_of(False), "chain_planar": chain_of(True)}

    def chain_token(name):
        ch = chains[name]

        def run(st=None):
            ch.run(stream=sh if st is None else st)
        return run

    def one_token_fused(st=None):
        h = sh if st is None else st
        for kind, a in fused:
            if kind == "swiglu":
                rc = lib.qk_gemv_swiglu(*a, h)
            elif kind == "ex":
                rc = lib.qk_gemv_ex(*a, h)
            else:
                rc = lib.qk_gemv_batch(*a, h)
            if rc != 0:
                raise binding.QKError(rc, kind)

    def one_token():
        for t in tensors:
            launcher.gemv(t["qtype"], t["W"][0].data_ptr(), t["x"].data_ptr(), t["y"].data_ptr(),
                          t["N"], t["K"], 1, sh)

    def one_token_batched(st=None):
        h = sh if st is None else st
        for arr, n in batches:
            rc = lib.qk_gemv_batch(arr, n, h)
            if rc != 0:
                raise binding.QKError(rc, "qk_gemv_batch")

    def spans_of(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        spans = []
        for _ in range(3):
            torch.cuda._sleep(int(2e7))
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            spans.append(a.elapsed_time(b) * 1e-3)
        return sorted(spans)[1]

    def graph_of(fn):
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn(s.cuda_stream)
        sp = graph_span(torch, g)
        del g
        return sp

    if only is not None:
        # one variant, `tokens` tokens back to back after a warm-up (for a
        # kernel trace: the last tokens * launches dispatches are the timed ones)
        fns = {"launches": one_token, "batched": one_token_batched, "fused": one_token_fused,
               "fused_planar": one_token_fused_planar, "chain": chain_token("chain"),
               "chain_planar": chain_token("chain_planar")}
        graph = only.endswith("_graph")
        fn = fns[only[:-6] if graph else only]
        launches = len(entries) if fn is one_token else 2 if only.startswith("chain") else len(groups)
        if graph:
            s2 = torch.cuda.Stream()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=s2):
                if fn is one_token:
                    for t in tensors:
                        launcher.gemv(t["qtype"], t["W"][0].data_ptr(), t["x"].data_ptr(), t["y"].data_ptr(),
                                      t["N"], t["K"], 1, s2.cuda_stream)
                else:
                    fn(s2.cuda_stream)
            run = gr.replay
        else:
            run = fn
        for _ in range(warm):
            run()
        torch.cuda._sleep(SPIN_CYCLES)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(tokens):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        sp = a.elapsed_time(b) * 1e-3 / tokens
        return {"variant": only, "tokens": tokens, "launches_per_token": launches, "warm_tokens": warm,
                "token_ms": round(sp * 1e3, 4), "tok_s": round(1 / sp, 2)}

    span = spans_of(one_token)
    g = capture(torch, launcher, [(t, 0) for t in tensors])
    gspan = graph_span(torch, g)
    del g
    bspan = spans_of(one_token_batched)
    bgspan = graph_of(one_token_batched)
    fspan = spans_of(one_token_fused)
    fgspan = graph_of(one_token_fused)
    fpgspan = graph_of(one_token_fused_planar)
    cspan = spans_of(chain_token("chain"))
    cpspan = spans_of(chain_token("chain_planar"))
    for ch in chains.values():
        if ch.status() != 0:
            raise RuntimeError("chain run gave up at a barrier")
    nbytes = synth.weight_bytes(entries)
    del tensors, batches, fused, fused_planar, planar_w, chains
    torch.cuda.empty_cache()

    def rec(sp, launches):
        return {"launches_per_token": launches, "token_ms": round(sp * 1e3, 4), "tok_s": round(1 / sp, 2),
                "weight_GBs": round(nbytes / sp / 1e9, 1)}
    return {"gemvs": len(entries), "weight_bytes": nbytes,
            "launches": rec(span, len(entries)), "graph": rec(gspan, len(entries)),
            "batched": rec(bspan, len(groups)), "batched_graph": rec(bgspan, len(groups)),
            "fused": rec(fspan, len(groups)), "fused_graph": rec(fgspan, len(groups)),
            "fused_planar_graph": rec(fpgspan, len(groups)),
            "chain": rec(cspan, 2), "chain_planar": rec(cpspan, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-stream", action="store_true", help="skip the 448-GEMV decode stream")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--stream-only", metavar="VARIANT",
                    choices=["launches", "launches_graph", "batched", "batched_graph", "fused", "fused_graph",
                             "fused_planar", "fused_planar_graph", "chain", "chain_planar"],
                    help="only time this decode-stream variant for --tokens tokens (for a kernel trace); "
                         "prints its own JSON line instead of the benchmark's")
    ap.add_argument("--tokens", type=int, default=5)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(row sharding across GPUs is a design note, not an implementation). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quant_dequant_gemv_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    launcher = Launcher()
    if args.stream_only:
        r = run_stream(torch, launcher, only=args.stream_only, tokens=args.tokens)
        r["device"] = device_info(torch)
        print(json.dumps(r))
        return

    entries = synth.Q4K_PROJECTIONS
    tensors = make_tensors(torch, entries)
    copies = add_rotation(tensors)
    step_bytes = sum(t["bytes"] for t in tensors)
    step_alg = sum(algorithmic_bytes(t["qtype"], t["N"], t["K"]) for t in tensors)
    # exactly K steps in one graph (step i reads rotation set i mod copies)
    timed = capture(torch, launcher, [(t, i % copies) for i in range(args.steps) for t in tensors])
    warm = capture(torch, launcher, [(t, i % copies) for i in range(max(1, args.warmup)) for t in tensors])
    warm.replay()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(SPIN_CYCLES)  # clocks at their steady state (see graph_span)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    timed.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = e0.elapsed_time(e1) * 1e-3
    value = args.steps * step_bytes / wall / 1e9
    per_step = len(tensors)
    launches = args.steps * per_step
    # dominant kernel: every launch of the timed region is the Q4_K one-column GEMV
    achieved = (step_alg / per_step) / (span / launches) / 1e9
    del timed, warm
    progress(f"timed steps: {value:.1f} GB/s")

    for t in tensors:
        t["W"] = t["W"][:1]
    torch.cuda.empty_cache()
    ceiling = read_ceiling(torch, [t["bytes"] for t in tensors])
    sustained = sustained_read(torch)
    # plain reads at the two graded tensor sizes (Q4_K 17408 x 5120, Q6_K 5120 x 17408)
    size_reads = {}
    for e in (entries[2], synth.MIXED[0]):
        nb = e["N"] * synth.row_bytes(e["qtype"], e["K"])
        size_reads[e["name"]] = read_ceiling(torch, [nb])
    shapes = per_shape(torch, launcher, tensors)
    del tensors
    torch.cuda.empty_cache()
    # the small Q4_K case (1024 x 5120), and IQ4_XS at the FFN shape, one and eight columns
    small = make_tensors(torch, [dict(synth.SMALL, name="small_q4k_1024x5120")])
    small_out = per_shape(torch, launcher, small)[0]
    del small
    # one GPU's share of an 8-way row split (N / 8 rows, the whole K): the kernel at a shard's real
    # shape (the split itself, x replicated and y gathered, is not part of this single-GPU build)
    shards = make_tensors(torch, [dict(name=f"shard8_{e['name']}", qtype=e["qtype"], N=e["N"] // 8, K=e["K"],
                                       seed=e["seed"] + 100)
                                  for e in list(entries[:1]) + list(entries[2:]) + list(synth.MIXED)])
    shard_out = per_shape(torch, launcher, shards)
    del shards
    iq4_out = []
    for nc in (1, 2, 4, 8, 16, 17):
        t = make_tensors(torch, [dict(name=f"iq4xs_ffn_up_ncols{nc}", qtype=synth.IQ4_XS, N=17408, K=5120, seed=1003,
                                      ncols=nc)])
        r = per_shape(torch, launcher, t)[0]
        r["ncols"] = nc
        iq4_out.append(r)
        del t
    torch.cuda.empty_cache()
    progress("read ceiling and per-shape figures")

    mixed = make_tensors(torch, synth.MIXED)
    mixed_out = per_shape(torch, launcher, mixed)
    del mixed
    torch.cuda.empty_cache()

    # the same shapes on PLANAR rows (qk_repack once, then qk_gemv with the flag)
    planar = make_planar(torch, list(entries) + list(synth.MIXED))
    planar_out = per_shape(torch, launcher, planar)
    for r in planar_out:
        r["layout"] = "PLANAR"
    del planar
    torch.cuda.empty_cache()
    progress("mixed types and PLANAR rows")

    # few-column verify: Q4_K 17408 x 5120, weights read once per call
    v = synth.VERIFY
    verify_out = []
    for nc in v["ncols"]:
        vt = make_tensors(torch, [dict(name=f"verify_ncols{nc}", qtype=v["qtype"], N=v["N"], K=v["K"],
                                       seed=v["seed"], ncols=nc)])
        r = per_shape(torch, launcher, vt)[0]
        r["ncols"] = nc
        r["TFLOPs"] = round(2.0 * v["N"] * v["K"] * nc / r["us"] / 1e6, 2)
        verify_out.append(r)
        del vt
        torch.cuda.empty_cache()

    # wider verification (column groups of <= 8, one launch): 16 and 17 columns
    for nc in (16, 17):
        vt = make_tensors(torch, [dict(name=f"verify_ncols{nc}", qtype=v["qtype"], N=v["N"], K=v["K"],
                                       seed=v["seed"], ncols=nc)])
        r = per_shape(torch, launcher, vt)[0]
        r["ncols"] = nc
        r["TFLOPs"] = round(2.0 * v["N"] * v["K"] * nc / r["us"] / 1e6, 2)
        verify_out.append(r)
        del vt
        torch.cuda.empty_cache()

    # the verify form on the mixed-type shapes (Q6_K FFN down, Q5_K output
    # projection) at 2, 4, 8, 16 and 17 columns
    verify_mixed = []
    for e in synth.MIXED:
        for nc in (2, 4, 8, 16, 17):
            vt = make_tensors(torch, [dict(e, name=f"{e['name']}_ncols{nc}", ncols=nc)])
            r = per_shape(torch, launcher, vt)[0]
            r["ncols"] = nc
            verify_mixed.append(r)
            del vt
            torch.cuda.empty_cache()

    progress("verify")
    fused_out = fused_epilogues(torch)
    progress("fused epilogues")

    stream_out = None if args.no_stream else run_stream(torch, launcher)
    progress("decode stream")
    cpu = None if args.no_cpu else cpu_baseline(entries)
    progress("cpu baseline")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "k-quant(u8) x f16 -> f32",
        "data": "synthetic (seeded k-quant superblocks, x ~ N(0,1) fp16)",
        "config": {"workload": "Q4_K one-column GEMV x3 per step: N=10240, 12288, 17408 at K=5120 "
                               "(fused DeltaNet QKV, attention Q, FFN gate/up of a 5120-hidden decoder)",
                   "ncols": 1, "weight_bytes_per_step": step_bytes, "rotation_copies": copies,
                   "timing": "the K timed steps replayed from one HIP graph after the W warm-up steps and a "
                             "GPU busy-wait (clocks at steady state); wall clock around the timed steps"},
        "roofline": {"bound": "hbm", "kernel": "gemv1_kernel<Q4_K>", "achieved": round(achieved, 1),
                     "avg_launch_us": round(span / launches * 1e6, 3),
                     "bytes_per_launch": round(step_alg / per_step),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for("gemv1_kernel<Q4_K>", None),
                     "read_ceiling_GBs": ceiling["GBs"],
                     "frac_of_read_ceiling": round(achieved / ceiling["GBs"], 4)},
        "read_ceiling": ceiling,
        "sustained_read": sustained,
        "read_at_size": size_reads,
        "cpu_baseline": cpu,
        "per_gemv": shapes,
        "small_gemv": small_out,
        "shard8": shard_out,
        "iq4_xs": iq4_out,
        "mixed_types": mixed_out,
        "planar_rows": planar_out,
        "verify": verify_out,
        "verify_mixed": verify_mixed,
        "fused_epilogues": fused_out,
        "decode_stream": stream_out,
        "event_span_ms_per_step": round(span / args.steps * 1e3, 5),
        "kernel_hash": kernel_hash(),
        "device": device_info(torch),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
