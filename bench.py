"""Benchmark of the W12 decode GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-stack]
                    [--no-cpu-baseline] [--workload qkv|gate_up|down] [--m M]

Prints ONE compact JSON line on stdout (the headline, its roofline and the
CPU oracle's rate); the full record -- sweep, shard shapes, W12-b, codec,
exception-list and stack figures -- goes to stderr as one "detail:" line and,
with --detail-out PATH, to a file.

The headline workload is the attention QKV projection of a ~27B dense
decoder at single-request decode: W [7168, 5120] packed to W12 (group 128),
x [1, 5120], y fp32.  One step = one w12_gemm launch over that weight (the
three planes streamed with x, BF16 rebuilt in registers, fp32 dot products,
epilogue).  `value` is the effective weight
stream rate: stored W12 bytes (planes + meta) per launch x launches / time.

Timing protocol (the pages warm up before timing and tune kernels against
the memory-bandwidth limit: HotRepo digest of StargazerX0/SpecPilot, quick
start; AI Radar summary of SpecPilot, English edition, opening paragraph):
  * inputs are resident in HBM before the timed region;
  * R distinct copies of the weight (>= 1 GB in total, above the 256 MB
    last-level cache) are used in rotation, so every launch streams from HBM;
  * the R launches are captured once in a HIP graph; W warm-up launches run,
    the graph is replayed for a short settling time (0.5 s for the headline:
    the clocks ramp up under load), then replayed until K launches are done,
    bracketed by synchronize + HIP events recorded on the launch stream.
The same protocol times the same-tiling BF16 control; `speedup_vs_bf16` is
the ratio of the two.  `cpu_baseline` times the CPU oracle (decode + fp64
GEMM, all host threads) on the same workload.

Beside the headline: the M sweep over the QKV, O, gate+up and down weights;
pack / unpack throughput on the QKV weight; the QKV GEMM on the raw
(unprojected) weight made lossless by its exception list; and one decode
step over the 64-layer linear stack (256 GEMMs, 31.9 GB of W12 weights,
captured as one graph) at M in {1, 4, 8, 16, 32}.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30           # >= 1 GiB of distinct weights per rotation
CALIB_BYTES = 256 << 20          # size of the counter-calibration copy
METRIC = "w12_gemm effective weight GB/s & % HBM peak; speedup vs BF16 GEMM, M=1–32"
WORKLOAD_NAMES = {"qkv": "QKV projection", "o": "attention output projection",
                  "gate_up": "MLP fused gate+up projection", "down": "MLP down projection"}
WORKLOAD_NAMES.update({k + "_tp8": v + ", one GPU's share under 8-way tensor parallelism"
                       for k, v in list(WORKLOAD_NAMES.items())})


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-sweep", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 64-layer linear-stack decode step")
    ap.add_argument("--stack-ms", type=str, default="1,4,8,16,32,64,128")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU-oracle work to time")
    ap.add_argument("--sweep-ms", type=str, default="1,2,4,8,16,32,64,128")
    ap.add_argument("--w12b-ms", type=str, default="1,4,16,32",
                    help="x rows for the W12-b (arbitrary-base) comparison ('' to skip)")
    ap.add_argument("--shard-ms", type=str, default="1,4,16,32",
                    help="x rows for the 8-way tensor-parallel shard shapes ('' to skip)")
    ap.add_argument("--workload", default="qkv",
                    choices=["qkv", "o", "gate_up", "down",
                             "qkv_tp8", "o_tp8", "gate_up_tp8", "down_tp8"],
                    help="headline weight (default: the QKV projection; *_tp8: one GPU's "
                         "share under 8-way tensor parallelism)")
    ap.add_argument("--exceptions-ms", type=str, default=None,
                    help="x rows for the raw (unprojected) weight with its exception list "
                         "(default: 1,4,8,16,32 with the sweep, none with --no-sweep)")
    ap.add_argument("--m", type=int, default=1, help="headline x rows (default 1)")
    ap.add_argument("--tiling", type=str, default="",
                    help="headline tiling instead of the default: kind,r,kw,depth,x_direct"
                         "[,splitk[,waves]] (kind 0 = GEMV, 1 = MFMA), for profiles of one variant")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "VARIANT"),
                    help="print a markdown summary of a rocprofv3 --stats kernel table")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "VARIANT"),
                    help="print a markdown summary of FETCH_SIZE / WRITE_SIZE counter runs")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("COUNTER_CSV", "VARIANT"),
                    help="print a markdown summary of any rocprofv3 --pmc run")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--read-sizes", type=str, default="",
                    help="only time the plain streaming-read kernel at these sizes (MB, "
                         "comma-separated) and print a markdown table: the launch floor and "
                         "the read rate a kernel reaching each byte once can reach")
    ap.add_argument("--detail-out", default="",
                    help="also write the full record (sweep, shards, codec, stack...) to this file")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="also run a plain elementwise kernel over 256 MiB (bitwise not: "
                         "reads and writes 256 MiB) 4 times, the known-size reference for "
                         "HBM byte counters")
    return ap.parse_args()


def source_sha() -> str:
    """Hash of the kernel sources, to tie stored counter readings to code."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "lossless_bit_weight_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class Workload:
    """One weight on the GPU in R rotated copies, W12 (allocation `fmt`) and
    BF16."""

    def __init__(self, case, torch, w12, fmt="v1"):
        from lossless_bit_weight_amd.inputs import GemmCase  # noqa: F401
        self.case = case
        self.fmt = fmt
        self.N, self.K = case.N, case.K
        raw = case.weights_raw()
        wd = torch.from_numpy(raw.view(np.int16)).cuda()
        # project onto the encodable set with the library itself, then repack
        first, self.raw_bad = w12.pack(wd, fmt=fmt)
        w_bf16 = w12.w12_unpack(first)
        wt, bad = w12.pack(w_bf16, fmt=fmt)
        if bad:
            raise RuntimeError("projected weights still have unencodable groups")
        self.w_tiled = w12.w12_bf16_tile(w_bf16)
        del wd, first, w_bf16
        self.w12_bytes = wt.nbytes
        self.bf16_bytes = self.w_tiled.nbytes
        r12 = max(2, math.ceil(ROTATE_BYTES / self.w12_bytes))
        r16 = max(2, math.ceil(ROTATE_BYTES / self.bf16_bytes))
        self.w12_copies = [wt] + [w12.W12Weight(wt.p0.clone(), wt.p1.clone(), wt.p2.clone(),
                                                wt.meta.clone(), self.N, self.K, fmt=fmt)
                                  for _ in range(r12 - 1)]
        self.bf16_copies = [self.w_tiled] + [w12.BF16Tiled(self.w_tiled.w.clone(), self.N, self.K)
                                             for _ in range(r16 - 1)]
        torch.cuda.synchronize()


def time_graph(torch, launches, steps, warmup, settle_s=0.05):
    """Capture `launches` (callables, in rotation) into one graph, replay it
    for at least `settle_s` seconds (the GPU's clocks ramp up under load:
    the first launches of a process ran a few percent slower), then replay
    it until `steps` launches ran; return average ms per launch measured
    with events on the launch stream."""
    R = len(launches)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(warmup, R)):
            launches[i % R]()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    reps = max(1, math.ceil(steps / R))
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * R), reps * R


def gemm_bytes(N, K, M, out_bytes, w_bytes):
    return w_bytes + 2 * M * K + out_bytes * M * N


def measure(torch, w12, wl: Workload, M, steps, warmup, out_dtype, settle_s=0.05, tiling=None):
    """W12 and the BF16 control on the same tiling (the default, or `tiling`)."""
    x = torch.from_numpy(wl.case.activations(M).view(np.int16)).cuda()
    y = torch.empty((M, wl.N), dtype=out_dtype, device="cuda")
    out_b = 4 if out_dtype == torch.float32 else 2
    # one zero-filled split-K workspace for every launch (allocated outside
    # the graph; each launch leaves its counters at zero)
    ws = torch.zeros(max(256, w12.w12_gemm_workspace_bytes(M, wl.N, wl.K, tiling)), dtype=torch.uint8,
                     device="cuda")
    l12 = [(lambda c=c: w12.w12_gemm(x, c, y=y, tiling=tiling, workspace=ws)) for c in wl.w12_copies]
    l16 = [(lambda c=c: w12.bf16_gemm(x, c, y=y, tiling=tiling, workspace=ws)) for c in wl.bf16_copies]
    ms12, n12 = time_graph(torch, l12, steps, warmup, settle_s)
    ms16, n16 = time_graph(torch, l16, steps, warmup, settle_s)
    b12 = gemm_bytes(wl.N, wl.K, M, out_b, wl.w12_bytes)
    b16 = gemm_bytes(wl.N, wl.K, M, out_b, wl.bf16_bytes)
    return {
        "workload": wl.case.name, "M": M,
        "w12_kernel": (w12.w12_gemm_variant(M, wl.N, wl.K, 2 if wl.fmt == "b" else 1) if tiling is None
                       else w12.w12_tiling_variant(M, wl.N, wl.K, tiling, 2 if wl.fmt == "b" else 1)),
        "bf16_kernel": (w12.w12_gemm_variant(M, wl.N, wl.K, False) if tiling is None
                        else w12.w12_tiling_variant(M, wl.N, wl.K, tiling, False)),
        "w12_us": ms12 * 1e3, "bf16_us": ms16 * 1e3,
        "w12_weight_gbps": wl.w12_bytes / (ms12 * 1e-3) / 1e9,
        "w12_bf16_equiv_gbps": wl.bf16_bytes / (ms12 * 1e-3) / 1e9,
        "bf16_weight_gbps": wl.bf16_bytes / (ms16 * 1e-3) / 1e9,
        "w12_alg_gbps": b12 / (ms12 * 1e-3) / 1e9,
        "bf16_alg_gbps": b16 / (ms16 * 1e-3) / 1e9,
        "w12_alg_bytes": b12, "bf16_alg_bytes": b16,
        "speedup_vs_bf16": ms16 / ms12,
        "launches": n12,
    }


def read_ceiling(torch, w12, nbytes, steps, warmup):
    """The library's plain streaming-read kernel (w12_read_probe) over
    buffers of `nbytes`, rotated like the weights (>= 1 GiB in total), timed
    with the same graph protocol: the rate a kernel that reads each byte
    once can reach at this size on this device."""
    nbytes = (nbytes + 15) // 16 * 16
    R = max(2, math.ceil(ROTATE_BYTES / nbytes))
    bufs = [torch.full((nbytes,), i & 255, dtype=torch.uint8, device="cuda") for i in range(R)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms, n = time_graph(torch, [(lambda b=b: w12.w12_read_probe(b, sink)) for b in bufs], steps, warmup)
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "us": ms * 1e3, "gbps": nbytes / (ms * 1e-3) / 1e9, "launches": n}


def read_sizes_table(torch, w12, sizes_mb, steps, warmup):
    """The read ceiling at each size, as a markdown table: time per launch
    (graph-replayed, buffers rotated over >= 1 GiB), the rate, and a
    least-squares line t = t0 + bytes / rate over the sizes >= 50 MB."""
    rows = []
    for mb in sizes_mb:
        nbytes = max(4096, int(mb * 1e6) // 4096 * 4096)
        r = read_ceiling(torch, w12, nbytes, steps, warmup)
        rows.append(r)
        print("read %.3f MB: %.3f us" % (nbytes / 1e6, r["us"]), file=sys.stderr, flush=True)
    lines = ["| bytes | us per launch | GB/s | launches timed |", "|---|---|---|---|"]
    for r in rows:
        lines.append("| %d | %.3f | %.0f | %d |" % (r["bytes"], r["us"], r["gbps"], r["launches"]))
    big = [r for r in rows if r["bytes"] >= 50e6]
    if len(big) >= 2:
        xs = [r["bytes"] for r in big]
        ys = [r["us"] for r in big]
        n = len(xs)
        mx, my = sum(xs) / n, sum(ys) / n
        slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sum((a - mx) ** 2 for a in xs)
        t0 = my - slope * mx
        lines += ["", "Least-squares line over the sizes >= 50 MB: t = %.2f us + bytes / %.0f GB/s."
                  % (t0, 1e-3 / slope)]
    print("\n".join(lines))


def attach_ceiling(r, c12, c16):
    """Fractions of the measured read ceiling (same bytes, same protocol)."""
    r["w12_frac_of_read_ceiling"] = r["w12_weight_gbps"] / c12["gbps"]
    r["bf16_frac_of_read_ceiling"] = r["bf16_weight_gbps"] / c16["gbps"]
    return r


def template_of(variant: str) -> str:
    """rocprofv3's demangled name of the kernel a variant name refers to, e.g.
    w12_gemv_m1_r1_kw4_d2_single ->
    gemm_kernel<w12::kern::FetchW12, false, 1, 1, 4, 2, false, false, 4>
    (the last argument is the wave count, 8 or 16 for a _w8 or _w16 suffix; a split-K
    suffix _sN does not change the kernel)."""
    parts = variant.split("_")
    f, kind, mr, r, kw, d, mode = parts[:7]
    nw = 16 if "w16" in parts[7:] else 8 if "w8" in parts[7:] else 4
    mr = mr.replace("mt", "").replace("m", "")
    tf = lambda b: "true" if b else "false"
    # w12x_: W12-v1 with an exception list (the kernel of a container that
    # carries one); w12b_: the arbitrary-base allocation
    fetch = {"w12": "FetchW12", "w12x": "FetchW12X", "w12b": "FetchW12B"}.get(f, "FetchBF16")
    return "gemm_kernel<w12::kern::%s, %s, %s, %s, %s, %s, %s, %s, %d>" % (
        fetch, tf(kind == "mfma"),
        mr, r[1:], kw[2:], d[1:], tf(mode == "chunked"), tf(mode == "xdirect"), nw)


TRAFFIC_TAG = "traffic_record: "


def stored_traffic(kernel: str, workload: str, M: int):
    """HBM bytes per launch of `kernel` on `workload` at M x rows from a
    committed counter summary under profiles/, if it was taken on the
    current kernel sources; else None."""
    pdir = os.path.join(HERE, "profiles")
    if not os.path.isdir(pdir):
        return None
    for fn in sorted(os.listdir(pdir)):
        if not fn.endswith(".md"):
            continue
        with open(os.path.join(pdir, fn)) as f:
            for line in f:
                if line.startswith(TRAFFIC_TAG):
                    rec = json.loads(line[len(TRAFFIC_TAG):])
                    if (rec.get("kernel") == kernel and rec.get("workload") == workload
                            and rec.get("M") == M and rec.get("source_sha") == source_sha()):
                        return rec.get("hbm_bytes_per_launch")
    return None


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(path, variant, command):
    rows = _read_csv(path)
    lines = ["# rocprofv3 kernel trace: %s" % variant, "",
             "Command (run from the repository root on the GPU box):", "",
             "    " + command, "",
             "Kernel-source hash: `%s`" % source_sha(), "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %s | %.0f | %s | %s |" % (r["Name"][:110], r["Calls"],
                                                        float(r["AverageNs"]), r["MinNs"], r["MaxNs"]))
    want = template_of(variant)
    hit = [r for r in rows if want in r["Name"]]
    if hit:
        lines += ["", "Average duration of `%s` (%s): %.3f us over %s calls (graph-replayed "
                  "launches plus warm-up launches)." % (variant, want, float(hit[0]["AverageNs"]) / 1e3,
                                                        hit[0]["Calls"])]
    st = dispatch_stats(path, want)
    if st:
        lines += ["", "Per-dispatch durations of that kernel (the kernel-trace file beside the "
                  "stats, first %d dispatches dropped as warm-up): n = %d, mean %.3f us (95%% "
                  "bootstrap CI %.3f-%.3f us, %d resamples), median %.3f us (CI %.3f-%.3f us), "
                  "p10 %.3f us, p90 %.3f us."
                  % (st["skipped"], st["n"], st["mean"] / 1e3,
                     st["mean_ci"][0] / 1e3, st["mean_ci"][1] / 1e3, st["resamples"],
                     st["median"] / 1e3, st["median_ci"][0] / 1e3, st["median_ci"][1] / 1e3,
                     st["p10"] / 1e3, st["p90"] / 1e3)]
    print("\n".join(lines))


def dispatch_stats(stats_path, want, skip=20, resamples=2000):
    """Mean, median, p10/p90 and 95% bootstrap confidence intervals of the
    mean and the median of one kernel's per-dispatch durations, from the
    rocprofv3 kernel-trace CSV written beside the --stats table (None if
    there is none)."""
    import numpy as np
    d = os.path.dirname(os.path.abspath(stats_path))
    names = sorted(f for f in os.listdir(d) if f.endswith("kernel_trace.csv"))
    if not names:
        return None
    rows = _read_csv(os.path.join(d, names[0]))
    if not rows or "Start_Timestamp" not in rows[0] or "Kernel_Name" not in rows[0]:
        return None
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in rows if want in r["Kernel_Name"]][skip:]
    if len(durs) < 50:
        return None
    a = np.asarray(durs, dtype=np.float64)
    rng = np.random.default_rng(0)
    means, meds = [], []
    for _ in range(resamples // 200):
        r = rng.choice(a, size=(200, a.size))
        means.append(r.mean(axis=1))
        meds.append(np.median(r, axis=1))
    ci = lambda v: tuple(float(c) for c in np.percentile(np.concatenate(v), [2.5, 97.5]))
    return {"n": int(a.size), "skipped": skip, "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(a.mean()), "mean_ci": ci(means), "median_ci": ci(meds),
            "resamples": resamples}


def summarize_pmc(fetch_path, write_path, variant, command):
    import statistics
    want = template_of(variant)
    def per_kernel(path):
        out = {}
        for r in _read_csv(path):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out
    fetch, write = per_kernel(fetch_path), per_kernel(write_path)
    calib_kib = CALIB_BYTES / 1024
    # The calibration kernel (bench.py --pmc-calibration) is the only bitwise
    # not; it reads and writes CALIB_BYTES.
    f_cal = statistics.median(v for k, vs in fetch.items() if "bitwise_not" in k for v in vs)
    w_cal = statistics.median(v for k, vs in write.items() if "bitwise_not" in k for v in vs)
    f_scale, w_scale = calib_kib / f_cal, calib_kib / w_cal
    fk = [k for k in fetch if want in k]
    wk = [k for k in write if want in k]
    f_med = statistics.median(fetch[fk[0]])
    w_med = statistics.median(write[wk[0]])
    hbm = f_med * 1024 * f_scale + w_med * 1024 * w_scale
    # the workload and x rows of the profiled run, from its command line
    wm = re.search(r"--workload (\S+)", command)
    mm = re.search(r"--m (\d+)", command)
    workload = wm.group(1) if wm else "qkv"
    m_rows = int(mm.group(1)) if mm else 1
    lines = ["# HBM bytes of %s (rocprofv3 FETCH_SIZE / WRITE_SIZE)" % variant, "",
             "Commands (run from the repository root on the GPU box, one counter per run):", "",
             "    " + command.replace("{CTR}", "FETCH_SIZE"),
             "    " + command.replace("{CTR}", "WRITE_SIZE"), "",
             "Kernel-source hash: `%s`" % source_sha(), "",
             "Calibration: a plain elementwise kernel over %d MiB (bitwise not, bench.py "
             "--pmc-calibration) reads FETCH_SIZE = %.1f KiB and writes WRITE_SIZE = %.1f KiB, "
             "so the counters are scaled by %.4f (fetch) and %.4f (write)."
             % (CALIB_BYTES >> 20, f_cal, w_cal, f_scale, w_scale), "",
             "| kernel | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) |",
             "|---|---|---|---|"]
    for k in sorted(fetch):
        if k in write:
            lines.append("| `%s` | %d | %.1f | %.1f |" % (k[:110], len(fetch[k]), statistics.median(fetch[k]),
                                                          statistics.median(write[k])))
    lines += ["", "HBM bytes per launch of `%s`: %.0f (fetch %.0f + write %.0f)."
              % (variant, hbm, f_med * 1024 * f_scale, w_med * 1024 * w_scale), "",
              TRAFFIC_TAG + json.dumps({"kernel": variant, "workload": workload, "M": m_rows,
                                        "source_sha": source_sha(),
                                        "hbm_bytes_per_launch": round(hbm),
                                        "fetch_kib": f_med, "write_kib": w_med,
                                        "fetch_scale": f_scale, "write_scale": w_scale})]
    print("\n".join(lines))


def summarize_counters(path, variant, command):
    """Per-kernel medians of the counters of one `rocprofv3 --pmc` run; with
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE, also the MFMA busy share
    (busy cycles summed over the SIMDs / (active cycles x SIMDs))."""
    import statistics
    rows = _read_csv(path)
    want = template_of(variant)
    vals = {}
    for r in rows:
        vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    kernels = sorted({k for k, _ in vals})
    ctrs = sorted({c for _, c in vals})
    lines = ["# rocprofv3 counters of %s" % variant, "",
             "Command (run from the repository root on the GPU box):", "",
             "    " + command, "",
             "Kernel-source hash: `%s`" % source_sha(), "",
             "| kernel | dispatches | " + " | ".join("%s (median)" % c for c in ctrs) + " |",
             "|---|---|" + "---|" * len(ctrs)]
    for k in kernels:
        n = max(len(vals.get((k, c), [])) for c in ctrs)
        cells = ["%.4g" % statistics.median(vals[(k, c)]) if (k, c) in vals else "" for c in ctrs]
        lines.append("| `%s` | %d | %s |" % (k[:110], n, " | ".join(cells)))
    hit = [k for k in kernels if want in k]
    if hit and (hit[0], "SQ_VALU_MFMA_BUSY_CYCLES") in vals and (hit[0], "GRBM_GUI_ACTIVE") in vals:
        busy = statistics.median(vals[(hit[0], "SQ_VALU_MFMA_BUSY_CYCLES")])
        active = statistics.median(vals[(hit[0], "GRBM_GUI_ACTIVE")])
        simds = 4 * 256
        lines += ["", "MFMA busy share of `%s`: %.2f%% (SQ_VALU_MFMA_BUSY_CYCLES / "
                  "(GRBM_GUI_ACTIVE x %d SIMDs))." % (variant, 100.0 * busy / (active * simds), simds)]
    print("\n".join(lines))


def time_codec(torch, w12, wl: Workload, steps):
    """Pack, unpack and control-layout throughput on the workload's weight
    (events around back-to-back launches; inputs resident in HBM)."""
    w = w12.w12_unpack(wl.w12_copies[0])
    out = w12.empty_weight(wl.N, wl.K)
    wb = torch.empty_like(w)
    res = {}
    for name, fn, nbytes in (
            ("pack", lambda: w12.w12_pack(w, out=out), 2 * wl.N * wl.K + wl.w12_bytes),
            ("unpack", lambda: w12.w12_unpack(wl.w12_copies[0], out=wb), 2 * wl.N * wl.K + wl.w12_bytes)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        n = max(10, steps // 10)
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        res[name] = {"us": round(ms * 1e3, 2), "gbps": round(nbytes / ms / 1e6, 1), "bytes": nbytes}
    return res


def stack_step(torch, w12, inputs, ms, steps, warmup):
    """One decode step over the 64-layer linear stack (QKV, O, gate+up, down
    per layer): 256 GEMMs back to back, W12 and the BF16 control."""
    layers = []
    raw_bad = 0
    w12_bytes = bf16_bytes = 0
    for layer in range(inputs.STACK_LAYERS):
        row = []
        for j, (N, K) in enumerate(inputs.STACK_SHAPES):
            w = inputs.device_weights(torch, N, K, 10000 + 10 * layer + j)
            first, bad = w12.pack(w)
            raw_bad += bad
            wc = w12.w12_unpack(first)
            del first
            wt, bad = w12.pack(wc)
            if bad:
                raise RuntimeError("projected stack weight still has unencodable groups")
            bt = w12.w12_bf16_tile(wc)
            del w, wc
            row.append((wt, bt))
            w12_bytes += wt.nbytes
            bf16_bytes += bt.nbytes
        layers.append(row)
    torch.cuda.synchronize()
    print("stack ready: %.2f GB W12, %.2f GB BF16 (raw unencodable groups %d)"
          % (w12_bytes / 1e9, bf16_bytes / 1e9, raw_bad), file=sys.stderr, flush=True)
    out = {"layers": inputs.STACK_LAYERS, "w12_gb": round(w12_bytes / 1e9, 3),
           "bf16_gb": round(bf16_bytes / 1e9, 3), "raw_unencodable_groups": raw_bad, "by_m": []}
    for M in ms:
        xs = {K: torch.from_numpy(inputs.gaussian_bf16((M, K), 1.0, 20000 + M).view(np.int16)).cuda()
              for K in {k for _, k in inputs.STACK_SHAPES}}
        ys = {N: torch.empty((M, N), dtype=torch.float32, device="cuda")
              for N in {n for n, _ in inputs.STACK_SHAPES}}
        ws = torch.zeros(max([256] + [w12.w12_gemm_workspace_bytes(M, N, K)
                                      for N, K in inputs.STACK_SHAPES]),
                         dtype=torch.uint8, device="cuda")
        def step(fn, idx):
            def run():
                for row in layers:
                    for (wt, bt), (N, K) in zip(row, inputs.STACK_SHAPES):
                        fn(xs[K], (wt, bt)[idx], y=ys[N], workspace=ws)
            return run
        ms12, _ = time_graph(torch, [step(w12.w12_gemm, 0)], max(3, steps // 100), max(1, warmup // 20))
        ms16, _ = time_graph(torch, [step(w12.bf16_gemm, 1)], max(3, steps // 100), max(1, warmup // 20))
        r = {"M": M, "w12_ms": round(ms12, 4), "bf16_ms": round(ms16, 4),
             "w12_weight_gbps": round(w12_bytes / ms12 / 1e6, 1),
             "bf16_weight_gbps": round(bf16_bytes / ms16 / 1e6, 1),
             "speedup_vs_bf16": round(ms16 / ms12, 4)}
        out["by_m"].append(r)
        print("stack M=%d: w12 %.3f ms (%.0f GB/s) bf16 %.3f ms speedup %.3f"
              % (M, ms12, r["w12_weight_gbps"], ms16, r["speedup_vs_bf16"]), file=sys.stderr, flush=True)
    del layers
    torch.cuda.empty_cache()
    return out


def measure_exceptions(torch, w12, case, ms, steps, warmup, fmt="v1"):
    """The raw (unprojected) weight packed with its exception list, so the
    container is lossless: list size, and the W12 GEMM against the BF16
    control on the same raw weight (same protocol as the headline)."""
    raw = torch.from_numpy(case.weights_raw().view(np.int16)).cuda()
    wt, bad = w12.pack(raw, exceptions=True, fmt=fmt)
    w_tiled = w12.w12_bf16_tile(raw)
    count = int(wt.exc_offsets[-1].item()) if wt.exc_offsets is not None else 0
    r = max(2, math.ceil(ROTATE_BYTES / wt.nbytes))
    clone = lambda t: None if t is None else t.clone()
    copies = [wt] + [w12.W12Weight(wt.p0.clone(), wt.p1.clone(), wt.p2.clone(), wt.meta.clone(),
                                   wt.N, wt.K, clone(wt.exc_offsets), clone(wt.exc_entries), fmt=fmt)
                     for _ in range(r - 1)]
    b16 = [w_tiled] + [w12.BF16Tiled(w_tiled.w.clone(), wt.N, wt.K)
                       for _ in range(max(2, math.ceil(ROTATE_BYTES / w_tiled.nbytes)) - 1)]
    out = {"workload": case.name + " raw (unprojected)", "format": fmt, "flagged_groups": bad,
           "exceptions": count, "list_bytes": wt.nbytes - 3 * wt.p0.numel() - wt.meta.numel(),
           "by_m": []}
    for M in ms:
        x = torch.from_numpy(case.activations(M).view(np.int16)).cuda()
        y = torch.empty((M, wt.N), dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(256, w12.w12_gemm_workspace_bytes(M, wt.N, wt.K)), dtype=torch.uint8,
                         device="cuda")
        ms12, _ = time_graph(torch, [(lambda c=c: w12.w12_gemm(x, c, y=y, workspace=ws)) for c in copies],
                             steps, warmup)
        ms16, _ = time_graph(torch, [(lambda c=c: w12.bf16_gemm(x, c, y=y, workspace=ws)) for c in b16],
                             steps, warmup)
        out["by_m"].append({"M": M, "w12_us": round(ms12 * 1e3, 3), "bf16_us": round(ms16 * 1e3, 3),
                            "w12_weight_gbps": round(wt.nbytes / ms12 / 1e6, 1),
                            "speedup_vs_bf16": round(ms16 / ms12, 4)})
    del copies, b16
    torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, M, seconds):
    """The CPU oracle as it stands: container decode + fp64 GEMM over the whole
    headline weight on all host threads, repeated until ~`seconds` passed;
    beside it the same on one thread (~seconds / 4) and one oracle pack of
    the weight."""
    import oracle
    nthreads = len(os.sched_getaffinity(0))
    raw = case.weights_raw()
    x = case.activations(M)
    # Oracle-side projection and container (no input from the HIP path).
    p0, p1, p2, meta, _ = oracle.pack(raw)
    w = oracle.unpack(p0, p1, p2, meta, case.N, case.K)
    t0 = time.perf_counter()
    q = oracle.pack(w)
    pack_s = time.perf_counter() - t0
    del raw, w
    wb = 3 * oracle.plane_bytes(case.N, case.K) + oracle.meta_bytes(case.N, case.K)

    def run(threads, budget):
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.gemm_w12_f64(x, *q[:4], case.N, nthreads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget or reps >= 10000:
                return reps, dt

    reps, dt = run(nthreads, seconds)
    reps1, dt1 = run(1, seconds / 4)
    del q
    # One layer of the 64-layer stack at M = 1 on host-generated weights of
    # the stack's shapes, one decode + fp64 GEMM pass each, times 64.
    from lossless_bit_weight_amd import inputs
    layer_s = 0.0
    layer_bytes = 0
    for j, (N, K) in enumerate(inputs.STACK_SHAPES):
        ql = oracle.pack(inputs.gaussian_bf16((N, K), 0.02, 30000 + j))
        xl = inputs.gaussian_bf16((1, K), 1.0, 30100 + j)
        t0 = time.perf_counter()
        oracle.gemm_w12_f64(xl, *ql[:4], N, nthreads=nthreads)
        layer_s += time.perf_counter() - t0
        layer_bytes += 3 * oracle.plane_bytes(N, K) + oracle.meta_bytes(N, K)
        del ql
    stack = {"layer_s": layer_s, "step_s_extrapolated": 64 * layer_s,
             "gbps": layer_bytes / layer_s / 1e9,
             "sample": "one pass over each of the 4 weights of one stack layer at M=1, "
                       "x64 (an extrapolation, not a measured 64-layer step)"}
    return {
        "value": reps * wb / dt / 1e9, "unit": "GB/s", "cores": nthreads, "kind": "oracle",
        "sample": "%d full passes over %s, M=%d (decode + fp64 GEMM), %.1f s"
                  % (reps, case.name, M, dt),
        "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
        "single_thread": {"value": reps1 * wb / dt1 / 1e9, "unit": "GB/s",
                          "sample": "%d passes, %.1f s" % (reps1, dt1)},
        "pack": {"seconds": pack_s, "bf16_gbps": 2 * case.N * case.K / pack_s / 1e9,
                 "sample": "one oracle pack of %s" % case.name},
        "stack_m1": stack,
    }


# hipDeviceAttribute_t values (ROCm 7 headers) of the memory clock (kHz) and
# the memory bus width (bits).
_HIP_ATTR_MEM_CLOCK_KHZ = 60
_HIP_ATTR_MEM_BUS_BITS = 59


def device_memory_peak():
    """Peak HBM bandwidth recomputed from the device's reported memory clock
    and bus width, beside the published 8 TB/s.  MI355X reports a 2 GHz
    clock on 8192 bits; its HBM3E moves 8 Gb/s per pin, four transfers per
    reported clock."""
    import ctypes
    # The HIP runtime torch has loaded (opening it by path again returns the
    # same handle; a second runtime in the process is never loaded).
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    if path is None:
        return None
    hip = ctypes.CDLL(path)
    clk, bus = ctypes.c_int(0), ctypes.c_int(0)
    if (hip.hipDeviceGetAttribute(ctypes.byref(clk), _HIP_ATTR_MEM_CLOCK_KHZ, 0) != 0
            or hip.hipDeviceGetAttribute(ctypes.byref(bus), _HIP_ATTR_MEM_BUS_BITS, 0) != 0):
        return None
    per_clock = clk.value * 1e3 * bus.value / 8 / 1e9
    return {"memory_clock_khz": clk.value, "bus_width_bits": bus.value,
            "gbps_one_transfer_per_clock": per_clock,
            "gbps_four_transfers_per_clock": 4 * per_clock,
            "published_gbps": HBM_PEAK_GBPS}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.command)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.command)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the W12 decode GEMM of one weight on "
              "one MI355X; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from lossless_bit_weight_amd import inputs, w12
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w12.lib()
    if args.read_sizes:
        read_sizes_table(torch, w12, [float(v) for v in args.read_sizes.split(",") if v],
                         args.steps, args.warmup)
        return
    props = torch.cuda.get_device_properties(0)
    print("device: %s, %d CUs" % (props.name, props.multi_processor_count), file=sys.stderr,
          flush=True)

    head_case = inputs.CASES.get(args.workload) or inputs.SHARD_CASES[args.workload]
    head_m = args.m
    wl = Workload(head_case, torch, w12)
    print("headline workload ready (%s, raw unencodable groups %d)" % (head_case.name, wl.raw_bad),
          file=sys.stderr, flush=True)
    head_tiling = tuple(int(v) for v in args.tiling.split(",")) if args.tiling else None
    head = measure(torch, w12, wl, head_m, args.steps, args.warmup, torch.float32, settle_s=0.5,
                   tiling=head_tiling)
    rotation = len(wl.w12_copies)
    ceilings = {}
    ceilings[args.workload] = (read_ceiling(torch, w12, wl.w12_bytes, args.steps, args.warmup),
                               read_ceiling(torch, w12, wl.bf16_bytes, args.steps, args.warmup))
    attach_ceiling(head, *ceilings[args.workload])
    print("headline: %s" % json.dumps(head), file=sys.stderr, flush=True)

    if args.pmc_calibration:
        # a kernel of its own (bitwise not) that reads and writes exactly
        # CALIB_BYTES, so the summary finds it among the other launches
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.int32, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(4):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    sweep = []
    if not args.no_sweep:
        ms = [int(m) for m in args.sweep_ms.split(",") if m]
        for name in ("qkv", "o", "gate_up", "down"):
            case = inputs.CASES[name]
            wlc = wl if name == args.workload else Workload(case, torch, w12)
            if name not in ceilings:
                ceilings[name] = (read_ceiling(torch, w12, wlc.w12_bytes, args.steps, args.warmup),
                                  read_ceiling(torch, w12, wlc.bf16_bytes, args.steps, args.warmup))
            for M in ms:
                r = attach_ceiling(measure(torch, w12, wlc, M, args.steps, args.warmup, torch.float32),
                                   *ceilings[name])
                sweep.append(r)
                print("sweep: %s M=%d w12 %.2f us (%.0f GB/s) bf16 %.2f us speedup %.3f"
                      % (name, M, r["w12_us"], r["w12_weight_gbps"], r["bf16_us"],
                         r["speedup_vs_bf16"]), file=sys.stderr, flush=True)
            if wlc is not wl:
                del wlc
                torch.cuda.empty_cache()

    shards = []
    if not args.no_sweep:
        for name, case in inputs.SHARD_CASES.items():
            ms = [int(m) for m in args.shard_ms.split(",") if m]
            if not ms:
                break
            wlc = Workload(case, torch, w12)
            for M in ms:
                r = measure(torch, w12, wlc, M, args.steps, args.warmup, torch.float32)
                shards.append(r)
                print("shard: %s M=%d w12 %.2f us (%.0f GB/s) bf16 %.2f us speedup %.3f"
                      % (name, M, r["w12_us"], r["w12_weight_gbps"], r["bf16_us"],
                         r["speedup_vs_bf16"]), file=sys.stderr, flush=True)
            del wlc
            torch.cuda.empty_cache()

    # W12-b, the arbitrary-base allocation: unencodable groups and exception
    # counts of the raw weights beside W12-v1's, and its GEMMs on its own
    # projection of the same weights.
    w12b = None
    bms = [int(m) for m in args.w12b_ms.split(",") if m]
    if not args.no_sweep and bms:
        w12b = {"by_workload": [], "gemm": []}
        v1_rows = {(r["workload"], r["M"]): r for r in sweep}
        for name in ("qkv", "o", "gate_up", "down"):
            case = inputs.CASES[name]
            raw = torch.from_numpy(case.weights_raw().view(np.int16)).cuda()
            groups = case.N * case.K // 128
            enc = {"workload": case.name, "groups": groups}
            for fmt in ("v1", "b"):
                wt, bad = w12.pack(raw, exceptions=True, fmt=fmt)
                count = int(wt.exc_offsets[-1].item()) if wt.exc_offsets is not None else 0
                enc[fmt] = {"flagged_groups": bad, "flagged_frac": round(bad / groups, 5),
                            "exceptions": count}
                del wt
            del raw
            w12b["by_workload"].append(enc)
            wlb = Workload(case, torch, w12, fmt="b")
            for M in bms:
                r = measure(torch, w12, wlb, M, args.steps, args.warmup, torch.float32)
                v1 = v1_rows.get((case.name, M))
                row = {"workload": case.name, "M": M, "w12b_kernel": r["w12_kernel"],
                       "w12b_us": round(r["w12_us"], 3), "bf16_us": round(r["bf16_us"], 3),
                       "w12b_weight_gbps": round(r["w12_weight_gbps"], 1),
                       "speedup_vs_bf16": round(r["speedup_vs_bf16"], 4),
                       "w12_v1_us": round(v1["w12_us"], 3) if v1 else None}
                w12b["gemm"].append(row)
                print("w12b: %s M=%d w12b %.2f us (v1 %s) bf16 %.2f us"
                      % (name, M, r["w12_us"], row["w12_v1_us"], r["bf16_us"]),
                      file=sys.stderr, flush=True)
            del wlb
            torch.cuda.empty_cache()
        w12b["exceptions"] = measure_exceptions(torch, w12, head_case, [1, 16], args.steps,
                                                args.warmup, fmt="b")
        print("w12b: %s" % json.dumps(w12b["by_workload"]), file=sys.stderr, flush=True)

    codec = time_codec(torch, w12, wl, args.steps)
    print("codec: %s" % json.dumps(codec), file=sys.stderr, flush=True)

    exc = None
    exc_ms = args.exceptions_ms if args.exceptions_ms is not None else (
        "" if args.no_sweep else "1,4,8,16,32")
    exc_ms = [int(m) for m in exc_ms.split(",") if m]
    if exc_ms:
        exc = measure_exceptions(torch, w12, head_case, exc_ms, args.steps, args.warmup)
        print("exceptions: %s" % json.dumps(exc), file=sys.stderr, flush=True)

    stack = None
    if not args.no_stack:
        del wl
        torch.cuda.empty_cache()
        stack = stack_step(torch, w12, inputs, [int(m) for m in args.stack_ms.split(",") if m],
                           args.steps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head_case, head_m, args.cpu_seconds)
        print("cpu baseline: %s" % json.dumps(cpu), file=sys.stderr, flush=True)

    kernel = head["w12_kernel"]
    traffic = stored_traffic(kernel, args.workload, head_m)
    detail = {
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "memory": device_memory_peak()},
        "headline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in head.items()},
        "read_ceiling": {k: {"w12_bytes_gbps": round(v[0]["gbps"], 1),
                             "bf16_bytes_gbps": round(v[1]["gbps"], 1)}
                         for k, v in ceilings.items()},
        "cpu_baseline": cpu,
        "sweep": [{k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
                  for r in sweep],
        "w12b": w12b,
        "tp8_shards": [{k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
                       for r in shards],
        "codec": codec,
        "exceptions": exc,
        "stack": stack,
        "source_sha": source_sha(),
    }
    # The full record goes to stderr (one line) and, if asked, to a file; the
    # one stdout line is the compact headline.
    print("detail: %s" % json.dumps(detail), file=sys.stderr, flush=True)
    if args.detail_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.detail_out)), exist_ok=True)
        with open(args.detail_out, "w") as f:
            json.dump(detail, f, indent=1)
    out = headline_record(head, args.workload, head_case, head_m, args.warmup, rotation,
                          ceilings[args.workload], traffic, cpu, sweep, stack)
    print(json.dumps(out, separators=(",", ":")), flush=True)


def headline_record(head, workload, case, M, warmup, rotation, ceiling, traffic, cpu, sweep,
                    stack):
    """The one JSON line bench.py prints on stdout (kept well under 2 KB):
    the headline launch's rate, its roofline and the CPU oracle's rate, plus
    the smallest W12 / BF16 speedup of the sweep at M = 1-32 and the stack
    step at M = 1.  Everything else is in the detail record."""
    achieved = head["w12_alg_gbps"]
    small = [r for r in sweep if r["M"] <= 32]
    worst = min(small, key=lambda r: r["speedup_vs_bf16"]) if small else None
    st1 = None
    if stack:
        st1 = next((r for r in stack["by_m"] if r["M"] == 1), None)
    cpu_short = None
    if cpu is not None:
        cpu_short = {"value": round(cpu["value"], 3), "unit": cpu["unit"], "cores": cpu["cores"],
                     "kind": cpu["kind"], "sample": cpu["sample"], "nproc": cpu["nproc"],
                     "cpu_model": cpu["cpu_model"],
                     "single_thread": round(cpu["single_thread"]["value"], 3)}
    return {
        "metric": METRIC,
        "value": round(head["w12_weight_gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["launches"],
        "warmup": warmup,
        "ms_per_step": round(head["w12_us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s W[%d,%d] W12 group 128, x[%d,%d] bf16, y fp32"
                               % (WORKLOAD_NAMES[workload], case.N, case.K, M, case.K),
                   "N": case.N, "K": case.K, "M": M, "rotation_copies": rotation},
        "pct_hbm_peak": round(100.0 * head["w12_weight_gbps"] / HBM_PEAK_GBPS, 2),
        "w12_us": round(head["w12_us"], 3),
        "bf16_us": round(head["bf16_us"], 3),
        "speedup_vs_bf16": round(head["speedup_vs_bf16"], 4),
        "read_ceiling_gbps": round(ceiling[0]["gbps"], 1),
        "roofline": {"bound": "hbm", "kernel": head["w12_kernel"], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": head["w12_alg_bytes"]},
        "cpu_baseline": cpu_short,
        "sweep_min_speedup_m1_32": None if worst is None else
            {"workload": worst["workload"], "M": worst["M"],
             "speedup": round(worst["speedup_vs_bf16"], 4)},
        "stack_m1": None if st1 is None else {"w12_ms": st1["w12_ms"],
                                              "speedup_vs_bf16": st1["speedup_vs_bf16"]},
    }


if __name__ == "__main__":
    main()
