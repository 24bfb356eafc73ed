"""Benchmark of the MI355X paged MQA indexer hot path.

One step = indexer_logits (histogram on) + topk_rows (top-2048, FP32 keys)
over the long-decode workload (B=8, next_n=1, L=131072, H=32, D=128, fp8
e4m3 Q/K, 64-token pages with a shuffled block table), inputs resident in
HBM.  Before every step a 1 GiB read sweep evicts the L2s and the 256 MiB
Infinity Cache (so K comes from HBM, as with the cold-L2 protocol of the
measurements this path is compared with) and the histogram is reset; both
happen outside the kernels' timed interval.  The sweep reads rather than
writes: a write sweep would leave the caches full of dirty lines whose
write-back then competes with the timed kernel's reads.

Kernel times come from HIP events that the library's own dispatches record
(indexer_time_next_call, hipExtLaunchKernel): a call's start event when its
first kernel begins and its stop event when its last kernel ends, the same
interval rocprofv3's kernel trace reports.  A step is timed from the start of
the logits kernel to the end of the last top-k kernel, so the gap between
the two calls counts.  Events recorded on the stream around the step are
reported beside them; they also hold the dispatch latency of the first
kernel.

HBM traffic of the logits kernel comes from two rocprofv3 counter runs of
this script (FETCH_SIZE, then WRITE_SIZE, with --copy-calibration so that a
plain device copy of known size is counted too); --traffic-from turns their
CSVs into bytes per launch, scaled by copy bytes / counted copy bytes, and
stores them under profiles/ with a digest of the kernel source, so a later
kernel change voids them.

Prints one JSON line (rank 0, N=1):
  value          mean us per step (logits + top-k kernels), lower is better
  roofline       the logits kernel against the 8 TB/s HBM peak (algorithmic
                 bytes per launch / mean launch time)
  cpu_baseline   the CPU oracle on the same workload, timed on the host
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA, MI355X
FLUSH_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20  # bytes read (and written) by the calibration copy
CALIBRATION_COPIES = 3  # copies run after the timing with --copy-calibration
# The logits kernel each workload launches, whose counters and trace are
# read: indexer_logits_kernel<rows per request, histogram, FP16 output, K
# format (0 FP8, 1 MXFP4), persistent grid> (varlen_decode: 64 one-row
# requests take the persistent grid), and the ragged prefill kernel
# indexer_prefill_logits_kernel<K format>.
COUNTED_KERNEL = {
    "tiny_decode": "indexer_logits_kernel<1, true, false, 0, false>",
    "long_decode": "indexer_logits_kernel<1, true, false, 0, false>",
    "spec_verify/fine": "indexer_logits_kernel<4, true, false, 0, false>",
    "spec_verify/unit": "indexer_logits_kernel<4, true, false, 0, false>",
    "spec_verify/mixed": "indexer_logits_kernel<4, true, false, 0, false>",
    "varlen_decode": "indexer_logits_kernel<1, true, false, 0, true>",
    "very_long": "indexer_logits_kernel<1, true, false, 0, false>",
    "long_decode/mxfp4": "indexer_logits_kernel<1, true, false, 1, false>",
    "spec_verify/mxfp4": "indexer_logits_kernel<4, true, false, 1, false>",
    "prefill/extend": "indexer_prefill_logits_kernel<0>",
    "prefill/extend_mxfp4": "indexer_prefill_logits_kernel<1>",
}
LOGITS_KERNEL = COUNTED_KERNEL["long_decode"]
# bench.py arguments of the profiled runs: one workload's step and nothing
# else (the prefill workloads run in the prefill leg, after two long-decode
# steps).
LEGS_OFF = ("--fp16-steps 0 --mxfp4-steps 0 --candidate-steps 0 --prefill-steps 0 --hist-steps 0 "
            "--sweep-steps 0 --scores-steps 0 --coissue-iters 0 --no-cpu-baseline")


def slug(workload: str) -> str:
    return workload.replace("/", "_")


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"logits_{slug(workload)}_traffic.json")


TRAFFIC_FILE = traffic_file("long_decode")


def profile_args(workload: str, steps: int = 5) -> str:
    """The bench.py arguments of a profiled run of one workload."""
    if workload.startswith("prefill/"):
        legs = LEGS_OFF.replace("--prefill-steps 0", f"--prefill-steps {steps}")
        return f"--workload long_decode --steps 2 --warmup 1 --spin-up-ms 1000 {legs}"
    return f"--workload {workload} --steps {steps} --warmup 2 --spin-up-ms 1000 {LEGS_OFF}"
KERNEL_SOURCES = ("paged_mqa_logits_indexer_amd/csrc/logits_kernel.hip",
                  "paged_mqa_logits_indexer_amd/csrc/indexer_common.h")


def measured_traffic(workload: str):
    """HBM bytes per launch from the workload's committed counter record,
    or None when there is none or the kernel sources changed since."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_src_sha") != kernel_source_digest() or tr.get("workload") != workload:
        return None
    return tr.get("bytes_per_launch")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(x) -> dict:
    """Bytes one indexer_logits launch must move at minimum (read + write)."""
    import numpy as np
    req_keys = x.request_keys().astype(np.int64)
    pages = (req_keys + 63) // 64
    lens = x.context_lens.astype(np.int64)
    if x.mxfp4:
        k = int(req_keys.sum()) * 68         # packed MXFP4 tokens (codes + block scales)
        scales = 0
    else:
        k = int(req_keys.sum()) * 128        # fp8 K rows, once per request
        scales = int(req_keys.sum()) * 4     # one fp32 scale per key
    logits = int(lens.sum()) * 4             # fp32 logits written
    table = int(pages.sum()) * 4             # block-table entries
    qw = x.rows * (32 * 128 + 32 * 4 + 4)    # Q, weights, lengths
    # histogram read-modify-write (the prefill kernel has none)
    hist = 0 if getattr(x, "cu_q", None) is not None else x.rows * 1024 * 4 * 2
    return {"k": k, "total": k + scales + logits + table + qw + hist}


def gpu_clock_mhz():
    """The current shader clock (MHz) of every card sysfs lists, from the
    active pp_dpm_sclk level; {} when the driver does not expose it."""
    import glob
    out = {}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        out[path.split("/")[4]] = int(line.split(":")[1].strip().rstrip("*").strip()
                                                      .lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            pass
    return out


def page_list(x):
    """The physical pages one logits call reads: each request's block-table
    row up to its last live page (int32, request after request)."""
    import numpy as np
    pages = (x.request_keys().astype(np.int64) + 63) // 64
    return np.concatenate([x.block_table[b, :int(pages[b])] for b in range(x.B)]).astype(np.int32)


def sampled_cpu_baseline(x, budget_rows_keys=3_000_000):
    """The oracle on a bounded sample of one workload -- whole requests in
    order until about budget (row, key) pairs -- scaled to the whole step by
    the (row, key) pairs: logits, histogram, top-2048 FP32 of those rows."""
    import numpy as np
    import oracle as O
    lens = x.context_lens.astype(np.int64)
    nn = max(x.next_n, 1)
    reqs, pairs = 0, 0
    while reqs < x.B and (reqs == 0 or pairs + int(lens[reqs * nn:(reqs + 1) * nn].sum()) <= budget_rows_keys):
        pairs += int(lens[reqs * nn:(reqs + 1) * nn].sum())
        reqs += 1
    rows = reqs * nn
    sub_q, sub_w, sub_bt, sub_l = x.q[:rows], x.weights[:rows], x.block_table[:reqs], x.context_lens[:rows]
    t0 = time.perf_counter()
    lg = O.indexer_logits(sub_q, x.kv_pages, x.k_scales, sub_w, sub_bt, sub_l, x.next_n, x.logits_stride)
    O.coarse_histogram(lg, sub_l)
    O.topk_rows(lg, sub_l, 2048, O.KEY_FP32)
    dt = time.perf_counter() - t0
    total = int(lens.sum())
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    return {"value": round(dt * total / pairs * 1e6, 1), "unit": "us/step", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{reqs} of {x.B} requests ({pairs} of {total} row-key pairs), {dt:.2f} s, "
                      f"scaled by the pairs"}


def pct(a, q):
    import numpy as np
    return float(np.percentile(np.asarray(a), q))


def cpu_baseline(x, budget_s: float):
    """The oracle (as it stands) on the whole workload, repeated ~budget_s."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        lg = O.indexer_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                              x.context_lens, x.next_n, x.logits_stride)
        O.coarse_histogram(lg, x.context_lens)
        O.topk_rows(lg, x.context_lens, 2048, O.KEY_FP32)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end:
            break
    mean_s = float(np.mean(times))
    return {"value": mean_s * 1e6, "unit": "us/step", "cores": int(threads), "kind": "oracle",
            "sample": f"whole {x.name} step (logits over all {x.rows} rows, histogram, "
                      f"top-2048 FP32) repeated {len(times)}x, {sum(times):.1f} s"}


def read_counters(directory: str, counter: str):
    """Per-dispatch values of one counter from a rocprofv3 --pmc CSV run:
    [(dispatch id, kernel name, value)] in dispatch order."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    if not rows:
        raise SystemExit(f"no {counter} rows under {directory}")
    return rows


def traffic_from(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """HBM bytes per launch of the workload's logits kernel from the
    FETCH_SIZE and WRITE_SIZE runs (KiB per dispatch), each scaled by the
    same counter on the calibration copies: the device-to-device copies
    after the kernel's last dispatch."""
    import numpy as np
    kernel = COUNTED_KERNEL[workload]
    out = {"workload": workload, "kernel": kernel, "kernel_src_sha": kernel_source_digest(),
           "copy_bytes": COPY_BYTES}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read_counters(d, counter)
        hits = [i for i, (_, name, _) in enumerate(rows) if kernel in name]
        if not hits:
            raise SystemExit(f"{counter}: no dispatch of {kernel} under {d}")
        last_logits = max(hits)
        logits = [v for _, name, v in rows if kernel in name]
        # the calibration copies are the run's last three copy kernels (other
        # copies, such as uploads of later inputs, may follow the kernel too)
        copies = [v for _, name, v in rows[last_logits + 1:] if "copy" in name.lower()][-CALIBRATION_COPIES:]
        if not copies:
            raise SystemExit(f"{counter}: no calibration copy after the last logits dispatch")
        copy_kib = float(np.mean(copies))
        factor = COPY_BYTES / (copy_kib * 1024.0)
        out[counter] = {"logits_kib_per_dispatch": float(np.mean(logits)), "dispatches": len(logits),
                        "copy_kib_per_dispatch": copy_kib, "copies": len(copies), "factor": factor,
                        "bytes_per_launch": float(np.mean(logits)) * 1024.0 * factor}
    out["bytes_per_launch"] = int(round(out["FETCH_SIZE"]["bytes_per_launch"]
                                        + out["WRITE_SIZE"]["bytes_per_launch"]))
    return out


def short_kernel_name(n: str) -> str:
    """A trace's kernel name without namespaces and parameter lists."""
    import re
    n = n.replace("pmqa::(anonymous namespace)::", "").replace("void ", "")
    if n.startswith("at::native") or "rocclr" in n:
        return "torch/runtime kernel (set-up, histogram reset, calibration copy)"
    m = re.match(r"([A-Za-z_0-9]+(<[^>]*>)?)", n)
    return m.group(1) if m else n[:60]


def profiled_command(tool: str, workload: str, steps: int) -> str:
    return (f"rocprofv3 {tool} -d <out> -o run --output-format csv -- \\\n"
            f"    python3 bench.py {profile_args(workload, steps)}")


def write_traffic_md(tr: dict, alg_bytes: int, out_dir: str = PROFILES) -> str:
    w = tr["workload"]
    path = os.path.join(out_dir, f"logits_{slug(w)}_traffic.md")
    lines = [f"# HBM traffic of {tr['kernel']}: {w}", "",
             "Two counter runs (one counter each) and the conversion, from the repository root "
             "with `TMPDIR=/tmp`:", "", "```"]
    for c, d in (("FETCH_SIZE", "<fetch>"), ("WRITE_SIZE", "<write>")):
        lines.append(profiled_command(f"--pmc {c}", w, 5).replace("<out>", d) + " --copy-calibration")
    lines += [f"python3 bench.py --workload {w} --traffic-from <fetch> <write>", "```", "",
              "Every dispatch follows a 1 GiB read sweep, so K comes from HBM.  The calibration "
              "copy is an int32 -> float32 elementwise copy of 256 MiB (reads and writes "
              "268,435,456 bytes), counted after the kernel's last dispatch.", "",
              "| counter | KiB / dispatch | dispatches | copy KiB / dispatch | factor | bytes / launch |",
              "|---|---|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = tr[c]
        lines.append(f"| {c} | {r['logits_kib_per_dispatch']:.1f} | {r['dispatches']} | "
                     f"{r['copy_kib_per_dispatch']:.1f} | {r['factor']:.4f} | {r['bytes_per_launch']:,.0f} |")
    lines += ["", f"Traffic per launch: {tr['bytes_per_launch']:,} bytes against {alg_bytes:,} "
              f"algorithmic bytes: ratio {tr['bytes_per_launch'] / alg_bytes:.4f}.  Kernel source digest "
              f"`{tr['kernel_src_sha']}` (bench.py reports the traffic only while the kernel sources "
              "still have this digest)."]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def write_stats_md(csv_path: str, workload: str, steps: int, out_dir: str = PROFILES) -> str:
    """A rocprofv3 --stats kernel table as markdown, with its command."""
    import csv
    with open(csv_path) as fh:
        rows = list(csv.DictReader(fh))
    path = os.path.join(out_dir, f"{slug(workload)}_kernel_trace.md")
    lines = [f"# Kernel trace: {workload}", "", "From the repository root with `TMPDIR=/tmp`:", "", "```",
             profiled_command("--kernel-trace --stats", workload, steps),
             f"python3 bench.py --workload {workload} --profile-steps {steps} --stats-md <out>/run_kernel_stats.csv",
             "```", "",
             f"Calls include warm-up, the timed steps, the per-call timing and the read-ceiling "
             f"probes of `bench.py`; `hbm_read_probe_kernel` also covers the 1 GiB cache sweeps before "
             f"every step.  The workload's logits kernel is `{COUNTED_KERNEL[workload]}`.", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    agg = {}  # kernels that share a short name are merged (calls-weighted average)
    for r in rows:
        n = short_kernel_name(r["Name"])
        c, a, lo, hi = int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])
        if n in agg:
            c0, a0, lo0, hi0 = agg[n]
            agg[n] = (c0 + c, (a0 * c0 + a * c) / (c0 + c), min(lo0, lo), max(hi0, hi))
        else:
            agg[n] = (c, a, lo, hi)
    for n, (c, a, lo, hi) in sorted(agg.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        lines.append(f"| {n} | {c} | {a / 1e3:.2f} | {lo / 1e3:.2f} | {hi / 1e3:.2f} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def counters_of(directory: str, kernel: str) -> dict:
    """Median per dispatch of every counter of one kernel in a --pmc run, and
    the median dispatch duration (profiler timestamps, us)."""
    import csv
    import glob
    import numpy as np
    per = {}
    dur = {}
    for f in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel not in r["Kernel_Name"]:
                    continue
                key = (r["Dispatch_Id"], r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                if r.get("Start_Timestamp"):
                    dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    if not per:
        raise SystemExit(f"no dispatch of {kernel} under {directory}")
    names = sorted({c for _, c in per})
    out = {c: float(np.median([v for (d, cc), v in per.items() if cc == c])) for c in names}
    out["dispatches"] = len(dur) or len({d for d, _ in per})
    out["duration_us"] = float(np.median(list(dur.values()))) if dur else None
    return out


MFMA_COUNTERS = "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_BUSY_CYCLES SQ_WAVES GRBM_GUI_ACTIVE"


def write_counters_md(directory: str, workload: str, out_dir: str = PROFILES) -> str:
    """MFMA use of the workload's kernel from one --pmc run (MFMA_COUNTERS)."""
    kernel = COUNTED_KERNEL[workload]
    c = counters_of(directory, kernel)
    path = os.path.join(out_dir, f"logits_{slug(workload)}_mfma.md")
    lines = [f"# MFMA use of {kernel}: {workload}", "", "One counter run, from the repository root with "
             "`TMPDIR=/tmp`:", "", "```", profiled_command(f"--pmc {MFMA_COUNTERS}", workload, 5),
             f"python3 bench.py --workload {workload} --counters-md <out>", "```", "",
             f"Medians over the kernel's {c['dispatches']} dispatches:", "", "| counter | per dispatch |",
             "|---|---|"]
    for k, v in c.items():
        if k.startswith(("SQ_", "GRBM_")):
            lines.append(f"| {k} | {v:,.0f} |")
    if c.get("duration_us"):
        lines.append(f"| dispatch duration (profiler timestamps) | {c['duration_us']:.2f} us |")
    busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
    if busy is not None and c.get("duration_us"):
        cyc = c["duration_us"] * 1e-6 * 2.4e9
        frac = busy / 1024 / cyc
        lines += ["", f"MFMA busy per SIMD: {busy:,.0f} / 1,024 SIMDs = {busy / 1024:,.0f} cycles of "
                  f"{cyc:,.0f} ({c['duration_us']:.2f} us at 2.4 GHz): {100 * frac:.1f} %."]
        if c.get("SQ_INSTS_MFMA"):
            lines.append(f"Busy cycles per MFMA: {busy / c['SQ_INSTS_MFMA']:.1f}; VALU instructions per "
                         f"MFMA: {c.get('SQ_INSTS_VALU', 0) / c['SQ_INSTS_MFMA']:.2f}.")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_decode")
    ap.add_argument("--fp16-steps", type=int, default=100,
                    help="steps of the second timing with FP16 score keys")
    ap.add_argument("--mxfp4-steps", type=int, default=100,
                    help="steps of the same shape with MXFP4 K (indexer_logits_mxfp4)")
    ap.add_argument("--candidate-steps", type=int, default=50,
                    help="steps of the two-level candidate chain on the dense logits")
    ap.add_argument("--prefill-steps", type=int, default=30,
                    help="steps of the ragged prefill (extend) logits on prefill/extend")
    ap.add_argument("--hist-steps", type=int, default=50,
                    help="steps of the logits kernel with and without the histogram (interleaved)")
    ap.add_argument("--sweep-steps", type=int, default=40,
                    help="steps per decode workload in the all-workload sweep (0: skip it)")
    ap.add_argument("--coissue-iters", type=int, default=4096,
                    help="rounds per wave of the MFMA / VALU co-issue probe (0: skip it)")
    ap.add_argument("--scores-steps", type=int, default=30,
                    help="steps of top-2048 over the very-long synthetic score rows (no histogram)")
    ap.add_argument("--candidate-blocks", type=int, default=512,
                    help="8-token blocks the source layer publishes per row")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cache eviction between steps (warm caches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timing, run plain 256 MiB device copies (counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of --workload into its traffic record (no GPU)")
    ap.add_argument("--stats-md", metavar="KERNEL_STATS_CSV",
                    help="write the kernel-trace summary of --workload under profiles/ (no GPU)")
    ap.add_argument("--counters-md", metavar="PMC_DIR",
                    help="write the MFMA counter summary of --workload under profiles/ (no GPU)")
    ap.add_argument("--profile-args", action="store_true",
                    help="print the bench.py arguments of a profiled run of --workload")
    ap.add_argument("--profile-steps", type=int, default=5)
    ap.add_argument("--spin-up-ms", type=float, default=0.0,
                    help="read sweeps for this long before the warmup, so that a short run is timed "
                         "at the clocks a sustained load reaches")
    args = ap.parse_args()

    if args.profile_args:
        print(profile_args(args.workload, args.profile_steps))
        return 0
    if args.traffic_from or args.stats_md or args.counters_md:
        import gen
        if args.traffic_from:
            tr = traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload)
            with open(traffic_file(args.workload), "w") as f:
                json.dump(tr, f, indent=1)
            print(write_traffic_md(tr, algorithmic_bytes(gen.config_inputs(args.workload))["total"]))
        if args.stats_md:
            print(write_stats_md(args.stats_md, args.workload, args.profile_steps))
        if args.counters_md:
            print(write_counters_md(args.counters_md, args.workload))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the indexer path has no multi-GPU part "
              "(each request's rows are independent; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gen
    import paged_mqa_logits_indexer_amd as pmqa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    x = gen.config_inputs(args.workload)
    def upload(x):
        return {k: (None if getattr(x, k) is None
                    else torch.from_numpy(np.ascontiguousarray(getattr(x, k))).to(dev))
                for k in ("q", "kv_pages", "k_scales", "weights", "block_table", "context_lens")}

    def call_logits(x, t, logits, hist, events):
        """indexer_logits, or indexer_logits_mxfp4 for packed MXFP4 pages."""
        if x.mxfp4:
            pmqa.indexer_logits_mxfp4(t["q"], t["kv_pages"], t["weights"], t["block_table"],
                                      t["context_lens"], x.next_n, logits, hist, events=events)
        else:
            pmqa.indexer_logits(t["q"], t["kv_pages"], t["k_scales"], t["weights"],
                                t["block_table"], t["context_lens"], x.next_n, logits, hist,
                                events=events)

    t = upload(x)
    logits = torch.full((x.rows, x.logits_stride), float("inf"), dtype=torch.float32, device=dev)
    hist = torch.zeros((x.rows, 1024), dtype=torch.int32, device=dev)
    K = 2048
    idx = torch.empty((x.rows, K), dtype=torch.int32, device=dev)
    ws = torch.zeros(pmqa.topk_workspace_bytes(x.rows, x.logits_stride, K), dtype=torch.uint8,
                     device=dev)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def evict():
        if not args.no_flush:
            pmqa.hbm_read_probe(flush, sink)

    stream = torch.cuda.current_stream(dev)

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)  # creates the HIP event before a dispatch records it
        return evs

    stride16 = -(-x.logits_stride // 8) * 8  # 16-byte rows of halves
    logits16 = torch.full((x.rows, stride16), float("inf"), dtype=torch.float16, device=dev)

    def run16(n_steps, record, split=False):
        """Steps with FP16 logits (indexer_logits_f16 + topk_rows_f16); as in
        run(), only the step's ends are recorded unless `split`."""
        out = []
        evs = []
        for i in range(n_steps):
            ls, le, te = new_events(3)
            evict()
            hist.zero_()
            pmqa.indexer_logits_f16(t["q"], t["kv_pages"], t["k_scales"], t["weights"],
                                    t["block_table"], t["context_lens"], x.next_n, logits16, hist,
                                    events=(ls, le if split else None))
            pmqa.topk_rows_f16(logits16, hist, t["context_lens"], K, idx, ws,
                               events=None if split else (None, te))
            evs.append((ls, le if split else te))
        torch.cuda.synchronize()
        if record:
            out = [a.elapsed_time(b) * 1e3 for a, b in evs]
        return out

    def run(n_steps, key, record, split=False, x=x, t=t, logits=logits, hist=hist, idx=idx, ws=ws):
        """Steps of logits + top-k.  Without `split` only the step's start
        (logits kernel begins) and end (last top-k kernel ends) are recorded,
        so no event sits between the two calls; with it each call is timed
        on its own."""
        lt, tt, st, wt = [], [], [], []
        evs = []
        for i in range(n_steps):
            ls, le, ts, te, ws0, ws1 = new_events(6)
            evict()
            hist.zero_()
            ws0.record(stream)
            call_logits(x, t, logits, hist, (ls, le if split else None))
            pmqa.topk_rows(logits, hist, t["context_lens"], K, key, idx, ws,
                           events=(ts if split else None, te))
            ws1.record(stream)
            evs.append((ls, le, ts, te, ws0, ws1))
        torch.cuda.synchronize()
        if record:
            for ls, le, ts, te, ws0, ws1 in evs:
                if split:
                    lt.append(ls.elapsed_time(le) * 1e3)
                    tt.append(ts.elapsed_time(te) * 1e3)
                else:
                    st.append(ls.elapsed_time(te) * 1e3)
                    wt.append(ws0.elapsed_time(ws1) * 1e3)
        return lt, tt, st, wt

    if args.spin_up_ms > 0:
        print(f"[bench] spin-up {args.spin_up_ms:.0f} ms", file=sys.stderr, flush=True)
        t_end = time.perf_counter() + args.spin_up_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(8):
                pmqa.hbm_read_probe(flush, sink)
            torch.cuda.synchronize()
    clock_before = gpu_clock_mhz()
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    run(args.warmup, pmqa.KEY_FP32, False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    _, _, step_us, stream_us = run(args.steps, pmqa.KEY_FP32, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] per-call timing {args.steps} steps", file=sys.stderr, flush=True)
    lt, tt, _, _ = run(args.steps, pmqa.KEY_FP32, True, split=True)
    print(f"[bench] FP16-key timing {args.fp16_steps} steps", file=sys.stderr, flush=True)
    if args.fp16_steps > 0 and not x.mxfp4:
        _, _, st16, _ = run(args.fp16_steps, pmqa.KEY_FP16, True)
        _, tt16, _, _ = run(args.fp16_steps, pmqa.KEY_FP16, True, split=True)
        print(f"[bench] FP16-logits timing {args.fp16_steps} steps", file=sys.stderr, flush=True)
        run16(3, False)
        st_h = run16(args.fp16_steps, True)
        lt_h = run16(args.fp16_steps, True, split=True)
        # The three step kinds once more, interleaved (order rotated every
        # step), so that clock and thermal drift between the legs above does
        # not decide their comparison.
        print(f"[bench] interleaved FP32 / FP16-key / FP16-logits steps {args.fp16_steps}",
              file=sys.stderr, flush=True)
        inter = {0: [], 1: [], 2: []}
        for i in range(args.fp16_steps):
            for v in ((0, 1, 2), (1, 2, 0), (2, 0, 1))[i % 3]:
                if v == 2:
                    inter[2] += run16(1, True)
                else:
                    inter[v] += run(1, pmqa.KEY_FP32 if v == 0 else pmqa.KEY_FP16, True)[2]
    else:
        st16, tt16, lt_h, st_h = [], [], [], []
        inter = None

    # the same shape with MXFP4 K pages (half the K bytes)
    mx_out = None
    mx_name = {"long_decode": "long_decode/mxfp4"}.get(args.workload)
    if mx_name is None and args.workload.startswith("spec_verify/") and not x.mxfp4:
        mx_name = "spec_verify/mxfp4"
    if args.mxfp4_steps > 0 and mx_name:
        print(f"[bench] {mx_name}: {args.mxfp4_steps} steps", file=sys.stderr, flush=True)
        xm = gen.config_inputs(mx_name)
        tm = upload(xm)
        lgm = torch.full((xm.rows, xm.logits_stride), float("inf"), dtype=torch.float32, device=dev)
        hm = torch.zeros((xm.rows, 1024), dtype=torch.int32, device=dev)
        mx_kw = dict(x=xm, t=tm, logits=lgm, hist=hm)
        run(5, pmqa.KEY_FP32, False, **mx_kw)
        _, _, st_m, _ = run(args.mxfp4_steps, pmqa.KEY_FP32, True, **mx_kw)
        lt_m, tt_m, _, _ = run(args.mxfp4_steps, pmqa.KEY_FP32, True, split=True, **mx_kw)
        abm = algorithmic_bytes(xm)
        lm = float(np.mean(lt_m))
        mx_out = {"workload": mx_name, "step_us_mean": round(float(np.mean(st_m)), 3),
                  "indexer_logits_mxfp4_mean": round(lm, 3),
                  "topk_rows_fp32_mean": round(float(np.mean(tt_m)), 3),
                  "k_bytes": abm["k"], "bytes_per_launch": abm["total"],
                  "achieved_gbps": round(abm["total"] / (lm * 1e-6) / 1e9, 1),
                  "frac": round(abm["total"] / (lm * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        del tm, lgm, hm

    # two-level candidate chain on this workload's dense logits (FP8 K):
    # publish = block maxima + block top-k + sorted table; select = sparse
    # logits over the published blocks + top-k inside the sparse row + map
    cand_out = None
    if args.candidate_steps > 0 and not x.mxfp4:
        kbk = args.candidate_blocks
        print(f"[bench] candidate chain ({kbk} blocks): {args.candidate_steps} steps",
              file=sys.stderr, flush=True)
        hist.zero_()
        call_logits(x, t, logits, None, None)
        width = -(-(-(-x.logits_stride // 8)) // 4) * 4
        am = torch.empty((x.rows, width), dtype=torch.float32, device=dev)
        ah = torch.zeros((x.rows, 1024), dtype=torch.int32, device=dev)
        blens = torch.empty(x.rows, dtype=torch.int32, device=dev)
        bsel = torch.empty((x.rows, kbk), dtype=torch.int32, device=dev)
        table = torch.empty_like(bsel)
        slots = torch.empty_like(bsel)
        slens = torch.empty(x.rows, dtype=torch.int32, device=dev)
        sparse = torch.empty((x.rows, kbk * 8), dtype=torch.float32, device=dev)
        ssel = torch.empty((x.rows, K), dtype=torch.int32, device=dev)
        pos = torch.empty_like(ssel)
        pos2 = torch.empty_like(ssel)
        ws_b = torch.zeros(pmqa.topk_workspace_bytes(x.rows, width, kbk), dtype=torch.uint8, device=dev)
        ws_s = torch.zeros(pmqa.topk_workspace_bytes(x.rows, kbk * 8, K), dtype=torch.uint8, device=dev)
        # select = sparse logits + sparse_topk (the top-k inside the sparse
        # row and the map to logical keys in one launch); the unfused pair
        # (topk_rows + sparse_to_logical) is timed after it for comparison
        names = ("block_amax8", "block_topk", "sort_candidate_blocks", "indexer_sparse_logits",
                 "sparse_topk", "sparse_topk_unfused", "sparse_to_logical")

        def chain(n_steps, record):
            per = {nm: [] for nm in names}
            pub, sel = [], []
            for i in range(n_steps):
                ev = new_events(14)
                evict()
                ah.zero_()
                pmqa.block_amax8(logits, t["context_lens"], am, ah, block_lens=blens, events=(ev[0], ev[1]))
                pmqa.topk_rows(am, ah, blens, kbk, pmqa.KEY_FP32, bsel, ws_b, events=(ev[2], ev[3]))
                pmqa.sort_candidate_blocks(bsel, t["context_lens"], x.logits_stride, t["block_table"],
                                           x.next_n, table, slots, slens, events=(ev[4], ev[5]))
                pmqa.indexer_sparse_logits(t["q"], t["kv_pages"], t["k_scales"], t["weights"], table,
                                           slots, t["context_lens"], sparse, events=(ev[6], ev[7]))
                pmqa.sparse_topk(sparse, None, slens, K, pmqa.KEY_FP32, table, pos, events=(ev[8], ev[9]))
                pmqa.topk_rows(sparse, None, slens, K, pmqa.KEY_FP32, ssel, ws_s, events=(ev[10], ev[11]))
                pmqa.sparse_to_logical(ssel, table, pos2, events=(ev[12], ev[13]))
                if record:
                    per["_ev"] = per.get("_ev", []) + [ev]
            torch.cuda.synchronize()
            if record:
                for ev in per.pop("_ev"):
                    for j, nm in enumerate(names):
                        per[nm].append(ev[2 * j].elapsed_time(ev[2 * j + 1]) * 1e3)
                    pub.append(ev[0].elapsed_time(ev[5]) * 1e3)
                    sel.append(ev[6].elapsed_time(ev[9]) * 1e3)
            return per, pub, sel

        chain(3, False)
        per, pub, sel = chain(args.candidate_steps, True)
        keys_listed = int(slens.sum().item())
        fused_matches_unfused = bool(torch.equal(torch.sort(pos, dim=1).values, torch.sort(pos2, dim=1).values))


        sp_bytes = keys_listed * (128 + 4 + 4) + x.rows * kbk * 8 + x.rows * (32 * 128 + 32 * 4 + 4)
        sp_us = float(np.mean(per["indexer_sparse_logits"]))
        cand_out = {"blocks_per_row": kbk, "k": K,
                    "publish_us_mean": round(float(np.mean(pub)), 3),
                    "select_us_mean": round(float(np.mean(sel)), 3),
                    "per_call_us_mean": {nm: round(float(np.mean(per[nm])), 3) for nm in names},
                    "sparse_logits_bytes": sp_bytes,
                    "sparse_logits_gbps": round(sp_bytes / (sp_us * 1e-6) / 1e9, 1),
                    "fused_matches_unfused": fused_matches_unfused,
                    "note": "select = indexer_sparse_logits + sparse_topk; the publish and select "
                            "spans include the gaps between their calls"}
        del am, ah, bsel, table, slots, slens, sparse, ssel, pos, pos2, ws_b, ws_s

    # cost of the fused histogram: the logits kernel with and without it,
    # interleaved (the pages' producer-cost measure: histogram extra)
    hx_out = None
    if args.hist_steps > 0:
        print(f"[bench] histogram on/off: {args.hist_steps} steps each", file=sys.stderr, flush=True)
        on_us, off_us = [], []
        for i in range(args.hist_steps + 2):
            for with_hist in (True, False):
                e0, e1 = new_events(2)
                evict()
                hist.zero_()
                call_logits(x, t, logits, hist if with_hist else None, (e0, e1))
                torch.cuda.synchronize()
                if i >= 2:
                    (on_us if with_hist else off_us).append(e0.elapsed_time(e1) * 1e3)
        hx_out = {"with_hist_us_mean": round(float(np.mean(on_us)), 3),
                  "without_hist_us_mean": round(float(np.mean(off_us)), 3),
                  "extra_us_mean": round(float(np.mean(on_us) - np.mean(off_us)), 3),
                  "extra_us_median": round(pct(on_us, 50) - pct(off_us, 50), 3)}

    # ragged prefill (extend) logits (SGLang PR #38944, SM90 FP8 prefill):
    # compute-bound, priced against the fp8 MFMA peak
    pf_out = None
    if args.prefill_steps > 0:
        pf_out = {}
        for pname in ("prefill/extend", "prefill/extend_mxfp4"):
            print(f"[bench] {pname}: {args.prefill_steps} steps", file=sys.stderr, flush=True)
            xp = gen.config_inputs(pname)
            tp = upload(xp)
            cu = torch.from_numpy(np.ascontiguousarray(xp.cu_q)).to(dev)
            lgp = torch.empty((xp.rows, xp.logits_stride), dtype=torch.float32, device=dev)
            pts_pf = []
            for i in range(args.prefill_steps + 3):
                e0, e1 = new_events(2)
                evict()
                pmqa.indexer_prefill_logits(tp["q"], tp["kv_pages"], tp["k_scales"], tp["weights"],
                                            tp["block_table"], cu, tp["context_lens"], lgp,
                                            events=(e0, e1))
                pts_pf.append((e0, e1))
            torch.cuda.synchronize()
            us = [a.elapsed_time(b) * 1e3 for a, b in pts_pf[3:]]
            pairs = int(xp.context_lens.astype(np.int64).sum())
            flop = pairs * 2 * 32 * 128
            pu = float(np.mean(us))
            pf_out[pname] = {
                "rows": xp.rows, "row_key_pairs": pairs, "us_mean": round(pu, 3),
                "us_median": round(pct(us, 50), 3), "mfma_flop": flop,
                "tflops": round(flop / (pu * 1e-6) / 1e12, 1),
                "mfma_peak_tflops": FP8_MFMA_PEAK_TFLOPS,
                "mfma_frac": round(flop / (pu * 1e-6) / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4),
                "logits_write_bytes": pairs * 4,
                "logits_write_gbps": round(pairs * 4 / (pu * 1e-6) / 1e9, 1)}
            del tp, cu, lgp

    # how far a SIMD's matrix and vector pipes overlap: fp8 MFMAs only, fp32
    # FMAs only (eight per MFMA, the logits epilogue's ratio), and both
    co_out = None
    if args.coissue_iters > 0:
        print(f"[bench] MFMA / VALU co-issue probe: {args.coissue_iters} rounds", file=sys.stderr, flush=True)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        co_out = {"rounds_per_wave": args.coissue_iters, "mfma_per_round": 4, "fma_per_round": 32}
        for wps in (1, 2):
            buf = torch.empty(cus * wps * 256, dtype=torch.float32, device=dev)
            us = {}
            for mode, name in ((0, "mfma_only_us"), (1, "valu_only_us"), (2, "both_us")):
                pmqa.mfma_valu_probe(mode, wps, args.coissue_iters, buf)
                evs = []
                for i in range(5):
                    e0, e1 = new_events(2)
                    pmqa.mfma_valu_probe(mode, wps, args.coissue_iters, buf, events=(e0, e1))
                    evs.append((e0, e1))
                torch.cuda.synchronize()
                us[name] = round(float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs])), 2)
            m, v, b = us["mfma_only_us"], us["valu_only_us"], us["both_us"]
            rounds = args.coissue_iters * wps  # per SIMD
            us.update({"both_over_sum": round(b / (m + v), 3), "both_over_max": round(b / max(m, v), 3),
                       "cycles_per_mfma_at_2400mhz": round(m * 2400.0 / (4 * rounds), 1),
                       "cycles_per_fma_at_2400mhz": round(v * 2400.0 / (32 * rounds), 2)})
            co_out[f"waves_per_simd_{wps}"] = us
            del buf

    # top-2048 over synthetic fp32 score rows [4, 1048576] (0.99 N(0, var 4) +
    # 0.01 N(40, var 10)), FP16 keys, no histogram: the selector's own first
    # pass, then threshold bin, collect and refine
    sc_out = None
    if args.scores_steps > 0:
        print(f"[bench] very_long/scores: {args.scores_steps} steps", file=sys.stderr, flush=True)
        sc = torch.from_numpy(gen.very_long_scores()).to(dev)
        sc_lens = torch.full((sc.shape[0],), sc.shape[1], dtype=torch.int32, device=dev)
        sc_idx = torch.empty((sc.shape[0], K), dtype=torch.int32, device=dev)
        sc_ws = torch.zeros(pmqa.topk_workspace_bytes(sc.shape[0], sc.shape[1], K), dtype=torch.uint8,
                            device=dev)
        sc_ev = []
        for i in range(args.scores_steps + 3):
            e0, e1 = new_events(2)
            evict()
            pmqa.topk_rows(sc, None, sc_lens, K, pmqa.KEY_FP16, sc_idx, sc_ws, events=(e0, e1))
            sc_ev.append((e0, e1))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in sc_ev[3:]]
        sc_out = {"rows": int(sc.shape[0]), "cols": int(sc.shape[1]), "k": K, "key": "fp16",
                  "hist": None, "us_mean": round(float(np.mean(us)), 3),
                  "us_median": round(pct(us, 50), 3),
                  "score_read_gbps": round(sc.numel() * 4 / (float(np.mean(us)) * 1e-6) / 1e9, 1)}
        del sc, sc_lens, sc_idx, sc_ws

    def probes(xw, tw, reps):
        """Read ceilings for one workload's K stream: a contiguous read of the
        same bytes (K codes + scales), and the paged gather of exactly the
        pages the logits call reads (FP8 pages only); times in us."""
        kb = algorithmic_bytes(xw)
        # MXFP4 tokens carry their scales; FP8 keys add one 4-byte scale per 128 bytes
        src = torch.ones((kb["k"] if xw.mxfp4 else kb["k"] + kb["k"] // 32) // 4, dtype=torch.int32,
                         device=dev)
        plist = torch.from_numpy(page_list(xw)).to(dev)
        rd, ga = [], []
        for i in range(reps + 3):
            e0, e1, e2, e3 = new_events(4)
            evict()
            pmqa.hbm_read_probe_nt(src, sink, events=(e0, e1))
            if not xw.mxfp4:
                evict()
                pmqa.hbm_gather_probe(tw["kv_pages"], tw["k_scales"], plist, sink, events=(e2, e3))
            torch.cuda.synchronize()
            if i >= 3:
                rd.append(e0.elapsed_time(e1) * 1e3)
                if not xw.mxfp4:
                    ga.append(e2.elapsed_time(e3) * 1e3)
        del src, plist
        return rd, ga

    # every decode workload: logits (histogram on) + top-2048, the roofline of
    # its logits kernel, the read ceilings of its K stream and the oracle on a
    # bounded sample of it
    sweep_out = None
    if args.sweep_steps > 0:
        sweep_out = {}
        for name in gen.CONFIG_NAMES:
            print(f"[bench] sweep {name}: {args.sweep_steps} steps", file=sys.stderr, flush=True)
            xw = x if name == x.name else gen.config_inputs(name)
            tw = t if name == x.name else upload(xw)
            lw = torch.full((xw.rows, xw.logits_stride), float("inf"), dtype=torch.float32, device=dev)
            hw = torch.zeros((xw.rows, 1024), dtype=torch.int32, device=dev)
            iw = torch.empty((xw.rows, K), dtype=torch.int32, device=dev)
            key = pmqa.KEY_FP16 if name == "varlen_decode" else pmqa.KEY_FP32
            kw = dict(x=xw, t=tw, logits=lw, hist=hw, idx=iw, ws=None)
            run(3, key, False, **kw)
            _, _, sw, _ = run(args.sweep_steps, key, True, **kw)
            lw_us, tw_us, _, _ = run(args.sweep_steps, key, True, split=True, **kw)
            rd, ga = probes(xw, tw, max(10, args.sweep_steps // 2))
            abw = algorithmic_bytes(xw)
            lm = float(np.mean(lw_us))
            ach = abw["total"] / (lm * 1e-6) / 1e9
            sweep_out[name] = {
                "B": xw.B, "next_n": xw.next_n, "key": "fp16" if key == pmqa.KEY_FP16 else "fp32",
                "step_us": {"mean": round(float(np.mean(sw)), 3), "p10": round(pct(sw, 10), 3),
                            "p50": round(pct(sw, 50), 3), "p90": round(pct(sw, 90), 3)},
                "indexer_logits_us": {"mean": round(lm, 3), "p10": round(pct(lw_us, 10), 3),
                                      "p50": round(pct(lw_us, 50), 3), "p90": round(pct(lw_us, 90), 3)},
                "topk_rows_us": {"mean": round(float(np.mean(tw_us)), 3), "p10": round(pct(tw_us, 10), 3),
                                 "p50": round(pct(tw_us, 50), 3), "p90": round(pct(tw_us, 90), 3)},
                "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(ach / HBM_PEAK_GBPS, 4), "bytes_per_launch": abw["total"],
                             "traffic": measured_traffic(name), "kernel": COUNTED_KERNEL[name],
                             "k_bytes": abw["k"],
                             "k_frac": round(abw["k"] / (lm * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
                "read_probe_us_p50": round(pct(rd, 50), 3),
                "gather_probe_us_p50": round(pct(ga, 50), 3),
                "logits_vs_gather_probe": round(pct(ga, 50) / pct(lw_us, 50), 4),
                "cpu_baseline": (None if args.no_cpu_baseline else sampled_cpu_baseline(xw)),
            }
            if name != x.name:
                del tw
            del lw, hw, iw
            torch.cuda.empty_cache()

    # practical read ceilings for the headline workload's K stream
    ab = algorithmic_bytes(x)
    rd_pts, ga_pts = probes(x, t, 30)
    probe_us = pct(rd_pts, 50)
    gather_us = pct(ga_pts, 50) if ga_pts else None
    clock_after = gpu_clock_mhz()

    if args.copy_calibration:
        # int32 -> float32: an elementwise copy kernel (a same-dtype copy may
        # go to a DMA engine, which the counters do not see); 4 B read and
        # 4 B written per element.
        src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        for i in range(CALIBRATION_COPIES):
            evict()
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    mean_logits = float(np.mean(lt))
    mfma_flop = int(x.context_lens.astype(np.int64).sum()) * 2 * 32 * 128
    achieved = ab["total"] / (mean_logits * 1e-6) / 1e9
    traffic = measured_traffic(x.name)
    value = float(np.mean(step_us))
    out = {
        "metric": "indexer logits+hist+top-2048 us/step and HBM GB/s (% peak), B=8 L=128K",
        "value": round(value, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(value / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-in/fp32-acc",
        "data": "synthetic",
        "config": {"workload": x.name, "B": x.B, "next_n": x.next_n,
                   "context_len": int(x.context_lens.max()), "heads": 32, "head_dim": 128,
                   "page_tokens": 64, "topk": K, "key": "fp32",
                   "cache": "cold (1 GiB read sweep before each step)" if not args.no_flush else "warm"},
        "breakdown_us": {
            "indexer_logits_mean": round(mean_logits, 3),
            "indexer_logits_p10": round(pct(lt, 10), 3),
            "indexer_logits_median": round(pct(lt, 50), 3),
            "indexer_logits_p90": round(pct(lt, 90), 3),
            "topk_rows_fp32_mean": round(float(np.mean(tt)), 3),
            "step_median": round(pct(step_us, 50), 3),
            "step_p10": round(pct(step_us, 10), 3),
            "step_p90": round(pct(step_us, 90), 3),
            "step_stream_events_mean": round(float(np.mean(stream_us)), 3),
        },
        "timing": "dispatch-recorded HIP events (hipExtLaunchKernel start/stop), mean over steps",
        "fp16_keys": ({"step_us_mean": round(float(np.mean(st16)), 3),
                       "topk_rows_fp16_mean": round(float(np.mean(tt16)), 3)} if st16 else None),
        # FP16 logits output: indexer_logits_f16 (halves) + topk_rows_f16 (FP16 keys)
        "fp16_logits": ({"step_us_mean": round(float(np.mean(st_h)), 3),
                         "indexer_logits_f16_mean": round(float(np.mean(lt_h)), 3)} if st_h else None),
        # The same three steps interleaved step by step (means and medians).
        "interleaved_steps": ({name: {"mean": round(float(np.mean(inter[v])), 3),
                                      "median": round(float(np.median(inter[v])), 3)}
                               for v, name in ((0, "fp32"), (1, "fp16_keys"), (2, "fp16_logits"))}
                              if inter else None),
        # the same shape with MXFP4 K: indexer_logits_mxfp4 + topk_rows (FP32 keys);
        # frac = algorithmic bytes / time against the HBM peak
        "mxfp4_k": mx_out,
        # two-level candidate indexer on this workload (SGLang PR #38944)
        "candidate_chain": cand_out,
        # logits kernel with the fused histogram minus without it
        "histogram_extra": hx_out,
        # ragged prefill (extend) logits: 4 requests x 2048 rows, contexts 2K..32K
        "prefill": pf_out,
        # top-2048 over synthetic score rows [4, 1048576], FP16 keys, hist=NULL
        "topk_scores_1m": sc_out,
        # MFMA / VALU co-issue probe (the prefill epilogue's bound)
        "mfma_valu_coissue": co_out,
        "hbm": {
            "k_bytes": ab["k"],
            "k_gbps": round(ab["k"] / (mean_logits * 1e-6) / 1e9, 1),
            "k_frac_of_peak": round(ab["k"] / (mean_logits * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            # contiguous read of the K codes + scales: non-temporal loads, the best streaming shape
            "read_probe_us_p50": round(probe_us, 3),
            "read_probe_us_p10_p90": [round(pct(rd_pts, 10), 3), round(pct(rd_pts, 90), 3)],
            "read_probe_gbps": round(ab["k"] * 33 / 32 / (probe_us * 1e-6) / 1e9, 1),
            # the same pages read through the block table, whole lines, no arithmetic
            "gather_probe_us_p50": round(gather_us, 3) if ga_pts else None,
            "gather_probe_us_p10_p90": [round(pct(ga_pts, 10), 3), round(pct(ga_pts, 90), 3)] if ga_pts else None,
            "logits_median_vs_gather_probe": round(gather_us / pct(lt, 50), 4) if ga_pts else None,
            "logits_median_vs_read_probe": round(probe_us / pct(lt, 50), 4),
        },
        "gpu_clock_mhz": {"before": clock_before, "after": clock_after},
        # every decode workload, each with its roofline and oracle baseline
        "workloads": sweep_out,
        # MFMA work of the same launch: 2*32*128 flop per (row, live key)
        "mfma": {"flop_per_launch": mfma_flop,
                 "tflops": round(mfma_flop / (mean_logits * 1e-6) / 1e12, 1),
                 "frac_of_fp8_peak": round(mfma_flop / (mean_logits * 1e-6) / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": COUNTED_KERNEL[x.name],
                     "bytes_per_launch": ab["total"]},
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_baseline_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
