"""Per-point kernel times from a rocprofv3 kernel trace of ``bench.py --points-out``,
or (``--sequence``) of the bench's own timed region.

    rocprofv3 --kernel-trace --output-format csv -d OUT -o t -- \\
        python3 bench.py --no-cpu --points-out points.json
    python -m latency_decode_gemm_amd.trace_points OUT/.../t_kernel_trace.csv points.json \\
        [plain.json]

``bench.py --points-out`` runs, for each workload point in turn, one K = 0
call (the zero-fill kernel, a marker), ``trace_warm`` warm-up calls and
``trace_calls`` timed calls, each of ``dispatches_per_call`` dispatches (two
for the two-pass split-K backend).  The library's dispatches are taken in
time order; the ones after the i-th marker belong to the i-th point.  A
call's kernel time is the sum of its dispatches' durations; the table gives
the median over the timed calls, the weight bandwidth (weight bytes: 2NK,
or 4NK over fp32 weights) / time and the
fraction of 8 TB/s, beside the bench's own figures for the point (the
library GEMM's graph time for the same product among them), taken from
``plain.json`` when given: the output of the same command run without the
profiler, whose event, eager and graph timings the tracing does not inflate.

    rocprofv3 --kernel-trace --output-format csv -d OUT -o t -- python3 bench.py > line.json
    python -m latency_decode_gemm_amd.trace_points --sequence OUT/.../t_kernel_trace.csv line.json

splits the timed region of a plain bench run (the calls after the two
marker calls that precede it, in step order) by point: each point's kernel
time inside the sequence, beside its back-to-back time from the same line.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys

PEAK_GBS = 8000.0
MARKER = "skg_zero_fill_kernel"


def load_trace(path):
    if os.path.isdir(path):
        path = glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)[0]
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if "skg::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows


def split_points(rows, points):
    """{point name: list of per-call kernel ns over the timed calls}."""
    order = sorted(points.items(), key=lambda kv: kv[1]["trace_order"])
    marks = [i for i, r in enumerate(rows) if MARKER in r["Kernel_Name"]]
    if len(marks) < len(order):
        raise ValueError(f"{len(marks)} markers for {len(order)} points")
    marks = marks[-len(order):]  # the report's markers are the last ones
    out = {}
    for (name, e), m in zip(order, marks):
        d = e["dispatches_per_call"]
        n = e["trace_warm"] + e["trace_calls"]
        seg = rows[m + 1:m + 1 + n * d]
        if len(seg) < n * d or any(MARKER in r["Kernel_Name"] for r in seg):
            raise ValueError(f"trace segment of {name} is incomplete")
        per_call = []
        for c in range(e["trace_warm"], n):
            per_call.append(sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                                for r in seg[c * d:(c + 1) * d]))
        out[name] = {"ns": per_call, "kernels": sorted({r["Kernel_Name"] for r in seg})}
    return out


def table(trace_path, points_path, plain_path=None):
    with open(points_path) as f:
        points = json.load(f)
    per = split_points(load_trace(trace_path), points)
    if plain_path:
        with open(plain_path) as f:
            plain = json.load(f)
        points = {k: dict(v, **{f: plain[k][f] for f in plain[k] if f not in (
            "trace_order", "trace_warm", "trace_calls", "dispatches_per_call")})
                  for k, v in points.items()}
    lines = ["| point | config (backend, inner, split, tiles, wn, wk, depth, rb/wg) | "
             "kernel µs (rocprof median) | µs events median | µs/call graph | µs/call hot | "
             "read ceiling µs | weight GB/s | of 8 TB/s | CPU µs all cores / 1 core | "
             "library GEMM µs/call graph | speed-up vs library |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, e in sorted(points.items(), key=lambda kv: kv[1]["trace_order"]):
        us = statistics.median(per[name]["ns"]) / 1000.0
        gbs = e["weight_bytes"] / us / 1e3
        c = e["config"]
        cfg = ",".join(str(c[k]) for k in ("backend", "inner", "split_k", "row_tiles", "waves_n",
                                           "waves_k", "depth", "rb_per_wg"))
        cpu = e.get("cpu_all_cores", {}).get("us_per_call"), e.get("cpu_one_core", {}).get(
            "us_per_call")
        lines.append(f"| {name} | {cfg} | {us:.2f} | {e['kernel_us_events_median']:.2f} | "
                     f"{e['us_per_call_graph']:.2f} | {e['us_per_call_hot_graph']:.2f} | "
                     f"{e['read_ceiling_us_eager']:.2f} | {gbs:.0f} | {gbs / PEAK_GBS:.3f} | "
                     f"{cpu[0]} / {cpu[1]} | {e.get('us_per_call_library_graph', '-')} | "
                     f"{e.get('speedup_vs_library_graph', '-')} |")
    return "\n".join(lines)


def split_sequence(rows, names, dispatches, steps):
    """{point name: per-call kernel ns} for the timed region of ``bench.py``:
    the ``steps`` x len(names) calls after the last pair of consecutive
    markers, the points in step order."""
    pairs = [i for i in range(len(rows) - 1)
             if MARKER in rows[i]["Kernel_Name"] and MARKER in rows[i + 1]["Kernel_Name"]]
    if not pairs:
        raise ValueError("no marker pair before the timed region")
    i = pairs[-1] + 2
    out = {n: [] for n in names}
    for _ in range(steps):
        for n in names:
            seg = rows[i:i + dispatches[n]]
            if len(seg) < dispatches[n] or any(MARKER in r["Kernel_Name"] for r in seg):
                raise ValueError("timed region of the trace is incomplete")
            out[n].append(sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in seg))
            i += dispatches[n]
    return out


def sequence_table(trace_path, line_path):
    """Per point of the bench step: kernel time inside the sequence (the
    timed region of the traced run) beside the same kernel back to back
    (``gated_points_kernel_us`` of the bench line, where present)."""
    with open(line_path) as f:
        line = json.loads([ln for ln in f.read().splitlines() if ln.strip().startswith("{")][-1])
    names = [n.strip() for n in line["config"]["workload"].split(":", 1)[1].split(",")]
    per = split_sequence(load_trace(trace_path), names, line["dispatches_per_call"],
                         line["steps"])
    alone = line.get("gated_points_kernel_us") or {}
    lines = ["| point (in step order) | kernel µs in sequence (median) | mean | p90 | "
             "back to back (events, median) | in sequence − back to back |",
             "|---|---|---|---|---|---|"]
    for n in names:
        ns = sorted(per[n])
        med = statistics.median(ns) / 1000.0
        mean = statistics.mean(ns) / 1000.0
        p90 = ns[min(len(ns) - 1, int(0.9 * len(ns)))] / 1000.0
        a = alone.get(n, {}).get("kernel_us")
        lines.append(f"| {n} | {med:.2f} | {mean:.2f} | {p90:.2f} | "
                     f"{'-' if a is None else f'{a:.2f}'} | "
                     f"{'-' if a is None else f'{med - a:+.2f}'} |")
    return "\n".join(lines)


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) == 3 and argv[0] == "--sequence":
        print(sequence_table(argv[1], argv[2]))
        return 0
    if len(argv) not in (2, 3):
        print(__doc__, file=sys.stderr)
        return 2
    print(table(*argv))
    return 0


if __name__ == "__main__":
    sys.exit(main())
