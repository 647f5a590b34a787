#!/usr/bin/env python3
"""Benchmark of the MI355X skinny GEMM (C = A . B^T, bf16, M <= 16).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--points-out FILE]

One step = one call of the GEMM for every (M, K, N) point of the workload, in
order, each on its own synthetic inputs already resident in HBM.  The weight
matrix of every call is one of several byte-identical copies at different
addresses, cycled so that the bytes touched between two uses of a copy exceed
the 256 MB Infinity Cache: every call reads its weights from HBM.

Prints ONE JSON line:
  value        = sum over the step's calls of the weight bytes 2*N*K, divided
                 by the measured time per step (GB/s, whole GPU);
  roofline     = the dominant kernel (the point with the largest time in the
                 step): algorithmic bytes per launch (2NK + 2MK + M*N*s_out)
                 divided by its average kernel duration, from HIP events that
                 its dispatches record (skinny_gemm_bf16_timed) on every step
                 of the timed region;
  cpu_baseline = the CPU oracle timed on this host over the same workload;
  gated_points_kernel_us = after the timed region, the median kernel time
                 of every point with N*K >= 7168*2112 (qkv_a-style, wide,
                 deep; the points the bandwidth target covers) and its
                 fraction of the 8 TB/s peak.
``--workload router_f32w`` measures the router GEMM over fp32 weights
(skinny_gemm_f32w; weight bytes 4*N*K) the same way, ``--workload mid_m`` the
middle tier (16 < M <= 64) on the projection shapes.
``--points-out FILE`` also writes, for every one of the 29 workload points,
the 12 fp32-weight router points and the 24 middle-tier points, the library
GEMM's time for the same
product (torch.nn.functional.linear: hipBLASLt), and
the kernel time per call (median of 200 dispatch-recorded event pairs), the
time per call eager, from HIP-graph replay and with one hot weight copy, the
streaming-read ceiling for the same weight bytes, and the CPU oracle on all
host cores and on one core (the CPU-baseline leg per point).  A K = 0 call
(the zero-fill kernel) precedes each point's dispatches, so that a rocprofv3
kernel trace of the run can be split by point:
``python -m latency_decode_gemm_amd.trace_points TRACE.csv FILE``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (weight read) and µs/call, bf16 skinny GEMM, M=1..16"
METRIC_F32W = ("achieved HBM GB/s (weight read) and µs/call, router GEMM over fp32 weights "
               "(bf16 activations), M=1..16")
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
ROTATE_BYTES = 1 << 30  # footprint between two uses of one weight copy
DEFAULT_WORKLOAD = "wide_deep"
GRAPH_STEPS = 4  # steps per captured graph (each weight copy recurs every 4 steps)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# what the counters depend on: the kernels' code (the configuration they were
# taken with is stored beside them and compared separately)
KERNEL_SOURCES = ["skg_device.h", "skg_internal.h", "skg_launch.hip", "skg_valu_lo.hip",
                  "skg_valu_hi.hip", "skg_valu_ga.hip", "skg_f32w_lo.hip", "skg_f32w_hi.hip",
                  "skg_f32w_ga.hip", "skg_mfma_mid.h", "skg_mfma_mt2.hip", "skg_mfma_mt3.hip",
                  "skg_mfma_mt4.hip", "skg_mfma_sync.hip", "skg_api.cpp"]
F32W_SUFFIX = "_w32"  # point names of the fp32-weight router GEMM


def code_tokens(text: str) -> str:
    """C++ source without its comments and with each run of whitespace made
    one space (string and character literals kept as written), so that
    editing a comment does not count as changing a kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored): the
    HBM counters in profiles/traffic.json hold for the code they were taken
    with."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "latency_decode_gemm_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--points-out", default=None,
                    help="write per-point us/call for all 29 points to this JSON file")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default=None,
                    help="profile helper: run only the point 'M,K,N' (no JSON checks)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a HIP graph (GRAPH_STEPS steps "
                         "captured with rotating weight copies): ms_per_step_graph")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the per-point report of the points the bandwidth target "
                         "covers (N*K >= 7168*2112), timed after the headline region")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="host only: from the counter collections of two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, then WRITE_SIZE) of `--only M,K,N --copy-probe-mb MB`, "
                         "write that point's HBM bytes per launch to profiles/traffic.json")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after the timed region, copy a buffer of this many MiB once "
                         "(a plain copy kernel of known size, for scaling HBM counters)")
    return ap.parse_args()


class Point:
    """Device buffers of one workload point (A, rotating B copies, C); a point
    with ``w == "f32"`` runs the fp32-weight entry points."""

    def __init__(self, torch, skg, inputs, p, b_pool):
        self.M, self.K, self.N = p["M"], p["K"], p["N"]
        self.f32w = p.get("w") == "f32"
        wsz = 4 if self.f32w else 2
        self.out = p["out"]
        self.ldc = p["ldc"] or self.N
        self.A_bits = inputs.make_a(self.M, self.K, self.N)
        self.A = torch.from_numpy(self.A_bits.view("int16")).cuda().view(torch.bfloat16)
        self.copies = b_pool[(self.K, self.N, self.f32w)]
        dt = torch.bfloat16 if self.out == "bf16" else torch.float32
        self.Cbuf = torch.zeros((self.M, self.ldc), dtype=dt, device="cuda")
        self.odt = skg.SKG_OUT_BF16 if self.out == "bf16" else skg.SKG_OUT_F32
        dispatch = skg.skinny_gemm_f32w_dispatch if self.f32w else skg.skinny_gemm_dispatch
        self.cfg = dispatch(self.M, self.K, self.N)
        self.s_out = 2 if self.out == "bf16" else 4
        self.weight_bytes = wsz * self.N * self.K
        self.alg_bytes = self.weight_bytes + 2 * self.M * self.K + self.M * self.N * self.s_out

    def key(self):
        return (self.K, self.N, self.f32w)

    def name(self):
        return f"M{self.M}_K{self.K}_N{self.N}_{self.out}" + (
            f"_ldc{self.ldc}" if self.ldc != self.N else "") + (F32W_SUFFIX if self.f32w else "")


class BPool:
    """Per (K, N, fp32 weights?): the seeded weights (bf16 bits, or float32)
    and byte-identical copies of them on the device."""

    def __init__(self, torch, inputs, shapes, rotate_bytes=ROTATE_BYTES):
        self.torch = torch
        self.bits = {}
        self.copies = {}
        for (K, N, f32w) in shapes:
            if f32w:
                bits = inputs.make_w_f32(K, N)
                base = torch.from_numpy(bits).cuda()
            else:
                bits = inputs.make_b(K, N)
                base = torch.from_numpy(bits.view("int16")).cuda().view(torch.bfloat16)
            self.bits[(K, N, f32w)] = bits
            n = max(2, math.ceil(rotate_bytes / (base.element_size() * N * K)))
            lst = [base] + [base.clone() for _ in range(n - 1)]
            self.copies[(K, N, f32w)] = {"list": lst, "next": 0}

    def __getitem__(self, key):
        return self.copies[key]


def call(lib, pt, B, stream_handle, events=None):
    if events is None:
        fn = lib.skinny_gemm_f32w if pt.f32w else lib.skinny_gemm_bf16
        st = fn(pt.A.data_ptr(), B.data_ptr(), pt.Cbuf.data_ptr(), pt.M, pt.N, pt.K, pt.K, pt.K,
                pt.ldc, pt.odt, stream_handle)
    else:
        fn = lib.skinny_gemm_f32w_timed if pt.f32w else lib.skinny_gemm_bf16_timed
        st = fn(pt.A.data_ptr(), B.data_ptr(), pt.Cbuf.data_ptr(), pt.M, pt.N, pt.K, pt.K, pt.K,
                pt.ldc, pt.odt, stream_handle, events[0].handle, events[1].handle)
    if st != 0:
        raise RuntimeError(f"skinny_gemm call failed for {pt.name()}: status {st}")


def next_copy(pt):
    c = pt.copies
    B = c["list"][c["next"]]
    c["next"] = (c["next"] + 1) % len(c["list"])
    return B


def check_parity(pt, bits_B, torch):
    """Sampled outputs (all M rows, up to 64 columns) against a plain float64
    product of the decoded inputs."""
    from latency_decode_gemm_amd import spot_check
    return spot_check.sampled_check(torch, pt.A_bits, bits_B, pt.Cbuf, pt.K, pt.out)


def time_points_graph(torch, lib, pts, stream, calls=200, warm=20):
    """us per call of each point: back-to-back calls replayed from a HIP graph
    (rotating weight copies), so host launch cost is excluded."""
    res = {}
    h = stream.cuda_stream
    for pt in pts:
        for _ in range(warm):
            call(lib, pt, next_copy(pt), h)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        n = min(calls, 4 * len(pt.copies["list"])) if pt.weight_bytes > (64 << 20) else calls
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                call(lib, pt, next_copy(pt), stream.cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / n
        res[pt.name()] = us
        del g
    return res


def time_library_graph(torch, pts, stream, calls=200, warm=20):
    """us per call of the library GEMM a caller would otherwise use for the
    same product (torch.nn.functional.linear, i.e. hipBLASLt: bf16 in, bf16
    out; over fp32 weights, the fp32 GEMM of the widened activations), timed
    like time_points_graph: back-to-back calls over the rotating weight
    copies, replayed from a HIP graph."""
    F = torch.nn.functional
    res = {}
    for pt in pts:
        A = pt.A.float() if pt.f32w else pt.A
        with torch.cuda.stream(stream):
            for _ in range(warm):
                F.linear(A, next_copy(pt))
        torch.cuda.synchronize()
        n = min(calls, 4 * len(pt.copies["list"])) if pt.weight_bytes > (64 << 20) else calls
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                F.linear(A, next_copy(pt))
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        res[pt.name()] = e0.elapsed_time(e1) * 1000.0 / n
        del g
    return res


def time_points_eager(torch, lib, pts, stream, calls=200, warm=20):
    res = {}
    h = stream.cuda_stream
    for pt in pts:
        for _ in range(warm):
            call(lib, pt, next_copy(pt), h)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record()
            for _ in range(calls):
                call(lib, pt, next_copy(pt), h)
            e1.record()
        torch.cuda.synchronize()
        res[pt.name()] = e0.elapsed_time(e1) * 1000.0 / calls
    return res


GATED_NK = 7168 * 2112  # the bandwidth target applies to N * K at least this


def gated_points_report(torch, skg, lib, inputs, stream, bpool, pts, calls=100, warm=10):
    """Every workload point with N * K >= 7168 * 2112 (qkv_a-style, wide and
    deep, M <= 16): median kernel time over `calls` dispatches that record
    their own start and end (skinny_gemm_bf16_timed), weights rotated past
    the Infinity Cache as in the timed region, and the weight bytes 2NK per
    second as a fraction of the 8 TB/s peak.  Run after the timed region, so
    it does not change ms_per_step."""
    h = stream.cuda_stream
    spec = [p for p in inputs.all_points() if p["N"] * p["K"] >= GATED_NK]
    have = {pt.name(): pt for pt in pts}
    shapes = [(K, N, False) for (K, N) in dict.fromkeys((p["K"], p["N"]) for p in spec)
              if (K, N, False) not in bpool.copies]
    extra = BPool(torch, inputs, shapes) if shapes else None
    out = {}
    ev = [(skg.HipEvent(), skg.HipEvent()) for _ in range(calls)]
    for p in spec:
        key = (p["K"], p["N"], False)
        pool = bpool if key in bpool.copies else extra
        pt = Point(torch, skg, inputs, p, pool)
        pt = have.get(pt.name(), pt)
        skg.skinny_gemm_warmup([(pt.K, pt.N)], [pt.M], stream=stream)
        for _ in range(warm):
            call(lib, pt, next_copy(pt), h)
        for i in range(calls):
            call(lib, pt, next_copy(pt), h, ev[i])
        torch.cuda.synchronize()
        us = median([a.elapsed_ms(b) * 1000.0 for a, b in ev])
        gbs = pt.weight_bytes / us / 1e3
        out[pt.name()] = {"kernel_us": round(us, 3), "weight_GBps": round(gbs, 1),
                          "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4)}
    del extra
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(oracle, pts, bpool, budget_s):
    """The oracle over the whole workload (every output), repeated until the
    time budget is used; rate = weight bytes per second."""
    threads = oracle.default_threads()
    passes, t_total, bytes_total = 0, 0.0, 0
    while passes == 0 or t_total < budget_s:
        for pt in pts:
            t0 = time.perf_counter()
            oracle_gemm(oracle, pt)(pt.A_bits, bpool.bits[pt.key()], pt.K, threads=threads)
            t_total += time.perf_counter() - t0
            bytes_total += pt.weight_bytes
        passes += 1
    return {"value": round(bytes_total / t_total / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole workload ({len(pts)} calls, every output), {passes} pass(es), "
                      f"{t_total:.1f} s; binary64 C loop, OpenMP over columns; "
                      f"{threads} threads of {os.cpu_count()} logical CPUs, {cpu_model()}"}


def oracle_gemm(oracle, pt):
    return oracle.gemm_f32w if pt.f32w else oracle.gemm_f64


def oracle_mod():
    import oracle
    return oracle


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def points_report(torch, np, skg, lib, inputs, oracle, stream, calls=200, warm=20):
    """Every workload point: kernel time per call from the dispatches' own
    events (median of `calls`), HIP-graph and eager time per call, the same
    with one hot weight copy, the streaming-read ceiling for the weight size,
    and the CPU oracle on all host cores and on one core (median of 3 after a
    warm-up).  Each point's timed dispatches follow one K = 0 call (the
    zero-fill kernel) that marks them in a kernel trace, so a rocprofv3
    kernel trace of this run can be attributed to points by order."""
    h = stream.cuda_stream
    spec = (inputs.all_points() + inputs.WORKLOADS_F32W["router_f32w"] +
            inputs.WORKLOADS_MID["mid_m"] + inputs.WORKLOADS_MID["mid_router"])

    def key_of(p):
        return (p["K"], p["N"], p.get("w") == "f32")

    shapes = list(dict.fromkeys(key_of(p) for p in spec))
    table = {}
    cpu_jobs = []  # (point, oracle function, A bits, B bits, K), timed at the end
    order = 0
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    for (K, N, f32w) in shapes:
        sub = [p for p in spec if key_of(p) == (K, N, f32w)]
        bp = BPool(torch, inputs, [(K, N, f32w)])
        ps = [Point(torch, skg, inputs, p, bp) for p in sub]
        warm_fn = skg.skinny_gemm_f32w_warmup if f32w else skg.skinny_gemm_warmup
        warm_fn([(K, N)], [p.M for p in ps], stream=stream)
        ev = [(skg.HipEvent(), skg.HipEvent()) for _ in range(calls)]
        for pt in ps:
            st = lib.skinny_gemm_bf16(pt.A.data_ptr(), pt.A.data_ptr(), pt.Cbuf.data_ptr(), pt.M,
                                      pt.N, 0, 8, 8, pt.ldc, pt.odt, h)  # trace marker (K = 0)
            if st != 0:
                raise RuntimeError(f"marker call failed: status {st}")
            for _ in range(warm):
                call(lib, pt, next_copy(pt), h)
            for i in range(calls):
                call(lib, pt, next_copy(pt), h, ev[i])
            torch.cuda.synchronize()
            ev_us = [a.elapsed_ms(b) * 1000.0 for a, b in ev]
            table[pt.name()] = {
                "M": pt.M, "K": pt.K, "N": pt.N, "out": pt.out, "ldc": pt.ldc,
                "config": pt.cfg.as_dict(), "trace_order": order, "trace_warm": warm,
                "trace_calls": calls,
                "weights": "f32" if pt.f32w else "bf16",
                "dispatches_per_call": 2 if pt.cfg.backend == skg.SKG_BACKEND_SPLITK_2PASS else 1,
                "kernel_us_events_median": round(median(ev_us), 3),
                "weight_bytes": pt.weight_bytes, "alg_bytes": pt.alg_bytes}
            order += 1
        eager = time_points_eager(torch, lib, ps, stream)
        graph = time_points_graph(torch, lib, ps, stream)
        libgemm = time_library_graph(torch, ps, stream)
        # streaming-read ceiling over the same rotating weight copies
        lst = bp[(K, N, f32w)]["list"]
        nb = lst[0].element_size() * N * K
        for i in range(4):
            lib.skinny_gemm_stream_read(lst[i % len(lst)].data_ptr(), nb, sink.data_ptr(), h)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record()
            for i in range(calls):
                lib.skinny_gemm_stream_read(lst[i % len(lst)].data_ptr(), nb, sink.data_ptr(), h)
            e1.record()
        torch.cuda.synchronize()
        read_us = e0.elapsed_time(e1) * 1000.0 / calls
        hot = BPool(torch, inputs, [(K, N, f32w)], rotate_bytes=0)
        for p in ps:
            p.copies = hot[(K, N, f32w)]
            p.copies["list"] = p.copies["list"][:1]
        hot_us = time_points_graph(torch, lib, ps, stream)
        for pt in ps:
            e = table[pt.name()]
            e.update({"us_per_call_eager": round(eager[pt.name()], 3),
                      "us_per_call_graph": round(graph[pt.name()], 3),
                      "us_per_call_library_graph": round(libgemm[pt.name()], 3),
                      "speedup_vs_library_graph": round(libgemm[pt.name()] / graph[pt.name()], 3),
                      "us_per_call_hot_graph": round(hot_us[pt.name()], 3),
                      "read_ceiling_us_eager": round(read_us, 3)})
            k_us = e["kernel_us_events_median"]
            e["weight_GBps_kernel_events"] = round(pt.weight_bytes / k_us / 1e3, 1)
            e["frac_of_8TBps_kernel_events"] = round(pt.weight_bytes / k_us / 1e3 / PEAK_HBM_GBS, 4)
            cpu_jobs.append((pt.name(), oracle_gemm(oracle, pt), pt.A_bits, bp.bits[(K, N, f32w)],
                             K))
        del ps, bp, hot
        torch.cuda.empty_cache()
        print(f"points: K={K} N={N} done", file=sys.stderr, flush=True)
    # CPU oracle per point, after all GPU work (host threads of the GPU
    # runtime no longer compete with the oracle's), the thread pool warmed
    # once first; per point one warm-up call, then the median of 3
    torch.cuda.synchronize()
    if cpu_jobs:
        name, fn, a_bits, b_bits, K = cpu_jobs[0]
        fn(a_bits, b_bits, K, threads=oracle.default_threads())
    for name, fn, a_bits, b_bits, K in cpu_jobs:
        e = table[name]
        for threads, key in ((oracle.default_threads(), "cpu_all_cores"), (1, "cpu_one_core")):
            ts = []
            for rep in range(4):
                t0 = time.perf_counter()
                fn(a_bits, b_bits, K, threads=threads)
                ts.append(time.perf_counter() - t0)
            e[key] = {"us_per_call": round(median(ts[1:]) * 1e6, 1), "threads": threads}
    return table


def load_traffic(dominant_name, config):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = t.get("points", {}).get(dominant_name)
    if not entry or entry.get("config") != config:
        return None
    return entry.get("hbm_bytes_per_launch")


def counter_per_dispatch(path, counter):
    """{dispatch id: [kernel name, counter summed over its instances]} from a
    rocprofv3 counter-collection CSV."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = per.setdefault(r["Dispatch_Id"], [r["Kernel_Name"], 0.0])
            d[1] += float(r["Counter_Value"])
    return per


def write_traffic(args):
    """HBM bytes per launch of the --only point's kernel: the median FETCH_SIZE
    and WRITE_SIZE (KiB) over its dispatches, each scaled by known bytes over
    what the same counter reads for the copy probe of the same run (the largest
    runtime copy: args.copy_probe_mb MiB read and written)."""
    from statistics import median

    import latency_decode_gemm_amd as skg
    from latency_decode_gemm_amd import inputs
    if not args.only or not args.copy_probe_mb:
        sys.exit("bench.py: --write-traffic needs --only M,K,N and --copy-probe-mb")
    M, K, N = (int(x) for x in args.only.split(","))
    p = [q for q in inputs.all_points() if (q["M"], q["K"], q["N"]) == (M, K, N)][0]
    cfg = skg.skinny_gemm_dispatch(M, K, N)
    probe = args.copy_probe_mb << 20
    out = {}
    for path, counter in zip(args.write_traffic, ("FETCH_SIZE", "WRITE_SIZE")):
        per = counter_per_dispatch(path, counter)
        copies = [v for k, v in per.values() if "copyBuffer" in k]
        # the GEMM kernels are the templates (skg_valu_kernel<...>, skg_mfma_...<...>);
        # the zero-fill marker and the scratch clear are not
        gemm = [(k, v) for k, v in per.values() if "skg_" in k and "_kernel<" in k]
        names = {k for k, _ in gemm}
        if not copies or len(names) != 1:
            sys.exit(f"bench.py: {path}: expected one GEMM kernel and the copy probe, "
                     f"found {sorted(names)} and {len(copies)} copies")
        kib = median(v for _, v in gemm)
        scale = probe / (max(copies) * 1024)
        out[counter] = (names.pop(), kib, scale, len(gemm))
    kernel = out["FETCH_SIZE"][0]
    s_out = 2 if p["out"] == "bf16" else 4
    alg = 2 * N * K + 2 * M * K + M * N * s_out
    fb = round(out["FETCH_SIZE"][1] * 1024 * out["FETCH_SIZE"][2])
    wb = round(out["WRITE_SIZE"][1] * 1024 * out["WRITE_SIZE"][2])
    name = f"M{M}_K{K}_N{N}_{p['out']}" + (f"_ldc{p['ldc']}" if p["ldc"] and p["ldc"] != N else "")
    rec = {
        "about": "HBM bytes per launch of the dominant bench kernel from rocprofv3 --pmc "
                 "FETCH_SIZE and WRITE_SIZE (separate runs), each scaled by the same counter on "
                 f"a {args.copy_probe_mb} MiB device copy in the same run; written by "
                 "bench.py --write-traffic",
        "kernel_source_hash": kernel_source_hash(),
        "fetch_scale": round(out["FETCH_SIZE"][2], 5),
        "write_scale": round(out["WRITE_SIZE"][2], 5),
        "points": {name: {
            "kernel": kernel.replace("void skg::(anonymous namespace)::", "").split("(")[0],
            "config": cfg.as_dict(),
            "dispatches": out["FETCH_SIZE"][3],
            "fetch_kib_raw": out["FETCH_SIZE"][1],
            "write_kib_raw": out["WRITE_SIZE"][1],
            "fetch_bytes": fb,
            "write_bytes": wb,
            "hbm_bytes_per_launch": fb + wb,
            "algorithmic_bytes": alg,
            "traffic_over_algorithmic": round((fb + wb) / alg, 3),
        }},
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["points"][name]))


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py: the GEMM runs on one GPU (asked for --gpus {args.gpus}); sharding "
              "it across GPUs (by rows of the weights, or by K with one all-reduce) is not "
              "implemented.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import latency_decode_gemm_amd as skg
    from latency_decode_gemm_amd import _capi, inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    lib = _capi.lib()
    if not skg.skinny_gemm_available():
        print("bench.py: libskinny_gemm.so has no gfx950 device/code to run", file=sys.stderr)
        sys.exit(1)

    groups = dict(inputs.WORKLOADS, **inputs.WORKLOADS_F32W, **inputs.WORKLOADS_MID,
                  **inputs.WORKLOADS_CHAIN)
    workload = groups[args.workload]
    if args.only:
        M, K, N = (int(x) for x in args.only.split(","))
        workload = [p for p in inputs.all_points() if (p["M"], p["K"], p["N"]) == (M, K, N)]
    shapes = list(dict.fromkeys((p["K"], p["N"], p.get("w") == "f32") for p in workload))
    bpool = BPool(torch, inputs, shapes)
    pts = [Point(torch, skg, inputs, p, bpool) for p in workload]
    # all work on one non-default stream (graph capture needs one)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    h = stream.cuda_stream
    for (K, N, f32w) in shapes:
        ms = sorted(set(p.M for p in pts if p.key() == (K, N, f32w)))
        warm_fn = skg.skinny_gemm_f32w_warmup if f32w else skg.skinny_gemm_warmup
        warm_fn([(K, N)], ms, stream=stream)

    # untimed warm-up steps; also find the dominant point (largest time per call)
    for _ in range(max(args.warmup, 1)):
        for pt in pts:
            call(lib, pt, next_copy(pt), h)
    torch.cuda.synchronize()
    probe = time_points_eager(torch, lib, pts, stream, calls=20, warm=2)
    dom = max(pts, key=lambda p: probe[p.name()])

    # two K = 0 calls (the zero-fill kernel) mark the start of the timed
    # region in a kernel trace (trace_points --sequence); they run before t0
    for _ in range(2):
        st = lib.skinny_gemm_bf16(pts[0].A.data_ptr(), pts[0].A.data_ptr(),
                                  pts[0].Cbuf.data_ptr(), pts[0].M, pts[0].N, 0, 8, 8,
                                  pts[0].ldc, pts[0].odt, h)
        if st != 0:
            raise RuntimeError(f"marker call failed: status {st}")

    # timed region: K steps; the dominant point's kernel records its own start
    # and end in HIP events (skinny_gemm_bf16_timed) on every step
    n_dom = args.steps
    ev_s = [skg.HipEvent() for _ in range(n_dom)]
    ev_e = [skg.HipEvent() for _ in range(n_dom)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for s in range(args.steps):
        for pt in pts:
            B = next_copy(pt)
            if pt is dom:
                call(lib, pt, B, h, (ev_s[s], ev_e[s]))
            else:
                call(lib, pt, B, h)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t0.elapsed_time(t1)
    ms_per_step = ms_total / args.steps
    weight_bytes_step = sum(p.weight_bytes for p in pts)
    value = weight_bytes_step / (ms_per_step * 1e-3) / 1e9
    dom_us = float(np.mean([a.elapsed_ms(b) for a, b in zip(ev_s, ev_e)])) * 1000.0
    achieved = dom.alg_bytes / (dom_us * 1e-6) / 1e9

    graph_ms = None
    if args.graph:
        # the same step captured (GRAPH_STEPS steps, rotating copies) and
        # replayed: no host launch work between the kernels of the chain
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(GRAPH_STEPS):
                for pt in pts:
                    call(lib, pt, next_copy(pt), h)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // GRAPH_STEPS)
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (reps * GRAPH_STEPS)
        del g

    # results are still right after the timed loop (sampled float64 check)
    bad = []
    if not args.only:
        for pt in pts:
            r = check_parity(pt, bpool.bits[pt.key()], torch)
            if not r["ok"]:
                bad.append((pt.name(), r))
    if bad:
        print(f"bench.py: results do not match the float64 check: {bad}", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe_mb:
        nbytes = args.copy_probe_mb << 20
        src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    gated = None
    if not args.no_gated and not args.only and not any(p.f32w for p in pts):
        gated = gated_points_report(torch, skg, lib, inputs, stream, bpool, pts)

    traffic = load_traffic(dom.name(), dom.cfg.as_dict())
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic,
                "kernel": dom.name(), "launch_us": round(dom_us, 3),
                "alg_bytes_per_launch": dom.alg_bytes,
                "config": dom.cfg.as_dict()}
    per_point = {p.name(): round(probe[p.name()], 3) for p in pts}
    cpu = None
    if not args.no_cpu and not args.only:
        import oracle
        cpu = cpu_baseline(oracle, pts, bpool, args.cpu_seconds)
    line = {
        "metric": METRIC_F32W if any(p.f32w for p in pts) else METRIC,
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if any(p.f32w for p in pts) else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload + ": " + ", ".join(p.name() for p in pts),
                   "accumulate": "f32", "weight_bytes_per_step": weight_bytes_step,
                   "parallelism": "single GPU", "weight_copies_rotated": True,
                   "host_wall_s": round(wall, 3)},
        "us_per_call_eager": per_point,
        "dispatches_per_call": {p.name(): 2 if p.cfg.backend == skg.SKG_BACKEND_SPLITK_2PASS
                                else 1 for p in pts},
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 5),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if gated is not None:
        line["gated_points_kernel_us"] = gated
        line["gated_points_min_frac"] = min(v["frac_of_8TBps"] for v in gated.values())
    if args.points_out:
        del pts, bpool
        torch.cuda.empty_cache()
        table = points_report(torch, np, skg, lib, inputs, oracle_mod(), stream)
        with open(args.points_out, "w") as f:
            json.dump(table, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
