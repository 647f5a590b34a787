"""The per-point trace splitter (host logic, no GPU): markers, two-dispatch
calls, warm-up calls skipped, incomplete traces rejected."""
import csv
import json

import pytest

from latency_decode_gemm_amd import trace_points


def _write(tmp_path, rows, points):
    tr = tmp_path / "t_kernel_trace.csv"
    with open(tr, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)
    pj = tmp_path / "points.json"
    pj.write_text(json.dumps(points))
    return str(tr), str(pj)


def _pt(order, d, warm=1, calls=3):
    return {"trace_order": order, "trace_warm": warm, "trace_calls": calls,
            "dispatches_per_call": d, "config": {k: 0 for k in (
                "backend", "inner", "split_k", "row_tiles", "waves_n", "waves_k", "depth",
                "rb_per_wg")},
            "kernel_us_events_median": 1.0, "us_per_call_graph": 1.0,
            "us_per_call_hot_graph": 1.0, "read_ceiling_us_eager": 1.0, "weight_bytes": 4000}


def test_split_and_median(tmp_path):
    t = [0]

    def k(name, dur):
        r = {"Kernel_Name": f"void skg::(anonymous namespace)::{name}(skg::KParams)",
             "Start_Timestamp": t[0], "End_Timestamp": t[0] + dur}
        t[0] += dur + 10
        return r
    rows = [k("skg_valu_kernel<1, 1, 4, true>", 999)]  # before any marker: ignored
    rows += [k("skg_zero_fill_kernel", 5)]
    rows += [k("skg_valu_kernel<1, 1, 4, true>", d) for d in (900, 100, 300, 200)]
    rows += [k("skg_zero_fill_kernel", 5)]
    for d in (700, 800, 1000, 50, 2000, 60, 3000, 70):  # pairs: main + reduce
        rows.append(k("skg_mfma_kernel<2, 1, 4>" if d >= 700 else "skg_splitk_reduce_kernel", d))
    rows.append({"Kernel_Name": "__amd_rocclr_copyBuffer", "Start_Timestamp": 1,
                 "End_Timestamp": 2})
    tr, pj = _write(tmp_path, rows, {"a": _pt(0, 1), "b": _pt(1, 2)})
    per = trace_points.split_points(trace_points.load_trace(tr), json.load(open(pj)))
    assert per["a"]["ns"] == [100, 300, 200]          # warm-up call (900) skipped
    assert per["b"]["ns"] == [1050, 2060, 3070]       # main + reduce per call
    text = trace_points.table(tr, pj)
    assert "| a |" in text and "| 0.20 |" in text and "| 2.06 |" in text


def test_incomplete_trace_rejected(tmp_path):
    rows = [{"Kernel_Name": "void skg::(anonymous namespace)::skg_zero_fill_kernel(void*)",
             "Start_Timestamp": 0, "End_Timestamp": 1},
            {"Kernel_Name": "void skg::(anonymous namespace)::skg_valu_kernel<1,1,4,true>(x)",
             "Start_Timestamp": 5, "End_Timestamp": 9}]
    tr, pj = _write(tmp_path, rows, {"a": _pt(0, 1)})
    with pytest.raises(ValueError):
        trace_points.split_points(trace_points.load_trace(tr), json.load(open(pj)))
    tr, pj = _write(tmp_path, rows[1:], {"a": _pt(0, 1)})
    with pytest.raises(ValueError):
        trace_points.split_points(trace_points.load_trace(tr), json.load(open(pj)))


def test_sequence_split_takes_the_timed_region_after_the_marker_pair(tmp_path):
    """The bench's timed region follows the last pair of marker calls; its
    calls are attributed to the points in step order (a two-dispatch call
    counts both), and dispatches before the pair are ignored."""
    rows, t = [], 0

    def add(name, dur):
        nonlocal t
        rows.append({"Kernel_Name": f"skg::{name}", "Start_Timestamp": t,
                     "End_Timestamp": t + dur})
        t += dur + 10

    add("a", 999)  # warm-up noise
    add(trace_points.MARKER, 5)  # a lone marker is not the pair
    add("b", 999)
    add(trace_points.MARKER, 5)
    add(trace_points.MARKER, 5)
    for step in range(3):
        add("p0", 1000 + step)
        add("p1", 2000)
        add("p1b", 500)  # second dispatch of p1
    add("after", 999)  # later work (not in the timed region)
    tr = tmp_path / "t_kernel_trace.csv"
    with open(tr, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)
    per = trace_points.split_sequence(trace_points.load_trace(str(tr)), ["P0", "P1"],
                                      {"P0": 1, "P1": 2}, 3)
    assert per == {"P0": [1000, 1001, 1002], "P1": [2500, 2500, 2500]}
    line = tmp_path / "line.json"
    line.write_text(json.dumps({"config": {"workload": "w: P0, P1"}, "steps": 3,
                                "dispatches_per_call": {"P0": 1, "P1": 2},
                                "gated_points_kernel_us": {"P1": {"kernel_us": 2.0}}}))
    out = trace_points.sequence_table(str(tr), str(line))
    assert "| P0 | 1.00 |" in out and "| P1 | 2.50 |" in out and "+0.50" in out
    with pytest.raises(ValueError):
        trace_points.split_sequence(trace_points.load_trace(str(tr)), ["P0", "P1"],
                                    {"P0": 1, "P1": 2}, 4)
