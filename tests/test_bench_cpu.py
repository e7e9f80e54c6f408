"""bench.py's profile summarizers on the CPU: a fabricated rocprofv3 kernel
trace and counter runs, split into phases by the run's dispatch layout."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _result(layout, per_kernel, dom, extra=None):
    d = {"metric": "m", "value": 5000.0, "pct_of_peak": 62.5, "steps": 2,
         "ms_per_step": 0.1, "config": {"workload": "w", "launch": "eager"},
         "per_kernel": per_kernel, "kernel_source_hash": "x",
         "roofline": {"kernel": dom, "avg_us": 51.0, "achieved": 1.0,
                      "frac": 0.5},
         "profile_layout": layout}
    d.update(extra or {})
    return json.dumps(d)


def _write_csv(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


import pytest


@pytest.mark.parametrize("timing", ["first_launch", "calls"])
def test_trace_summary_uses_the_timed_region_only(tmp_path, timing):
    # setup: 2 dispatches, then per step: "a" (kivi::ka) and "b" (kivi::kb,
    # two launches), 2 timed steps, then 2 armed steps; torch kernels mixed
    # in are ignored
    names = {"a": "void kivi::ka<0>(int)", "b": "void kivi::kb<1>(int)"}
    seq = ["a", "b", "b"] * 2
    disp = ([("a", 500)] * 2 + [(k, 40) for k in seq]
            + [(k, 50 if k == "a" else 10) for k in seq]
            + [(k, 70) for k in seq])
    rows, t, i = [], 1000, 0
    for k, dur in disp:
        i += 1
        rows.append({"Dispatch_Id": i, "Kernel_Name": names[k],
                     "Start_Timestamp": t, "End_Timestamp": t + dur * 1000})
        t += dur * 1000 + 10
        i += 1
        rows.append({"Dispatch_Id": i, "Kernel_Name": "at::fill<float>()",
                     "Start_Timestamp": t, "End_Timestamp": t + 5})
        t += 20
    _write_csv(str(tmp_path / "trace" / "x" / "bench_kernel_trace.csv"), rows,
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                "End_Timestamp"])
    layout = {"dispatches_before_timed": 8, "timed_dispatches": 6,
              "step_launches": ["a", "b", "b#2"], "per_kernel_timing": timing}
    pk = {"a": {"avg_us": 51.0, "algorithmic_bytes": 400000},
          "b": {"avg_us": 10.0, "algorithmic_bytes": 1000}}
    for f in ("plain.json", "profiled.json"):
        (tmp_path / f).write_text("noise\n" + _result(layout, pk, "a") + "\n")
    out = subprocess.run(
        [sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-trace",
         str(tmp_path), "--workload", "roundtrip"],
        capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    text = out.stdout
    # timed "a" dispatches last 50 us: 400000 B / 50 us = 8 GB/s
    assert "400000 algorithmic bytes / 50.00 us" in text, text
    assert "frac 0.0010" in text
    lines = [ln for ln in text.splitlines() if ln.startswith("b#2 ")]
    assert lines and " 10.00 " in lines[0]
    if timing == "calls":    # the call "b" is its two launches
        lines = [ln for ln in text.splitlines() if ln.startswith("b ")]
        assert any(" 20.00 " in ln for ln in lines), text


def _counter_csv(path, disp, counter):
    """A rocprofv3 counter_collection.csv: disp = [(kernel name, KiB)], each
    dispatch split over two rows (two counter instances) as the tool does."""
    rows, t = [], 1000
    for i, (name, kib) in enumerate(disp, 1):
        for half in (0.25, 0.75):
            rows.append({"Dispatch_Id": i, "Kernel_Name": name,
                         "Counter_Name": counter, "Counter_Value": kib * half,
                         "Start_Timestamp": t, "End_Timestamp": t + 500})
        t += 1000
    _write_csv(path, rows, ["Dispatch_Id", "Kernel_Name", "Counter_Name",
                            "Counter_Value", "Start_Timestamp",
                            "End_Timestamp"])


@pytest.mark.parametrize("timing", ["first_launch", "calls"])
def test_traffic_summary_per_launch_or_per_call(tmp_path, timing):
    # per step: "r" three times (a label that recurs, as a ring store per
    # decode token does) and "c" with two launches (c, c#2); one setup
    # dispatch before the two timed steps, one armed step after
    names = {"r": "void kivi::kr<0>(int)", "c": "void kivi::kc<1>(int)",
             "c#2": "void kivi::kc2(int)"}
    step = ["r", "r", "r", "c", "c#2"]
    kib = {"r": 10.0, "c": 100.0, "c#2": 20.0}
    disp = ([(names["c"], 9999.0)]
            + [(names[k], kib[k]) for k in step * 2]
            + [(names[k], 7777.0) for k in step])
    disp.insert(3, ("void at::fill<float>(int)", 5555.0))   # not the library's
    for sub, counter in (("pmc_fetch", "FETCH_SIZE"),
                         ("pmc_write", "WRITE_SIZE")):
        _counter_csv(str(tmp_path / "run" / sub / "x" /
                         "bench_counter_collection.csv"), disp, counter)
    layout = {"dispatches_before_timed": 1, "timed_dispatches": 10,
              "step_launches": ["r", "r", "r", "c", "c#2"],
              "per_kernel_timing": timing}
    pk = {"r": {"avg_us": 1.0, "algorithmic_bytes": 20480},
          "c": {"avg_us": 9.0, "algorithmic_bytes": 245760}}
    for f in ("fetch.json", "write.json"):
        (tmp_path / "run" / f).write_text(_result(layout, pk, "c") + "\n")
    # the copy: 1 MiB per launch; FETCH_SIZE reads half of it, WRITE_SIZE all
    for sub, k in (("fetch", 512.0), ("write", 1024.0)):
        _counter_csv(str(tmp_path / "copy" / sub / "x" /
                         "copy_counter_collection.csv"),
                     [("__amd_rocclr_copyBuffer", k)] * 3, "X")
        (tmp_path / "copy" / (sub + ".json")).write_text(
            json.dumps({"calibration": {}, "size_bytes": 1 << 20}) + "\n")
    rec = tmp_path / "traffic.json"
    out = subprocess.run(
        [sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-traffic",
         str(tmp_path / "run"), "--copy-dir", str(tmp_path / "copy"),
         "--workload", "cache-decode", "--traffic-json", str(rec)],
        capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    data = json.loads(rec.read_text())
    r = data["r@cache-decode"]
    # every "r" launch: 10 KiB fetched (x2 by the copy's scale), 10 written
    assert (r["fetch_bytes"], r["write_bytes"]) == (20480, 10240), out.stdout
    c = data["c@cache-decode"]
    if timing == "calls":       # the call: both launches summed
        assert (c["fetch_bytes"], c["write_bytes"]) == (245760, 122880)
    else:                       # the first launch only; c#2 has no bytes
        assert (c["fetch_bytes"], c["write_bytes"]) == (204800, 102400)


def test_dispatch_order_is_submission_order():
    # back-to-back kernels of one stream whose profiler start timestamps
    # land out of order (the second one stamped 100 ns before the first)
    # stay in dispatch order; other namespaces are ignored
    sys.path.insert(0, ROOT)
    import bench
    rows = [
        {"Dispatch_Id": "7", "Kernel_Name": "void kivi::chunk<0>(int)",
         "Start_Timestamp": "1000", "End_Timestamp": "2000"},
        {"Dispatch_Id": "8", "Kernel_Name": "at::fill<float>()",
         "Start_Timestamp": "2010", "End_Timestamp": "2020"},
        {"Dispatch_Id": "9", "Kernel_Name": "void kivi::merge<0>(int)",
         "Start_Timestamp": "2100", "End_Timestamp": "2500"},
        {"Dispatch_Id": "10", "Kernel_Name": "void kivi::chunk<0>(int)",
         "Start_Timestamp": "2000", "End_Timestamp": "3000"},
    ]
    got = bench._library_dispatches(rows)
    assert [g[0] for g in got] == ["void kivi::chunk<0>(int)",
                                   "void kivi::merge<0>(int)",
                                   "void kivi::chunk<0>(int)"]
    assert [g[1] for g in got] == [1000, 2100, 2000]
