"""Host logic of bench.py (no GPU): the kernel-span report splits a
rocprofv3 kernel trace at the flush kernels and takes per-op medians."""
import csv
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _trace(path, events):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, (name, b, e) in enumerate(events):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Start_Timestamp": b, "End_Timestamp": e})


def test_span_report_segments_and_medians(tmp_path):
    b = _bench()
    fl = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, x>"
    ev = [(fl, 0, 100), ("setup", 200, 300),                      # skip segment
          (fl, 1000, 1100), ("rmsn::fwd_kernel", 2000, 5000),     # fwd 3.0 us
          (fl, 6000, 6100), ("rmsn::fwd_kernel", 7000, 11000),    # fwd 4.0 us
          (fl, 12000, 12100), ("rmsn::fwd_kernel", 13000, 18000),  # fwd 5.0 us
          (fl, 20000, 20100), ("rmsn::bwd_kernel", 21000, 29000),  # bwd span 8.0 + reduce
          ("rmsn::dw_reduce_kernel", 30000, 33000),               # -> 12.0 us, 2 kernels
          (fl, 40000, 40100), ("next shape setup", 41000, 42000)]
    _trace(tmp_path / "t.csv", ev)
    labels = ["skip", "H8 T1|fwd", "H8 T1|fwd", "H8 T1|fwd", "H8 T1|bwd_det", "skip"]
    (tmp_path / "seq.json").write_text(json.dumps(labels))
    rep = b.span_report(str(tmp_path / "t.csv"), str(tmp_path / "seq.json"))
    assert rep["H8 T1"]["fwd"] == {"median_us": 4.0, "n": 3, "kernels": 1}
    assert rep["H8 T1"]["bwd_det"] == {"median_us": 12.0, "n": 1, "kernels": 2}


def test_span_report_rejects_mismatched_labels(tmp_path):
    import pytest
    b = _bench()
    fl = "FillFunctor<float>"
    _trace(tmp_path / "t.csv", [(fl, 0, 1), ("k", 2, 3)])
    (tmp_path / "seq.json").write_text(json.dumps(["skip", "H8 T1|fwd"]))
    with pytest.raises(SystemExit):
        b.span_report(str(tmp_path / "t.csv"), str(tmp_path / "seq.json"))


def test_sweep_shapes_cover_the_pages_tables():
    b = _bench()
    names = {b.shape_name(*s) for s in b.SWEEP_SHAPES}
    assert len(names) == len(b.SWEEP_SHAPES) == 115
    assert {"H4096 T65536", "H6144 T1 res w32", "H5120 T321", "H512 T256"} <= names
    assert set(b.shape_name(*s) for s in b.SMALL_T_SHAPES) <= names


def test_profile_report_scales_counters_and_averages_the_last_run(tmp_path):
    b = _bench()
    W, K = 1, 2
    fwd = "void rmsn::fwd_kernel<768, 1, 4, false, true, false>(rmsn::FwdParams)"
    bwd = "void rmsn::bwd_kernel<256, 3, 1, false, false, false>(rmsn::BwdParams)"
    red = "rmsn::dw_reduce_kernel(double const*, int, int, float*)"
    copy = "__amd_rocclr_copyBuffer"
    # W + 2K steps of (fwd, fwd, bwd, reduce); the last K steps are slower
    events, t = [], 0
    for step in range(W + 2 * K):
        d = 1200 if step >= W + K else 1000
        for name, dur in ((fwd, d), (fwd, d), (bwd, 700), (red, 5)):
            events.append((name, t, t + dur * 1000))
            t += dur * 1000 + 100
    (tmp_path / "ktrace").mkdir()
    _trace(tmp_path / "ktrace" / "run_kernel_trace.csv", events)
    with open(tmp_path / "ktrace" / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        for name in (fwd, bwd, red):
            ds = [e - s for n, s, e in events if n == name]
            w.writerow({"Name": name, "Calls": len(ds), "AverageNs": sum(ds) / len(ds), "MinNs": min(ds),
                        "MaxNs": max(ds)})
    for kind, copy_val, per in (("fetch", 524288.0, {fwd: 1000.0, bwd: 500.0, red: 1.0}),
                                ("write", 1048576.0, {fwd: 2000.0, bwd: 250.0, red: 0.5})):
        (tmp_path / kind).mkdir()
        with open(tmp_path / kind / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Value"])
            w.writeheader()
            i = 0
            for _ in range(3):
                i += 1
                w.writerow({"Dispatch_Id": i, "Kernel_Name": copy, "Counter_Value": copy_val})
            for name, v in per.items():
                i += 1
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Value": v})
    line = {"roofline": {"us_per_launch_mean": 1200.0}, "roofline_bwd": {"us_per_call_mean": 705.0}}
    (tmp_path / "ktrace.log").write_text("[bench] x\n" + json.dumps(line) + "\n")
    md = b.profile_report(str(tmp_path), "T131072_H6144_res", K, W)
    rec = json.loads(md.split("```json\n")[1].split("\n```")[0])
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert rec["kernels"]["fwd_kernel"]["traffic_bytes"] == (1000 * 2 + 2000) * 1024
    assert rec["trace_last_run_avg_us"]["fwd_kernel"] == 1200.0
    nb = b.fwd_bytes(131072, 6144, 2, True)
    assert f"| fwd | {nb:,} |" in md and f"1200.00 ({nb / 1200e-6 / 8e12:.4f})" in md
    assert "python3 R/bench.py --profile-report OUT T131072_H6144_res 2 1" in md


def test_profile_hash_follows_code_not_comments():
    # a profile summary stays valid across comment and layout edits of the
    # sources, and goes stale on any change to the code itself (string and
    # character literals that hold comment markers are code)
    import bench
    a = 'int f(int x) { // sum\n  return x + 1; /* one */ }\nconst char* s = "a // b";\n'
    b = '/* header */\nint f(int x) {\n    return x + 1;   // one\n}\nconst char* s = "a // b";'
    c = 'int f(int x) { return x + 2; }\nconst char* s = "a // b";'
    d = 'int f(int x) { return x + 1; }\nconst char* s = "a // c";'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert bench.code_text(a) != bench.code_text(d)
    assert bench.code_text("char q = '\\''; // x") == "char q = '\\'';"
    assert len(bench.source_hash("bwd_kernel")) == 16
