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
