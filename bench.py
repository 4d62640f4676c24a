"""Benchmark of the MI355X training RMSNorm on one GPU.

Workload (default): T=65536 rows of H=4096 BF16 values, FP32 weight
w = 1 + 0.1 N(0,1), x and dy ~ N(0,1), eps = 1e-6, plain rows -- the shape the
pages' headline comparison is quoted on.  A step is the pages' checkpointed
training step "2xfwd+bwd" (forward, forward recompute, backward; p2
"Key": op 2xfwd+bwd), here with the deterministic backward.

Printed: ONE JSON line.  `value` is the step's effective HBM throughput
(algorithmic bytes of fwd + fwd + bwd over the measured step time, back to
back with inputs resident in HBM).  Beside it the line carries, per op and
mode, latency with L2 and the 256 MB last-level cache flushed before every
launch (the pages' protocol: cold L2, median of many launches), the
per-kernel roofline of the dominant kernel from HIP events, and the CPU
oracle timed on the host as a baseline.

Algorithmic bytes (what the operation must move; workspace traffic excluded):
  fwd = 4 R H (+4 R H with a residual) + 4 R + sw H
  bwd = 6 R H (+2 R H with dres) + 4 R + sw H + 4 H,  sw = 2 (BF16 w) or 4 (FP32 w)
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E
EPS = 1e-6

WORKLOADS = {
    # name: (T, heads, H, stride_t, stride_h, w dtype, residual)
    "T65536_H4096_w32": (65536, 1, 4096, 4096, 4096, "f32", False),
    "T4096_H1536": (4096, 1, 1536, 1536, 1536, "bf16", False),
    "T131072_H6144_res": (131072, 1, 6144, 6144, 6144, "bf16", True),
    "T131072_H6144_res_w32": (131072, 1, 6144, 6144, 6144, "f32", True),
    "T32768_24x256_s8192": (32768, 24, 256, 8192, 256, "bf16", False),
    "T32768_4x256": (32768, 4, 256, 1024, 256, "bf16", False),
    "T65536_H5120": (65536, 1, 5120, 5120, 5120, "bf16", False),
    "T65536_H5120_w32": (65536, 1, 5120, 5120, 5120, "f32", False),
    "T32768_H5120": (32768, 1, 5120, 5120, 5120, "bf16", False),
    "T19968_H5120": (19968, 1, 5120, 5120, 5120, "bf16", False),
    "T6144_H5120": (6144, 1, 5120, 5120, 5120, "bf16", False),
    "T2048_H5120": (2048, 1, 5120, 5120, 5120, "bf16", False),
    # the SiLU-gated variant (y = RMSNorm(x) * w * silu(g)) at the headline shape
    "T65536_H4096_w32_gate": (65536, 1, 4096, 4096, 4096, "f32", "gate"),
    "T65536_H6144_gate": (65536, 1, 6144, 6144, 6144, "bf16", "gate"),
}
DEFAULT_WORKLOAD = "T65536_H4096_w32"


def fwd_bytes(R, H, sw, res, gate=False):
    return (8 if res else 6 if gate else 4) * R * H + 4 * R + sw * H


def bwd_bytes(R, H, sw, dres, gate=False):
    return (8 if dres else 10 if gate else 6) * R * H + 4 * R + sw * H + 4 * H


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def percentile(v, q):
    return float(np.percentile(np.asarray(v), q))


class Workload:
    def __init__(self, name, seed=0):
        import torch

        import rmsnorm_fwd_amd as rn
        import synth

        self.name = name
        T, heads, H, st, sh, wdt, res = WORKLOADS[name]
        self.gate = res == "gate"
        res = res is True
        self.T, self.heads, self.H, self.st, self.sh, self.wdt, self.res = T, heads, H, st, sh, wdt, res
        self.R = T * heads
        self.sw = 4 if wdt == "f32" else 2
        dev = "cuda"
        t0 = time.time()
        self.x_h = synth.rows(seed, "x", 0, self.R, H)
        self.dy_h = synth.rows(seed, "dy", 0, self.R, H)
        self.r_h = synth.rows(seed, "r", 0, self.R, H) if res else None
        self.w_h = synth.weight(seed, H, wdt)
        log(f"generated inputs in {time.time() - t0:.1f}s")

        def place(rows):
            n = (T - 1) * st + (heads - 1) * sh + H
            buf = torch.zeros(n, dtype=torch.bfloat16, device=dev)
            v = self.view(buf)
            v.copy_(torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).to(dev).view(v.shape))
            return buf

        self.view = lambda buf: (torch.as_strided(buf, (T, H), (st, 1)) if heads == 1 else
                                 torch.as_strided(buf, (T, heads, H), (st, sh, 1)))
        self.x = self.view(place(self.x_h))
        self.dy = self.view(place(self.dy_h))
        self.r = self.view(place(self.r_h)) if res else None
        # the incoming gradient of h for the residual backward's second form
        # (dres ~ N(0,1)); the step itself takes dres = NULL
        self.dres = self.view(place(synth.rows(seed, "dres", 0, self.R, H))) if res else None
        self.g_h = synth.rows(seed, "g", 0, self.R, H) if self.gate else None
        self.g = self.view(place(self.g_h)) if self.gate else None
        self.dg = self.view(place(self.x_h)) if self.gate else None
        self.w = (torch.from_numpy(self.w_h).to(dev) if wdt == "f32" else
                  torch.from_numpy(self.w_h.view(np.int16)).view(torch.bfloat16).to(dev))
        self.y = self.view(place(self.x_h))
        self.h = self.view(place(self.x_h)) if res else None
        self.dx = self.view(place(self.x_h))
        self.rstd = torch.empty(self.R, dtype=torch.float32, device=dev)
        self.dw = torch.empty(H, dtype=torch.float32, device=dev)
        self.ws = rn.rmsnorm_bwd_workspace(T, heads, H, dev)
        self.fwd_bytes = fwd_bytes(self.R, H, self.sw, res, self.gate)
        self.bwd_bytes = bwd_bytes(self.R, H, self.sw, False, self.gate)
        self.step_bytes = 2 * self.fwd_bytes + self.bwd_bytes
        self.rn = rn

    def fwd(self):
        if self.gate:
            self.rn.rmsnorm_gated_fwd(self.x, self.g, self.w, EPS, y=self.y, rstd=self.rstd)
            return
        self.rn.rmsnorm_fwd(self.x, self.w, EPS, residual=self.r, y=self.y, residual_out=self.h,
                            rstd=self.rstd)

    def bwd(self, det=True, dres=None):
        if self.gate:
            self.rn.rmsnorm_gated_bwd(self.dy, self.x, self.g, self.rstd, self.w, deterministic=det, dx=self.dx,
                                      dg=self.dg, dw=self.dw, workspace=self.ws)
            return
        u = self.h if self.res else self.x
        self.rn.rmsnorm_bwd(self.dy, u, self.rstd, self.w, residual=dres, deterministic=det, dx=self.dx,
                            dw=self.dw, workspace=self.ws)

    def step(self, det=True):
        self.fwd()
        self.fwd()
        self.bwd(det)


def time_cold(ops, rounds, reps, flush_buf):
    """Cache-flushed launch times (us) of every op in `ops` (name -> fn).

    Before each launch L2 and the last-level cache are flushed by a 1 GiB
    write on the same stream, outside the events.  The ops are interleaved
    launch by launch, in an order rotated every round, so that drift of the
    machine hits all of them alike.  Returns name -> list of `rounds` lists."""
    import torch

    names = list(ops)
    out = {n: [[] for _ in range(rounds)] for n in names}
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    for rd in range(rounds):
        order = names[rd % len(names):] + names[:rd % len(names)]
        for _ in range(reps):
            for n in order:
                flush_buf.fill_(1)
                a.record()
                ops[n]()
                b.record()
                b.synchronize()
                out[n][rd].append(a.elapsed_time(b) * 1e3)
    return out


def summarize(rounds_us):
    ts = [t for r in rounds_us for t in r]
    return {"median_us": round(statistics.median(ts), 2), "p10_us": round(percentile(ts, 10), 2),
            "p90_us": round(percentile(ts, 90), 2), "launches": len(ts),
            "round_medians_us": [round(statistics.median(r), 2) for r in rounds_us]}


def time_warm(fn, reps):
    """Average microseconds per launch of fn, launches back to back, bracketed
    by HIP events on the library's stream."""
    import torch

    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl: Workload, min_seconds=10.0, max_seconds=30.0):
    """The oracle (FP64, OpenMP) on the host: fwd + fwd + bwd over a bounded
    sample of the workload's rows, as GB/s of the same byte model.  The
    sample is the whole workload when one step takes under ~10 s, else the
    leading rows; the step repeats until about 10 s of work is done.  The
    forward and backward are also timed on their own (medians)."""
    import oracle

    nthreads = oracle.num_threads()
    probe_rows = min(wl.R, 2048)
    t0 = time.time()
    _step_oracle(wl, probe_rows)
    per_row = (time.time() - t0) / probe_rows
    rows = int(min(wl.R, max(probe_rows, 10.0 / max(per_row, 1e-9))))
    steps, fwds, bwds = [], [], []
    t_start = time.time()
    while (time.time() - t_start) < min_seconds or len(steps) < 3:
        tf1, tf2, tb = _step_oracle(wl, rows)
        steps.append(tf1 + tf2 + tb)
        fwds += [tf1, tf2]
        bwds.append(tb)
        if time.time() - t_start > max_seconds:
            break
    sec = statistics.median(steps)
    sample_bytes = 2 * fwd_bytes(rows, wl.H, wl.sw, wl.res, wl.gate) + bwd_bytes(rows, wl.H, wl.sw, False, wl.gate)
    return {"value": sample_bytes / sec / 1e9, "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"2xfwd+bwd over rows 0..{rows - 1} of {wl.R} (H={wl.H}), median of {len(steps)} "
                      f"repeats, {sec:.2f} s per step, {time.time() - t_start:.1f} s in all",
            "step_seconds": sec, "fwd_seconds": statistics.median(fwds), "bwd_seconds": statistics.median(bwds),
            "rows": rows, "cpu_model": cpu_model()}


def profiled_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 summary
    for this workload, or None if there is none or the kernel's sources have
    changed since it was taken."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"rmsnorm_kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get("kernels", {}).get(kernel)
    if not rec:
        return None
    srcs = {"fwd_kernel": ["fwd.hip", "device_common.h", "kernels.h", "layouts.h"],
            "bwd_kernel": ["bwd.hip", "device_common.h", "kernels.h", "layouts.h"]}[kernel]
    h = hashlib.sha256()
    for f in srcs:
        with open(os.path.join(ROOT, "rmsnorm_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return rec["traffic_bytes"] if h.hexdigest()[:16] == rec["source_hash"] else None


# The pages' latency tables (p1 #8577, per-shape fwd/bwd/step rows) cover
# T = 1..64 at H = 2048, 4096 (BF16 and FP32 w), 5120 and 6144 (plain, FP32
# w, residual, residual with FP32 w).  (H, T, w dtype, residual):
SMALL_T_SHAPES = (
    [(H, T, w, False) for H in (2048, 4096) for T in (1, 4, 16, 64) for w in ("bf16", "f32")]
    + [(5120, T, "bf16", False) for T in (1, 4, 16, 64)]
    + [(6144, T, w, r) for T in (1, 4, 16, 64) for w in ("bf16", "f32") for r in (False, True)])

# The whole shape list of those tables (bench.py --shape-sweep).
SWEEP_SHAPES = (
    [(H, T, "bf16", False) for H in (512, 1536) for T in (256, 1024, 4096, 14928, 16384, 32768, 65536)]
    + [(H, T, w, False) for H in (2048, 4096) for T in (1, 4, 16, 64) for w in ("bf16", "f32")]
    + [(H, T, "bf16", False) for H in (2048, 4096) for T in (256, 1024, 4096, 14928, 16384, 32768, 65536)]
    + [(5120, T, "bf16", False) for T in (1, 4, 16, 64, 321, 512, 896)]
    + [(5120, T, w, False) for T in (256, 1024, 4096, 14928, 16384, 32768, 65536) for w in ("bf16", "f32")]
    + [(6144, T, w, r) for T in (1, 4, 16, 64, 256, 1024, 4096, 14928, 16384, 32768, 65536)
       for w in ("bf16", "f32") for r in (False, True)]
    + [(6144, T, w, False) for T in (449, 768, 1152) for w in ("bf16", "f32")])


def shape_name(H, T, wdt, res):
    return f"H{H} T{T}" + (" res" if res else "") + (" w32" if wdt == "f32" else "")


class DeviceCase:
    """Inputs of one (H, T, w dtype, residual) shape drawn on the device from
    a seeded torch generator (latency does not depend on the values), x, r,
    dy ~ N(0,1), w = 1 + 0.1 N(0,1)."""

    def __init__(self, H, T, wdt, res, seed=0):
        import torch

        import rmsnorm_fwd_amd as rn

        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        bf = torch.bfloat16
        self.rn, self.res = rn, res
        self.x = torch.randn(T, H, generator=g, device="cuda").to(bf)
        self.r = torch.randn(T, H, generator=g, device="cuda").to(bf) if res else None
        self.dy = torch.randn(T, H, generator=g, device="cuda").to(bf)
        w = 1 + 0.1 * torch.randn(H, generator=g, device="cuda")
        self.w = w if wdt == "f32" else w.to(bf)
        self.y = torch.empty_like(self.x)
        self.h = torch.empty_like(self.x) if res else None
        self.dx = torch.empty_like(self.x)
        self.rstd = torch.empty(T, dtype=torch.float32, device="cuda")
        self.dw = torch.empty(H, dtype=torch.float32, device="cuda")
        self.ws = rn.rmsnorm_bwd_workspace(T, 1, H, "cuda")

    def fwd(self):
        self.rn.rmsnorm_fwd(self.x, self.w, EPS, residual=self.r, y=self.y, residual_out=self.h,
                            rstd=self.rstd)

    def bwd(self, det=True):
        self.rn.rmsnorm_bwd(self.dy, self.h if self.res else self.x, self.rstd, self.w, deterministic=det,
                            dx=self.dx, dw=self.dw, workspace=self.ws)

    def step(self):
        self.fwd()
        self.fwd()
        self.bwd(True)


def graphed(fn):
    """fn captured once in a HIP graph (after an eager warm-up on the capture
    stream); returns the replay function.  The library's calls allocate
    nothing and never synchronise, so the whole op can be captured."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g.replay


def shape_latencies(shapes, flush_buf, rounds, reps):
    """Cache-flushed median latency (us) of fwd, bwd (both modes) and the
    deterministic 2xfwd+bwd step for each shape -- the backward and the step
    also as one HIP-graph replay each (the pages time graph replays) -- plus
    the floor: the same timing around a one-element torch fill."""
    import torch

    tiny = torch.empty(1, dtype=torch.float32, device="cuda")
    floor = time_cold({"fill": lambda: tiny.fill_(0)}, rounds, reps, flush_buf)["fill"]
    rows = []
    for H, T, wdt, res in shapes:
        c = DeviceCase(H, T, wdt, res)
        ops = {"fwd": c.fwd, "bwd_det": lambda: c.bwd(True), "bwd_nondet": lambda: c.bwd(False),
               "step_det": c.step}
        for fn in ops.values():
            fn()
        ops["bwd_det_graph"] = graphed(lambda: c.bwd(True))
        ops["step_det_graph"] = graphed(c.step)
        raw = time_cold(ops, rounds, reps, flush_buf)
        row = {"shape": shape_name(H, T, wdt, res)}
        for k, v in raw.items():
            row[k + "_us"] = round(statistics.median([t for r in v for t in r]), 2)
        rows.append(row)
        del c
    return {"floor_us": round(statistics.median([t for r in floor for t in r]), 2),
            "launches_per_op": rounds * reps, "rows": rows}


# ---- kernel spans (the pages' latency: first kernel start to last kernel
# end of one op after a cache flush, from the GPU's own timestamps) --------
#
# `--span-sweep SEQ` runs, for every shape, `reps` x [flush, op] per op and
# writes the list of segment labels to SEQ; run it under
#   rocprofv3 --kernel-trace --output-format csv -d OUT -o run -- python3 bench.py --span-sweep SEQ
# and `--span-report TRACE SEQ` turns OUT/.../run_kernel_trace.csv into
# per-shape medians.  Every segment starts with the flush (the only float
# fill kernel); setup and warm-up kernels sit in segments labelled "skip".

FLUSH_KERNEL = "FillFunctor<float>"


def span_sweep(shapes, reps, seq_path):
    import torch

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    labels = []

    def mark(label):
        flush.fill_(1)
        labels.append(label)

    mark("skip")
    for H, T, wdt, res in shapes:
        c = DeviceCase(H, T, wdt, res)
        ops = {"fwd": c.fwd, "bwd_det": lambda: c.bwd(True), "bwd_nondet": lambda: c.bwd(False),
               "step_det": c.step}
        for fn in ops.values():
            fn()
        for name, fn in ops.items():
            for _ in range(reps):
                mark(f"{shape_name(H, T, wdt, res)}|{name}")
                fn()
        mark("skip")
        torch.cuda.synchronize()
        del c
    with open(seq_path, "w") as f:
        json.dump(labels, f)
    return len(labels)


def span_report(trace_csv, seq_path):
    """Median kernel span (us) per shape and op from a rocprofv3 kernel trace."""
    import csv

    labels = json.load(open(seq_path))
    rows = list(csv.DictReader(open(trace_csv)))
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else "Start_Timestamp"
    rows.sort(key=lambda r: int(r[key]))
    segs = []
    for r in rows:
        if FLUSH_KERNEL in r["Kernel_Name"]:
            segs.append([])
        elif segs:
            segs[-1].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    if len(segs) != len(labels):
        raise SystemExit(f"{len(segs)} flush-delimited segments in the trace, {len(labels)} labels")
    spans, kernels = {}, {}
    for lab, seg in zip(labels, segs):
        if lab == "skip":
            continue
        if not seg:
            raise SystemExit(f"segment {lab} has no kernels")
        spans.setdefault(lab, []).append((max(e for _, e, _ in seg) - min(b for b, _, _ in seg)) / 1e3)
        kernels[lab] = len(seg)
    out = {}
    for lab, v in spans.items():
        shape, op = lab.split("|")
        out.setdefault(shape, {})[op] = {"median_us": round(statistics.median(v), 2), "n": len(v),
                                         "kernels": kernels[lab]}
    return out


def _step_oracle(wl, rows):
    """One oracle step over the leading `rows` rows; seconds of its three ops."""
    import oracle

    x = _rows_view(wl.x_h, rows)
    r = _rows_view(wl.r_h, rows) if wl.res else None
    dy = _rows_view(wl.dy_h, rows)
    if wl.gate:
        g = _rows_view(wl.g_h, rows)
        t0 = time.perf_counter()
        oracle.gated_fwd_bf16(x, g, wl.w_h, EPS)
        t1 = time.perf_counter()
        _, rstd = oracle.gated_fwd_bf16(x, g, wl.w_h, EPS)
        t2 = time.perf_counter()
        oracle.gated_bwd_bf16(x, g, dy, wl.w_h, rstd.astype(np.float32))
        t3 = time.perf_counter()
        return t1 - t0, t2 - t1, t3 - t2
    t0 = time.perf_counter()
    oracle.fwd_bf16(x, wl.w_h, EPS, r)
    t1 = time.perf_counter()
    y, h, rstd = oracle.fwd_bf16(x, wl.w_h, EPS, r)
    t2 = time.perf_counter()
    oracle.bwd_bf16(h if wl.res else x, dy, wl.w_h, rstd.astype(np.float32))
    t3 = time.perf_counter()
    return t1 - t0, t2 - t1, t3 - t2


def _rows_view(a, rows):
    return a[:rows] if a is not None else None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--cold-reps", type=int, default=210,
                    help="cache-flushed launches per op, split over --cold-rounds interleaved rounds")
    ap.add_argument("--cold-rounds", type=int, default=3)
    ap.add_argument("--no-small-t", action="store_true", help="skip the small-T latency sweep")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="also time every shape of the pages' latency tables (a few minutes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only warmup + timed steps (for rocprofv3 runs), no per-op extras")
    ap.add_argument("--span-sweep", metavar="SEQ",
                    help="run the pages' shapes as flush-delimited ops for a rocprofv3 kernel trace; "
                         "write the segment labels to SEQ and exit")
    ap.add_argument("--span-report", nargs=2, metavar=("TRACE_CSV", "SEQ"),
                    help="print per-shape median kernel spans from a --span-sweep trace and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counter scaling)")
    args = ap.parse_args()

    if args.span_report:
        rep = span_report(*args.span_report)
        print(json.dumps({"kernel_spans_us": rep}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows split across GPUs with no exchange; dw would need one all-reduce of H values). "
              "Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    import rmsnorm_fwd_amd as rn

    rn.lib()  # fail loudly if the HIP library is not built
    if args.span_sweep:
        n = span_sweep(SWEEP_SHAPES, 20, args.span_sweep)
        torch.cuda.synchronize()
        log(f"span sweep: {n} flush-delimited segments, labels in {args.span_sweep}")
        return
    if args.copy_calibration:
        # the first three device-to-device copies of the process: 1 GiB each
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x copy of 1 GiB done")
    wl = Workload(args.workload)
    log(f"workload {wl.name}: R={wl.R} H={wl.H} w={wl.wdt} res={wl.res}")

    # warmup + timed steps (deterministic backward), back to back
    for _ in range(args.warmup):
        wl.step(True)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        wl.step(True)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = wl.step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, {value:.0f} GB/s (wall {wall:.3f}s)")

    out = {
        "metric": "RMSNorm fwd/bwd/2xfwd+bwd \u00b5s and effective HBM GB/s (% of peak) at [T,H]",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic the kernels compute in: FP32 products, FP64 row and
        # column sums; activations are stored as BF16
        "dtype": "f32",
        "storage_dtype": "bf16",
        "accumulation": "f64 row sums and dw column sums",
        "data": "synthetic (seeded N(0,1) x and dy, w = 1 + 0.1 N(0,1))",
        "config": {"workload": wl.name, "T": wl.T, "heads": wl.heads, "H": wl.H, "w_dtype": wl.wdt,
                   "residual": wl.res, "silu_gate": wl.gate,
                   "step": "fwd + fwd (recompute) + bwd (deterministic)",
                   "step_bytes": wl.step_bytes, "pct_of_peak": round(100 * value / PEAK_GBS, 2)},
    }

    if not args.profile:
        # per-op latency, cold caches; "fwd_aa" is the forward again, timed as
        # if it were another implementation (the A/A floor of the method)
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        ops = {
            "fwd": (wl.fwd, wl.fwd_bytes),
            "fwd_aa": (wl.fwd, wl.fwd_bytes),
            "bwd_det": (lambda: wl.bwd(True), wl.bwd_bytes),
            "bwd_nondet": (lambda: wl.bwd(False), wl.bwd_bytes),
            **({"bwd_det_dres": (lambda: wl.bwd(True, wl.dres), bwd_bytes(wl.R, wl.H, wl.sw, True))}
               if wl.res else {}),
            "step_det": (lambda: wl.step(True), wl.step_bytes),
            "step_nondet": (lambda: wl.step(False), wl.step_bytes),
        }
        ops["step_det_graph"] = (graphed(lambda: wl.step(True)), wl.step_bytes)
        for fn, _ in ops.values():
            for _ in range(3):
                fn()
        reps = max(1, -(-args.cold_reps // args.cold_rounds))
        raw = time_cold({k: v[0] for k, v in ops.items()}, args.cold_rounds, reps, flush)
        lat = {}
        for name, (_, nbytes) in ops.items():
            c = summarize(raw[name])
            c["gbs"] = round(nbytes / (c["median_us"] * 1e-6) / 1e9, 1)
            c["pct_peak"] = round(100 * c["gbs"] / PEAK_GBS, 2)
            c["bytes"] = nbytes
            lat[name] = c
            log(f"cold {name}: {c['median_us']:.1f} us  {c['gbs']:.0f} GB/s ({c['pct_peak']:.1f}%)")
        lat["aa_floor_pct"] = round(100 * abs(lat["fwd"]["median_us"] - lat["fwd_aa"]["median_us"])
                                    / lat["fwd"]["median_us"], 3)
        # deterministic over non-deterministic backward time (> 1: non-det faster)
        lat["mode_ratio_bwd"] = round(lat["bwd_det"]["median_us"] / lat["bwd_nondet"]["median_us"], 4)
        out["latency_cold"] = lat

        if not args.no_small_t:
            t0 = time.time()
            out["small_t"] = shape_latencies(SMALL_T_SHAPES, flush, args.cold_rounds, 20)
            log(f"small-T latencies: {len(SMALL_T_SHAPES)} shapes in {time.time() - t0:.1f}s")
        if args.shape_sweep:
            t0 = time.time()
            out["shape_sweep"] = shape_latencies(SWEEP_SHAPES, flush, args.cold_rounds, 20)
            log(f"shape sweep: {len(SWEEP_SHAPES)} shapes in {time.time() - t0:.1f}s")

        # roofline of the dominant kernels: per-launch duration from HIP events
        # around back-to-back launches on the stream the library uses
        fwd_us = time_warm(wl.fwd, 40)
        bwd_nd_us = time_warm(lambda: wl.bwd(False), 40)
        bwd_d_us = time_warm(lambda: wl.bwd(True), 40)
        # The forward kernel runs twice per step and takes the larger share
        # of it; the backward (row kernel + fixed-order dw reduce) is shown
        # beside it.
        fwd_gbs = wl.fwd_bytes / (fwd_us * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": "fwd_kernel", "achieved": round(fwd_gbs, 1),
                           "peak": PEAK_GBS, "unit": "GB/s", "frac": round(fwd_gbs / PEAK_GBS, 4),
                           "traffic": profiled_traffic(wl.name, "fwd_kernel"),
                           "us_per_launch": round(fwd_us, 2), "bytes_per_launch": wl.fwd_bytes}
        bwd_gbs = wl.bwd_bytes / (bwd_d_us * 1e-6) / 1e9
        out["roofline_bwd"] = {"bound": "hbm", "kernel": "bwd_kernel + dw_reduce_kernel (deterministic)",
                               "achieved": round(bwd_gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                               "frac": round(bwd_gbs / PEAK_GBS, 4),
                               "traffic_row_kernel": profiled_traffic(wl.name, "bwd_kernel"),
                               "us_per_call": round(bwd_d_us, 2), "bytes_per_call": wl.bwd_bytes,
                               "nondet_us_per_call": round(bwd_nd_us, 2)}
        log(f"warm fwd {fwd_us:.1f} us, bwd nondet {bwd_nd_us:.1f} us, bwd det {bwd_d_us:.1f} us")
        route = {}
        for det in (1, 0):
            f, chunks = rn.rmsnorm_bwd_route(wl.T, wl.heads, wl.H, 1 if wl.wdt == "f32" else 0, wl.res, det)
            route["det" if det else "nondet"] = {"form": "pair" if f == 0 else "atomic", "chunks": chunks}
        out["route"] = route

        if not args.no_cpu_baseline:
            t0 = time.time()
            out["cpu_baseline"] = cpu_baseline(wl)
            log(f"cpu baseline: {out['cpu_baseline']['value']:.2f} GB/s on {out['cpu_baseline']['cores']} "
                f"threads ({time.time() - t0:.1f}s)")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
