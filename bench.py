"""Benchmark of the MI355X training RMSNorm on one GPU.

Workload (default): the largest of the measured workloads, T=131072 rows of
H=6144 with the fused residual add -- x, r, dy ~ N(0,1) BF16, BF16 weight
w = 1 + 0.1 N(0,1), eps = 1e-6; the forward reads x and r and writes h and
y, the backward reads h and dy (dres = NULL, the workload names only dy).
A step is the pages' checkpointed training step "2xfwd+bwd" (forward,
forward recompute, backward; p2 "Key": op 2xfwd+bwd), here with the
deterministic backward.

Printed: ONE JSON line.  `value` is the step's effective HBM throughput
(algorithmic bytes of fwd + fwd + bwd over the measured step time, back to
back with inputs resident in HBM).  Beside it the line carries, per op and
mode, latency with L2 and the 256 MB last-level cache flushed before every
launch (the pages' protocol: cold L2, median of many launches), the
roofline of the dominant kernel (the forward) and of the backward from
HIP events around every launch of a second run of K steps, the same
figures for the T=65536 x H=4096 FP32-weight workload, and the CPU oracle
timed on the host as a baseline.

Roofline basis.  `roofline.achieved` = algorithmic bytes per launch / the
mean duration of the kernel's launches, each launch bracketed by HIP events
on the library's stream, over the warm-up steps and both runs of K steps.
`rocprofv3 --kernel-trace --stats` of `bench.py --profile` (which runs
exactly those steps and nothing else) averages the same launches;
`--profile-report` writes that summary under profiles/ with both figures.

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
DEFAULT_WORKLOAD = "T131072_H6144_res"
EXTRA_WORKLOADS = ("T65536_H4096_w32",)


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
        # one workspace for the calls with and without dres
        self.ws = rn.rmsnorm_bwd_workspace(T, heads, H, dev, w_dtype=rn.RMSN_W_F32 if wdt == "f32" else rn.RMSN_W_BF16)
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
    return rec["traffic_bytes"] if source_hash(kernel) == rec["source_hash"] else None


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
        # one workspace for the calls with and without dres
        self.ws = rn.rmsnorm_bwd_workspace(T, 1, H, "cuda", w_dtype=rn.RMSN_W_F32 if wdt == "f32" else rn.RMSN_W_BF16)

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


def span_markdown(rep, seq_path):
    """The span report as the committed summary: a table per shape, and the
    figures as JSON."""
    ops = ("fwd", "bwd_det", "bwd_nondet", "step_det")
    out = ["# Kernel spans over the pages' shape list (rocprofv3 kernel trace)", "",
           "One span = first kernel start to last kernel end of one op, from the GPU timestamps of a rocprofv3 kernel "
           "trace, after a 1 GiB flush of L2 and the last-level cache (the pages time CUPTI spans of one graph replay "
           "after an L2 flush).  Median of the spans per op; `k` = kernels per op (the step is fwd + fwd + bwd).  "
           "The backward's kernels follow the route of each shape: one column-form launch at small T, the column "
           "form and the fixed-order reduce at mid T, the row kernel and the reduce above.", "",
           "Commands (from /tmp with TMPDIR=/tmp on one MI355X; R = repository root, OUT = an output directory):", "",
           "```",
           "rocprofv3 --kernel-trace --output-format csv -d OUT -o run -- python3 R/bench.py --span-sweep OUT/seq.json",
           "python3 R/bench.py --span-report OUT/run_kernel_trace.csv OUT/seq.json",
           "```", "",
           "| shape | " + " | ".join(f"{o} us (k)" for o in ops) + " |", "|---|" + "---|" * len(ops)]
    for shape, r in rep.items():
        cells = [f"{r[o]['median_us']:.2f} ({r[o]['kernels']})" if o in r else "-" for o in ops]
        out.append(f"| {shape} | " + " | ".join(cells) + " |")
    out += ["", "```json", json.dumps({"kernel_spans_us": rep}), "```", ""]
    return "\n".join(out)


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


class LaunchTimer:
    """HIP events around every launch of the ops it wraps, on torch's current
    stream (the stream the library's calls are enqueued on)."""

    def __init__(self):
        self.ev = {}

    def __call__(self, name, fn):
        import torch

        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.ev.setdefault(name, []).append((a, b))

    def us(self, name):
        import torch

        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in self.ev.get(name, [])]


def timed_step(wl, timer, det=True):
    timer("fwd", wl.fwd)
    timer("fwd", wl.fwd)
    timer("bwd", lambda: wl.bwd(det))


def roofline_of(wl, fwd_us, bwd_us, basis):
    """The forward (two launches per step, the larger share of it) is the
    dominant kernel; the backward (row kernel, plus the fixed-order reduce
    where the route has one) beside it."""
    f_mean, b_mean = statistics.fmean(fwd_us), statistics.fmean(bwd_us)
    f_gbs = wl.fwd_bytes / (f_mean * 1e-6) / 1e9
    b_gbs = wl.bwd_bytes / (b_mean * 1e-6) / 1e9
    roof = {"bound": "hbm", "kernel": "fwd_kernel", "achieved": round(f_gbs, 1), "peak": PEAK_GBS,
            "unit": "GB/s", "frac": round(f_gbs / PEAK_GBS, 4),
            "traffic": profiled_traffic(wl.name, "fwd_kernel"), "basis": basis,
            "us_per_launch_mean": round(f_mean, 2), "us_per_launch_median": round(statistics.median(fwd_us), 2),
            "launches": len(fwd_us), "bytes_per_launch": wl.fwd_bytes}
    roof_b = {"bound": "hbm", "kernel": "bwd_kernel (+ dw_reduce_kernel when routed), deterministic",
              "achieved": round(b_gbs, 1), "peak": PEAK_GBS, "unit": "GB/s", "frac": round(b_gbs / PEAK_GBS, 4),
              "traffic_row_kernel": profiled_traffic(wl.name, "bwd_kernel"), "basis": basis,
              "us_per_call_mean": round(b_mean, 2), "us_per_call_median": round(statistics.median(bwd_us), 2),
              "calls": len(bwd_us), "bytes_per_call": wl.bwd_bytes}
    return roof, roof_b


def measure_workload(wl, args):
    """Warm-up, K timed steps (whole-step events), K more steps with every
    launch bracketed (roofline); returns the step time and the per-launch
    lists of the bracketed run.  With --profile nothing else runs, so a
    profiler sees exactly these launches."""
    import torch

    for _ in range(args.warmup):
        wl.step(True)
    torch.cuda.synchronize()
    log(f"{wl.name}: warmup {args.warmup} steps done")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        wl.step(True)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    timer = LaunchTimer()
    for _ in range(args.steps):
        timed_step(wl, timer)
    fwd_us, bwd_us = timer.us("fwd"), timer.us("bwd")
    log(f"{wl.name}: timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall:.3f}s); "
        f"per launch fwd {statistics.fmean(fwd_us):.1f} us, bwd {statistics.fmean(bwd_us):.1f} us")
    return ms_per_step, fwd_us, bwd_us


def cold_latencies(wl, args, flush):
    """Per-op latency with cold caches; "fwd_aa" is the forward again, timed
    as if it were another implementation (the A/A floor of the method)."""
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
        log(f"{wl.name}: cold {name}: {c['median_us']:.1f} us  {c['gbs']:.0f} GB/s ({c['pct_peak']:.1f}%)")
    lat["aa_floor_pct"] = round(100 * abs(lat["fwd"]["median_us"] - lat["fwd_aa"]["median_us"])
                                / lat["fwd"]["median_us"], 3)
    # deterministic over non-deterministic backward time (> 1: non-det faster)
    lat["mode_ratio_bwd"] = round(lat["bwd_det"]["median_us"] / lat["bwd_nondet"]["median_us"], 4)
    return lat


def route_of(wl, rn):
    """The backward routes of the step (dres NULL; the gated backward's own
    for a gated workload) in both modes, and with a residual the
    deterministic route of the backward with dres."""
    route = {}
    names = {0: "pair", 1: "atomic", 2: "cols", 3: "cols_ticket"}
    wd = 1 if wl.wdt == "f32" else 0
    for key, det, dres in (("det", 1, False), ("nondet", 0, False), ("det_dres", 1, True)):
        if dres and not wl.res:
            continue
        f, chunks, cc, cv, pf = (rn.rmsnorm_gated_bwd_route(wl.T, wl.heads, wl.H, wd, det) if wl.gate else
                                 rn.rmsnorm_bwd_route(wl.T, wl.heads, wl.H, wd, dres, det))
        route[key] = {"form": names.get(f, f), "chunks": chunks, "col_chunks": cc, "col_vecs": cv, "prefetch": pf}
    return route


# ---- rocprofv3 summaries (profiles/rmsnorm_kernels_<workload>.md) --------

PROFILE_KERNELS = ("fwd_kernel", "bwd_kernel", "bwd_cols_kernel", "dw_reduce_kernel")
PROFILE_SOURCES = {"fwd_kernel": ["fwd.hip", "device_common.h", "kernels.h", "layouts.h"],
                   "bwd_kernel": ["bwd.hip", "device_common.h", "kernels.h", "layouts.h"],
                   "bwd_cols_kernel": ["bwd.hip", "device_common.h", "kernels.h", "layouts.h"],
                   "dw_reduce_kernel": ["bwd.hip", "device_common.h", "kernels.h", "layouts.h"]}


def code_text(src):
    """C/C++ source without its comments, whitespace collapsed: what a
    profile's figures depend on (string and character literals are kept)."""
    import re

    tok = re.compile(r'("(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\')|//[^\n]*|/\*.*?\*/', re.S)
    body = tok.sub(lambda m: m.group(1) if m.group(1) else " ", src)
    return re.sub(r"\s+", " ", body).strip()


def source_hash(kernel):
    """Hash of the code (not the comments) of the sources a kernel is built
    from; a profile summary whose hash no longer matches is stale."""
    import hashlib

    h = hashlib.sha256()
    for f in PROFILE_SOURCES[kernel]:
        with open(os.path.join(ROOT, "rmsnorm_fwd_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def profile_commands(workload, steps, warmup):
    base = f"python3 R/bench.py --profile --steps {steps} --warmup {warmup} --workload {workload} --copy-calibration"
    return [f"rocprofv3 --kernel-trace --stats --output-format csv -d OUT/ktrace -o run -- {base} > OUT/ktrace.log",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- {base}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- {base}",
            f"python3 R/bench.py --profile-report OUT {workload} {steps} {warmup}"]


def profile_report(out_dir, workload, steps, warmup):
    """The markdown summary of three rocprofv3 runs of `bench.py --profile`
    (a kernel trace with --stats, then FETCH_SIZE, then WRITE_SIZE): kernel
    statistics, HBM bytes per dispatch scaled by a plain 1 GiB device copy
    in the same process, and the bench's own event-based roofline from the
    trace run's JSON line beside the trace's averages."""
    import csv
    import glob

    def one(pattern):
        hits = sorted(glob.glob(os.path.join(out_dir, pattern), recursive=True))
        if not hits:
            raise SystemExit(f"no {pattern} under {out_dir}")
        return hits[0]

    def key_of(name):
        for k in PROFILE_KERNELS:
            if f"rmsn::{k}" in name:
                return k
        return None

    stats = list(csv.DictReader(open(one("ktrace/**/*kernel_stats.csv"))))
    trace = list(csv.DictReader(open(one("ktrace/**/*kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Dispatch_Id"]))
    durs = {}
    for r in trace:
        k = key_of(r["Kernel_Name"])
        if k:
            durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    # bench.py --profile runs W warm-up steps, K timed steps, then K steps
    # with every launch bracketed: two forwards and one backward per step
    per_step = {"fwd_kernel": 2, "bwd_kernel": 1, "bwd_cols_kernel": 1, "dw_reduce_kernel": 1}
    last_run = {k: v[-per_step[k] * steps:] for k, v in durs.items() if len(v) >= per_step[k] * (warmup + 2 * steps)}

    def counters(kind):
        rows = list(csv.DictReader(open(one(f"{kind}/**/*counter_collection.csv"))))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        per = {}
        for r in rows:
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return copies[:3], {k: sum(v) / len(v) for k, v in per.items()}

    fc, fetch = counters("fetch")
    wc, write = counters("write")
    gib_kib = 1048576.0
    fscale = gib_kib / (sum(fc) / len(fc))
    wscale = gib_kib / (sum(wc) / len(wc))
    bench_line = None
    for path in glob.glob(os.path.join(out_dir, "ktrace*.log")) + glob.glob(os.path.join(out_dir, "*.json")):
        for line in open(path):
            if line.startswith("{") and '"roofline"' in line:
                bench_line = json.loads(line)
    wl_bytes = None
    if workload in WORKLOADS:
        T, heads, H, st, sh, wdt, res = WORKLOADS[workload]
        sw = 4 if wdt == "f32" else 2
        wl_bytes = {"fwd_kernel": fwd_bytes(T * heads, H, sw, res is True, res == "gate"),
                    "bwd_kernel": bwd_bytes(T * heads, H, sw, False, res == "gate")}
    out = [f"# rocprofv3 summary: workload {workload}", "",
           "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; R = repository root, OUT = an output "
           "directory; the first run's stdout goes to OUT/ktrace.log):", "", "```", *profile_commands(workload, steps, warmup),
           "```", "", "## Kernel statistics (--kernel-trace --stats)", "",
           "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    avg = {}
    for r in stats:
        k = key_of(r["Name"])
        if k and k not in avg:
            avg[k] = float(r["AverageNs"]) / 1e3
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    if wl_bytes:
        out += ["", "## Roofline (algorithmic bytes / duration / 8 TB/s)", "",
                f"`all launches`: the --stats average over every launch of the process; `last run`: the trace's "
                f"average over the {steps} steps whose launches bench.py brackets with HIP events (the last "
                f"{steps} steps of the run); `bench events`: bench.py's own mean over those launches, from its JSON "
                f"line in the same run (OUT/ktrace.log).  For the backward the row kernel and the reduce kernel "
                f"(when the route has one) are added.", "",
                "| op | algorithmic bytes | all launches us (frac) | last run us (frac) | bench events us (frac) |",
                "|---|---|---|---|---|"]
        ev = {}
        if bench_line:
            ev["fwd"] = bench_line["roofline"]["us_per_launch_mean"]
            ev["bwd"] = bench_line["roofline_bwd"]["us_per_call_mean"]

        def cell(t, nbytes):
            return f"{t:.2f} ({nbytes / (t * 1e-6) / 8e12:.4f})" if t else "-"

        for op, ks, nb in (("fwd", ("fwd_kernel",), wl_bytes["fwd_kernel"]),
                           ("bwd", ("bwd_kernel", "bwd_cols_kernel", "dw_reduce_kernel"), wl_bytes["bwd_kernel"])):
            t_all = sum(avg.get(k, 0.0) for k in ks)
            t_last = sum(statistics.fmean(last_run[k]) for k in ks if k in last_run)
            out.append(f"| {op} | {nb:,} | {cell(t_all, nb)} | {cell(t_last, nb)} | {cell(ev.get(op), nb)} |")
    out += ["", "## HBM traffic per dispatch (--pmc FETCH_SIZE, WRITE_SIZE; KiB)", "",
            f"Scale: a plain 1 GiB device copy (the first three copies of the process, `__amd_rocclr_copyBuffer`, "
            f"1,048,576 KiB each way) reads FETCH_SIZE = {sum(fc) / len(fc):,.0f} KiB and WRITE_SIZE = "
            f"{sum(wc) / len(wc):,.0f} KiB, so FETCH_SIZE is scaled by {fscale:.4f} and WRITE_SIZE by {wscale:.4f}.",
            "", "| kernel | FETCH_SIZE raw | WRITE_SIZE raw | scaled bytes per dispatch | source hash |",
            "|---|---|---|---|---|"]
    rec = {"workload": workload, "fetch_scale": fscale, "write_scale": wscale, "kernels": {}, "trace_avg_us": avg,
           "trace_last_run_avg_us": {k: statistics.fmean(v) for k, v in last_run.items()}}
    for name in sorted(set(fetch) | set(write)):
        k = key_of(name)
        if not k:
            continue
        fb, wb = fetch.get(name, 0.0), write.get(name, 0.0)
        total = int(round((fb * fscale + wb * wscale) * 1024))
        out.append(f"| `{name[:90]}` | {fb:,.1f} | {wb:,.1f} | {total:,} | {source_hash(k)} |")
        if k not in rec["kernels"]:
            rec["kernels"][k] = {"traffic_bytes": total, "source_hash": source_hash(k), "kernel": name}
    out += ["", "Machine-readable (read by bench.py; a source hash (of the code, comments excluded) that no longer matches the sources means the "
            "figure is stale):", "", "```json", json.dumps(rec, indent=1), "```", ""]
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--cold-reps", type=int, default=210,
                    help="cache-flushed launches per op, split over --cold-rounds interleaved rounds")
    ap.add_argument("--cold-rounds", type=int, default=3)
    ap.add_argument("--no-small-t", action="store_true", help="skip the small-T latency sweep")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra workloads (T65536_H4096_w32)")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="also time every shape of the pages' latency tables (a few minutes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only warmup + the two runs of timed steps (for rocprofv3 runs), no per-op extras")
    ap.add_argument("--span-sweep", metavar="SEQ",
                    help="run the pages' shapes as flush-delimited ops for a rocprofv3 kernel trace; "
                         "write the segment labels to SEQ and exit")
    ap.add_argument("--span-report", nargs=2, metavar=("TRACE_CSV", "SEQ"),
                    help="print per-shape median kernel spans from a --span-sweep trace and exit")
    ap.add_argument("--profile-report", nargs=4, metavar=("OUT", "WORKLOAD", "STEPS", "WARMUP"),
                    help="print the markdown summary of the three rocprofv3 runs under OUT and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counter scaling)")
    args = ap.parse_args()

    if args.span_report:
        print(span_markdown(span_report(*args.span_report), args.span_report[1]))
        return
    if args.profile_report:
        o, w, k, wu = args.profile_report
        print(profile_report(o, w, int(k), int(wu)))
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
    ms_per_step, fwd_us, bwd_us = measure_workload(wl, args)
    flush = None if args.profile else torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    value = wl.step_bytes / (ms_per_step * 1e-3) / 1e9
    basis = (f"HIP events around each launch on the library's stream, mean over a second run of {args.steps} "
             f"steps after the warm-up and the timed run ({len(fwd_us)} forward launches, {len(bwd_us)} backward "
             f"calls); the committed rocprofv3 summary of bench.py --profile gives the kernel trace's average over "
             f"the same launches beside it")
    roof, roof_b = roofline_of(wl, fwd_us, bwd_us, basis)

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
        "data": "synthetic (seeded N(0,1) x, r and dy, w = 1 + 0.1 N(0,1))",
        "config": {"workload": wl.name, "T": wl.T, "heads": wl.heads, "H": wl.H, "w_dtype": wl.wdt,
                   "residual": wl.res, "silu_gate": wl.gate,
                   "step": "fwd + fwd (recompute) + bwd (deterministic)",
                   "step_bytes": wl.step_bytes, "pct_of_peak": round(100 * value / PEAK_GBS, 2)},
        "roofline": roof,
        "roofline_bwd": roof_b,
        "route": route_of(wl, rn),
    }
    log(f"{wl.name}: {ms_per_step * 1e3:.1f} us/step, {value:.0f} GB/s; fwd frac {roof['frac']}, "
        f"bwd frac {roof_b['frac']}")

    if not args.profile:
        out["latency_cold"] = cold_latencies(wl, args, flush)
        if not args.no_small_t:
            t0 = time.time()
            out["small_t"] = shape_latencies(SMALL_T_SHAPES, flush, args.cold_rounds, 20)
            log(f"small-T latencies: {len(SMALL_T_SHAPES)} shapes in {time.time() - t0:.1f}s")
        if args.shape_sweep:
            t0 = time.time()
            out["shape_sweep"] = shape_latencies(SWEEP_SHAPES, flush, args.cold_rounds, 20)
            log(f"shape sweep: {len(SWEEP_SHAPES)} shapes in {time.time() - t0:.1f}s")
        if not args.no_cpu_baseline:
            t0 = time.time()
            out["cpu_baseline"] = cpu_baseline(wl)
            log(f"cpu baseline: {out['cpu_baseline']['value']:.2f} GB/s on {out['cpu_baseline']['cores']} "
                f"threads ({time.time() - t0:.1f}s)")
        if not args.no_extra:
            extra = {}
            for name in EXTRA_WORKLOADS:
                if name == wl.name:
                    continue
                xw = Workload(name)
                ms, fu, bu = measure_workload(xw, args)
                r1, r2 = roofline_of(xw, fu, bu, "as roofline.basis")
                extra[name] = {"ms_per_step": round(ms, 5),
                               "value": round(xw.step_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                               "roofline": r1, "roofline_bwd": r2, "route": route_of(xw, rn),
                               "latency_cold": cold_latencies(xw, argparse.Namespace(
                                   cold_reps=60, cold_rounds=args.cold_rounds), flush)}
                del xw
                torch.cuda.empty_cache()
            out["other_workloads"] = extra

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
