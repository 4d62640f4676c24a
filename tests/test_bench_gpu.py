"""bench.py's own call pattern on the GPU, at reduced row counts: every
configured workload (same width, heads, strides, weight dtype, residual or
gate) builds its buffers and runs the timed step in both modes and, with a
residual, the backward with dres, on the one workspace it allocates.  The
row counts are chosen past the next-row tile's window, where the routes
with and without dres take different chunk counts."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", sorted(__import__("bench").WORKLOADS))
def test_bench_workload_calls(name, monkeypatch):
    import torch

    import bench
    T, heads, H, st, sh, wdt, res = bench.WORKLOADS[name]
    small = {name: (max(1, 9000 // heads), heads, H, st, sh, wdt, res)}
    monkeypatch.setattr(bench, "WORKLOADS", small)
    wl = bench.Workload(name)
    for det in (True, False):
        wl.step(det)
    if wl.res:
        wl.bwd(True, wl.dres)
        wl.bwd(False, wl.dres)
    torch.cuda.synchronize()
    assert torch.isfinite(wl.dw).all()
