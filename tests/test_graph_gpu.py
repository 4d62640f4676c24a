"""The library's calls inside a captured HIP graph: they allocate nothing,
never synchronise and clear nothing with memset nodes, so a graph of the
checkpointed step (forward, forward recompute, backward) replays to the
same bits as eager calls.  Each replay is checked, with eager work and a
synchronisation between replays, and the eager result is checked against
the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import (EPS, Report, check_dw, check_dx, check_fwd, prepared_bytes, to_dev_bf16, to_host_bits,
                           weight_dev)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,wdt,res,route", [
    (4096, 1536, "bf16", False, None),
    (2048, 4096, "f32", False, None),
    (300, 6144, "bf16", True, None),
    (3, 4096, "f32", False, None),        # one workgroup writes dw directly
    (777, 2048, "bf16", False, (1, 64)),  # atomic form: ticket and accumulator clear themselves
])
def test_step_replays_bitwise(T, H, wdt, res, route):
    import rmsnorm_fwd_amd as rn
    x_h = synth.rows(11, "x", 0, T, H)
    r_h = synth.rows(11, "r", 0, T, H) if res else None
    dy_h = synth.rows(11, "dy", 0, T, H)
    w_h = synth.weight(11, H, wdt)
    x, dy, w = to_dev_bf16(x_h).view(T, H), to_dev_bf16(dy_h).view(T, H), weight_dev(w_h)
    r = to_dev_bf16(r_h).view(T, H) if res else None
    y, h = torch.empty_like(x), (torch.empty_like(x) if res else None)
    dx = torch.empty_like(x)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    nbytes = (rn.rmsnorm_bwd_workspace_size_for_route(T, 1, H, route) if route
              else rn.rmsnorm_bwd_workspace_size(T, 1, H, rn.RMSN_W_F32 if wdt == "f32" else rn.RMSN_W_BF16, res))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    det = route is None

    def step():
        rn.rmsnorm_fwd(x, w, EPS, residual=r, y=y, residual_out=h, rstd=rstd)
        rn.rmsnorm_fwd(x, w, EPS, residual=r, y=y, residual_out=h, rstd=rstd)
        u = h if res else x
        if route:
            rn.rmsnorm_bwd_routed(dy, u, rstd, w, route, deterministic=False, dx=dx, dw=dw, workspace=ws)
        else:
            rn.rmsnorm_bwd(dy, u, rstd, w, deterministic=det, dx=dx, dw=dw, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # eager, on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [to_host_bits(y), to_host_bits(dx), rstd.cpu().numpy().copy(), dw.cpu().numpy().copy()]
    if res:
        eager.append(to_host_bits(h))

    rep = Report()
    ref_y, ref_h, ref_rstd = oracle.fwd_bf16(x_h, w_h, EPS, r_h)
    check_fwd(eager[0], eager[4] if res else None, eager[2], ref_y, ref_h, ref_rstd, rep)
    ref_dx, _, ref_dw = oracle.bwd_bf16(eager[4] if res else x_h, dy_h, w_h, eager[2])
    check_dx(eager[1], ref_dx, rep)
    check_dw(eager[3], ref_dw, rep)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for i in range(4):
        for t in (y, dx, dw, rstd) + ((h,) if res else ()):
            t.fill_(0)  # eager work between replays; the replay must rewrite all of it
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [to_host_bits(y), to_host_bits(dx), rstd.cpu().numpy(), dw.cpu().numpy()]
        if res:
            got.append(to_host_bits(h))
        for k, (a, b) in enumerate(zip(eager, got)):
            if k == 3 and not det:  # atomic dw: reproducible only within its budget
                check_dw(b, ref_dw, rep)
            else:
                assert np.array_equal(a, b), f"replay {i}: output {k} differs from the eager step"
    if route:
        assert int(ws[:prepared_bytes(H)].count_nonzero()) == 0
    print(T, H, wdt, res, route, rep)


def test_gated_step_replays_bitwise():
    # the gated forward / recompute / backward captured once and replayed
    import rmsnorm_fwd_amd as rn
    T, H = 1000, 4096
    x = to_dev_bf16(synth.rows(12, "x", 0, T, H)).view(T, H)
    g = to_dev_bf16(synth.rows(12, "g", 0, T, H)).view(T, H)
    dy = to_dev_bf16(synth.rows(12, "dy", 0, T, H)).view(T, H)
    w = weight_dev(synth.weight(12, H, "f32"))
    y, dx, dg = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.zeros(rn.rmsnorm_bwd_workspace_size(T, 1, H, rn.RMSN_W_F32), dtype=torch.uint8, device="cuda")

    def step():
        rn.rmsnorm_gated_fwd(x, g, w, EPS, y=y, rstd=rstd)
        rn.rmsnorm_gated_fwd(x, g, w, EPS, y=y, rstd=rstd)
        rn.rmsnorm_gated_bwd(dy, x, g, rstd, w, dx=dx, dg=dg, dw=dw, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, rstd, dx, dg, dw)]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        step()
    for i in range(3):
        for t in (y, rstd, dx, dg, dw):
            t.fill_(0)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, (y, rstd, dx, dg, dw)):
            assert torch.equal(a, b), f"replay {i} differs"
