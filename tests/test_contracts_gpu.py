"""Calling contracts of the C ABI that the parity tests do not exercise:
in-place outputs and workspaces that hold garbage.

Aliasing.  The forward may write y over x and h over x or over r; the
backward may write dx over dy or over dres; the gated backward may write
dg over g and dx over dy.  An in-place call must give the same bits as the
call with separate outputs, and those bits are checked against the oracle.

Workspace.  The fixed-order pair writes every chunk partial before the
reduce reads it, so a deterministic call is correct whatever the workspace
held before.  The atomic form needs only its accumulator and ticket zeroed
(rmsnorm_bwd_workspace_init), whatever the rest holds, and leaves them zero
again.  The pages ask for a workspace that serves mixed forms (p1 #8577
commit text, its "mixed-form workspace" test)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import (EPS, Layout, Report, check_dw, check_dx, check_fwd, gen_case, prepared_bytes, to_host_bits,
                           weight_dev)

pytestmark = pytest.mark.gpu

LAYOUTS = [
    Layout.plain(301, 2048),                      # one-pass column form
    Layout.plain(1000, 2048),                     # two-launch column form (row-block partials)
    Layout.plain(4099, 1536),                     # prime row count, row kernel + fixed-order reduce
    Layout.plain(3, 4096),                        # one-pass column form, three rows
    Layout.heads_view(64, 24, 256, 8192, 256),    # per-head view of a [T, 8192] buffer (two-launch column form)
]
IDS = ["T301_H2048", "T1000_H2048", "T4099_H1536", "T3_H4096", "T64x24x256"]


def _bufs(L, wdt, res, dres, seed):
    x, r, dy, dr, w = gen_case(seed, L, wdt, res, dres)
    return dict(x=x, r=r, dy=dy, dr=dr, w=w)


def _fwd(L, c, alias):
    """Forward with the outputs named by `alias` written over an input."""
    import torch
    import rmsnorm_fwd_amd as rn
    res = c["r"] is not None
    xb, rb = L.place(c["x"]), (L.place(c["r"]) if res else None)
    yb = xb if "y=x" in alias else L.empty()
    hb = None
    if res:
        hb = xb if "h=x" in alias else (rb if "h=r" in alias else L.empty())
    rstd = torch.empty(L.R, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(L.view(xb), weight_dev(c["w"]), EPS, residual=L.view(rb) if res else None,
                   y=L.view(yb), residual_out=L.view(hb) if res else None, rstd=rstd)
    torch.cuda.synchronize()
    return L.rows_of(yb), (L.rows_of(hb) if res else None), rstd.cpu().numpy()


@pytest.mark.parametrize("L", LAYOUTS, ids=IDS)
@pytest.mark.parametrize("res,alias", [(False, "y=x"), (True, "y=x"), (True, "h=x"), (True, "h=r"),
                                       (True, "y=x,h=r")])
def test_forward_in_place(L, res, alias):
    c = _bufs(L, "bf16", res, False, seed=40 + L.H)
    y0, h0, rstd0 = _fwd(L, c, "")
    y1, h1, rstd1 = _fwd(L, c, alias)
    assert np.array_equal(y0, y1), f"y differs in place ({alias})"
    assert np.array_equal(rstd0, rstd1)
    if res:
        assert np.array_equal(h0, h1), f"h differs in place ({alias})"
    ry, rh, rr = oracle.fwd_bf16(c["x"], c["w"], EPS, c["r"])
    check_fwd(y1, h1, rstd1, ry, rh, rr, Report())


def _bwd(L, c, u, rstd, alias, det):
    import torch
    import rmsnorm_fwd_amd as rn
    dres = c["dr"] is not None
    ub, dyb = L.place(u), L.place(c["dy"])
    drb = L.place(c["dr"]) if dres else None
    dxb = dyb if alias == "dx=dy" else (drb if alias == "dx=dres" else L.empty())
    dx, dw = rn.rmsnorm_bwd(L.view(dyb), L.view(ub), rstd, weight_dev(c["w"]),
                            residual=L.view(drb) if dres else None, deterministic=det, dx=L.view(dxb))
    torch.cuda.synchronize()
    return L.rows_of(dxb), dw.cpu().numpy()


@pytest.mark.parametrize("L", LAYOUTS, ids=IDS)
@pytest.mark.parametrize("dres,alias", [(False, "dx=dy"), (True, "dx=dy"), (True, "dx=dres")])
@pytest.mark.parametrize("det", [True, False])
def test_backward_in_place(L, dres, alias, det):
    import torch
    import rmsnorm_fwd_amd as rn
    c = _bufs(L, "f32", False, dres, seed=50 + L.H)
    _, rstd, _ = rn.rmsnorm_fwd(L.view(L.place(c["x"])), weight_dev(c["w"]), EPS)
    dx0, dw0 = _bwd(L, c, c["x"], rstd, "", det)
    dx1, dw1 = _bwd(L, c, c["x"], rstd, alias, det)
    assert np.array_equal(dx0, dx1), f"dx differs in place ({alias})"
    if det:
        assert np.array_equal(dw0, dw1), "deterministic dw differs in place"
    ref_dx, _, ref_dw = oracle.bwd_bf16(c["x"], c["dy"], c["w"], rstd.cpu().numpy(), c["dr"])
    rep = Report()
    check_dx(dx1, ref_dx, rep)
    check_dw(dw1, ref_dw, rep)


@pytest.mark.parametrize("L", [Layout.plain(257, 2048), Layout.plain(2, 6144),
                               Layout.heads_view(64, 4, 256, 1024, 256)], ids=["T257_H2048", "T2_H6144", "T64x4x256"])
def test_gated_backward_in_place(L):
    """dg over g and dx over dy give the bits of separate outputs."""
    import torch
    import rmsnorm_fwd_amd as rn
    x, dy = synth.rows(60, "x", 0, L.R, L.H), synth.rows(60, "dy", 0, L.R, L.H)
    g, w = synth.rows(60, "g", 0, L.R, L.H), synth.weight(60, L.H, "bf16")
    wd = weight_dev(w)
    _, rstd = rn.rmsnorm_gated_fwd(L.view(L.place(x)), L.view(L.place(g)), wd, EPS)

    def run(in_place):
        xb, gb, dyb = L.place(x), L.place(g), L.place(dy)
        dxb, dgb = (dyb, gb) if in_place else (L.empty(), L.empty())
        _, _, dw = rn.rmsnorm_gated_bwd(L.view(dyb), L.view(xb), L.view(gb), rstd, wd,
                                        dx=L.view(dxb), dg=L.view(dgb))
        torch.cuda.synchronize()
        return L.rows_of(dxb), L.rows_of(dgb), dw.cpu().numpy()

    dx0, dg0, dw0 = run(False)
    dx1, dg1, dw1 = run(True)
    assert np.array_equal(dx0, dx1) and np.array_equal(dg0, dg1) and np.array_equal(dw0, dw1)


@pytest.mark.parametrize("L", LAYOUTS, ids=IDS)
def test_deterministic_workspace_may_hold_garbage(L):
    import torch
    import rmsnorm_fwd_amd as rn
    c = _bufs(L, "bf16", False, False, seed=70 + L.H)
    xv, wd = L.view(L.place(c["x"])), weight_dev(c["w"])
    _, rstd, _ = rn.rmsnorm_fwd(xv, wd, EPS)
    dyv = L.view(L.place(c["dy"]))
    clean = rn.rmsnorm_bwd_workspace(L.T, L.heads, L.H, "cuda")
    dx0, dw0 = rn.rmsnorm_bwd(dyv, xv, rstd, wd, deterministic=True, workspace=clean)
    for byte in (0xFF, 0x7F, 0x00):                # NaN doubles, huge doubles, zeros
        ws = torch.full_like(clean, byte)
        dx1, dw1 = rn.rmsnorm_bwd(dyv, xv, rstd, wd, deterministic=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(dw0, dw1) and torch.equal(dx0, dx1), f"workspace filled with {byte:#x}"


@pytest.mark.parametrize("H", [256, 1536, 4096])
def test_atomic_form_needs_only_its_header_zeroed(H):
    """A garbage-filled workspace, prepared by rmsnorm_bwd_workspace_init,
    serves the atomic form, then the pair, then the atomic form again."""
    import torch
    import rmsnorm_fwd_amd as rn
    L = Layout.plain(333, H)
    c = _bufs(L, "f32", False, False, seed=80 + H)
    xv, wd = L.view(L.place(c["x"])), weight_dev(c["w"])
    _, rstd, _ = rn.rmsnorm_fwd(xv, wd, EPS)
    dyv = L.view(L.place(c["dy"]))
    routes = [(rn.RMSN_FORM_ATOMIC, 64), (rn.RMSN_FORM_PAIR, 64), (rn.RMSN_FORM_ATOMIC, 7)]
    need = max(rn.rmsnorm_bwd_workspace_size_for_route(L.T, 1, H, r) for r in routes)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    rn.rmsnorm_bwd_workspace_init(ws, H)
    ref_dx, _, ref_dw = oracle.bwd_bf16(c["x"], c["dy"], c["w"], rstd.cpu().numpy())
    dxs = []
    for route in routes:
        det = route[0] == rn.RMSN_FORM_PAIR
        dx, dw = rn.rmsnorm_bwd_routed(dyv, xv, rstd, wd, route, deterministic=det, workspace=ws)
        torch.cuda.synchronize()
        rep = Report()
        check_dx(to_host_bits(dx), ref_dx, rep)
        check_dw(dw.cpu().numpy(), ref_dw, rep)
        dxs.append(to_host_bits(dx))
    assert all(np.array_equal(dxs[0], d) for d in dxs[1:])
    assert int(ws[:prepared_bytes(H)].count_nonzero()) == 0, "atomic form did not leave its header zero"


def test_binding_rejects_what_the_abi_cannot_check():
    """Lengths, contiguity and dtypes of the vectors (rstd, w, dw), the
    activations' dtype and the workspace layout are checked in the binding
    before any launch; nothing is enqueued for a rejected call."""
    import torch
    import rmsnorm_fwd_amd as rn
    T, H = 16, 512
    x = torch.randn(T, H, device="cuda").bfloat16()
    w = torch.ones(H, device="cuda")
    y, rstd, _ = rn.rmsnorm_fwd(x, w)
    bad = [
        (ValueError, "rstd must be a contiguous", lambda: rn.rmsnorm_fwd(x, w, rstd=torch.empty(T - 1, device="cuda"))),
        (ValueError, "w must be a contiguous", lambda: rn.rmsnorm_fwd(x, torch.ones(H - 8, device="cuda"))),
        (ValueError, "w must be a contiguous", lambda: rn.rmsnorm_fwd(x, torch.ones(2 * H, device="cuda")[::2])),
        (TypeError, "w must be", lambda: rn.rmsnorm_fwd(x, w.half())),
        (TypeError, "y must be bfloat16", lambda: rn.rmsnorm_fwd(x, w, y=torch.empty(T, H, device="cuda"))),
        (TypeError, "dy must be bfloat16", lambda: rn.rmsnorm_bwd(x.float(), x, rstd, w)),
        (ValueError, "rstd must be a contiguous", lambda: rn.rmsnorm_bwd(x, x, rstd[:-1], w)),
        (TypeError, "dw must be", lambda: rn.rmsnorm_bwd(x, x, rstd, w, dw=torch.empty(H, device="cuda").half())),
        (ValueError, "dw must be a contiguous", lambda: rn.rmsnorm_bwd(x, x, rstd, w, dw=torch.empty(H + 8, device="cuda"))),
        (ValueError, "workspace must be contiguous",
         lambda: rn.rmsnorm_bwd(x, x, rstd, w, workspace=torch.zeros(2 << 20, dtype=torch.uint8, device="cuda")[::2])),
        (TypeError, "g must be bfloat16", lambda: rn.rmsnorm_gated_fwd(x, x.float(), w)),
        (TypeError, "dg must be bfloat16",
         lambda: rn.rmsnorm_gated_bwd(x, x, x, rstd, w, dg=torch.empty(T, H, device="cuda"))),
    ]
    for exc, msg, call in bad:
        with pytest.raises(exc, match=msg):
            call()
    torch.cuda.synchronize()
    # the good call still works after the rejected ones
    dx, dw = rn.rmsnorm_bwd(x, x, rstd, w)
    torch.cuda.synchronize()
    assert torch.isfinite(dw).all()


@pytest.mark.parametrize("T,H", [(64, 1536), (4, 4096), (1000, 256)])
def test_non_finite_rows_stay_in_their_rows(T, H):
    """NaN and Inf inputs propagate by IEEE rules within their own row only:
    every other row's y, rstd and dx are bitwise those of the clean input
    (dw sums over rows, so its affected columns are not compared)."""
    import torch
    import rmsnorm_fwd_amd as rn
    g = torch.Generator().manual_seed(T + H)
    x = torch.randn(T, H, generator=g).bfloat16().cuda()
    dy = torch.randn(T, H, generator=g).bfloat16().cuda()
    w = (1 + 0.1 * torch.randn(H, generator=g)).cuda()
    bad = x.clone()
    bad[1, 3] = float("nan")
    bad[T - 1, 0] = float("inf")
    keep = torch.ones(T, dtype=torch.bool, device="cuda")
    keep[1] = keep[T - 1] = False
    y0, r0, _ = rn.rmsnorm_fwd(x, w)
    y1, r1, _ = rn.rmsnorm_fwd(bad, w)
    dx0, _ = rn.rmsnorm_bwd(dy, x, r0, w)
    dx1, _ = rn.rmsnorm_bwd(dy, bad, r1, w)
    torch.cuda.synchronize()
    assert torch.equal(y0[keep], y1[keep]) and torch.equal(r0[keep], r1[keep])
    assert torch.equal(dx0[keep], dx1[keep])
    assert torch.isnan(r1[1]) and torch.isnan(y1[1]).all()
