"""GPU parity of the HIP path against the FP64 oracle at sizes the oracle
finishes in seconds: every width layout, ragged widths, padded rows, strided
per-head views, both weight dtypes, residual in and out, both modes."""
import numpy as np
import pytest

import oracle

from tests.helpers import Layout, prepared_bytes, run_case

pytestmark = pytest.mark.gpu


def test_config1_shape_exact():
    # T=4096, H=1536, BF16 w, seed 0, plain rows, both modes
    rep = run_case(Layout.plain(4096, 1536), "bf16", det_repeats=10)
    print("config1", rep)


# every forward / backward layout, and the widths just past each boundary
WIDTHS = [8, 64, 72, 128, 136, 256, 264, 512, 520, 1024, 1032, 1536, 1544, 2048, 2056, 3072,
          4096, 4104, 5120, 6144, 6152, 8192, 8200, 16384]


@pytest.mark.parametrize("H", WIDTHS)
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_widths(H, wdt):
    T = 37 if H >= 4096 else 301
    rep = run_case(Layout.plain(T, H), wdt, seed=H)
    print(H, wdt, rep)


@pytest.mark.parametrize("H", [256, 1536, 4096, 5120, 6144, 8192, 8200, 16384])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("dres", [False, True])
def test_residual(H, wdt, dres):
    rep = run_case(Layout.plain(257, H), wdt, res=True, dres=dres, seed=7)
    print(H, wdt, dres, rep)


@pytest.mark.parametrize("H", [1536, 4096, 5120, 6144, 8192, 16384])
def test_forward_tables_give_the_same_rows(H):
    # The plain forward takes another table from 65536 rows on, and the
    # residual forward another from 32768 rows on; all keep the row layout, so
    # every row's y and rstd are the same bits whichever table ran: a long run
    # (with a ragged tail) against shorter plain runs over the same rows, and
    # the residual forward, long and short, against the plain forward over
    # its h.
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import EPS
    g = torch.Generator(device="cuda").manual_seed(H)
    R = 65536 + 37
    x = torch.randn(R, H, generator=g, device="cuda").bfloat16()
    r = torch.randn(R, H, generator=g, device="cuda").bfloat16()
    for wdt in (torch.bfloat16, torch.float32):
        w = (1 + 0.1 * torch.randn(H, generator=g, device="cuda")).to(wdt)
        y, rstd, _ = rn.rmsnorm_fwd(x, w, EPS)
        y0, rstd0, _ = rn.rmsnorm_fwd(x[:65535], w, EPS)
        y1, rstd1, _ = rn.rmsnorm_fwd(x[-100:], w, EPS)
        assert torch.equal(y[:65535], y0) and torch.equal(rstd[:65535], rstd0), "long run, head rows"
        assert torch.equal(y[-100:], y1) and torch.equal(rstd[-100:], rstd1), "long run, tail rows"
        del y0, y1
        for n in (R, 32768, 32767, 257):
            yr, rstdr, h = rn.rmsnorm_fwd(x[:n], w, EPS, residual=r[:n])
            assert torch.equal(h, (x[:n].float() + r[:n].float()).bfloat16()), "residual output"
            yp, rstdp, _ = rn.rmsnorm_fwd(h, w, EPS)
            assert torch.equal(yr, yp) and torch.equal(rstdr, rstdp), f"residual forward, {n} rows"
            del yr, h, yp
        del y
    torch.cuda.synchronize()


@pytest.mark.parametrize("heads,H,res", [(4, 4096, False), (5, 5120, False), (4, 6144, True), (3, 5120, True)])
def test_forward_tables_on_head_views(heads, H, res):
    # strided [T, heads, H] views whose row count T*heads crosses into the
    # long-run tables: every row's y, rstd (and h) must be the bits the same
    # rows give as a contiguous [T*heads, H] run of the short-run table
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import EPS
    R_min = 32768 if res else 65536
    T = -(-R_min // heads) + 7
    g = torch.Generator(device="cuda").manual_seed(H + heads)
    pad = 24
    xb = torch.randn(T, heads, H + pad, generator=g, device="cuda").bfloat16()
    rb = torch.randn(T, heads, H + pad, generator=g, device="cuda").bfloat16() if res else None
    x = xb[..., :H]
    r = rb[..., :H] if res else None
    w = (1 + 0.1 * torch.randn(H, generator=g, device="cuda")).bfloat16()
    sentinel = torch.tensor(-12345.0, dtype=torch.bfloat16, device="cuda")
    yb = sentinel.expand(T, heads, H + pad).clone()
    hb = sentinel.expand(T, heads, H + pad).clone() if res else None
    y, rstd, h = rn.rmsnorm_fwd(x, w, EPS, residual=r, y=yb[..., :H], residual_out=hb[..., :H] if res else None)
    assert T * heads >= R_min
    xc = x.reshape(T * heads, H).contiguous()
    rc = r.reshape(T * heads, H).contiguous() if res else None
    half = (T * heads) // 2  # two short runs, each below the threshold
    for lo, hi in ((0, half), (half, T * heads)):
        yc, rstdc, hc = rn.rmsnorm_fwd(xc[lo:hi], w, EPS, residual=rc[lo:hi] if res else None)
        assert torch.equal(y.reshape(T * heads, H)[lo:hi], yc), (lo, hi, "y")
        assert torch.equal(rstd[lo:hi], rstdc), (lo, hi, "rstd")
        if res:
            assert torch.equal(h.reshape(T * heads, H)[lo:hi], hc), (lo, hi, "h")
    # the padding between heads is left alone
    assert bool((yb[..., H:] == sentinel).all()), "y padding written"
    if res:
        assert bool((hb[..., H:] == sentinel).all()), "h padding written"
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 2, 3, 5, 17, 63, 64, 65, 127, 1000])
def test_row_counts(T):
    run_case(Layout.plain(T, 2048), "bf16", seed=T)
    run_case(Layout.plain(T, 256), "f32", seed=T)


def test_padded_rows():
    run_case(Layout.plain(129, 1024, pad=64), "bf16", res=True, dres=True, seed=3)
    run_case(Layout.plain(65, 4096, pad=8), "f32", seed=4)


@pytest.mark.parametrize("layout", [
    Layout.heads_view(512, 24, 256, 8192, 256),     # q slice of a [T, 8192] buffer
    Layout.heads_view(512, 24, 256, 12288, 512),    # strides (12288, 512, 1)
    Layout.heads_view(1024, 4, 256, 1024, 256),     # contiguous [T, 4, 256]
    Layout.heads_view(33, 3, 1024, 4096, 1280),
])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_head_views(layout, wdt):
    rep = run_case(layout, wdt, seed=11)
    print(layout, wdt, rep)


@pytest.mark.parametrize("T,heads,H,st,sh,res", [
    (1024, 24, 256, 8192, 256, False),    # pair with the next-row tile, one row per row group
    (1024, 24, 200, 8192, 256, True),     # the same at H 200, residual and dres
    (3000, 24, 256, 8192, 256, False),    # above the tile's window (72000 rows)
    (3000, 8, 256, 4096, 512, True),      # gaps between heads too
    (20000, 4, 256, 1024, 256, False),    # contiguous: two rows per row group
])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_gapped_head_views_row_kernel(T, heads, H, st, sh, res, wdt):
    # views with gaps between rows take one row per row group in the row
    # kernel at H 129-256; these sizes route to the pair
    import rmsnorm_fwd_amd as rn
    assert rn.rmsnorm_bwd_route(T, heads, H, 0, res, 1)[0] == rn.RMSN_FORM_PAIR
    rep = run_case(Layout.heads_view(T, heads, H, st, sh), wdt, res=res, dres=res, seed=T + H)
    print(T, heads, H, st, sh, res, wdt, rep)


@pytest.mark.parametrize("family", ["normal", "outlier", "offset"])
def test_input_families(family):
    rep = run_case(Layout.plain(2048, 4096), "f32", family=family, seed=5)
    print(family, rep)


def test_zero_rows_backward_writes_zero_dw():
    import torch
    import rmsnorm_fwd_amd as rn
    x = torch.empty(0, 512, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(512, dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(0, dtype=torch.float32, device="cuda")
    dw = torch.full((512,), 7.0, device="cuda")
    y, r, _ = rn.rmsnorm_fwd(x, w)
    dx, dw = rn.rmsnorm_bwd(x, x, rstd, w, dw=dw)
    torch.cuda.synchronize()
    assert y.numel() == 0 and int(dw.count_nonzero()) == 0


@pytest.mark.parametrize("H", [256, 1536, 4096, 6144])
def test_routes_agree(H):
    # both sides of every route choice: pair and atomic forms at several
    # chunk counts (including more chunks than row groups); dx must be
    # bitwise the same for all of them and dw within budget for each
    routes = [(0, 1), (0, 2), (0, 7), (0, 512), (0, 1000), (1, 1), (1, 5), (1, 256)]
    rep = run_case(Layout.plain(333, H), "bf16", seed=21, routes=routes)
    print(H, rep)


# column forms: (form, row tasks, row blocks per slice, vectors per slice);
# row-task and row-block counts above, at and below the row count, every
# slice width, a ragged last slice where H is not a multiple of the slice
COLUMN_ROUTES = [(0, 512), (2, 1, 1, 8), (2, 7, 1, 4), (2, 64, 3, 2), (2, 1000, 16, 1), (2, 40, 400, 8),
                 (3, 13, 2, 8), (3, 5, 5, 4), (3, 300, 64, 1), (3, 2, 333, 2)]


@pytest.mark.parametrize("H", [8, 72, 256, 264, 1032, 1536, 2056, 4096, 4104, 6144, 6152, 8200, 16384])
def test_column_forms_agree(H):
    # dx bitwise equal to the pair's, dw within budget, for every column route
    rep = run_case(Layout.plain(333, H), "f32" if H % 16 else "bf16", seed=31 + H, routes=COLUMN_ROUTES)
    print(H, rep)


@pytest.mark.parametrize("layout", [Layout.heads_view(40, 24, 256, 8192, 256), Layout.heads_view(97, 4, 256, 1024, 256),
                                    Layout.plain(65, 4096, pad=64)], ids=["24x256_s8192", "4x256", "padded"])
def test_column_forms_on_views_and_residual(layout):
    rep = run_case(layout, "bf16", res=True, dres=True, seed=5, routes=COLUMN_ROUTES)
    print(layout, rep)


@pytest.mark.parametrize("T,H", [(1, 4096), (5, 2048), (64, 6144), (1000, 1536)])
def test_column_form_dw_is_the_same_with_and_without_tickets(T, H):
    """With the same row blocks the deterministic column form (partials summed
    by the reduce kernel) and the ticket form (summed by the slice's last
    column task) add the same partials in the same order, and one block per
    slice needs neither: all give dw bit for bit, over repeated calls."""
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import gen_case, to_dev_bf16, weight_dev
    x, _, dy, _, w = gen_case(41, Layout.plain(T, H), "bf16", False, False)
    X, DY, W = to_dev_bf16(x).view(T, H), to_dev_bf16(dy).view(T, H), weight_dev(w)
    _, rstd, _ = rn.rmsnorm_fwd(X, W)
    ws = rn.rmsnorm_bwd_workspace(T, 1, H, "cuda", nbytes=rn.rmsnorm_bwd_workspace_size_for_route(
        T, 1, H, (2, 8, 16, 2)))
    for cc in (2, 16):
        got = []
        for route, det in [((2, 8, cc, 2), True), ((3, 8, cc, 2), False), ((2, 8, cc, 2), True), ((3, 3, cc, 2), False)]:
            dx, dw = rn.rmsnorm_bwd_routed(DY, X, rstd, W, route, deterministic=det, workspace=ws)
            got.append((dx, dw))
        torch.cuda.synchronize()
        for dx, dw in got[1:]:
            assert torch.equal(dx, got[0][0]) and torch.equal(dw, got[0][1])
    one = [rn.rmsnorm_bwd_routed(DY, X, rstd, W, (2, 4, 1, v), deterministic=True, workspace=ws) for v in (8, 8)]
    torch.cuda.synchronize()
    assert torch.equal(one[0][1], one[1][1]) and torch.equal(one[0][0], got[0][0])
    assert int(ws[:prepared_bytes(H)].count_nonzero()) == 0


def _route_edges(heads, H, t_max, res=False):
    """Token counts T where the default route's form, one-pass column form or
    next-row tile differs from T - 1's."""
    import rmsnorm_fwd_amd as rn
    edges, prev = [], rn.rmsnorm_bwd_route(1, heads, H, 0, res, 1)
    for T in range(2, t_max + 1):
        r = rn.rmsnorm_bwd_route(T, heads, H, 0, res, 1)
        if r[0] != prev[0] or (r[2] == 1) != (prev[2] == 1) or r[4] != prev[4]:
            edges.append(T)
        prev = r
    return edges


@pytest.mark.parametrize("heads,H,res", [(4, 256, False), (1, 1536, False), (1, 4096, False), (1, 6144, False),
                                         (1, 8192, False), (1, 1024, True), (1, 5120, True)])
def test_route_edges_from_both_sides(heads, H, res):
    # each change of backward form (one-pass column form -> two-launch column
    # form -> pair, with then without the next-row tile) is run on both
    # sides, in both modes, against the oracle (p3 commit message: each new
    # edge is exercised from both sides)
    edges = _route_edges(heads, H, 16384 // heads + 64, res)
    assert len(edges) >= 1
    for T in edges:
        for t in (T - 1, T):
            L = Layout.heads_view(t, heads, H, heads * H, H) if heads > 1 else Layout.plain(t, H)
            rep = run_case(L, "bf16", res=res, dres=res, seed=t, det_repeats=2)
            print(heads, H, res, t, rep)


@pytest.mark.parametrize("H", [64, 256, 512, 1024, 1536, 2048, 3072, 4096, 6144, 8192, 16384])
@pytest.mark.parametrize("dres,wdt", [(False, "bf16"), (True, "bf16"), (False, "f32")])
def test_next_row_tile_changes_no_bit(H, dres, wdt):
    """The row kernel with and without the next-row tile, at the same chunk
    counts (a row group per workgroup, several iterations each, a ragged last
    iteration), with and without dres: dx and the deterministic dw bit for bit
    the same, and within budget of the oracle."""
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import gen_case, to_dev_bf16, weight_dev
    T = 1000 if H <= 2048 else 301
    x, _, dy, dr, w = gen_case(61 + H, Layout.plain(T, H), wdt, False, dres)
    X, DY, W = to_dev_bf16(x).view(T, H), to_dev_bf16(dy).view(T, H), weight_dev(w)
    DR = to_dev_bf16(dr).view(T, H) if dres else None
    _, rstd, _ = rn.rmsnorm_fwd(X, W)
    for chunks in (3, 37, 256, 1000):
        got = [rn.rmsnorm_bwd_routed(DY, X, rstd, W, (0, chunks, 0, 0, pf), residual=DR, deterministic=True)
               for pf in (0, 1, 1)]
        torch.cuda.synchronize()
        for dx, dw in got[1:]:
            assert torch.equal(dx, got[0][0]) and torch.equal(dw, got[0][1]), (H, chunks)
        nd = rn.rmsnorm_bwd_routed(DY, X, rstd, W, (1, chunks, 0, 0, 1), residual=DR, deterministic=False)
        torch.cuda.synchronize()
        assert torch.equal(nd[0], got[0][0])
    rep = run_case(Layout.plain(T, H), wdt, res=dres, dres=dres, seed=61 + H,
                   routes=[(0, 256, 0, 0, 1), (0, 37, 0, 0, 1), (1, 64, 0, 0, 1)])
    print(H, dres, wdt, rep)


def test_deterministic_dw_repeats_at_scale():
    # ten repeats of the deterministic backward on a large case
    rep = run_case(Layout.plain(16384, 4096), "f32", seed=2, det_repeats=10)
    print(rep)


@pytest.mark.parametrize("H", [64, 256, 1536, 4096, 6144])
@pytest.mark.parametrize("T", [1, 5, 300])
def test_one_chunk_writes_dw_directly(T, H):
    # with one chunk the row kernel writes dw itself; it must equal the
    # reduce kernel's result for one partial bit for bit, and dx must not move
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import to_dev_bf16, weight_dev, gen_case, EPS
    L = Layout.plain(T, H)
    x, _, dy, _, w = gen_case(T + H, L, "bf16", False, False)
    xd, dyd, wd = to_dev_bf16(x), to_dev_bf16(dy), weight_dev(w)
    _, rstd, _ = rn.rmsnorm_fwd(xd, wd, EPS)
    dx1, dw1 = rn.rmsnorm_bwd_routed(dyd, xd, rstd, wd, (rn.RMSN_FORM_PAIR, 1))
    dx2, dw2 = rn.rmsnorm_bwd_routed(dyd, xd, rstd, wd, (rn.RMSN_FORM_PAIR, 1))
    dx3, dw3 = rn.rmsnorm_bwd_routed(dyd, xd, rstd, wd, (rn.RMSN_FORM_PAIR, 2))
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw2) and torch.equal(dx1, dx3)
    ref = oracle.dw_bf16(x, dy, rstd.cpu().numpy())
    from tests.helpers import check_dw, Report
    check_dw(dw1.cpu().numpy(), ref, Report())
    check_dw(dw3.cpu().numpy(), ref, Report())


@pytest.mark.parametrize("heads", [1, 3])
def test_offsets_beyond_32_bits(heads):
    # rows (or tokens) 2^30 + 1536 elements apart: the last rows start past
    # 2^32 elements (8 GiB) into their buffers, so every row address needs
    # 64-bit arithmetic.  Rows are compared with the oracle; the elements on
    # both sides of every row must keep their sentinel.
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import (EPS, SENTINEL, Report, check_dw, check_dx, check_fwd, gen_case,
                               to_host_bits, weight_dev)
    T, H = 5, 1536
    L = Layout.heads_view(T, heads, H, (1 << 30) + 1536, H if heads == 1 else 2048)
    assert (T - 1) * L.stride_t > (1 << 32)
    x, _, dy, _, w = gen_case(31, L, "bf16", False, False)
    xb, dyb, yb, dxb = L.place(x), L.place(dy), L.empty(), L.empty()
    wd = weight_dev(w)
    rstd = torch.empty(L.R, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(L.view(xb), wd, EPS, y=L.view(yb), rstd=rstd)
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    rn.rmsnorm_bwd(L.view(dyb), L.view(xb), rstd, wd, dx=L.view(dxb), dw=dw)
    torch.cuda.synchronize()
    rep = Report()
    ref_y, _, ref_rstd = oracle.fwd_bf16(x, w, EPS)
    rstd_h = rstd.cpu().numpy()
    check_fwd(L.rows_of(yb), None, rstd_h, ref_y, None, ref_rstd, rep)
    ref_dx, _, ref_dw = oracle.bwd_bf16(x, dy, w, rstd_h)
    check_dx(L.rows_of(dxb), ref_dx, rep)
    check_dw(dw.cpu().numpy(), ref_dw, rep)
    for buf in (yb, dxb):
        for t in range(T):
            for hd in range(heads):
                s = t * L.stride_t + hd * L.stride_h
                for lo, hi in ((s - 8, s), (s + H, s + H + 8)):
                    lo, hi = max(lo, 0), min(hi, L.buffer_elems())
                    if lo < hi:
                        assert np.all(to_host_bits(buf[lo:hi]) == SENTINEL), (t, hd, lo)
    print(heads, rep)


def test_max_rows_periodic():
    # The largest row count the library takes, R = 2^30 - 1, at H = 8.  The
    # rows repeat a block of P seeded rows, so the oracle needs only the
    # block: sampled rows of y, rstd and dx must match the oracle's values
    # for their block row, and dw = (R // P) * dw(block) + dw(first R % P
    # rows of the block) in FP64.
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import (EPS, Report, check_dw, check_dx, check_fwd, gen_case, to_dev_bf16,
                               to_host_bits, weight_dev)
    H, P = 8, 4096
    R = (1 << 30) - 1
    reps, rem = divmod(R, P)
    x, _, dy, _, w = gen_case(41, Layout.plain(P, H), "f32", False, False)
    wd = weight_dev(w)

    def tiled(rows):
        blk = to_dev_bf16(rows).view(P, H)
        t = torch.empty(R, H, dtype=torch.bfloat16, device="cuda")
        t[:reps * P].view(reps, P, H).copy_(blk.unsqueeze(0).expand(reps, P, H))
        t[reps * P:].copy_(blk[:rem])
        return t

    X, DY = tiled(x), tiled(dy)
    y, rstd, _ = rn.rmsnorm_fwd(X, wd, EPS)
    rng = np.random.default_rng(3)
    sample = np.unique(np.concatenate([[0, 1, P - 1, P, R - rem - 1, R - rem, R - 1],
                                       rng.integers(0, R, 2000)]))
    idx = torch.from_numpy(sample).cuda()
    base = sample % P
    rstd_blk = rstd[:P].cpu().numpy()
    rep = Report()
    ref_y, _, ref_rstd = oracle.fwd_bf16(x, w, EPS)
    check_fwd(to_host_bits(y[idx]), None, rstd[idx].cpu().numpy(), ref_y[base], None, ref_rstd[base], rep)
    assert np.array_equal(rstd[idx].cpu().numpy(), rstd_blk[base]), "a repeated row got another rstd"
    ref_dx, _, ref_dw_blk = oracle.bwd_bf16(x, dy, w, rstd_blk)
    _, _, ref_dw_rem = oracle.bwd_bf16(x[:rem], dy[:rem], w, rstd_blk[:rem])
    ref_dw = reps * ref_dw_blk + ref_dw_rem
    del y
    for det in (True, False):
        dx, dw = rn.rmsnorm_bwd(DY, X, rstd, wd, deterministic=det)
        torch.cuda.synchronize()
        check_dx(to_host_bits(dx[idx]), ref_dx[base], rep)
        check_dw(dw.cpu().numpy(), ref_dw, rep)
        del dx
    print(rep)


def test_two_streams_with_own_workspaces():
    # the library keeps no state between calls: two streams, each with its
    # own workspace, running forward and backward at the same time give
    # bitwise the results of running them one after the other
    import torch
    import rmsnorm_fwd_amd as rn
    from tests.helpers import EPS, to_dev_bf16, weight_dev
    import synth
    cases = []
    for k, (T, H) in enumerate(((3000, 4096), (5000, 1536))):
        x = to_dev_bf16(synth.rows(60 + k, "x", 0, T, H)).view(T, H)
        dy = to_dev_bf16(synth.rows(60 + k, "dy", 0, T, H)).view(T, H)
        w = weight_dev(synth.weight(60 + k, H, "bf16"))
        cases.append((x, dy, w, rn.rmsnorm_bwd_workspace(T, 1, H, "cuda")))

    def run(c, stream):
        x, dy, w, ws = c
        with torch.cuda.stream(stream):
            y, rstd, _ = rn.rmsnorm_fwd(x, w, EPS)
            dx, dw = rn.rmsnorm_bwd(dy, x, rstd, w, workspace=ws)
        return y, rstd, dx, dw

    s0 = torch.cuda.current_stream()
    ref = [run(c, s0) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for s in streams:
            s.wait_stream(s0)
        got = [run(c, s) for c, s in zip(cases, streams)]
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            for t, u in zip(a, b):
                assert torch.equal(t, u)
