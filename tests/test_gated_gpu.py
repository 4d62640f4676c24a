"""SiLU-gated variant (y = RMSNorm(x) * w * silu(g)) through the C ABI against
the oracle.

Tolerances.  The kernels evaluate silu in FP32: sigmoid(g) = 1 / (1 + exp(-g))
is within ~4 units in the last place of FP32 while it is a normal number, so
silu and silu' carry a relative error below EPS_S = 2^-20 (a margin of ~3 over
that bound); for g < -87.3 sigmoid is FP32-subnormal and its absolute error
stays below 2^-149 (plus the same relative part), far below the BF16
subnormal spacing 2^-133 that every check below allows at least.
  * y: within 1 BF16 unit (its FP32 error stays far below half a BF16 unit).
  * rstd: as in the plain forward (the gate does not enter the norm).
  * dx: within 1 BF16 unit, or within one unit plus the bound that silu's
    error sets: EPS_S * rho * (|w e| + |x| rho^2 sum_i |x_i w_i e_i| / H),
    e = dy * silu(g).  The kernel forms the gated dx in FP32 (and rounds
    x * dy * silu(g) once in FP32 before its FP64 sums): those roundings,
    ~3 * 2^-24 of the same terms, sit inside that bound.
  * dg: within 1 BF16 unit, or one unit plus EPS_S * |dy * xhat * w| *
    sigmoid(g) * (1 + 2 |g|) (silu' = sigmoid (1 + g (1 - sigmoid)) cancels
    near g = -1.28).
  * dw: the plain budget 1e-4 + 1e-4 |dw| plus EPS_S * sum over rows of
    |e * xhat|.
dx and dg are bitwise the same in both modes; deterministic dw repeats
bitwise."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import EPS, Layout, to_dev_bf16, to_host_bits, ulp_dist, weight_dev

pytestmark = pytest.mark.gpu

EPS_S = 2.0 ** -20


def _bf16_ulp(v):
    """Spacing of BF16 numbers at |v| (subnormal floor included)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _close(got_bits, ref64, bound):
    got = oracle.bf16_to_f64(got_bits)
    ok = ulp_dist(got_bits, oracle.bf16_round(ref64)) <= 1
    ok |= np.abs(got - ref64) <= _bf16_ulp(ref64) + bound
    return ok


def gen_gate(seed, R, H, kind):
    g = synth.rows(seed, "g", 0, R, H, "offset" if kind == "open" else "normal")
    if kind == "mixed":
        gf = oracle.bf16_to_f64(g).reshape(-1)
        gf[::7] *= 6.0                         # wide gates, both tails
        gf[1::11] = 0.0                        # closed gate
        gf[2::13] = -1.28125                   # near silu's minimum (silu' ~ 0)
        gf[3::17] = 30.0                       # saturated: silu = g, silu' = 1
        gf[4::19] = -88.0                      # sigmoid below FP32's normal range
        gf[5::23] = -90.0
        gf[6::29] = -100.0                     # silu below BF16's subnormal spacing
        gf[8::37] = -1.0e4                     # sigmoid underflows to 0
        g = oracle.bf16_round(gf).reshape(R, H)
    return g


def run_gated(L: Layout, wdt="bf16", seed=0, kind="mixed", det_repeats=2):
    import torch
    import rmsnorm_fwd_amd as rn
    x = synth.rows(seed, "x", 0, L.R, L.H)
    dy = synth.rows(seed, "dy", 0, L.R, L.H)
    g = gen_gate(seed, L.R, L.H, kind)
    w = synth.weight(seed, L.H, wdt)
    xb, dyb, gb = L.place(x), L.place(dy), L.place(g)
    wd = weight_dev(w)
    gaps = L.gap_mask() if L.R else np.zeros(0, bool)

    outs = []
    for det in (True, False):
        yb = L.empty()
        rstd = torch.empty(L.R, dtype=torch.float32, device="cuda")
        rn.rmsnorm_gated_fwd(L.view(xb), L.view(gb), wd, EPS, deterministic=det, y=L.view(yb), rstd=rstd)
        outs.append((L.rows_of(yb), rstd.cpu().numpy()))
        if gaps.any():
            assert np.all(to_host_bits(yb)[gaps] == 0x7FC0), "write outside the view"
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    y_k, rho = outs[0]
    ref_y, ref_rstd = oracle.gated_fwd_bf16(x, g, w, EPS)
    assert ulp_dist(y_k, ref_y).max(initial=0) <= 1, "y off by more than one unit"
    if L.R:
        assert (np.abs(rho.astype(np.float64) - ref_rstd) / ref_rstd).max() <= 1e-6

    ref_dx, ref_dg, dx64, dg64, ref_dw = oracle.gated_bwd_bf16(x, g, dy, w, rho, want_f64=True)
    # tolerance terms from the FP64 inputs
    xf, gf, df = oracle.bf16_to_f64(x), oracle.bf16_to_f64(g), oracle.bf16_to_f64(dy)
    wf = oracle.bf16_to_f64(w) if wdt == "bf16" else w.astype(np.float64)
    r = rho.astype(np.float64)[:, None]
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-gf))
    e = df * gf * sg
    xhat = xf * r
    bx = EPS_S * r * (np.abs(wf * e) + np.abs(xf) * r * r * np.abs(xf * wf * e).sum(1, keepdims=True) / L.H)
    bg = EPS_S * np.abs(df * xhat * wf) * sg * (1 + 2 * np.abs(gf))
    bw = 1e-4 + 1e-4 * np.abs(ref_dw) + EPS_S * np.abs(e * xhat).sum(0)
    ws = rn.rmsnorm_bwd_workspace(L.T, L.heads, L.H, "cuda")
    first = {}
    for det in (True, False):
        for rep in range(det_repeats if det else 1):
            dxb, dgb = L.empty(), L.empty()
            dw = torch.empty(L.H, dtype=torch.float32, device="cuda")
            rn.rmsnorm_gated_bwd(L.view(dyb), L.view(xb), L.view(gb), torch.from_numpy(rho).cuda(), wd,
                                 deterministic=det, dx=L.view(dxb), dg=L.view(dgb), dw=dw, workspace=ws)
            torch.cuda.synchronize()
            dx_k, dg_k, dw_k = L.rows_of(dxb), L.rows_of(dgb), dw.cpu().numpy()
            if not first:
                assert _close(dx_k, dx64, bx).all(), "dx outside its tolerance"
                assert _close(dg_k, dg64, bg).all(), "dg outside its tolerance"
                assert (np.abs(dw_k.astype(np.float64) - ref_dw) <= bw).all(), "dw outside its tolerance"
                first = dict(dx=dx_k, dg=dg_k, dw=dw_k)
                if gaps.any():
                    for buf in (dxb, dgb):
                        assert np.all(to_host_bits(buf)[gaps] == 0x7FC0), "write outside the view"
            else:
                assert np.array_equal(dx_k, first["dx"]) and np.array_equal(dg_k, first["dg"])
                if det:
                    assert np.array_equal(dw_k, first["dw"]), "deterministic dw not reproducible"
                else:
                    assert (np.abs(dw_k.astype(np.float64) - ref_dw) <= bw).all()
    return ulp_dist(first["dx"], ref_dx).max(initial=0), ulp_dist(first["dg"], ref_dg).max(initial=0)


@pytest.mark.parametrize("H", [8, 64, 256, 264, 1024, 1536, 2048, 4096, 5120, 6144, 8192, 8200, 16384])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_gated_widths(H, wdt):
    T = 37 if H >= 4096 else 301
    print(H, wdt, run_gated(Layout.plain(T, H), wdt, seed=H))


@pytest.mark.parametrize("T", [0, 1, 2, 3, 5, 17, 64, 65, 1000])
def test_gated_row_counts(T):
    print(T, run_gated(Layout.plain(T, 4096), "f32", seed=T + 1))


@pytest.mark.parametrize("kind", ["normal", "open", "mixed"])
def test_gated_gate_families(kind):
    print(kind, run_gated(Layout.plain(2048, 2048), "bf16", seed=7, kind=kind))


@pytest.mark.parametrize("H", [64, 512, 1536, 3072, 4096, 5120, 6144, 16384])
def test_gated_moderate_gates_widths(H):
    # N(0,1) gates: no gate reaches the scaled branch of the sigmoid (g below
    # about -44), so every lane of the eight-gate form takes its direct path
    T = 37 if H >= 4096 else 301
    print(H, run_gated(Layout.plain(T, H), "bf16", seed=H + 11, kind="normal"))


@pytest.mark.parametrize("H", [64, 2048, 6144])
def test_gated_infinite_gates_forward(H):
    # g = -inf gives silu = -inf * 0 = NaN and g = +inf gives +inf, as the
    # formula g * sigmoid(g) reads in IEEE arithmetic (the oracle's FP64
    # evaluation and torch's silu agree); the gate never enters the norm, so
    # rstd and every other element of those rows keep their values
    import torch
    import rmsnorm_fwd_amd as rn
    T = 40
    x = synth.rows(9, "x", 0, T, H)
    g = gen_gate(9, T, H, "mixed")
    gf = oracle.bf16_to_f64(g)
    gf[::3, 5] = -np.inf
    gf[1::3, H - 1] = np.inf
    gf[2::5, 0] = -np.inf
    g = oracle.bf16_round(gf)
    w = synth.weight(9, H, "bf16")
    y, rstd = rn.rmsnorm_gated_fwd(to_dev_bf16(x).view(T, H), to_dev_bf16(g).view(T, H), weight_dev(w), EPS)
    torch.cuda.synchronize()
    ref_y, ref_rstd = oracle.gated_fwd_bf16(x, g, w, EPS)
    yk = to_host_bits(y)
    yf, rf = oracle.bf16_to_f64(yk), oracle.bf16_to_f64(ref_y)
    assert np.array_equal(np.isnan(yf), np.isnan(rf)) and np.isnan(rf).sum() == (np.isneginf(gf)).sum()
    fin = ~np.isnan(rf)
    assert np.array_equal(yf[~np.isfinite(rf) & fin], rf[~np.isfinite(rf) & fin])
    assert ulp_dist(yk[np.isfinite(rf)], ref_y[np.isfinite(rf)]).max() <= 1
    assert (np.abs(rstd.cpu().numpy().astype(np.float64) - ref_rstd) / ref_rstd).max() <= 1e-6


@pytest.mark.parametrize("T,H", [(4099, 2048), (4099, 3072), (4099, 4096), (70000, 1536), (4099, 6144)])
def test_gated_rows_over_several_iterations_moderate_gates(T, H):
    # N(0,1) gates (no lane takes the sigmoid's scaled branch) through the
    # row kernel with several iterations per workgroup, on the layouts that
    # keep sigmoid(g) between the two passes
    import rmsnorm_fwd_amd as rn
    assert rn.rmsnorm_gated_bwd_route(T, 1, H, 0, 1)[0] == rn.RMSN_FORM_PAIR
    print(T, H, run_gated(Layout.plain(T, H), "bf16", seed=T + H + 5, kind="normal"))


def test_gated_head_view():
    print(run_gated(Layout.heads_view(512, 24, 256, 8192, 256), "bf16", seed=3))


@pytest.mark.parametrize("T,H,wdt", [(4099, 1536, "bf16"), (4099, 3072, "bf16"), (4099, 5120, "bf16"),
                                     (4099, 6144, "bf16"), (60000, 64, "bf16"), (4099, 2048, "f32"),
                                     (4099, 4096, "bf16"), (1500, 8192, "f32"), (1500, 8200, "bf16"),
                                     (1100, 16384, "bf16")])
def test_gated_rows_over_several_iterations(T, H, wdt):
    # gated rows up to H 8192 load a workgroup's next rows while reducing the
    # current ones (one- and two-vector rows, and the H 8192 rows run as 512
    # lanes x 2 vectors), wider ones do not; these row counts take the row
    # kernel with several iterations per workgroup and a ragged last one
    import rmsnorm_fwd_amd as rn
    assert rn.rmsnorm_gated_bwd_route(T, 1, H, 0, 1)[0] == rn.RMSN_FORM_PAIR
    print(T, H, wdt, run_gated(Layout.plain(T, H), wdt, seed=T + H))


def test_gated_large():
    print(run_gated(Layout.plain(16384, 4096), "f32", seed=5, det_repeats=3))


@pytest.mark.parametrize("recompute", [False, True])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_gated_autograd(wdt, recompute):
    # the autograd form gives the C-ABI results bitwise: x.grad = dx, g.grad = dg,
    # w.grad = dw (cast to w's dtype), for an upstream gradient dy
    import torch
    import rmsnorm_fwd_amd as rn
    from rmsnorm_fwd_amd.autograd import rmsnorm_gated
    T, H = 300, 2048
    x_h, g_h, dy_h = synth.rows(8, "x", 0, T, H), gen_gate(8, T, H, "mixed"), synth.rows(8, "dy", 0, T, H)
    w_h = synth.weight(8, H, wdt)
    x = to_dev_bf16(x_h).view(T, H).requires_grad_(True)
    g = to_dev_bf16(g_h).view(T, H).requires_grad_(True)
    w = weight_dev(w_h).requires_grad_(True)
    dy = to_dev_bf16(dy_h).view(T, H)
    y = rmsnorm_gated(x, g, w, EPS, deterministic=True, recompute=recompute)
    y.backward(dy)
    y2, rstd = rn.rmsnorm_gated_fwd(x.detach(), g.detach(), w.detach(), EPS)
    dx, dg, dw = rn.rmsnorm_gated_bwd(dy, x.detach(), g.detach(), rstd, w.detach())
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2)
    assert torch.equal(x.grad, dx) and torch.equal(g.grad, dg)
    assert torch.equal(w.grad, dw if wdt == "f32" else dw.to(torch.bfloat16))


def test_gated_full_size_headline_shape():
    # T=65536 x H=4096, FP32 w (the benchmark's gated workload): y, dx, dg on
    # sampled rows, dw against the oracle's full column sums, dx/dg across
    # modes and deterministic dw across repeats over the whole tensors
    import torch
    import rmsnorm_fwd_amd as rn
    T, H = 65536, 4096
    x, dy = synth.rows(0, "x", 0, T, H), synth.rows(0, "dy", 0, T, H)
    g = gen_gate(0, T, H, "mixed")
    w = synth.weight(0, H, "f32")
    X, G, DY = (to_dev_bf16(a).view(T, H) for a in (x, g, dy))
    W = weight_dev(w)
    y, rstd = rn.rmsnorm_gated_fwd(X, G, W, EPS)
    rows = np.unique(np.concatenate([[0, 1, T // 2, T - 1], np.random.default_rng(1).integers(0, T, 384)]))
    idx = torch.from_numpy(rows).cuda()
    rho = rstd.cpu().numpy()
    ref_y, ref_rstd = oracle.gated_fwd_bf16(x[rows], g[rows], w, EPS)
    assert ulp_dist(to_host_bits(y.index_select(0, idx)), ref_y).max() <= 1
    assert (np.abs(rho[rows].astype(np.float64) - ref_rstd) / ref_rstd).max() <= 1e-6
    dx, dg, dw = rn.rmsnorm_gated_bwd(DY, X, G, rstd, W, deterministic=True)
    _, _, dx64, dg64, _ = oracle.gated_bwd_bf16(x[rows], g[rows], dy[rows], w, rho[rows], want_f64=True)
    xf, gf, df = oracle.bf16_to_f64(x[rows]), oracle.bf16_to_f64(g[rows]), oracle.bf16_to_f64(dy[rows])
    r = rho[rows].astype(np.float64)[:, None]
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-gf))
    e = df * gf * sg
    bx = EPS_S * r * (np.abs(w * e) + np.abs(xf) * r * r * np.abs(xf * w * e).sum(1, keepdims=True) / H)
    bg = EPS_S * np.abs(df * xf * r * w) * sg * (1 + 2 * np.abs(gf))
    assert _close(to_host_bits(dx.index_select(0, idx)), dx64, bx).all()
    assert _close(to_host_bits(dg.index_select(0, idx)), dg64, bg).all()
    # dw over all rows, with its bound sum |e * xhat| accumulated in row blocks
    _, _, _, _, ref_dw = oracle.gated_bwd_bf16(x, g, dy, w, rho)
    absum = np.zeros(H)
    for r0 in range(0, T, 8192):
        sl = slice(r0, r0 + 8192)
        gb = oracle.bf16_to_f64(g[sl])
        with np.errstate(over="ignore"):
            eb = oracle.bf16_to_f64(dy[sl]) * gb / (1.0 + np.exp(-gb))
        absum += np.abs(eb * oracle.bf16_to_f64(x[sl]) * rho[sl].astype(np.float64)[:, None]).sum(0)
    bw = 1e-4 + 1e-4 * np.abs(ref_dw) + EPS_S * absum
    assert (np.abs(dw.cpu().numpy().astype(np.float64) - ref_dw) <= bw).all()
    for _ in range(3):
        dx2, dg2, dw2 = rn.rmsnorm_gated_bwd(DY, X, G, rstd, W, deterministic=True)
        assert torch.equal(dx2, dx) and torch.equal(dg2, dg) and torch.equal(dw2, dw)
    dx3, dg3, dw3 = rn.rmsnorm_gated_bwd(DY, X, G, rstd, W, deterministic=False)
    assert torch.equal(dx3, dx) and torch.equal(dg3, dg)
    assert (np.abs(dw3.cpu().numpy().astype(np.float64) - ref_dw) <= bw).all()


@pytest.mark.parametrize("H", [1536, 4096, 6144])
def test_gated_route_edges_from_both_sides(H):
    # each change of the gated backward's form (one-pass column form ->
    # two-launch column form -> pair) is run on both sides against the oracle
    import rmsnorm_fwd_amd as rn
    edges, prev = [], rn.rmsnorm_gated_bwd_route(1, 1, H, 0, 1)
    for T in range(2, 8192):
        r = rn.rmsnorm_gated_bwd_route(T, 1, H, 0, 1)
        assert r[4] == 0
        if r[0] != prev[0] or (r[2] == 1) != (prev[2] == 1):
            edges.append(T)
        prev = r
    assert len(edges) >= 1
    for T in edges:
        for t in (T - 1, T):
            print(H, t, run_gated(Layout.plain(t, H), "bf16", seed=t))

