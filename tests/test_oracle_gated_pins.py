"""Pins for the SiLU-gated oracle (y = RMSNorm(u) * w * silu(g)): torch's own
FP64 rms_norm, silu and autograd, central finite differences in x, g and w,
and the closed forms of a closed gate (g = 0) and a saturated one (large g),
which reduce to the plain oracle (pinned on its own).  CPU only."""
import numpy as np
import pytest
import torch

import oracle
import synth

EPS = 1e-6


def _rand(shape, seed, scale=1.0, loc=0.0):
    return loc + scale * np.random.default_rng(seed).standard_normal(shape)


def _torch_gated(u, g, w, eps):
    U = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    G = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    W = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.rms_norm(U, (U.shape[-1],), weight=W, eps=eps) * torch.nn.functional.silu(G)
    return U, G, W, y


@pytest.mark.parametrize("R,H,eps", [(5, 64, EPS), (3, 1000, 0.25)])
def test_gated_matches_torch_autograd_fp64(R, H, eps):
    u, g = _rand((R, H), 1), _rand((R, H), 2, 2.0)
    w, dy = _rand(H, 3, 0.1, 1.0), _rand((R, H), 4)
    y, rstd = oracle.gated_fwd_f64(u, g, w, eps)
    U, G, W, Y = _torch_gated(u, g, w, eps)
    np.testing.assert_allclose(y, Y.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt((u * u).mean(axis=1) + eps), rtol=1e-14)
    (Y * torch.tensor(dy)).sum().backward()
    dx, dg, dw = oracle.gated_bwd_f64(u, g, dy, w, rstd)
    np.testing.assert_allclose(dx, U.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg, G.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw, W.grad.numpy(), rtol=1e-10, atol=1e-12)


def _loss(u, g, w, dy, eps):
    y, _ = oracle.gated_fwd_f64(u, g, w, eps)
    return float((dy * y).sum())


def test_gated_central_finite_differences_4x8():
    u, g = _rand((4, 8), 11), _rand((4, 8), 12, 1.5)
    w, dy = _rand(8, 13, 0.1, 1.0), _rand((4, 8), 14)
    _, rstd = oracle.gated_fwd_f64(u, g, w, EPS)
    dx, dg, dw = oracle.gated_bwd_f64(u, g, dy, w, rstd)

    def fd(arr, idx, f):
        h = 1e-6 * max(1.0, abs(arr[idx]))
        p, m = arr.copy(), arr.copy()
        p[idx] += h
        m[idx] -= h
        return (f(p) - f(m)) / (2 * h)

    fd_x = np.array([[fd(u, (i, j), lambda a: _loss(a, g, w, dy, EPS)) for j in range(8)] for i in range(4)])
    fd_g = np.array([[fd(g, (i, j), lambda a: _loss(u, a, w, dy, EPS)) for j in range(8)] for i in range(4)])
    fd_w = np.array([fd(w, (j,), lambda a: _loss(u, g, a, dy, EPS)) for j in range(8)])
    for got, ref in ((dx, fd_x), (dg, fd_g), (dw, fd_w)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-7 * np.abs(got).max())


def test_closed_gate_and_saturated_gate_reduce_to_plain():
    u, dy = _rand((6, 48), 21), _rand((6, 48), 22)
    w = _rand(48, 23, 0.1, 1.0)
    y0, rstd = oracle.fwd_f64(u, w, EPS)
    # g = 0: silu = 0, silu' = 1/2 -> no output, no dx or dw, dg = dy * y_plain / 2
    z = np.zeros_like(u)
    yg, rg = oracle.gated_fwd_f64(u, z, w, EPS)
    dx, dg, dw = oracle.gated_bwd_f64(u, z, dy, w, rstd)
    assert np.array_equal(rg, rstd) and not yg.any() and not dx.any() and not dw.any()
    np.testing.assert_allclose(dg, dy * y0 / 2, rtol=1e-14, atol=1e-16)
    # g = 60: sigmoid rounds to 1 in double, silu = g, silu' = 1
    big = np.full_like(u, 60.0)
    yg, _ = oracle.gated_fwd_f64(u, big, w, EPS)
    dx, dg, dw = oracle.gated_bwd_f64(u, big, dy, w, rstd)
    px, pw = oracle.bwd_f64(u, 60.0 * dy, w, rstd)
    np.testing.assert_allclose(yg, 60.0 * y0, rtol=1e-14)
    np.testing.assert_allclose(dx, px, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dw, pw, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dg, dy * y0, rtol=1e-14, atol=1e-16)


def test_deep_negative_and_infinite_gates():
    # For g < 0, sigmoid(g) = e^g / (1 + e^g) needs no e^-g, so it stays
    # accurate (and free of overflow) down to where e^g underflows; silu and
    # silu' from that form pin the oracle's 1 / (1 + e^-g) far into the
    # negative tail, where a capped or overflowing exponential goes wrong.
    # g = -1e4 underflows to -0; g = -inf gives NaN and +inf gives +inf (the
    # formula g * sigmoid(g) in IEEE arithmetic, like torch's FP64 silu).
    deep = np.array([-30.0, -88.0, -90.0, -100.0, -300.0, -700.0])
    R, H = len(deep), 16
    u, dy = _rand((R, H), 41), _rand((R, H), 42)
    w = _rand(H, 43, 0.1, 1.0)
    g = _rand((R, H), 44)
    g[:, 3] = deep
    y, rstd = oracle.gated_fwd_f64(u, g, w, EPS)
    dx, dg, dw = oracle.gated_bwd_f64(u, g, dy, w, rstd)
    a = u * rstd[:, None] * w
    t = np.exp(deep)
    s = t / (1.0 + t)
    silu = deep * s
    dsilu = s * (1.0 + deep * (1.0 - s))
    np.testing.assert_allclose(y[:, 3], a[:, 3] * silu, rtol=1e-14, atol=0)
    np.testing.assert_allclose(dg[:, 3], dy[:, 3] * a[:, 3] * dsilu, rtol=1e-13, atol=0)
    assert np.all(y[:, 3] != 0) and np.all(np.abs(y[:, 3]) < 1e-10)
    np.testing.assert_allclose(y[:, 3], torch.nn.functional.silu(torch.tensor(g)).numpy()[:, 3] * a[:, 3],
                               rtol=1e-14, atol=0)
    # underflow and infinities
    g2 = _rand((3, H), 45)
    g2[0, 0], g2[1, 1], g2[2, 2] = -1.0e4, -np.inf, np.inf
    with np.errstate(over="ignore", invalid="ignore"):
        y2, r2 = oracle.gated_fwd_f64(u[:3], g2, w, EPS)
    assert y2[0, 0] == 0.0 and np.signbit(y2[0, 0]) != np.signbit(u[0, 0] * w[0])
    assert np.isnan(y2[1, 1]) and np.isinf(y2[2, 2]) and np.sign(y2[2, 2]) == np.sign(u[2, 2] * w[2])
    assert np.isfinite(np.delete(y2, [0, 1 * H + 1, 2 * H + 2])).all()
    ref = torch.nn.functional.silu(torch.tensor(g2)).numpy()
    assert np.isnan(ref[1, 1]) and np.isinf(ref[2, 2]) and ref[0, 0] == 0.0


def test_gated_dx_dw_are_plain_at_the_gated_gradient():
    u, g, dy = _rand((7, 96), 31), _rand((7, 96), 32, 3.0), _rand((7, 96), 33)
    w = _rand(96, 34, 0.1, 1.0)
    _, rstd = oracle.fwd_f64(u, w, EPS)
    dx, _, dw = oracle.gated_bwd_f64(u, g, dy, w, rstd)
    e = dy * torch.nn.functional.silu(torch.tensor(g)).numpy()
    px, pw = oracle.bwd_f64(u, e, w, rstd)
    np.testing.assert_allclose(dx, px, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dw, pw, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_gated_bf16_path_equals_fp64_core(wdt):
    R, H = 40, 264
    x, g, dy = synth.rows(4, "x", 0, R, H), synth.rows(4, "g", 0, R, H), synth.rows(4, "dy", 0, R, H)
    w = synth.weight(4, H, wdt)
    wd = oracle.bf16_to_f64(w) if wdt == "bf16" else w.astype(np.float64)
    y, rstd = oracle.gated_fwd_bf16(x, g, w, EPS)
    y64, rstd64 = oracle.gated_fwd_f64(oracle.bf16_to_f64(x), oracle.bf16_to_f64(g), wd, EPS)
    assert np.array_equal(y, oracle.bf16_round(y64)) and np.array_equal(rstd, rstd64)
    rho = rstd.astype(np.float32)
    dx, dg, dx64, dg64, dw = oracle.gated_bwd_bf16(x, g, dy, w, rho, want_f64=True)
    cx, cg, cw = oracle.gated_bwd_f64(oracle.bf16_to_f64(x), oracle.bf16_to_f64(g), oracle.bf16_to_f64(dy),
                                      wd, rho.astype(np.float64))
    np.testing.assert_allclose(dx64, cx, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dg64, cg, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dw, cw, rtol=1e-13, atol=1e-13)
    assert np.array_equal(dx, oracle.bf16_round(dx64)) and np.array_equal(dg, oracle.bf16_round(dg64))
