"""Pins for the FP64 CPU oracle: every check ties it to something other than
itself -- finite differences, torch's own FP64 rms_norm and autograd, exact
rational arithmetic, closed forms of special rows, and algebraic identities
that link the forward's outputs to the backward's.  CPU only."""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
import synth

EPS = 1e-6  # every measurement on the pages uses eps = 1e-6 (p1 #8577 "Baselines and measurement")


def _rand(shape, seed, scale=1.0, loc=0.0):
    return loc + scale * np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------- BF16 ----

def _bits(v):
    return int(oracle.bf16_round([v])[0])


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),                 # exact tie -> even (1.0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # exact tie -> even (1 + 2^-6)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # just above the tie; a float32 detour would land on the tie
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite BF16
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),    # tie above it rounds to even = inf
    (2.0 ** -133, 0x0001),                     # smallest BF16 subnormal
    (2.0 ** -134, 0x0000),                     # tie between 0 and 2^-133 -> even
    (1.5 * 2.0 ** -133, 0x0002),               # tie between 1 and 2 units -> even
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
])
def test_bf16_round_hand_cases(value, bits):
    assert _bits(value) == bits


def test_bf16_round_matches_torch_on_float32_values():
    # torch rounds float32 -> bfloat16 to nearest even; on float32 inputs a
    # single rounding from double must agree with it bit for bit.
    v32 = np.random.default_rng(1).standard_normal(200_000).astype(np.float32) * np.float32(7.0)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(v32.astype(np.float64))
    assert np.array_equal(got, ref)


def _bf16_value(bits):
    return Fraction(float(oracle.bf16_to_f64(np.array([bits], dtype=np.uint16))[0]))


def test_bf16_round_brute_force_nearest_even():
    # Exact rational comparison against the neighbouring BF16 values.
    rng = np.random.default_rng(2)
    vals = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    for v in vals:
        b = _bits(float(v))
        exact = Fraction(float(v))
        cands = [(b + k) & 0xFFFF for k in (-1, 0, 1)]
        best = None
        for c in cands:
            if (c & 0x7F80) == 0x7F80:
                continue
            d = abs(_bf16_value(c) - exact)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                best = (d, c)
        assert best[1] == b, (v, hex(b), hex(best[1]))


def test_bf16_widening_exact():
    b = np.arange(0, 0x10000, 7, dtype=np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.bf16_to_f64(b), ref)


# ------------------------------------------------------------- residual ----

def test_residual_add_matches_torch_and_exact():
    x = synth.rows(0, "x", 0, 64, 256)
    r = synth.rows(0, "r", 0, 64, 256)
    h = oracle.residual_add(x, r)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    ref = (tx.float() + tr.float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ref)
    # a few elements against exact rationals
    for i in range(0, x.size, 997):
        s = _bf16_value(int(x.flat[i])) + _bf16_value(int(r.flat[i]))
        assert _bits(float(s)) == int(h.flat[i])


# ------------------------------------------------- forward: library pins ----

@pytest.mark.parametrize("R,H,eps", [(5, 8, EPS), (7, 64, EPS), (3, 1536, EPS), (4, 8, 0.25)])
def test_fwd_matches_torch_rms_norm_fp64(R, H, eps):
    u = _rand((R, H), 3)
    w = _rand(H, 4, 0.1, 1.0)
    y, rstd = oracle.fwd_f64(u, w, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(u), (H,), torch.from_numpy(w), eps).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)
    # rstd recovered from torch's y: y = u * rstd * w
    rs = (ref / (u * w[None, :])).mean(axis=1)
    np.testing.assert_allclose(rstd, rs, rtol=1e-12)


# ------------------------------------------------ backward: library pins ----

@pytest.mark.parametrize("R,H,eps,with_dres", [(5, 8, EPS, False), (6, 96, EPS, True),
                                               (3, 1024, EPS, False), (4, 8, 0.5, True)])
def test_bwd_matches_torch_autograd_fp64(R, H, eps, with_dres):
    u = _rand((R, H), 5)
    w = _rand(H, 6, 0.1, 1.0)
    dy = _rand((R, H), 7)
    dres = _rand((R, H), 8) if with_dres else None
    _, rstd = oracle.fwd_f64(u, w, eps)
    dx, dw = oracle.bwd_f64(u, dy, w, rstd, dres)
    tu = torch.from_numpy(u).requires_grad_(True)
    tw = torch.from_numpy(w).requires_grad_(True)
    y = torch.nn.functional.rms_norm(tu, (H,), tw, eps)
    loss = (y * torch.from_numpy(dy)).sum()
    if with_dres:
        loss = loss + (tu * torch.from_numpy(dres)).sum()
    loss.backward()
    np.testing.assert_allclose(dx, tu.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-11, atol=1e-13)


# -------------------------------------------- central finite differences ----

def _loss(u, w, dy, eps):
    y, _ = oracle.fwd_f64(u, w, eps)
    return float((dy * y).sum())


@pytest.mark.parametrize("eps", [EPS, 0.3])
def test_bwd_central_finite_differences_4x8(eps):
    u = _rand((4, 8), 11)
    w = _rand(8, 12, 0.1, 1.0)
    dy = _rand((4, 8), 13)
    _, rstd = oracle.fwd_f64(u, w, eps)
    dx, dw = oracle.bwd_f64(u, dy, w, rstd)
    fd_x = np.zeros_like(u)
    for i in range(4):
        for j in range(8):
            h = 1e-6 * max(1.0, abs(u[i, j]))
            up, um = u.copy(), u.copy()
            up[i, j] += h
            um[i, j] -= h
            fd_x[i, j] = (_loss(up, w, dy, eps) - _loss(um, w, dy, eps)) / (2 * h)
    fd_w = np.zeros_like(w)
    for j in range(8):
        h = 1e-6 * max(1.0, abs(w[j]))
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        fd_w[j] = (_loss(u, wp, dy, eps) - _loss(u, wm, dy, eps)) / (2 * h)
    scale_x = np.abs(dx).max()
    np.testing.assert_allclose(dx, fd_x, rtol=0, atol=1e-7 * scale_x)
    np.testing.assert_allclose(dw, fd_w, rtol=0, atol=1e-7 * np.abs(dw).max())


# ------------------------------------------------------------ invariants ----

def test_linearity_in_dy():
    u = _rand((6, 40), 21)
    w = _rand(40, 22, 0.1, 1.0)
    d1, d2 = _rand((6, 40), 23), _rand((6, 40), 24)
    _, rho = oracle.fwd_f64(u, w, EPS)
    a, b = 0.75, -1.5
    dx1, dw1 = oracle.bwd_f64(u, d1, w, rho)
    dx2, dw2 = oracle.bwd_f64(u, d2, w, rho)
    dx3, dw3 = oracle.bwd_f64(u, a * d1 + b * d2, w, rho)
    np.testing.assert_allclose(dx3, a * dx1 + b * dx2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw3, a * dw1 + b * dw2, rtol=1e-12, atol=1e-12)


def test_dw_independent_of_w_and_its_dtype():
    H = 256
    u = synth.rows(3, "x", 0, 100, H)
    dy = synth.rows(3, "dy", 0, 100, H)
    rho = np.random.default_rng(5).uniform(0.5, 2.0, 100).astype(np.float32)
    w_bf = synth.weight(0, H, "bf16")
    w_32 = synth.weight(1, H, "f32")
    _, _, dw_a = oracle.bwd_bf16(u, dy, w_bf, rho)
    _, _, dw_b = oracle.bwd_bf16(u, dy, w_32, rho)
    assert np.array_equal(dw_a, dw_b)


def test_orthogonality_identity():
    # sum_j u_j dx_j = eps * rstd^2 * sum_j y_j dy_j   (rstd exact for u)
    for eps in (EPS, 0.05):
        u = _rand((8, 24), 31)
        w = _rand(24, 32, 0.1, 1.0)
        dy = _rand((8, 24), 33)
        y, rstd = oracle.fwd_f64(u, w, eps)
        dx, _ = oracle.bwd_f64(u, dy, w, rstd)
        lhs = (u * dx).sum(axis=1)
        rhs = eps * rstd ** 2 * (y * dy).sum(axis=1)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-12 * np.abs(u * dx).sum(axis=1).max())


def test_weight_identity():
    # sum_j w_j dw_j = sum over rows of sum_j y_j dy_j
    u = _rand((16, 32), 41)
    w = _rand(32, 42, 0.1, 1.0)
    dy = _rand((16, 32), 43)
    y, rstd = oracle.fwd_f64(u, w, EPS)
    _, dw = oracle.bwd_f64(u, dy, w, rstd)
    np.testing.assert_allclose((w * dw).sum(), (y * dy).sum(), rtol=1e-12)


# --------------------------------------------------------- special rows ----

def test_zero_row():
    H = 16
    w = _rand(H, 51, 0.1, 1.0)
    dy = _rand((1, H), 52)
    u = np.zeros((1, H))
    y, rstd = oracle.fwd_f64(u, w, EPS)
    assert np.all(y == 0)
    assert rstd[0] == pytest.approx(1000.0, rel=1e-12)   # 1/sqrt(1e-6)
    dx, dw = oracle.bwd_f64(u, dy, w, rstd)
    np.testing.assert_allclose(dx, rstd[0] * w * dy, rtol=1e-15)
    assert np.all(dw == 0)


@pytest.mark.parametrize("a", [1.0, -3.0, 0.001])
def test_constant_row(a):
    H = 32
    w = _rand(H, 61, 0.1, 1.0)
    u = np.full((1, H), a)
    y, rstd = oracle.fwd_f64(u, w, EPS)
    assert rstd[0] == pytest.approx(1.0 / math.sqrt(a * a + EPS), rel=1e-14)
    np.testing.assert_allclose(y[0], a * w / math.sqrt(a * a + EPS), rtol=1e-14)


def test_width_one_closed_form():
    # H = 1: dx = w dy eps (u^2 + eps)^(-3/2)
    u = np.array([[0.7], [-2.0], [0.0]])
    w = np.array([1.3])
    dy = np.array([[0.4], [-1.1], [2.0]])
    eps = 0.2
    _, rstd = oracle.fwd_f64(u, w, eps)
    dx, dw = oracle.bwd_f64(u, dy, w, rstd)
    np.testing.assert_allclose(dx[:, 0], w[0] * dy[:, 0] * eps * (u[:, 0] ** 2 + eps) ** -1.5, rtol=1e-13)
    np.testing.assert_allclose(dw[0], (dy[:, 0] * u[:, 0] / np.sqrt(u[:, 0] ** 2 + eps)).sum(), rtol=1e-13)


def test_single_row_dw_is_dy_times_xhat():
    H = 48
    u = _rand((1, H), 71)
    w = _rand(H, 72, 0.1, 1.0)
    dy = _rand((1, H), 73)
    rho = np.array([0.8125])
    _, dw = oracle.bwd_f64(u, dy, w, rho)
    np.testing.assert_allclose(dw, dy[0] * u[0] * 0.8125, rtol=1e-15)


# ------------------------------------------------ BF16 storage wrappers ----

@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("res", [False, True])
def test_bf16_path_against_torch_fp64(wdt, res):
    R, H = 37, 136
    x = synth.rows(9, "x", 0, R, H)
    r = synth.rows(9, "r", 0, R, H) if res else None
    dy = synth.rows(9, "dy", 0, R, H)
    dres = synth.rows(9, "dres", 0, R, H) if res else None
    w = synth.weight(9, H, wdt)
    y, h, rstd = oracle.fwd_bf16(x, w, EPS, r)
    u = h if res else x
    if res:
        assert np.array_equal(h, oracle.residual_add(x, r))
    w64 = w.astype(np.float64) if wdt == "f32" else oracle.bf16_to_f64(w)
    tu = torch.from_numpy(oracle.bf16_to_f64(u)).requires_grad_(True)
    tw = torch.from_numpy(w64).requires_grad_(True)
    ty = torch.nn.functional.rms_norm(tu, (H,), tw, EPS)
    ref_y = torch.from_numpy(ty.detach().numpy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # torch's float64 -> bfloat16 may round twice; allow one unit where it does
    diff = np.abs(y.astype(np.int32) - ref_y.astype(np.int32))
    assert diff.max() <= 1
    assert np.array_equal(y, oracle.bf16_round(ty.detach().numpy()))
    # backward at the FP32 rstd, as the kernel would hand it over
    rho32 = rstd.astype(np.float32)
    dx, dx64, dw = oracle.bwd_bf16(u, dy, w, rho32, dres, want_dx64=True)
    dx_ref, dw_ref = oracle.bwd_f64(oracle.bf16_to_f64(u), oracle.bf16_to_f64(dy), w64,
                                    rho32.astype(np.float64),
                                    oracle.bf16_to_f64(dres) if res else None)
    np.testing.assert_allclose(dx64, dx_ref, rtol=1e-13, atol=1e-13)
    assert np.array_equal(dx, oracle.bf16_round(dx_ref))
    np.testing.assert_allclose(dw, dw_ref, rtol=1e-13, atol=1e-13)
    # and against autograd at the FP64 rstd (differs only through rho32)
    (ty * torch.from_numpy(oracle.bf16_to_f64(dy))).sum().backward()
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-6, atol=1e-6)


def test_dw_alone_equals_backward_dw():
    R, H = 300, 200
    u = synth.rows(4, "x", 0, R, H)
    dy = synth.rows(4, "dy", 0, R, H)
    rho = np.random.default_rng(6).uniform(0.5, 2.0, R).astype(np.float32)
    _, _, dw = oracle.bwd_bf16(u, dy, synth.weight(4, H, "bf16"), rho)
    assert np.array_equal(oracle.dw_bf16(u, dy, rho), dw)
