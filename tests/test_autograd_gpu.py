"""The autograd facade (functional form, Function, Module) against the oracle:
gradients of x, w and the residual, both weight dtypes, both modes, with and
without the checkpointed recompute; recompute and mode must not change dx."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import EPS, check_dw, check_dx, Report, to_dev_bf16, to_host_bits, ulp_dist, weight_dev

pytestmark = pytest.mark.gpu


def _run(T, H, wdt, res, det, recompute, seed=0):
    from rmsnorm_fwd_amd.autograd import rmsnorm
    x_h = synth.rows(seed, "x", 0, T, H)
    r_h = synth.rows(seed, "r", 0, T, H) if res else None
    g_h = synth.rows(seed, "dy", 0, T, H)
    g2_h = synth.rows(seed, "dres", 0, T, H) if res else None
    w_h = synth.weight(seed, H, wdt)
    x = to_dev_bf16(x_h).requires_grad_(True)
    r = to_dev_bf16(r_h).requires_grad_(True) if res else None
    w = weight_dev(w_h).requires_grad_(True)
    out = rmsnorm(x, w, EPS, residual=r, deterministic=det, recompute=recompute)
    G = to_dev_bf16(g_h)
    if res:
        y, h = out
        loss = (y * G).float().sum() + (h * to_dev_bf16(g2_h)).float().sum()
    else:
        y = out
        loss = (y * G).float().sum()
    loss.backward()
    return x, r, w, x_h, r_h, g_h, g2_h, w_h


@pytest.mark.parametrize("recompute", [False, True])
@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("res", [False, True])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_autograd_matches_oracle(wdt, res, det, recompute):
    import rmsnorm_fwd_amd as rn
    T, H = 257, 1536
    x, r, w, x_h, r_h, g_h, g2_h, w_h = _run(T, H, wdt, res, det, recompute)
    # the forward's rstd (bitwise what the backward used)
    _, rstd, h = rn.rmsnorm_fwd(to_dev_bf16(x_h), weight_dev(w_h), EPS,
                                residual=to_dev_bf16(r_h) if res else None)
    rho = rstd.cpu().numpy()
    u = to_host_bits(h) if res else x_h
    # dy reaches the kernel as bf16(G) (autograd casts the float grad back)
    ref_dx, _, _ = oracle.bwd_bf16(u, g_h, w_h, rho, g2_h)
    ref_dw = oracle.dw_bf16(u, g_h, rho)
    rep = Report()
    check_dx(to_host_bits(x.grad), ref_dx, rep)
    if res:
        assert torch.equal(x.grad, r.grad)
    if wdt == "f32":
        check_dw(w.grad.cpu().numpy(), ref_dw, rep)
    else:
        # the BF16 parameter receives dw rounded once to BF16
        assert ulp_dist(to_host_bits(w.grad), oracle.bf16_round(ref_dw)).max() <= 1


@pytest.mark.parametrize("res", [False, True])
def test_recompute_and_mode_do_not_change_dx(res):
    base = _run(129, 4096, "bf16", res, True, False, seed=3)
    for det, rec in ((True, True), (False, False), (False, True)):
        other = _run(129, 4096, "bf16", res, det, rec, seed=3)
        assert torch.equal(other[0].grad, base[0].grad)
        if det:
            assert torch.equal(other[2].grad, base[2].grad)


def test_module_and_views():
    from rmsnorm_fwd_amd.autograd import RMSNorm
    T, heads, H = 64, 4, 256
    m = RMSNorm(H, dtype=torch.float32, device="cuda")
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(synth.weight(5, H, "f32")))
    buf = to_dev_bf16(synth.rows(5, "x", 0, T, 8 * H)).requires_grad_(True)
    q = buf.view(T, 8, H)[:, :heads]          # a strided per-head view
    y = m(q)
    g = to_dev_bf16(synth.rows(5, "dy", 0, T * heads, H)).view(T, heads, H)
    (y * g).float().sum().backward()
    import rmsnorm_fwd_amd as rn
    _, rstd, _ = rn.rmsnorm_fwd(q.detach(), m.weight.detach())
    u = to_host_bits(q.detach().reshape(T * heads, H))
    ref_dx, _, _ = oracle.bwd_bf16(u, to_host_bits(g.reshape(T * heads, H)), synth.weight(5, H, "f32"),
                                   rstd.cpu().numpy())
    got = to_host_bits(buf.grad.view(T, 8, H)[:, :heads].reshape(T * heads, H))
    assert ulp_dist(got, ref_dx).max() <= 1
    assert int(buf.grad.view(T, 8, H)[:, heads:].count_nonzero()) == 0


@pytest.mark.parametrize("res", [False, True])
def test_leading_dims_fold_into_rows(res):
    # [B, S, N, H] inputs (contiguous, and a permuted one that needs a copy)
    # give bitwise the outputs and gradients of the same rows as [R, H]
    from rmsnorm_fwd_amd.autograd import rmsnorm
    B, S, N, H = 2, 3, 11, 1536
    R = B * S * N
    x_h = synth.rows(9, "x", 0, R, H)
    r_h = synth.rows(9, "r", 0, R, H)
    g_h = synth.rows(9, "dy", 0, R, H)
    w_h = synth.weight(9, H, "f32")

    def run(shape_fn, unshape_fn):
        x = shape_fn(to_dev_bf16(x_h).view(R, H)).detach().requires_grad_(True)
        r = shape_fn(to_dev_bf16(r_h).view(R, H)).detach() if res else None
        w = weight_dev(w_h).requires_grad_(True)
        out = rmsnorm(x, w, EPS, residual=r)
        y = out[0] if res else out
        loss = (y.float() * shape_fn(to_dev_bf16(g_h).view(R, H)).float()).sum()
        if res:
            loss = loss + out[1].float().sum()
        loss.backward()
        return unshape_fn(y.detach()), unshape_fn(x.grad), w.grad

    flat = run(lambda t: t, lambda t: t)
    four = run(lambda t: t.view(B, S, N, H), lambda t: t.reshape(R, H))
    perm = run(lambda t: t.view(S, B, N, H).permute(1, 0, 2, 3),
               lambda t: t.permute(1, 0, 2, 3).reshape(R, H))
    for other in (four, perm):
        for a, b in zip(flat[:2], other[:2]):
            assert torch.equal(a, b)
    assert torch.equal(flat[2], four[2])
    torch.testing.assert_close(flat[2], perm[2], rtol=1e-5, atol=1e-5)  # rows in another order
