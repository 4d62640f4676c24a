"""rmsnorm_bwd_noalloc, the backward for callers that cannot allocate, through
the C ABI: two calls in a row on the library's own scratch, the second with a
smaller input, each checked against rmsnorm_bwd on a workspace of its own
(dx bit for bit; dw bit for bit in deterministic mode, where both take the
same route and kernels, and within the dw budget in the other) and against
the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from tests.helpers import EPS, Layout, Report, check_dw, check_dx, gen_case, to_host_bits, weight_dev

pytestmark = pytest.mark.gpu


def _run(rn, L, wdt, det, seed, dres):
    import torch
    x, _, dy, dr, w = gen_case(seed, L, wdt, False, dres)
    xb, dyb = L.place(x), L.place(dy)
    drb = L.place(dr) if dres else None
    wd = weight_dev(w)
    _, rstd, _ = rn.rmsnorm_fwd(L.view(xb), wd, EPS)
    torch.cuda.synchronize()
    T, heads, H, st, sh = rn.geometry(L.view(xb))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dx_n, dw_n = L.empty(), torch.full((H,), float("nan"), device="cuda")
    status = rn.lib().rmsnorm_bwd_noalloc(
        ctypes.c_void_p(L.view(dyb).data_ptr()), ctypes.c_void_p(L.view(xb).data_ptr()),
        ctypes.c_void_p(rstd.data_ptr()), ctypes.c_void_p(wd.data_ptr()), rn._w_dtype(wd),
        ctypes.c_void_p(L.view(drb).data_ptr()) if dres else None, ctypes.c_void_p(L.view(dx_n).data_ptr()),
        ctypes.c_void_p(dw_n.data_ptr()), T, heads, H, st, sh, int(det), stream)
    assert status == rn.RMSN_OK, rn.status_string(status)
    dx_r, dw_r = rn.rmsnorm_bwd(L.view(dyb), L.view(xb), rstd, wd, residual=L.view(drb) if dres else None,
                                deterministic=det)
    torch.cuda.synchronize()
    assert np.array_equal(L.rows_of(dx_n), to_host_bits(dx_r.reshape(L.R, H))), "dx differs from rmsnorm_bwd"
    ref_dx, _, ref_dw = oracle.bwd_bf16(x, dy, w, rstd.cpu().numpy(), dr)
    rep = Report()
    check_dx(L.rows_of(dx_n), ref_dx, rep)
    check_dw(dw_n.cpu().numpy(), ref_dw, rep)
    if det:
        assert torch.equal(dw_n, dw_r), "deterministic dw differs from rmsnorm_bwd"
    else:
        check_dw(dw_r.cpu().numpy(), ref_dw, rep)
    return rep


# (larger, smaller) shape pairs covering the routes: the fixed-order pair with
# its partials in the scratch, one workgroup writing dw, and per-head views
CASES = [
    ((Layout.plain(4096, 1536), "bf16"), (Layout.plain(300, 1536), "bf16")),
    ((Layout.plain(16384, 4096), "f32"), (Layout.plain(3, 4096), "f32")),
    ((Layout.heads_view(2048, 24, 256, 8192, 256), "bf16"), (Layout.heads_view(100, 4, 256, 1024, 256), "bf16")),
    ((Layout.plain(8192, 6144), "bf16"), (Layout.plain(1000, 2048), "bf16")),
]


@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_rmsnorm_bwd_twice(case, det):
    import rmsnorm_fwd_amd as rn
    (big, wb), (small, ws) = CASES[case]
    print(f"noalloc case {case} det={det}: {big} then {small}", flush=True)
    r1 = _run(rn, big, wb, det, seed=90 + case, dres=case == 1)
    r2 = _run(rn, small, ws, det, seed=95 + case, dres=False)
    print(r1, r2)


def test_noalloc_refuses_a_route_beyond_its_scratch():
    import torch
    import rmsnorm_fwd_amd as rn
    T, H = 65536, 16384  # 256 chunk partials of 16384 doubles: 32 MiB and more
    assert rn.rmsnorm_bwd_workspace_size(T, 1, H) > rn.RMSN_NOALLOC_SCRATCH_BYTES
    t = torch.empty(8, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    status = rn.lib().rmsnorm_bwd_noalloc(p, p, p, p, 0, None, p, ctypes.c_void_p(dw.data_ptr()), T, 1, H, H, H, 1,
                                          None)
    assert status == rn.RMSN_ERR_WORKSPACE
