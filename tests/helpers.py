"""Shared test plumbing: move seeded inputs to the GPU in the layout a case
asks for, run the library through its C ABI, run the oracle on the same
inputs, and compare with the stated tolerances.

Tolerances (checked element by element):
  * h (residual output): bit-exact.
  * y and dx: within 1 BF16 unit in the last place of the oracle's FP64 value
    rounded once to BF16 (dx evaluated at the kernel's FP32 rstd).
  * rstd: relative error <= 1e-6 against the oracle's FP64 rstd.
  * dw: |dw - ref| <= 1e-4 + 1e-4 |ref| per element, ref being the FP64
    value evaluated at the kernel's FP32 rstd (p1 #8577 "Baselines and
    measurement"; p1 #8208 commit message).
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
with open(os.path.join(GOLDEN, "page_constants.json")) as _f:
    PAGE = {k: v["value"] for k, v in json.load(_f).items() if not k.startswith("_")}

EPS = PAGE["eps"]
DW_ATOL = PAGE["dw_atol"]
DW_RTOL = PAGE["dw_rtol"]
RSTD_RTOL = 1e-6
ULP_TOL = 1
SENTINEL = 0x7FC0  # a BF16 NaN written into the gaps of strided buffers


def torch():
    import torch as _t
    return _t


def bf16_ord(b: np.ndarray) -> np.ndarray:
    """Monotone integer image of BF16 bit patterns (+0 and -0 map to 0)."""
    b = b.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ord(a) - bf16_ord(b))


def max_ulp(a: np.ndarray, b: np.ndarray) -> int:
    """Largest ulp_dist over the elements, computed on the differing bit
    patterns only (most are equal), so that whole full-size tensors compare
    in seconds."""
    ne = a != b
    if not ne.any():
        return 0
    return int(ulp_dist(a[ne], b[ne]).max())


def to_dev_bf16(a: np.ndarray, device="cuda"):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to(device)


def to_host_bits(t) -> np.ndarray:
    tt = torch()
    return t.detach().contiguous().view(tt.int16).cpu().numpy().view(np.uint16)


@dataclass
class Layout:
    """How [T, heads, H] activations sit in their device buffers."""
    T: int
    heads: int
    H: int
    stride_t: int
    stride_h: int

    @property
    def R(self):
        return self.T * self.heads

    @staticmethod
    def plain(T, H, pad=0):
        return Layout(T, 1, H, H + pad, H)

    @staticmethod
    def heads_view(T, heads, H, stride_t, stride_h):
        return Layout(T, heads, H, stride_t, stride_h)

    def buffer_elems(self):
        if self.R == 0:
            return 0
        return (self.T - 1) * self.stride_t + (self.heads - 1) * self.stride_h + self.H

    def view(self, buf):
        t = torch()
        if self.heads == 1:
            return t.as_strided(buf, (self.T, self.H), (self.stride_t, 1))
        return t.as_strided(buf, (self.T, self.heads, self.H), (self.stride_t, self.stride_h, 1))

    def gap_mask(self) -> np.ndarray:
        """True for buffer elements that no row covers."""
        m = np.ones(self.buffer_elems(), dtype=bool)
        if self.R:
            starts = (np.arange(self.T)[:, None] * self.stride_t +
                      np.arange(self.heads)[None, :] * self.stride_h).ravel()
            m[(starts[:, None] + np.arange(self.H)[None, :]).ravel()] = False
        return m

    def place(self, rows: np.ndarray, device="cuda"):
        """Device buffer (sentinel in the gaps) holding rows[R, H] at this layout."""
        t = torch()
        buf = t.full((self.buffer_elems(),), SENTINEL, dtype=t.int16, device=device).view(t.bfloat16)
        if self.R:
            v = self.view(buf)
            v.copy_(to_dev_bf16(rows, device).view(v.shape))
        return buf

    def empty(self, device="cuda"):
        """Device buffer for an output, every element set to the sentinel."""
        t = torch()
        return t.full((self.buffer_elems(),), SENTINEL, dtype=t.int16, device=device).view(t.bfloat16)

    def rows_of(self, buf) -> np.ndarray:
        if self.R == 0:
            return np.zeros((0, self.H), np.uint16)
        return to_host_bits(self.view(buf).reshape(self.R, self.H))


def prepared_bytes(H: int) -> int:
    """Bytes at the start of a backward workspace that the non-deterministic
    forms keep zero between calls (header, FP64 accumulator, per-slice
    tickets; the layout include/rmsnorm.h's workspace calls describe)."""
    pad = lambda b: (b + 255) // 256 * 256  # noqa: E731
    return 256 + pad(8 * H) + pad(4 * ((H + 7) // 8))


def weight_dev(w: np.ndarray, device="cuda"):
    t = torch()
    if w.dtype == np.float32:
        return t.from_numpy(w).to(device)
    return to_dev_bf16(w, device)


@dataclass
class Report:
    y_ulp: int = 0
    dx_ulp: int = 0
    rstd_rel: float = 0.0
    dw_ratio: float = 0.0  # worst |err| / (atol + rtol |ref|)
    notes: dict = field(default_factory=dict)


def check_fwd(y, h, rstd, ref_y, ref_h, ref_rstd, rep: Report):
    if ref_h is not None:
        assert np.array_equal(h, ref_h), "residual output h differs from bf16(x + r)"
    rep.y_ulp = max(rep.y_ulp, max_ulp(y, ref_y))
    assert rep.y_ulp <= ULP_TOL, f"y off by {rep.y_ulp} ulp"
    if ref_rstd.size:
        rel = np.abs(rstd.astype(np.float64) - ref_rstd) / ref_rstd
        rep.rstd_rel = max(rep.rstd_rel, float(rel.max()))
    assert rep.rstd_rel <= RSTD_RTOL, f"rstd rel error {rep.rstd_rel}"


def check_dx(dx, ref_dx, rep: Report):
    rep.dx_ulp = max(rep.dx_ulp, max_ulp(dx, ref_dx))
    assert rep.dx_ulp <= ULP_TOL, f"dx off by {rep.dx_ulp} ulp"


def check_dw(dw, ref_dw, rep: Report):
    err = np.abs(dw.astype(np.float64) - ref_dw)
    bound = DW_ATOL + DW_RTOL * np.abs(ref_dw)
    ratio = float((err / bound).max()) if err.size else 0.0
    rep.dw_ratio = max(rep.dw_ratio, ratio)
    assert ratio <= 1.0, f"dw error {ratio:.3f} of the budget"


def gen_case(seed, L: Layout, wdt: str, res: bool, dres: bool, family="normal"):
    x = synth.rows(seed, "x", 0, L.R, L.H, family)
    r = synth.rows(seed, "r", 0, L.R, L.H) if res else None
    dy = synth.rows(seed, "dy", 0, L.R, L.H)
    dr = synth.rows(seed, "dres", 0, L.R, L.H) if dres else None
    w = synth.weight(seed, L.H, wdt)
    return x, r, dy, dr, w


def run_case(L: Layout, wdt: str = "bf16", res: bool = False, dres: bool = False, seed: int = 0,
             family: str = "normal", det_repeats: int = 1, routes=None) -> Report:
    """Forward and backward (both modes) of one case through the C ABI,
    compared with the oracle element by element.  Also checks that the gaps
    of strided buffers stay untouched, that the forward is bitwise the same
    when repeated and under deterministic=False, that dx is bitwise the same
    in both modes, and that deterministic dw repeats bitwise."""
    import rmsnorm_fwd_amd as rn
    t = torch()
    rep = Report()
    x, r, dy, dr, w = gen_case(seed, L, wdt, res, dres, family)
    xb = L.place(x)
    rb = L.place(r) if res else None
    dyb = L.place(dy)
    drb = L.place(dr) if dres else None
    wd = weight_dev(w)
    gaps = L.gap_mask()

    def fwd(det):
        yb = L.empty()
        hb = L.empty() if res else None
        rstd = t.empty(L.R, dtype=t.float32, device="cuda")
        rn.rmsnorm_fwd(L.view(xb), wd, EPS, residual=L.view(rb) if res else None, deterministic=det,
                       y=L.view(yb), residual_out=L.view(hb) if res else None, rstd=rstd)
        return yb, hb, rstd

    yb, hb, rstd = fwd(True)
    ref_y, ref_h, ref_rstd = oracle.fwd_bf16(x, w, EPS, r)
    t.cuda.synchronize()
    y_h = L.rows_of(yb)
    h_h = L.rows_of(hb) if res else None
    rstd_h = rstd.cpu().numpy()
    check_fwd(y_h, h_h, rstd_h, ref_y, ref_h, ref_rstd, rep)
    for buf in (yb, hb):
        if buf is not None and gaps.any():
            assert np.all(to_host_bits(buf)[gaps] == SENTINEL), "write outside the view"
    yb2, hb2, rstd2 = fwd(False)
    assert np.array_equal(L.rows_of(yb2), y_h) and np.array_equal(rstd2.cpu().numpy(), rstd_h)
    if res:
        assert np.array_equal(L.rows_of(hb2), h_h)

    ub = hb if res else xb
    u = h_h if res else x
    ref_dx, _, ref_dw = oracle.bwd_bf16(u, dy, w, rstd_h, dr)
    ws = rn.rmsnorm_bwd_workspace(L.T, L.heads, L.H, "cuda")
    dx_bits = {}
    dw_det = None
    route_list = routes if routes is not None else [None]
    for det in (True, False):
        for route in route_list:
            if route is not None and det and route[0] not in (rn.RMSN_FORM_PAIR, rn.RMSN_FORM_COLS):
                continue
            for rep_i in range(det_repeats if det else 1):
                dxb = L.empty()
                dw = t.empty(L.H, dtype=t.float32, device="cuda")
                if route is None:
                    rn.rmsnorm_bwd(L.view(dyb), L.view(ub), rstd, wd, residual=L.view(drb) if dres else None,
                                   deterministic=det, dx=L.view(dxb), dw=dw, workspace=ws)
                else:
                    need = rn.rmsnorm_bwd_workspace_size_for_route(L.T, L.heads, L.H, route)
                    wsr = ws if need <= ws.numel() else rn.rmsnorm_bwd_workspace(L.T, L.heads, L.H, "cuda", nbytes=need)
                    rn.rmsnorm_bwd_routed(L.view(dyb), L.view(ub), rstd, wd, route,
                                          residual=L.view(drb) if dres else None, deterministic=det,
                                          dx=L.view(dxb), dw=dw, workspace=wsr)
                t.cuda.synchronize()
                dx_h = L.rows_of(dxb)
                dw_h = dw.cpu().numpy()
                if rep_i == 0:
                    check_dx(dx_h, ref_dx, rep)
                    check_dw(dw_h, ref_dw, rep)
                    if gaps.any():
                        assert np.all(to_host_bits(dxb)[gaps] == SENTINEL), "write outside the view"
                    key = "ref"
                    if key in dx_bits:
                        assert np.array_equal(dx_bits[key], dx_h), "dx differs between modes or routes"
                    else:
                        dx_bits[key] = dx_h
                if det:
                    if dw_det is None or route is not None:
                        dw_det = dw_h
                    else:
                        assert np.array_equal(dw_det, dw_h), "deterministic dw not reproducible"
    # the atomic and ticket forms leave their accumulator and tickets at zero
    assert int(ws[:prepared_bytes(L.H)].count_nonzero()) == 0, "non-deterministic workspace not left clean"
    return rep


def run_full(L: Layout, wdt: str = "bf16", res: bool = False, dres: bool = False, seed: int = 0,
             family: str = "normal", det_repeats: int = 9, block_elems: int = 1 << 27) -> Report:
    """Full-size case: the whole forward and backward run on the GPU, and y,
    h, rstd and dx of EVERY row are compared with the oracle, in blocks of
    tokens of about block_elems elements (the oracle runs each block on the
    host cores); dw against the oracle's full column sums in both modes; the
    forward bitwise across repeats and modes, dx bitwise between modes, and
    the deterministic dw bitwise over 1 + det_repeats calls, on the device."""
    import rmsnorm_fwd_amd as rn
    t = torch()
    rep = Report()
    R, H = L.R, L.H
    x, r, dy, dr, w = gen_case(seed, L, wdt, res, dres, family)
    xb = L.place(x)
    rb = L.place(r) if res else None
    dyb = L.place(dy)
    drb = L.place(dr) if dres else None
    wd = weight_dev(w)

    def fwd(det):
        yb = L.empty()
        hb = L.empty() if res else None
        rstd = t.empty(R, dtype=t.float32, device="cuda")
        rn.rmsnorm_fwd(L.view(xb), wd, EPS, residual=L.view(rb) if res else None, deterministic=det,
                       y=L.view(yb), residual_out=L.view(hb) if res else None, rstd=rstd)
        return yb, hb, rstd

    yb, hb, rstd = fwd(True)
    yb2, hb2, rstd2 = fwd(False)
    assert t.equal(L.view(yb2), L.view(yb)) and t.equal(rstd2, rstd), "forward not bitwise repeatable"
    if res:
        assert t.equal(L.view(hb2), L.view(hb))
    del yb2, hb2, rstd2
    rstd_h = rstd.cpu().numpy()

    ub = hb if res else xb
    ws = rn.rmsnorm_bwd_workspace(L.T, L.heads, L.H, "cuda", w_dtype=rn.RMSN_W_F32 if wdt == "f32" else rn.RMSN_W_BF16,
                                  has_residual=dres)

    def bwd(det):
        dxb = L.empty()
        dw = t.empty(H, dtype=t.float32, device="cuda")
        rn.rmsnorm_bwd(L.view(dyb), L.view(ub), rstd, wd, residual=L.view(drb) if dres else None,
                       deterministic=det, dx=L.view(dxb), dw=dw, workspace=ws)
        return dxb, dw

    dx_det, dw_det = bwd(True)
    for _ in range(det_repeats):
        dxb, dw = bwd(True)
        assert t.equal(dw, dw_det), "deterministic dw not reproducible"
        del dxb
    dx_nd, dw_nd = bwd(False)
    assert t.equal(L.view(dx_nd), L.view(dx_det)), "dx differs between modes"
    del dx_nd

    # every row, in blocks of tokens
    per_token = L.heads * H
    bt = max(1, block_elems // per_token)
    for t0 in range(0, L.T, bt):
        t1 = min(L.T, t0 + bt)
        rows = slice(t0 * L.heads, t1 * L.heads)

        def blk(buf):
            return to_host_bits(L.view(buf)[t0:t1].reshape(-1, H))

        ref_y, ref_h, ref_rstd = oracle.fwd_bf16(x[rows], w, EPS, r[rows] if res else None)
        check_fwd(blk(yb), blk(hb) if res else None, rstd_h[rows], ref_y, ref_h, ref_rstd, rep)
        u_rows = ref_h if res else x[rows]
        ref_dx, _, _ = oracle.bwd_bf16(u_rows, dy[rows], w, rstd_h[rows], dr[rows] if dres else None)
        check_dx(blk(dx_det), ref_dx, rep)
    u_full = oracle.residual_add(x, r) if res else x
    ref_dw = oracle.dw_bf16(u_full, dy, rstd_h)
    check_dw(dw_det.cpu().numpy(), ref_dw, rep)
    check_dw(dw_nd.cpu().numpy(), ref_dw, rep)
    return rep
