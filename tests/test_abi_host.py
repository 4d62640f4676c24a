"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/rmsnorm.h declares, and rejects bad arguments before
making any HIP call; the workspace-size and route queries are pure."""
import ctypes
import os
import re
import subprocess

import pytest

import rmsnorm_fwd_amd as rn
from tests.helpers import prepared_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rmsnorm_\w+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(rn.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = rn.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rn.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(_declared()) <= exported


def test_library_is_gfx950_only():
    # the offload bundle of the built library names its code-object targets
    blob = open(rn.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}


BAD = ctypes.c_void_p(0x1001)     # never dereferenced: validation rejects it first
GOOD = ctypes.c_void_p(0x10000)   # 64 KiB aligned fake device address


def _fwd(**kw):
    a = dict(x=GOOD, r=None, w=GOOD, wd=0, y=GOOD, h=None, rstd=GOOD, T=4, heads=1, H=64,
             st=64, sh=64, eps=1e-6)
    a.update(kw)
    return rn.lib().rmsnorm_fwd(a["x"], a["r"], a["w"], a["wd"], a["y"], a["h"], a["rstd"], a["T"],
                                a["heads"], a["H"], a["st"], a["sh"], a["eps"], 1, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=12, st=12, sh=12), rn.RMSN_ERR_UNSUPPORTED),
    (dict(H=rn.RMSN_MAX_H + 8, st=rn.RMSN_MAX_H + 8), rn.RMSN_ERR_UNSUPPORTED),
    (dict(H=0), rn.RMSN_ERR_INVALID_ARG),
    (dict(T=-1), rn.RMSN_ERR_INVALID_ARG),
    (dict(heads=0), rn.RMSN_ERR_INVALID_ARG),
    (dict(wd=7), rn.RMSN_ERR_INVALID_ARG),
    (dict(eps=-1.0), rn.RMSN_ERR_INVALID_ARG),
    (dict(eps=float("nan")), rn.RMSN_ERR_INVALID_ARG),
    (dict(st=32), rn.RMSN_ERR_INVALID_ARG),                      # rows overlap
    (dict(heads=4, st=128, sh=64), rn.RMSN_ERR_INVALID_ARG),     # tokens overlap
    (dict(heads=4, st=256, sh=32), rn.RMSN_ERR_INVALID_ARG),     # heads overlap
    (dict(st=68), rn.RMSN_ERR_MISALIGNED),
    (dict(x=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(y=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(x=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(rstd=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(r=GOOD), rn.RMSN_ERR_INVALID_ARG),                     # residual without residual_out
    (dict(h=GOOD), rn.RMSN_ERR_INVALID_ARG),
    (dict(T=1 << 31), rn.RMSN_ERR_INVALID_ARG),
])
def test_fwd_rejects_bad_arguments(kw, status):
    assert _fwd(**kw) == status


def test_fwd_zero_rows_is_a_no_op():
    assert _fwd(T=0, x=None, y=None, rstd=None) == rn.RMSN_OK


def _bwd(**kw):
    a = dict(dy=GOOD, x=GOOD, rstd=GOOD, w=GOOD, wd=0, dres=None, dx=GOOD, dw=GOOD, ws=GOOD,
             wsb=1 << 30, T=4, heads=1, H=64, st=64, sh=64, det=1)
    a.update(kw)
    return rn.lib().rmsnorm_bwd(a["dy"], a["x"], a["rstd"], a["w"], a["wd"], a["dres"], a["dx"],
                                a["dw"], a["ws"], a["wsb"], a["T"], a["heads"], a["H"], a["st"],
                                a["sh"], a["det"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=20, st=20, sh=20), rn.RMSN_ERR_UNSUPPORTED),
    (dict(wd=2), rn.RMSN_ERR_INVALID_ARG),
    (dict(dw=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(ws=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(dy=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(dx=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(dres=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(ws=ctypes.c_void_p(0x10080)), rn.RMSN_ERR_MISALIGNED),  # not 256-byte aligned
    (dict(wsb=16), rn.RMSN_ERR_WORKSPACE),
    (dict(wsb=16, det=0), rn.RMSN_ERR_WORKSPACE),
])
def test_bwd_rejects_bad_arguments(kw, status):
    assert _bwd(**kw) == status


def test_workspace_size_follows_the_route():
    # the size is that of the route rmsnorm_bwd takes for the same arguments
    # (without dres at least that: it covers the gated backward's route too),
    # a pure function of them, never below the prepared part, and 0 for
    # invalid shapes or weight dtypes
    for (T, heads, H) in [(4096, 1, 1536), (65536, 1, 4096), (131072, 1, 6144), (32768, 24, 256),
                          (1, 1, 8), (0, 1, 64), (64, 1, 4096), (777, 1, 2048)]:
        for det in (0, 1):
            for wd in (0, 1):
                for res in (0, 1):
                    a = rn.rmsnorm_bwd_workspace_size(T, heads, H, wd, res, det)
                    assert a == rn.rmsnorm_bwd_workspace_size(T, heads, H, wd, res, det)
                    route = rn.rmsnorm_bwd_route(T, heads, H, wd, res, det)
                    own = rn.rmsnorm_bwd_workspace_size_for_route(T, heads, H, route)
                    assert a >= own > 0 and (a == own or not res)
                    assert a >= prepared_bytes(H)
                    if det:
                        assert route[0] in (rn.RMSN_FORM_PAIR, rn.RMSN_FORM_COLS)
    assert rn.rmsnorm_bwd_workspace_size(10, 1, 12) == 0
    assert rn.rmsnorm_bwd_workspace_size(-1, 1, 64) == 0
    assert rn.rmsnorm_bwd_workspace_size(10, 1, 64, w_dtype=2) == 0
    # the binding's workspace helper serves both modes with one allocation
    for (T, H) in [(64, 4096), (65536, 4096)]:
        both = max(rn.rmsnorm_bwd_workspace_size(T, 1, H, 0, False, d) for d in (0, 1))
        assert both == max(rn.rmsnorm_bwd_workspace_size(T, 1, H, deterministic=d) for d in (True, False))


def test_route_chunks_depend_only_on_shape():
    # deterministic dw is fixed by the chunking; it must not vary with anything
    # but the shape (and never with the device's compute-unit count).
    r1 = rn.rmsnorm_bwd_route(65536, 1, 4096, 1, 0, 1)
    r2 = rn.rmsnorm_bwd_route(65536, 1, 4096, 1, 0, 1)
    assert r1 == r2 and r1[1] >= 1


def _routed(route, det=1, T=4, H=64):
    return rn.lib().rmsnorm_bwd_routed(GOOD, GOOD, GOOD, GOOD, 0, None, GOOD, GOOD, GOOD, 1 << 30,
                                       T, 1, H, H, H, det, rn.RmsnRoute(*route), None)


@pytest.mark.parametrize("route,det", [
    ((rn.RMSN_FORM_ATOMIC, 4), 1),              # atomic accumulation is not deterministic
    ((rn.RMSN_FORM_PAIR, 0), 0),                # no workgroups
    ((rn.RMSN_FORM_PAIR, 65537), 0),            # too many
    ((7, 8), 0),                                # no such form
    ((rn.RMSN_FORM_PAIR, 8, 1, 8), 0),          # column fields on a row form
    ((rn.RMSN_FORM_COLS, 8, 0, 8), 1),          # no row blocks
    ((rn.RMSN_FORM_COLS, 8, 4097, 8), 1),       # too many row blocks
    ((rn.RMSN_FORM_COLS, 8, 1, 3), 1),          # slice width not a power of two
    ((rn.RMSN_FORM_COLS, 8, 1, 16), 1),         # slice wider than 8 vectors
    ((rn.RMSN_FORM_COLS_TICKET, 8, 4, 8), 1),   # tickets need the prepared workspace
    ((rn.RMSN_FORM_COLS_TICKET, 8, 1, 8), 0),   # a ticket needs two row blocks at least
    ((rn.RMSN_FORM_PAIR, 8, 0, 0, 2), 1),       # prefetch is 0 or 1
    ((rn.RMSN_FORM_PAIR, 8, 0, 0, -1), 1),
    ((rn.RMSN_FORM_COLS, 8, 2, 8, 1), 1),       # no next-row tile in the column forms
])
def test_routed_rejects_malformed_routes(route, det):
    assert _routed(route, det) == rn.RMSN_ERR_INVALID_ARG
    assert rn.rmsnorm_bwd_workspace_size_for_route(4, 1, 64, route) == 0 or det


def _noalloc(**kw):
    a = dict(dy=GOOD, x=GOOD, rstd=GOOD, w=GOOD, wd=0, dres=None, dx=GOOD, dw=GOOD, T=4, heads=1, H=64, st=64,
             sh=64, det=1)
    a.update(kw)
    return rn.lib().rmsnorm_bwd_noalloc(a["dy"], a["x"], a["rstd"], a["w"], a["wd"], a["dres"], a["dx"], a["dw"],
                                        a["T"], a["heads"], a["H"], a["st"], a["sh"], a["det"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=20, st=20, sh=20), rn.RMSN_ERR_UNSUPPORTED),
    (dict(wd=2), rn.RMSN_ERR_INVALID_ARG),
    (dict(dw=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(dy=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(dx=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(dres=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(st=32), rn.RMSN_ERR_INVALID_ARG),
    # H 16384 at 65536 rows routes to 256 chunks x 16384 FP64 partials: beyond the scratch
    (dict(T=65536, H=16384, st=16384, sh=16384), rn.RMSN_ERR_WORKSPACE),
])
def test_noalloc_rejects_bad_arguments(kw, status):
    # every one of these is refused on the host, before the scratch is touched
    assert _noalloc(**kw) == status


def test_noalloc_scratch_covers_every_width_up_to_8192():
    # the allocation-free call runs rmsnorm_bwd's route (with and without
    # dres) on its scratch
    for H in range(8, 8193, 8):
        for T in (1, 64, 4096, 65536, (1 << 30) // 8192 - 1):
            for det in (0, 1):
                for res in (0, 1):
                    route = rn.rmsnorm_bwd_route(T, 1, H, 0, res, det)
                    need = rn.rmsnorm_bwd_workspace_size_for_route(T, 1, H, route)
                    assert 0 < need <= rn.RMSN_NOALLOC_SCRATCH_BYTES, (H, T, det, res, need)


def test_status_strings():
    for s in range(6):
        assert rn.status_string(s)
    assert rn.status_string(99) == "unknown status"


def test_row_map_division_is_exact(tmp_path):
    # compiled with the host compiler against the library's internal header
    src = os.path.join(ROOT, "tests", "host", "row_map_check.cpp")
    exe = str(tmp_path / "row_map_check")
    csrc = os.path.join(ROOT, "rmsnorm_fwd_amd", "csrc")
    subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{csrc}", "-I/opt/rocm/include",
                    src, "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    assert " 0 failures" in out.stdout


# Host code under AddressSanitizer and UBSan (the GPU code is not built with
# sanitizers; these drivers need neither a GPU nor the HIP runtime).
SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def test_abi_layer_under_sanitizers(tmp_path):
    """api.cpp and route.cpp with stub launchers: every error path, and for a
    sweep of shapes every workspace access inside rmsnorm_bwd_workspace_size."""
    csrc = os.path.join(ROOT, "rmsnorm_fwd_amd", "csrc")
    exe = str(tmp_path / "abi_check")
    subprocess.run(["g++", "-std=c++17", *SANITIZE, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
                    os.path.join(ROOT, "tests", "host", "abi_check.cpp"), os.path.join(csrc, "api.cpp"),
                    os.path.join(csrc, "route.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout + out.stderr


def test_oracle_under_sanitizers(tmp_path):
    """Every exported oracle function on small and edge shapes, buffers of
    exact size."""
    exe = str(tmp_path / "oracle_check")
    subprocess.run(["gcc", "-std=c11", *SANITIZE, "-fopenmp", "-ffp-contract=off",
                    os.path.join(ROOT, "tests", "host", "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm", "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, env={**os.environ, "OMP_NUM_THREADS": "4"})
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout + out.stderr


def test_route_table_moves_from_column_forms_to_the_pair():
    # as rows grow: the one-pass column form (one launch, no partials), then
    # the two-launch column form, then the fixed-order pair; never back.  Both
    # modes and both weight dtypes take the same route (every routed form is
    # deterministic); with dres the same form and never more workgroups (so
    # a workspace sized without dres serves it); chunk counts stay within
    # their bounds
    order = {(rn.RMSN_FORM_COLS, True): 0, (rn.RMSN_FORM_COLS, False): 1, (rn.RMSN_FORM_PAIR, False): 2}
    for H in (256, 512, 1536, 2048, 4096, 5120, 6144, 8192, 16384):
        prev = 0
        for T in [1, 2, 3, 4, 7, 16, 64, 100, 256, 384, 449, 512, 768, 1024, 2048, 4096, 6143, 6144, 8192, 8193,
                  16384, 16385, 65536, 131072]:
            r = rn.rmsnorm_bwd_route(T, 1, H, 0, 0, 1)
            assert r == rn.rmsnorm_bwd_route(T, 1, H, 1, 0, 0)
            rr = rn.rmsnorm_bwd_route(T, 1, H, 0, 1, 1)
            assert rr == rn.rmsnorm_bwd_route(T, 1, H, 1, 1, 0)
            assert rr[0] == r[0] and rr[1] <= r[1], (H, T, r, rr)
            assert rn.rmsnorm_bwd_workspace_size(T, 1, H, 0, True) <= rn.rmsnorm_bwd_workspace_size(T, 1, H, 0, False)
            form, chunks, cc, cv, pf = r
            stage = order[(form, cc == 1)]
            assert stage >= prev, (H, T, r)
            prev = stage
            if form == rn.RMSN_FORM_PAIR:
                assert 1 <= chunks <= 512 and cc == cv == 0 and pf in (0, 1)
            else:
                assert 1 <= chunks <= min(T, 512 if cc > 1 else T) and cv in (1, 2, 4, 8) and 1 <= cc <= 64
                assert pf == 0
        assert rn.rmsnorm_bwd_route(1, 1, H, 0, 0, 1)[:3] == (rn.RMSN_FORM_COLS, 1, 1)
        assert prev == 2 and rn.rmsnorm_bwd_route(65536, 1, H, 0, 0, 1)[1] >= 256


def test_gated_route_table():
    # the gated backward's chunking (measured, see route.cpp): where it takes
    # the pair, 512 workgroups at H 1025-1536, 256 at every row count from
    # H 1537 to 6144, 256 up to 65536 rows and 512 above at H 6145-8192;
    # never more workgroups than row groups; the next-row tile is not a
    # route field there; both modes and weight dtypes alike
    for H in (1032, 1536, 1544, 2048, 3072, 4096, 4104, 5120, 6144, 6152, 8192):
        for T in (16384, 16385, 32768, 65536, 65537, 131072):
            r = rn.rmsnorm_gated_bwd_route(T, 1, H, 0, 1)
            assert r == rn.rmsnorm_gated_bwd_route(T, 1, H, 1, 0)
            form, chunks, cc, cv, pf = r
            assert form == rn.RMSN_FORM_PAIR and cc == cv == pf == 0
            want = 512 if H <= 1536 else (256 if H <= 6144 or T <= 65536 else 512)
            assert chunks == want, (H, T, r)
            # the size query without dres covers the gated route
            assert rn.rmsnorm_bwd_workspace_size(T, 1, H, 0, False) >= rn.rmsnorm_bwd_workspace_size_for_route(T, 1, H, r)


def test_row_count_limit_is_below_2_pow_30():
    r = rn.RmsnRoute()
    L = rn.lib()
    for heads in (1, 3, 24):
        last = ((1 << 30) - 1) // heads  # largest T with T * heads < 2^30
        assert L.rmsnorm_bwd_route(last, heads, 256, 0, 0, 1, ctypes.byref(r)) == rn.RMSN_OK
        assert L.rmsnorm_bwd_route(last + 1, heads, 256, 0, 0, 1, ctypes.byref(r)) == rn.RMSN_ERR_INVALID_ARG
        assert rn.rmsnorm_bwd_workspace_size(last, heads, 256) > 0
        assert rn.rmsnorm_bwd_workspace_size(last + 1, heads, 256) == 0


def _gfwd(**kw):
    a = dict(x=GOOD, g=GOOD, w=GOOD, wd=0, y=GOOD, rstd=GOOD, T=4, heads=1, H=64, st=64, sh=64, eps=1e-6)
    a.update(kw)
    return rn.lib().rmsnorm_gated_fwd(a["x"], a["g"], a["w"], a["wd"], a["y"], a["rstd"], a["T"], a["heads"],
                                      a["H"], a["st"], a["sh"], a["eps"], 1, None)


def _gbwd(**kw):
    a = dict(dy=GOOD, x=GOOD, g=GOOD, rstd=GOOD, w=GOOD, wd=0, dx=GOOD, dg=GOOD, dw=GOOD, ws=GOOD,
             wsb=1 << 30, T=4, heads=1, H=64, st=64, sh=64, det=1)
    a.update(kw)
    return rn.lib().rmsnorm_gated_bwd(a["dy"], a["x"], a["g"], a["rstd"], a["w"], a["wd"], a["dx"], a["dg"],
                                      a["dw"], a["ws"], a["wsb"], a["T"], a["heads"], a["H"], a["st"], a["sh"],
                                      a["det"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(g=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(H=12, st=12, sh=12), rn.RMSN_ERR_UNSUPPORTED),
    (dict(eps=-1.0), rn.RMSN_ERR_INVALID_ARG),
    (dict(st=32), rn.RMSN_ERR_INVALID_ARG),
    (dict(y=None), rn.RMSN_ERR_INVALID_ARG),
])
def test_gated_fwd_rejects_bad_arguments(kw, status):
    assert _gfwd(**kw) == status


def test_gated_fwd_zero_rows_is_a_no_op():
    assert _gfwd(T=0, x=None, g=None, y=None, rstd=None) == rn.RMSN_OK


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(dg=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(g=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(dg=BAD), rn.RMSN_ERR_MISALIGNED),
    (dict(dw=None), rn.RMSN_ERR_INVALID_ARG),
    (dict(wsb=16), rn.RMSN_ERR_WORKSPACE),
    (dict(wd=5), rn.RMSN_ERR_INVALID_ARG),
])
def test_gated_bwd_rejects_bad_arguments(kw, status):
    assert _gbwd(**kw) == status
