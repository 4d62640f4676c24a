"""Seeded random shapes through the C ABI against the oracle: row counts
from 0 up, 1-24 heads, widths from 8 to 16384 (any multiple of 8, so every
layout and ragged tails), padded token and head strides, both weight dtypes,
residual with and without dres.  Each case also runs one random explicit
backward route (pair, atomic, one-pass or row-blocked column form, ticket
form) beside the default one and checks the gaps of its strided buffers, the
forward's repeatability, dx across modes and routes and the workspace left
clean (see tests.helpers.run_case).  The SiLU-gated forward and backward get
seeded random shapes of their own."""
import numpy as np
import pytest

from tests.helpers import Layout, run_case
from tests.test_gated_gpu import run_gated

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(8 * rng.choice([rng.integers(1, 64), rng.integers(64, 1025), rng.integers(1025, 2049)],
                               p=[0.3, 0.5, 0.2]))
        heads = int(rng.choice([1, 1, 2, 3, 5, 24]))
        T = int(rng.choice([0, 1, 2, rng.integers(3, 64), rng.integers(64, 600)], p=[0.05, 0.1, 0.1, 0.35, 0.4]))
        if T * heads * H > 12_000_000:
            T = max(1, 12_000_000 // (heads * H))
        sh = H + 8 * int(rng.integers(0, 4)) if heads > 1 else H
        st = heads * sh + 8 * int(rng.integers(0, 6))
        wdt = str(rng.choice(["bf16", "f32"]))
        res = bool(rng.random() < 0.3)
        dres = res and bool(rng.random() < 0.5)
        route = _random_route(rng)
        out.append(pytest.param(T, heads, H, st, sh, wdt, res, dres, route, i,
                                id=f"{i}-T{T}x{heads}-H{H}-f{route[0]}"))
    return out


def _random_route(rng):
    """(form, chunks[, col_chunks, col_vecs]) within the limits the ABI accepts."""
    form = int(rng.integers(0, 4))
    chunks = int(rng.choice([1, rng.integers(2, 64), rng.integers(64, 1200)]))
    if form < 2:
        return (form, chunks)
    cc = int(rng.choice([1, rng.integers(2, 16), rng.integers(16, 600)]))
    if form == 3:
        cc = max(cc, 2)
    return (form, chunks, cc, int(rng.choice([1, 2, 4, 8])))


@pytest.mark.parametrize("T,heads,H,st,sh,wdt,res,dres,route,seed", _cases())
def test_random_shape(T, heads, H, st, sh, wdt, res, dres, route, seed):
    L = Layout.heads_view(T, heads, H, st, sh) if heads > 1 else Layout.plain(T, H, pad=st - H)
    rep = run_case(L, wdt, res=res, dres=dres, seed=100 + seed, routes=[None, route])
    print(T, heads, H, st, sh, wdt, res, dres, route, rep)


def _gated_cases(n=16, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(8 * rng.choice([rng.integers(1, 128), rng.integers(128, 1025), rng.integers(1025, 2049)],
                               p=[0.3, 0.5, 0.2]))
        heads = int(rng.choice([1, 1, 3, 8]))
        T = int(rng.choice([0, 1, rng.integers(2, 100), rng.integers(100, 3000)], p=[0.05, 0.1, 0.45, 0.4]))
        if T * heads * H > 6_000_000:
            T = max(1, 6_000_000 // (heads * H))
        sh = H + 8 * int(rng.integers(0, 3)) if heads > 1 else H
        st = heads * sh + 8 * int(rng.integers(0, 4))
        wdt = str(rng.choice(["bf16", "f32"]))
        kind = str(rng.choice(["mixed", "normal", "open"]))
        out.append(pytest.param(T, heads, H, st, sh, wdt, kind, i, id=f"g{i}-T{T}x{heads}-H{H}-{kind}"))
    return out


@pytest.mark.parametrize("T,heads,H,st,sh,wdt,kind,seed", _gated_cases())
def test_random_gated_shape(T, heads, H, st, sh, wdt, kind, seed):
    L = Layout.heads_view(T, heads, H, st, sh) if heads > 1 else Layout.plain(T, H, pad=st - H)
    print(T, heads, H, st, sh, wdt, kind, run_gated(L, wdt, seed=300 + seed, kind=kind))
