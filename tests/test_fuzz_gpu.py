"""Seeded random shapes through the C ABI against the oracle: row counts
from 0 up, 1-24 heads, widths from 8 to 16384 (any multiple of 8, so every
layout and ragged tails), padded token and head strides, both weight dtypes,
residual with and without dres.  Each case also checks the gaps of its
strided buffers, the forward's repeatability, dx across modes and the
workspace left clean (see tests.helpers.run_case)."""
import numpy as np
import pytest

from tests.helpers import Layout, run_case

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
        out.append(pytest.param(T, heads, H, st, sh, wdt, res, dres, i, id=f"{i}-T{T}x{heads}-H{H}"))
    return out


@pytest.mark.parametrize("T,heads,H,st,sh,wdt,res,dres,seed", _cases())
def test_random_shape(T, heads, H, st, sh, wdt, res, dres, seed):
    L = Layout.heads_view(T, heads, H, st, sh) if heads > 1 else Layout.plain(T, H, pad=st - H)
    rep = run_case(L, wdt, res=res, dres=dres, seed=100 + seed)
    print(T, heads, H, st, sh, wdt, res, dres, rep)
