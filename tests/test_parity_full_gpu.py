"""GPU parity at the workloads' full sizes: T=65536 x H=4096 (FP32 w, three
input families, five seeds), T=131072 x H=6144 with the fused residual (BF16
and FP32 w, with and without dres), the per-head views [32768,24,256] (token
stride 8192) and [32768,4,256], and the H=5120 token sweep.  y, h, rstd and
dx are checked on every row against the oracle (in row blocks), dw against
the oracle's full column sums in both modes, dx across modes and the
deterministic dw across ten calls over the whole tensors."""
import pytest

from tests.helpers import Layout, run_full

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("family", ["normal", "outlier", "offset"])
def test_t65536_h4096_w32(family, seed):
    rep = run_full(Layout.plain(65536, 4096), "f32", family=family, seed=seed)
    print(family, seed, rep)


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("dres", [False, True])
def test_t131072_h6144_residual(wdt, dres):
    rep = run_full(Layout.plain(131072, 6144), wdt, res=True, dres=dres, seed=0)
    print(wdt, dres, rep)


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("layout", [Layout.heads_view(32768, 24, 256, 8192, 256),
                                    Layout.heads_view(32768, 4, 256, 1024, 256)],
                         ids=["24x256_stride8192", "4x256_contiguous"])
def test_t32768_head_views(layout, wdt):
    rep = run_full(layout, wdt, seed=0)
    print(layout, wdt, rep)


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("T", [2048, 6144, 19968, 32768, 65536])
def test_h5120_token_sweep(T, wdt):
    rep = run_full(Layout.plain(T, 5120), wdt, seed=T)
    print(T, wdt, rep)
