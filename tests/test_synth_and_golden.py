"""Input generator properties and the oracle regression fixture (CPU)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_rows_are_reproducible_and_sliceable():
    a = synth.rows(7, "x", 0, 3 * synth.ROW_BLOCK + 5, 64)
    b = synth.rows(7, "x", 700, 300, 64)
    assert np.array_equal(a[700:1000], b)
    ids = [0, 1, 511, 512, 1536, 1540]
    assert np.array_equal(synth.sampled_rows(7, "x", ids, 64), a[ids])
    assert not np.array_equal(synth.rows(8, "x", 0, 10, 64), a[:10])
    assert not np.array_equal(synth.rows(7, "dy", 0, 10, 64), a[:10])


@pytest.mark.parametrize("family,mean,std", [("normal", 0.0, 1.0), ("offset", 3.0, 0.5)])
def test_family_moments(family, mean, std):
    v = synth.bf16_bits_to_f32(synth.rows(0, "x", 0, 256, 1024, family)).astype(np.float64)
    assert abs(v.mean() - mean) < 0.01
    assert abs(v.std() - std) < 0.01 * std + 0.005


def test_outlier_family():
    base = synth.bf16_bits_to_f32(synth.rows(0, "x", 0, 256, 1024, "normal"))
    v = synth.bf16_bits_to_f32(synth.rows(0, "x", 0, 256, 1024, "outlier"))
    frac = np.mean(np.abs(v) > 8.0)
    assert 0.0004 < frac < 0.0012   # about 0.1 % of elements are x50 (most exceed 8)
    assert np.abs(v).max() > 100 and np.abs(base).max() < 7


def test_weights():
    w32 = synth.weight(0, 4096, "f32")
    wbf = synth.weight(0, 4096, "bf16")
    assert w32.dtype == np.float32 and wbf.dtype == np.uint16
    assert np.array_equal(synth.f32_to_bf16_bits(w32), wbf)
    assert abs(w32.mean() - 1.0) < 0.01 and abs(w32.std() - 0.1) < 0.01


def test_f32_to_bf16_is_nearest_even():
    v = np.random.default_rng(0).standard_normal(50_000).astype(np.float32)
    assert np.array_equal(synth.f32_to_bf16_bits(v), oracle.bf16_round(v.astype(np.float64)))


def test_oracle_regression_fixture():
    from tests.golden import make_golden  # noqa: F401  (module imports only oracle/synth)
    with open(os.path.join(GOLDEN, "oracle_small.json")) as f:
        ref = json.load(f)
    got = make_golden.case()
    assert got == ref
