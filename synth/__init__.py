"""Seeded synthetic inputs for the training-RMSNorm workloads.

This module only draws random numbers and stores them as BF16 bit patterns
or float32; it holds none of the normalisation arithmetic.  Both the oracle
side and the HIP side of every test and of the benchmark take their inputs
from here.

Reproducibility: a tensor is cut into blocks of ``ROW_BLOCK`` rows and each
block draws from its own PCG64 stream seeded by ``SeedSequence([seed, tensor
id, block])``.  Any row range can therefore be regenerated on its own (the
full-size parity tests regenerate only the rows they sample), and blocks can
be drawn in parallel without changing a bit.

Distributions (the workloads' recipe):
  * ``normal``  -- N(0, 1)
  * ``outlier`` -- N(0, 1), then each element independently, with
    probability 0.001, multiplied by 50
  * ``offset``  -- N(3, 0.5)
  * weights     -- 1 + 0.1 * N(0, 1), drawn in float32; the BF16 weight is the
    round-to-nearest-even of that float32 draw.
Values are drawn in float32 and stored as BF16 with round-to-nearest-even.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os

import numpy as np

ROW_BLOCK = 512

TENSOR_IDS = {"x": 1, "r": 2, "dy": 3, "w": 4, "dres": 5, "g": 6}
FAMILIES = ("normal", "outlier", "offset")


def _rng(seed: int, tensor: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), TENSOR_IDS[tensor], int(block)])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_block(seed, tensor, block, H, family):
    g = _rng(seed, tensor, block)
    n = ROW_BLOCK * H
    if family == "normal":
        v = g.standard_normal(n, dtype=np.float32)
    elif family == "outlier":
        v = g.standard_normal(n, dtype=np.float32)
        mask = g.random(n, dtype=np.float32) < np.float32(0.001)
        v[mask] *= np.float32(50.0)
    elif family == "offset":
        v = np.float32(3.0) + np.float32(0.5) * g.standard_normal(n, dtype=np.float32)
    else:
        raise ValueError(f"unknown family {family!r}")
    return f32_to_bf16_bits(v).reshape(ROW_BLOCK, H)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rows(seed: int, tensor: str, row0: int, nrows: int, H: int,
         family: str = "normal") -> np.ndarray:
    """BF16 bits for rows [row0, row0 + nrows) of an [*, H] tensor."""
    out = np.empty((nrows, H), dtype=np.uint16)
    if nrows == 0:
        return out
    b0 = row0 // ROW_BLOCK
    b1 = (row0 + nrows - 1) // ROW_BLOCK

    def fill(b):
        blk = _draw_block(seed, tensor, b, H, family)
        lo = max(row0, b * ROW_BLOCK)
        hi = min(row0 + nrows, (b + 1) * ROW_BLOCK)
        out[lo - row0:hi - row0] = blk[lo - b * ROW_BLOCK:hi - b * ROW_BLOCK]

    blocks = range(b0, b1 + 1)
    if len(blocks) <= 2:
        for b in blocks:
            fill(b)
    else:
        with _fut.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, blocks))
    return out


def sampled_rows(seed: int, tensor: str, row_ids, H: int, family: str = "normal") -> np.ndarray:
    """BF16 bits of the listed rows only (each regenerated from its block)."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    out = np.empty((row_ids.size, H), dtype=np.uint16)
    cache = {}
    for i, r in enumerate(row_ids):
        b = int(r) // ROW_BLOCK
        if b not in cache:
            cache[b] = _draw_block(seed, tensor, b, H, family)
        out[i] = cache[b][int(r) - b * ROW_BLOCK]
    return out


def weight(seed: int, H: int, dtype: str = "bf16") -> np.ndarray:
    """w = 1 + 0.1 * N(0, 1): BF16 bits (dtype='bf16') or float32 ('f32')."""
    g = _rng(seed, "w", 0)
    w32 = (np.float32(1.0) + np.float32(0.1) * g.standard_normal(H, dtype=np.float32)).astype(np.float32)
    if dtype == "f32":
        return w32
    if dtype == "bf16":
        return f32_to_bf16_bits(w32)
    raise ValueError(dtype)
