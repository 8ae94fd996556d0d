"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module draws random bytes and numbers and nothing else: it holds none of
the product's arithmetic (no dequantization, no dot products, no layout or
padding rules).  Every stream comes from

    numpy PCG64(SeedSequence(1234, spawn_key=(config, matrix, stream)))

with stream 0 = quants, 1 = scales, 2 = activations, 3 = token ids.

Distributions (the workloads' statement of them):
  * Q8_0 quants: integers uniform in [-127, 127], stored as int8 bytes;
  * Q4_0 quants: nibbles uniform in [0, 15].  Two independent uniform nibbles
    make a uniform byte, so the packed array is drawn as uniform bytes;
  * scales: uniform in [1e-3, 1e-2), rounded to IEEE f16 or f32 (numpy's
    round-to-nearest-even casts);
  * activations: standard normal float32; bfloat16 activations are those
    float32 values rounded to nearest even on the top 16 bits;
  * token ids: uniform integers in [lo, hi].
"""
from __future__ import annotations

import numpy as np

SEED = 1234
STREAM_QUANTS, STREAM_SCALES, STREAM_ACT, STREAM_IDS = 0, 1, 2, 3


def rng(config: int, matrix: int, stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence(SEED, spawn_key=(config, matrix, stream))
    return np.random.Generator(np.random.PCG64(ss))


def q8_quants(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows*cols int8 quants in [-127, 127] (as a flat int8 array)."""
    return g.integers(-127, 128, size=rows * cols, dtype=np.int16).astype(np.int8)


def q4_quants(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows*cols/2 bytes, each holding two uniform nibbles."""
    return g.integers(0, 256, size=rows * cols // 2, dtype=np.int16).astype(np.uint8)


def scales(g: np.random.Generator, n: int, f16: bool,
           lo: float = 1e-3, hi: float = 1e-2) -> np.ndarray:
    v = g.uniform(lo, hi, size=n)
    return v.astype(np.float16) if f16 else v.astype(np.float32)


def act_f32(g: np.random.Generator, batch: int, cols: int) -> np.ndarray:
    return g.standard_normal(size=(batch, cols), dtype=np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bits
    as uint16.  NaNs stay quiet NaNs."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def act_bf16(g: np.random.Generator, batch: int, cols: int) -> np.ndarray:
    return f32_to_bf16_bits(act_f32(g, batch, cols))


def token_ids(g: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    return g.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)
