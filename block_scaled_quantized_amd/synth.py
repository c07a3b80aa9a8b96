"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers (numpy PCG64). It contains none of the method's arithmetic:
no quantisation, no scale rule, no decoding. Both the GPU path and the CPU oracle receive what it
returns and quantise it themselves.

Recipe: seed = 1000 + 10 * workload + operand (0 = left operand / activations, 1 = right operand /
weights). Sources are fp32: ``standard_normal(dtype=float32) * sigma`` for N(0, sigma^2) and
``2 * random(dtype=float32) - 1`` for U(-1, 1).
"""
from __future__ import annotations

import numpy as np

# Workload numbering used for seeds.
MXFP8_SMALL = 0      # MXFP8 GEMM M=128, N=256, K=128
F16_SQUARE = 1       # fp16 GEMM M=N=K=4096
MXFP8_PREFILL = 2    # MXFP8 GEMM M=2048, N=14336, K=4096
MATVEC = 3           # dequant matvec K=4096, N=14336, M in {1, 8}
MXFP4_LARGE = 4      # MXFP4 GEMM M=4096, N=8192, K=8192
WQ_PREFILL = 5       # int8/int4-weight GEMM, fp16 block scales: M=128 N=12288 K=4096; M=64 N=4096 K=4096


def seed_for(workload: int, operand: int) -> int:
    return 1000 + 10 * workload + operand


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(shape, sigma: float, seed: int) -> np.ndarray:
    """fp32 N(0, sigma^2)."""
    x = rng(seed).standard_normal(size=shape, dtype=np.float32)
    return x if sigma == 1.0 else (x * np.float32(sigma)).astype(np.float32)


def uniform_pm1(shape, seed: int) -> np.ndarray:
    """fp32 U(-1, 1)."""
    return (np.float32(2.0) * rng(seed).random(size=shape, dtype=np.float32) - np.float32(1.0)).astype(np.float32)


def random_bytes(shape, seed: int, exclude=()) -> np.ndarray:
    """Uniform random bytes; values listed in ``exclude`` are redrawn."""
    g = rng(seed)
    out = g.integers(0, 256, size=shape, dtype=np.uint8)
    if exclude:
        ex = np.array(sorted(exclude), dtype=np.uint8)
        bad = np.isin(out, ex)
        while bad.any():
            out[bad] = g.integers(0, 256, size=int(bad.sum()), dtype=np.uint8)
            bad = np.isin(out, ex)
    return out


def random_ints(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as uint8 (for scale codes)."""
    return rng(seed).integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.uint8)


def sample_points(M: int, N: int, count: int, seed: int):
    """Random (m, n) output positions, always including the four corners."""
    g = rng(seed)
    ms = g.integers(0, M, size=count, dtype=np.int64)
    ns = g.integers(0, N, size=count, dtype=np.int64)
    ms[:4] = [0, 0, M - 1, M - 1]
    ns[:4] = [0, N - 1, 0, N - 1]
    return ms, ns
