"""Seeded synthetic operands for the dense GEMM workloads.

This module holds no GEMM arithmetic.  It draws the input matrices, quantises
them to FP16 / BF16 bit patterns, and names the workloads; both the HIP path's
tests and benchmark and the CPU oracle's tests take their inputs from here, and
it imports neither of them.

Workloads (shapes and value distributions as the pages state them):

* ``single_tile``  -- "TIRx GEMM on Blackwell", section "V1: One tile, one
  path": one 128 x 128 x 64 tile, D = A @ B.T, FP16.
* ``k_loop``       -- same page, "V2: Add the K-loop": 128 x 128 with a long K.
* ``square_nt``    -- same page, "The short version": M = N = K = 4096, FP16.
* ``large_nn``     -- TileFoundry "Choosing schedules and instructions for a
  backend", section 1: a (8192, 5120) times b (5120, 17408), BF16.
* ``ragged_nt``    -- shapes that divide no tile size (3000 x 5000 x 4000), for
  the edge paths the pages leave unstated.

Generator: ``numpy.random.Generator(PCG64(seed))``; A is drawn first, then B,
in float64.  FP16 patterns come from numpy's round-to-nearest-even cast; BF16
patterns from a round-to-nearest-even cast to float32 followed by
round-half-even on the upper 16 bits.  The quantised arrays are the inputs.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    layout: str      # "nt": D = A @ B.T (B is N x K); "nn": D = A @ B (B is K x N)
    fmt: str         # "f16" or "bf16" (inputs and output)
    M: int
    N: int
    K: int
    dist: str        # "uniform" (U[-1, 1]) or "normal"
    sigma: float     # standard deviation for "normal"
    seed: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "single_tile": Workload("single_tile", "nt", "f16", 128, 128, 64, "uniform", 0.0, 1),
    "k_loop": Workload("k_loop", "nt", "f16", 128, 128, 4096, "uniform", 0.0, 2),
    "square_nt": Workload("square_nt", "nt", "f16", 4096, 4096, 4096, "normal", 0.125, 3),
    "large_nn": Workload("large_nn", "nn", "bf16", 8192, 17408, 5120, "normal", 0.02, 4),
    "ragged_nt": Workload("ragged_nt", "nt", "f16", 3000, 5000, 4000, "uniform", 0.0, 5),
}


def f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to FP16 (numpy's RNE cast) and return the bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16 via float32 and return the bits.

    The float32 value's upper 16 bits are kept after adding the round-half-
    even bias 0x7FFF + (bit 16); NaN stays a quiet NaN.
    """
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f32)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def to_bits(fmt: str, x: np.ndarray) -> np.ndarray:
    return f16_bits(x) if fmt == "f16" else bf16_bits(x)


def _draw(rng: np.random.Generator, w: Workload, shape) -> np.ndarray:
    if w.dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape)
    if w.dist == "normal":
        return rng.standard_normal(size=shape) * w.sigma
    raise ValueError("unknown distribution %r" % w.dist)


def operand_shapes(layout: str, M: int, N: int, K: int):
    """Row-major shapes of (A, B): A is M x K; B is N x K ("nt") or K x N ("nn")."""
    return (M, K), ((N, K) if layout == "nt" else (K, N))


def make_operands(w: Workload, seed: int | None = None, M=None, N=None, K=None):
    """Draw (A, B) as uint16 bit patterns for workload ``w``.

    ``M``, ``N``, ``K`` override the workload's sizes (same distribution) for
    scaled-down parity cases.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    sa, sb = operand_shapes(w.layout, M, N, K)
    A = to_bits(w.fmt, _draw(rng, w, sa))
    B = to_bits(w.fmt, _draw(rng, w, sb))
    return A, B


def small_integers(fmt: str, shape, seed: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Integers uniform in [lo, hi] as FP16/BF16 bits (exactly representable)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return to_bits(fmt, rng.integers(lo, hi + 1, size=shape).astype(np.float64))


def identity(fmt: str, n: int) -> np.ndarray:
    return to_bits(fmt, np.eye(n))


def ones(fmt: str, shape) -> np.ndarray:
    return to_bits(fmt, np.ones(shape))


def random_finite_bits(fmt: str, shape, seed: int) -> np.ndarray:
    """Uniformly random finite bit patterns (every exponent, subnormals, +-0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    emask = 0x7C00 if fmt == "f16" else 0x7F80
    bad = (out & emask) == emask
    while bad.any():
        out[bad] = rng.integers(0, 1 << 16, size=int(bad.sum()), dtype=np.uint32).astype(np.uint16)
        bad = (out & emask) == emask
    return out


def sample_indices(M: int, N: int, n: int, seed: int):
    """``n`` (row, col) pairs for spot checks of large outputs: uniform draws,
    with an eighth of them moved onto the last row, an eighth onto the last
    column, and the four corners (the ragged edges of the tiling)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = rng.integers(0, M, size=n).astype(np.int64)
    cols = rng.integers(0, N, size=n).astype(np.int64)
    q = n // 8
    rows[:q] = M - 1
    cols[q:2 * q] = N - 1
    if n >= 2 * q + 4:
        rows[2 * q:2 * q + 4] = [0, 0, M - 1, M - 1]
        cols[2 * q:2 * q + 4] = [0, N - 1, 0, N - 1]
    return rows, cols
