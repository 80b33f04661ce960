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

# One GPU's share of the 8192 x 17408 x 5120 BF16 A @ B product when it is
# split over g GPUs with no exchange between them (output tiles are
# independent): "rows<g>" takes M / g rows of A and D and all of B;
# "cols<g>" takes N / g columns of B and D and all of A.  Same distribution
# as the whole product, a seed of its own per shard.
SHARD_WORKLOADS = {
    "large_nn_%s%d" % (how, g): Workload(
        "large_nn_%s%d" % (how, g), "nn", "bf16", 8192 // g if how == "rows" else 8192,
        17408 // g if how == "cols" else 17408, 5120, "normal", 0.02,
        40 + g + (10 if how == "cols" else 0))
    for how in ("rows", "cols") for g in (2, 4, 8)
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


def small_integers_large(fmt: str, shape, seed: int, lo: int = -1, hi: int = 1,
                         chunk: int = 1 << 26) -> np.ndarray:
    """Integers uniform in [lo, hi] as FP16/BF16 bits, for operands of
    gigabytes: drawn as int8 in chunks of ``chunk`` values and encoded through
    a table of the few distinct values (a stream of its own, not the one
    ``small_integers`` draws)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    table = to_bits(fmt, np.arange(lo, hi + 1, dtype=np.float64))
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    for i in range(0, out.size, chunk):
        n = min(chunk, out.size - i)
        out[i:i + n] = table[rng.integers(0, hi - lo + 1, size=n, dtype=np.int8)]
    return out.reshape(shape)


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


# ---- FP8 block-scaled (MX) operands ----------------------------------------
#
# E4M3 element codes and E8M0 scale codes (one per 32 consecutive K values of
# a row), as byte arrays.  Two recipes:
#
# * "quantised": A then B drawn N(0, sigma^2) in float64; each block of 32
#   takes the power-of-two scale 2^e with e = floor(log2(max |x|)) - 8 (8 is
#   the exponent of E4M3's largest binade), and each value x / 2^e, clipped
#   to +-448, is rounded to E4M3 by torch's float8_e4m3fn cast (via float32).
#   This is the OCP microscaling recipe; it puts each block's largest values
#   in E4M3's top binade, as real quantised tensors do.
# * "codes": every finite E4M3 code equally likely (subnormals and both
#   zeros included) and scale codes uniform in [lo, hi].

E4M3_FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _quantise_blocks(x: np.ndarray):
    rows, K = x.shape
    nb = K // 32
    blocks = x.reshape(rows, nb, 32)
    amax = np.abs(blocks).max(axis=2)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0).astype(np.int64)
    e = np.clip(e, -127, 127)
    scaled = np.clip(blocks / np.exp2(e)[:, :, None], -448.0, 448.0).reshape(rows, K)
    return _e4m3_codes(scaled), (e + 127).astype(np.uint8)


@dataclass(frozen=True)
class MxWorkload:
    name: str
    M: int
    N: int
    K: int
    kind: str    # recipe of mx_operands
    seed: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The pages time their FP8 block-scaled GEMM on eight shapes they do not list;
# these two stand in: the FP16 page's size doubled in every dimension, and
# the BF16 tutorial's (8192, 5120) x (5120, 17408) product.
MX_WORKLOADS = {
    "mx_square": MxWorkload("mx_square", 8192, 8192, 8192, "quantised", 31),
    "mx_large": MxWorkload("mx_large", 8192, 17408, 5120, "quantised", 32),
}


def mx_operands(M: int, N: int, K: int, seed: int, kind: str = "quantised", sigma: float = 1.0,
                lo: int = 118, hi: int = 136):
    """(A, SA, B, SB) byte arrays: A M x K and B N x K E4M3 codes, SA M x K/32
    and SB N x K/32 E8M0 codes (K a multiple of 32)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "quantised":
        A, SA = _quantise_blocks(rng.standard_normal(size=(M, K)) * sigma)
        B, SB = _quantise_blocks(rng.standard_normal(size=(N, K)) * sigma)
        return A, SA, B, SB
    if kind == "codes":
        A = rng.choice(E4M3_FINITE, size=(M, K))
        B = rng.choice(E4M3_FINITE, size=(N, K))
        SA = rng.integers(lo, hi + 1, size=(M, K // 32)).astype(np.uint8)
        SB = rng.integers(lo, hi + 1, size=(N, K // 32)).astype(np.uint8)
        return A, SA, B, SB
    raise ValueError("unknown kind %r" % kind)


def mx_small_integers(M: int, N: int, K: int, seed: int, lo: int = -3, hi: int = 3):
    """Integer-valued E4M3 codes in [lo, hi] with scales 2^0 or 2^1: every
    product and partial sum is an integer far below 2^24, so the FP32
    accumulation is exact in any order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    A = _e4m3_codes(rng.integers(lo, hi + 1, size=(M, K)).astype(np.float64))
    B = _e4m3_codes(rng.integers(lo, hi + 1, size=(N, K)).astype(np.float64))
    SA = rng.integers(127, 129, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(127, 129, size=(N, K // 32)).astype(np.uint8)
    return A, SA, B, SB


def mx_small_integers_large(M: int, N: int, K: int, seed: int, lo: int = -1, hi: int = 1,
                            chunk: int = 1 << 26):
    """Integer-valued E4M3 codes in [lo, hi] with unit scales (2^0) for
    operands of gigabytes, drawn as int8 in chunks and encoded through a
    table: every partial sum is an integer of magnitude at most
    K * max(|lo|, |hi|)^2."""
    rng = np.random.Generator(np.random.PCG64(seed))
    table = _e4m3_codes(np.arange(lo, hi + 1, dtype=np.float64))

    def draw(rows):
        out = np.empty(rows * K, dtype=np.uint8)
        for i in range(0, out.size, chunk):
            n = min(chunk, out.size - i)
            out[i:i + n] = table[rng.integers(0, hi - lo + 1, size=n, dtype=np.int8)]
        return out.reshape(rows, K)

    A = draw(M)
    B = draw(N)
    SA = np.full((M, K // 32), 127, dtype=np.uint8)
    SB = np.full((N, K // 32), 127, dtype=np.uint8)
    return A, SA, B, SB


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
