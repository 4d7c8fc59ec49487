"""Seeded synthetic inputs for the GEMM workloads.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds no matrix-multiplication arithmetic: it only draws operands.

Generator: numpy's PCG64 (``numpy.random.default_rng(seed)``).  A is drawn
first and B second, from one generator.

Distributions:
  * ``uniform``: i.i.d. uniform on [-1, 1), as ``2 * u - 1`` with ``u`` a
    float32 draw on [0, 1).  Every value is a multiple of 2**-23, so the
    transform is exact in float32 and -1 is attainable.
  * ``int4``: i.i.d. integers uniform on {-4, ..., 4}, stored as float32.
    Every partial sum of products is an integer of magnitude at most 16 * K,
    exact in float32 for K < 2**20, so any summation order gives the same
    bits.
  * ``normal``: A ~ N(0, 1); B ~ N(0, 0.02**2) (0.02 read as the standard
    deviation, the usual weight-initialisation scale), both float32.

Workloads (sizes are M x N x K; A is M x K, B is K x N, all row-major):
  * ``square256``    256 x 256 x 256, uniform (and ``square256_int4``)
  * ``square4096``   4096 x 4096 x 4096, uniform
  * ``square8192``   8192 x 8192 x 8192, uniform (the headline shape), and
                     ``square8192_int4`` with integer inputs: partial sums stay
                     below 16 * 8192 = 2**17, so the whole product is exact
  * ``ragged``       1000 x 1023 x 777, uniform (and ``ragged_int4``); no
                     dimension is a multiple of 32 or 64
  * ``ffn``          M = 8192 tokens, K = 4096, N = 14336, normal (an FFN
                     up-projection shape), and ``ffn_int4`` with integer inputs
  * ``batched64_1024`` 64 independent 1024 x 1024 x 1024 products, uniform
                     (A is 64 x M x K, B is 64 x K x N, drawn in that order)
  * ``deepk``        1024 x 1024 x 65536, uniform: few output tiles and a long
                     K, the shape that split-K serves
  * ``square8000``   8000 x 8000 x 8000, uniform: a large product whose M and N
                     are not whole 256-row tiles (rows still 16-byte aligned)
  * ``square8191``   8191 x 8191 x 8191, uniform: no dimension a multiple of 4,
                     so no row is 16-byte aligned
  * ``ktail8100``    8192 x 8192 x 8100, uniform: K is not a whole number of
                     32-k steps, rows are 16-byte aligned
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str
    seed: int = 0
    batch: int = 1

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("square256", 256, 256, 256, "uniform"),
        Workload("square256_int4", 256, 256, 256, "int4"),
        Workload("square4096", 4096, 4096, 4096, "uniform"),
        Workload("square8192", 8192, 8192, 8192, "uniform"),
        Workload("square8192_int4", 8192, 8192, 8192, "int4"),
        Workload("ragged", 1000, 1023, 777, "uniform"),
        Workload("ragged_int4", 1000, 1023, 777, "int4"),
        Workload("ffn", 8192, 14336, 4096, "normal"),
        Workload("ffn_int4", 8192, 14336, 4096, "int4"),
        Workload("batched64_1024", 1024, 1024, 1024, "uniform", batch=64),
        Workload("deepk", 1024, 1024, 65536, "uniform"),
        Workload("square8000", 8000, 8000, 8000, "uniform"),
        Workload("square8191", 8191, 8191, 8191, "uniform"),
        Workload("ktail8100", 8192, 8192, 8100, "uniform"),
    )
}

HEADLINE = "square8192"


def draw(rng: np.random.Generator, shape: tuple[int, ...], dist: str,
         scale: float = 1.0) -> np.ndarray:
    """One float32 matrix of the given distribution."""
    if dist == "uniform":
        u = rng.random(shape, dtype=np.float32)
        return (np.float32(2.0) * u - np.float32(1.0)).astype(np.float32, copy=False)
    if dist == "int4":
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        return x
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(M: int, N: int, K: int, dist: str = "uniform",
                seed: int = 0, batch: int = 1) -> tuple[np.ndarray, np.ndarray]:
    """Returns (A, B): A is M x K and B is K x N, float32, C-contiguous; with
    batch > 1, A is batch x M x K and B is batch x K x N."""
    rng = np.random.default_rng(seed)
    lead = (batch,) if batch > 1 else ()
    A = draw(rng, lead + (M, K), dist)
    B = draw(rng, lead + (K, N), dist, scale=0.02 if dist == "normal" else 1.0)
    return A, B


def workload_inputs(name: str, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    w = WORKLOADS[name]
    return make_inputs(w.M, w.N, w.K, w.dist, w.seed if seed is None else seed, w.batch)
