"""Helpers for the GPU parity tests: device transfer, the acceptance
tolerance, and sampled checks at full size."""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def to_host(t) -> np.ndarray:
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(C: np.ndarray, ref64: np.ndarray, K: int, what: str = "") -> dict:
    """Acceptance bar for float inputs: no NaN, max |C - ref| <= 1e-4 sqrt(K)
    and relative Frobenius error <= 1e-5, against the FP64 sums."""
    assert C.shape == ref64.shape, (C.shape, ref64.shape)
    assert not np.isnan(C).any(), f"{what}: NaN in result"
    err = np.abs(C.astype(np.float64) - ref64)
    max_err = float(err.max()) if err.size else 0.0
    norm = float(np.linalg.norm(ref64))
    rel = float(np.linalg.norm(C.astype(np.float64) - ref64)) / norm if norm > 0 else 0.0
    bound = 1e-4 * math.sqrt(max(K, 1))
    assert max_err <= bound, f"{what}: max abs error {max_err:.3e} > {bound:.3e}"
    assert rel <= 1e-5, f"{what}: relative Frobenius error {rel:.3e} > 1e-5"
    return {"max_err": max_err, "rel_fro": rel}


def assert_exact(C: np.ndarray, ref32: np.ndarray, what: str = "") -> None:
    """Bit-exact comparison of values (+0 and -0 compare equal)."""
    assert C.shape == ref32.shape
    bad = np.argwhere(C != ref32)
    assert bad.size == 0, (f"{what}: {len(bad)} cells differ, first at {tuple(bad[0])}: "
                           f"{C[tuple(bad[0])]} vs {ref32[tuple(bad[0])]}")


def sample_rows(M: int, tile: int = 256, count: int = 24, seed: int = 0) -> list[int]:
    """Rows to check at full size: the first and last row of the matrix,
    first/last rows of a few tile rows, and seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, min(tile - 1, M - 1), min(tile, M - 1)}
    n_tiles = (M + tile - 1) // tile
    for t in rng.choice(n_tiles, size=min(4, n_tiles), replace=False):
        rows.add(int(t) * tile)
        rows.add(min(int(t) * tile + tile - 1, M - 1))
    while len(rows) < count:
        rows.add(int(rng.integers(0, M)))
    return sorted(rows)


def freivalds(A: np.ndarray, B: np.ndarray, C: np.ndarray, seed: int = 0, trials: int = 2) -> float:
    """Relative residual ||C x - A (B x)|| / ||A (B x)|| for random sign
    vectors x, in FP64; O(N^2) work, independent of the O(N^3) product.
    For random signs its expected square equals the squared relative
    Frobenius error of C, so it is compared against the same 1e-5 bar."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for _ in range(trials):
        x = rng.choice([-1.0, 1.0], size=B.shape[1])
        ref = A.astype(np.float64) @ (B.astype(np.float64) @ x)
        got = C.astype(np.float64) @ x
        worst = max(worst, float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    return worst


def oracle_rows(A: np.ndarray, B: np.ndarray, rows: list[int]):
    return oracle.gemm(A, B, rows=rows, return_f64=True)
