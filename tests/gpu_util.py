"""Helpers for the GPU parity tests: device transfer and the acceptance
bars (tolerance for float inputs, bit-exactness for integer inputs)."""

from __future__ import annotations

import math
import sys

import numpy as np


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
