"""CPU oracle for row-major FP32 ``C = A x B`` (FP64 accumulation).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It shares no code with the GPU path in
``dense_fp32_gemm_row_amd`` and never imports it.

The arithmetic lives in ``gemm_oracle.c`` (plain C, built with gcc): each
output cell is the dot product of a row of A with a column of B ("Tiled
Matrix Multiplication in CUDA", section 1; "Tiled GEMM: Matrix Multiplication
in CUDA", section 1), stored row-major ("Tiled Matrix Multiplication in CUDA",
section 2), with products and the running sum in FP64 and a single rounding
to FP32 at the end.  This module only marshals numpy arrays into that call.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(worked example, identity and permutation products, brute force in exact
integer arithmetic, closed forms, block identities, FP64 library cross-check).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gemm_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_gemm.so")

# Flags: no fast-math, no contraction; OpenMP over output rows.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall"]

_i64 = ctypes.c_int64
_fp = ctypes.POINTER(ctypes.c_float)
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, "-o", output, source]
    subprocess.run(cmd, check=True)
    return output


def _bind(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [
        _i64, _i64, _i64,
        _fp, _i64,
        _fp, _i64,
        _lp, _i64,
        _fp, _i64,
        _dp, _i64,
        ctypes.c_int,
    ]
    lib.oracle_default_threads.restype = ctypes.c_int
    lib.oracle_default_threads.argtypes = []
    return lib


_LIB: ctypes.CDLL | None = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library.

    With ``path`` given, loads that library instead of the default one; the
    mutation tests use this to run the pins against deliberately broken
    copies of the oracle.
    """
    global _LIB
    if path is not None:
        return _bind(path)
    if _LIB is None:
        if not os.path.exists(LIBRARY) or (
            os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)
        ):
            build()
        _LIB = _bind(LIBRARY)
    return _LIB


def default_threads(lib: ctypes.CDLL | None = None) -> int:
    return int((lib or load()).oracle_default_threads())


def _as_rows(x: np.ndarray, name: str) -> tuple[np.ndarray, int]:
    """Returns (array, leading dimension) for a row-major float32 2-D array.

    Rows may be strided (a column slice of a wider array); elements within a
    row must be contiguous.
    """
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    rows, cols = x.shape
    if cols > 1 and x.strides[1] != 4:
        x = np.ascontiguousarray(x)
    ld = x.strides[0] // 4 if rows > 1 else max(cols, 1)
    if x.strides[0] % 4 or ld < max(cols, 1):
        x = np.ascontiguousarray(x)
        ld = max(cols, 1)
    return x, ld


def gemm(A: np.ndarray, B: np.ndarray, *, rows=None, threads: int = 0,
         return_f64: bool = False, lib: ctypes.CDLL | None = None):
    """``C = A x B`` for float32 row-major A (M x K) and B (K x N).

    ``rows``: optional sequence of row indices; the result then holds only
    those rows of the product, in that order.  Returns the FP32 result, and
    with ``return_f64`` also the FP64 sums.
    """
    lib = lib or load()
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} x {B.shape}")
    M, K = A.shape
    N = B.shape[1]
    A, lda = _as_rows(A, "A")
    B, ldb = _as_rows(B, "B")
    if rows is None:
        rows_arr = None
        nrows = M
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.shape[0]
    C = np.zeros((nrows, N), dtype=np.float32)
    C64 = np.zeros((nrows, N), dtype=np.float64) if return_f64 else None
    rc = lib.oracle_gemm(
        M, N, K,
        A.ctypes.data_as(_fp), lda,
        B.ctypes.data_as(_fp), ldb,
        rows_arr.ctypes.data_as(_lp) if rows_arr is not None else None, nrows,
        C.ctypes.data_as(_fp), max(N, 1),
        C64.ctypes.data_as(_dp) if C64 is not None else None, max(N, 1),
        int(threads),
    )
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed with code {rc}")
    return (C, C64) if return_f64 else C
