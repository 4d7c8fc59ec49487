"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``pin_*`` function takes a ``gemm(A, B, rows=None, return_f64=False)``
callable (the oracle, or a deliberately broken copy of it) and raises
``AssertionError`` on a mismatch.  ``tests/test_oracle_pins.py`` runs them on
the real oracle; ``tests/test_oracle_mutants.py`` runs them on broken copies
and expects at least one to fail for every planted mistake.

What pins the oracle:
  * the worked 4 x 4 example ("Tiled GEMM: Matrix Multiplication in CUDA",
    sections 3 and 5): the printed sums of block (0, 0) after each phase;
  * products with identity and permutation matrices, bit-exact for any
    float data (every product is x * 1 or x * 0, every sum adds exact zeros);
  * brute force in Python's exact integer arithmetic on small shapes;
  * closed forms: all-ones operands give K everywhere; rank-1 operands give
    K * a_i * b_j;
  * block identities (K-split additivity, row stacking, transposition);
  * an FP64 cross-check against numpy's float64 matmul (a library routine
    with its own summation order, so only agreement within FP64 rounding);
  * leading-dimension handling, row selection, empty shapes, thread-count
    invariance.

Run as a script (``python tests/oracle_pins.py --lib PATH``) it applies every
pin to the oracle library at PATH and exits non-zero if any pin fails.
"""

from __future__ import annotations

import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

from dense_fp32_gemm_row_amd.workloads import make_inputs  # noqa: E402

GOLDEN = os.path.join(_ROOT, "tests", "golden", "worked_example_4x4.txt")


def read_golden(path: str = GOLDEN) -> dict[str, np.ndarray]:
    """Parses the ``[name]`` / rows-of-numbers text fixture."""
    out: dict[str, list[list[float]]] = {}
    cur = None
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = line[1:-1]
                out[cur] = []
                continue
            out[cur].append([float(v) for v in line.split()])
    return {k: np.array(v, dtype=np.float32) for k, v in out.items()}


def brute_force_int(A: np.ndarray, B: np.ndarray) -> list[list[int]]:
    """Exact product in Python integers (inputs must hold integer values)."""
    M, K = A.shape
    N = B.shape[1]
    a = [[int(v) for v in row] for row in A]
    b = [[int(v) for v in row] for row in B]
    return [[sum(a[i][k] * b[k][j] for k in range(K)) for j in range(N)]
            for i in range(M)]


def _exact(C: np.ndarray, ref) -> None:
    ref = np.array(ref, dtype=np.float64).reshape(C.shape)
    assert C.shape == ref.shape, (C.shape, ref.shape)
    bad = np.argwhere(C.astype(np.float64) != ref)
    assert bad.size == 0, f"{len(bad)} cells differ, first at {bad[0]}"


def _bits_equal(X: np.ndarray, Y: np.ndarray) -> None:
    assert X.shape == Y.shape, (X.shape, Y.shape)
    # +0 and -0 compare equal (values, not encodings), NaN never expected
    assert not np.isnan(X).any()
    bad = np.argwhere(X != Y)
    assert bad.size == 0, f"{len(bad)} cells differ, first at {bad[0]}"


def _ints(rng, shape, lo=-4, hi=4):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_worked_example(gemm) -> None:
    g = read_golden()
    A, B = g["A"], g["B"]
    C = gemm(A, B)
    # final sums of block (0, 0), section 5 of the page
    _exact(C[:2, :2], g["final_block00"])
    # phase t = 0 covers k in {0, 1}: the product of the first K-slice
    P0 = gemm(np.ascontiguousarray(A[:, 0:2]), np.ascontiguousarray(B[0:2, :]))
    _exact(P0[:2, :2], g["phase0_block00"])
    # phase t = 1 adds k in {2, 3}; the two slices sum to the full product
    P1 = gemm(np.ascontiguousarray(A[:, 2:4]), np.ascontiguousarray(B[2:4, :]))
    _exact(P0 + P1, C)
    # the rest of the 4 x 4 result, by exact integer arithmetic
    _exact(C, brute_force_int(A, B))


def pin_identity(gemm) -> None:
    rng = np.random.default_rng(11)
    A = (2 * rng.random((37, 53), dtype=np.float32) - 1).astype(np.float32)
    B = rng.standard_normal((29, 41), dtype=np.float32)
    _bits_equal(gemm(A, np.eye(53, dtype=np.float32)), A)
    _bits_equal(gemm(np.eye(29, dtype=np.float32), B), B)


def pin_permutation(gemm) -> None:
    rng = np.random.default_rng(12)
    n = 45
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0  # row r of P selects column perm[r]
    B = rng.standard_normal((n, 31), dtype=np.float32)
    A = rng.standard_normal((23, n), dtype=np.float32)
    # (P B)[r] = B[perm[r]]
    _bits_equal(gemm(P, B), B[perm])
    # (A P)[:, perm[r]] = A[:, r]
    expect = np.empty_like(A)
    expect[:, perm] = A
    _bits_equal(gemm(A, P), expect)


def pin_small_int_brute_force(gemm) -> None:
    rng = np.random.default_rng(13)
    for M in range(0, 5):
        for N in range(0, 5):
            for K in range(0, 5):
                A = _ints(rng, (M, K))
                B = _ints(rng, (K, N))
                C = gemm(A, B)
                assert C.shape == (M, N)
                _exact(C, brute_force_int(A, B))
    for (M, N, K) in [(33, 65, 17), (9, 7, 31), (1, 40, 12), (40, 1, 12)]:
        A = _ints(rng, (M, K))
        B = _ints(rng, (K, N))
        _exact(gemm(A, B), brute_force_int(A, B))


def pin_closed_forms(gemm) -> None:
    # all-ones: every cell equals K
    for (M, N, K) in [(100, 103, 77), (3, 5, 1000)]:
        C = gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
        _exact(C, np.full((M, N), K))
    # rank one: A[i][k] = a_i, B[k][j] = b_j  ->  C[i][j] = K a_i b_j
    rng = np.random.default_rng(14)
    M, N, K = 57, 61, 91
    a = rng.integers(-9, 10, size=M)
    b = rng.integers(-9, 10, size=N)
    A = np.repeat(a[:, None], K, axis=1).astype(np.float32)
    B = np.repeat(b[None, :], K, axis=0).astype(np.float32)
    _exact(gemm(A, B), K * np.outer(a, b))
    # a single non-zero term: A = e_p e_q^T, so C = e_p (row q of B)
    A = np.zeros((M, K), np.float32)
    A[5, 17] = 1.0
    Bf = rng.standard_normal((K, N), dtype=np.float32)
    expect = np.zeros((M, N), np.float32)
    expect[5] = Bf[17]
    _bits_equal(gemm(A, Bf), expect)


def pin_block_identities(gemm) -> None:
    rng = np.random.default_rng(15)
    M, N, K = 41, 39, 77
    A = _ints(rng, (M, K))
    B = _ints(rng, (K, N))
    C = gemm(A, B)
    # K-split additivity at a split that is no tile multiple
    k1 = 13
    C1 = gemm(np.ascontiguousarray(A[:, :k1]), np.ascontiguousarray(B[:k1]))
    C2 = gemm(np.ascontiguousarray(A[:, k1:]), np.ascontiguousarray(B[k1:]))
    _exact(C1 + C2, C)
    # row stacking
    m1 = 17
    _exact(np.vstack([gemm(np.ascontiguousarray(A[:m1]), B),
                      gemm(np.ascontiguousarray(A[m1:]), B)]), C)
    # transposition: (A B)^T = B^T A^T, bit-exact even for float data since
    # the same exact products are summed in the same k order
    Af = rng.standard_normal((M, K), dtype=np.float32)
    Bf = rng.standard_normal((K, N), dtype=np.float32)
    _bits_equal(gemm(np.ascontiguousarray(Bf.T), np.ascontiguousarray(Af.T)).T,
                gemm(Af, Bf))


def pin_fp64_library(gemm) -> None:
    A, B = make_inputs(67, 45, 1000, "uniform", seed=16)
    C32, C64 = gemm(A, B, return_f64=True)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    scale = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64)
    # both sides are FP64 sums of the same exact products: they agree within
    # K * 2**-53 * sum|a||b| (any summation order)
    assert np.all(np.abs(C64 - ref) <= 1000 * 2.0**-53 * scale + 1e-300)
    # one rounding from FP64 to FP32
    _bits_equal(C32, C64.astype(np.float32))
    A, B = make_inputs(40, 50, 300, "normal", seed=17)
    C32, C64 = gemm(A, B, return_f64=True)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    scale = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64)
    assert np.all(np.abs(C64 - ref) <= 300 * 2.0**-53 * scale + 1e-300)


def pin_leading_dimensions(gemm) -> None:
    rng = np.random.default_rng(18)
    M, N, K = 29, 33, 21
    Awide = rng.standard_normal((M, K + 7), dtype=np.float32)
    Bwide = rng.standard_normal((K, N + 5), dtype=np.float32)
    A = Awide[:, 3:3 + K]  # lda = K + 7, offset start
    B = Bwide[:, :N]       # ldb = N + 5
    _bits_equal(gemm(A, B), gemm(np.ascontiguousarray(A), np.ascontiguousarray(B)))


def pin_row_selection(gemm) -> None:
    A, B = make_inputs(50, 37, 64, "uniform", seed=19)
    full = gemm(A, B)
    rows = [5, 0, 49, 17, 17]
    _bits_equal(gemm(A, B, rows=rows), full[rows])


def pin_empty(gemm) -> None:
    rng = np.random.default_rng(20)
    C = gemm(np.zeros((6, 0), np.float32), np.zeros((0, 9), np.float32))
    _exact(C, np.zeros((6, 9)))
    assert gemm(np.zeros((0, 4), np.float32), _ints(rng, (4, 3))).shape == (0, 3)
    assert gemm(_ints(rng, (3, 4)), np.zeros((4, 0), np.float32)).shape == (3, 0)


def pin_multi_row_accumulator_reset(gemm) -> None:
    # many rows per thread: a row accumulator carried over between rows shows
    A = np.ones((64, 3), np.float32)
    B = np.ones((3, 5), np.float32)
    _exact(gemm(A, B), np.full((64, 5), 3))


PINS = [
    pin_worked_example,
    pin_identity,
    pin_permutation,
    pin_small_int_brute_force,
    pin_closed_forms,
    pin_block_identities,
    pin_fp64_library,
    pin_leading_dimensions,
    pin_row_selection,
    pin_empty,
    pin_multi_row_accumulator_reset,
]


def _main(argv: list[str]) -> int:
    import argparse
    import functools

    import oracle

    ap = argparse.ArgumentParser()
    ap.add_argument("--lib", required=True)
    ap.add_argument("--threads", type=int, default=2)
    args = ap.parse_args(argv)
    lib = oracle.load(args.lib)
    gemm = functools.partial(oracle.gemm, lib=lib, threads=args.threads)
    failed = []
    for pin in PINS:
        try:
            pin(gemm)
        except Exception as e:  # noqa: BLE001 - report every failing pin
            failed.append(pin.__name__)
            print(f"FAIL {pin.__name__}: {type(e).__name__}: {e}", flush=True)
        else:
            print(f"ok   {pin.__name__}", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(_main(sys.argv[1:]))
