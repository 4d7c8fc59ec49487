"""The no-allocation split-K entry point (gemm_f32_splitk_noalloc) against
the one that takes a caller's workspace (gemm_f32_splitk), through the C
ABI: the same kernels run on the library's static scratch instead, so the
results must agree bit for bit, and both must meet the oracle's bar
(integer inputs exact, float inputs within tolerance).  Two calls in a row,
the second smaller, so the second runs on scratch that still holds the
first call's partial products."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_fp32_gemm_row_amd import binding as b
from dense_fp32_gemm_row_amd.workloads import make_inputs
from tests.gpu_util import assert_close, assert_exact, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _pair(A, B, splits):
    import torch

    M, N = A.shape[0], B.shape[1]
    dA, dB = to_dev(A), to_dev(B)
    ref = b.gemm_splitk(dA, dB, splits)
    out = torch.full((M, N + 2), float("nan"), device="cuda:0")
    b.gemm_splitk(dA, dB, splits, out[:, :N], noalloc=True)
    got = to_host(out)
    assert np.isnan(got[:, N:]).all(), "write outside C's columns"
    return got[:, :N], to_host(ref)


@pytest.mark.parametrize("dist", ["int4", "uniform"])
def test_noalloc_splitk_matches_workspace_splitk(dist):
    import torch

    assert torch.cuda.is_available()
    b.load()
    # larger call first, then a smaller one on the same scratch
    for M, N, K, splits, seed in [(700, 650, 3000, 5, 91), (300, 277, 1029, 3, 92),
                                  (256, 256, 4160, 4, 93)]:
        log(f"noalloc split-K {M}x{N}x{K} splits {splits} {dist}")
        A, B = make_inputs(M, N, K, dist, seed=seed)
        got, ref = _pair(A, B, splits)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
            f"{M}x{N}x{K}: differs from gemm_f32_splitk"
        if dist == "int4":
            assert_exact(got, oracle.gemm(A, B), f"{M}x{N}x{K} noalloc")
        else:
            _, ref64 = oracle.gemm(A, B, return_f64=True)
            assert_close(got, ref64, K, f"{M}x{N}x{K} noalloc")


def test_noalloc_library_choice_and_limit():
    """splits = 0 takes the library's choice capped to what fits the scratch
    (8 slices of 1024 x 1024 fill its 32 MiB); an explicit request above the
    scratch is refused with nothing enqueued."""
    import torch

    M, N, K = 1024, 1024, 8192
    A, B = make_inputs(M, N, K, "int4", seed=94)
    dA, dB = to_dev(A), to_dev(B)
    out = torch.empty((M, N), device="cuda:0")
    b.gemm_splitk(dA, dB, 0, out, noalloc=True)
    assert_exact(to_host(out), oracle.gemm(A, B), "noalloc library choice")
    with pytest.raises(b.GemmError) as e:
        b.gemm_splitk(dA, dB, 16, out, noalloc=True)  # 16 slices of 4 MiB = 64 MiB
    assert e.value.code == b.GEMM_F32_EINVAL
