"""Parity of every HIP kernel with the CPU oracle, through the C ABI.

Bars: integer-valued inputs bit-exact; float inputs within
max |C - ref| <= 1e-4 sqrt(K) and relative Frobenius error <= 1e-5 against
the oracle's FP64 sums; no NaN anywhere.  Every test compares every cell of
C with the oracle, the full-size shapes included: they run in the launch
configuration the benchmark times (gemm_f32's own choice), and the oracle
computes the whole product on the host's cores (about 12 s at 8192^3 on 16
cores).
"""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from dense_fp32_gemm_row_amd import binding as b
from dense_fp32_gemm_row_amd.workloads import WORKLOADS, make_inputs, workload_inputs
from tests import oracle_pins
from tests.gpu_util import assert_close, assert_exact, log, to_dev, to_host

pytestmark = pytest.mark.gpu

ALL_CONFIGS = [(v, c, b.gemm_f32_config_name(v, c)) for v in range(4)
               for c in range(b.gemm_f32_config_count(v))] if os.path.exists(b.LIBRARY) else []
CONFIG_IDS = [name for _, _, name in ALL_CONFIGS]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    b.load()
    oracle.load()
    yield
    torch.cuda.synchronize()


def run(A: np.ndarray, B: np.ndarray, variant=None, config=-1, ldc_pad=0):
    import torch

    M, N = A.shape[0], B.shape[1]
    dA, dB = to_dev(A), to_dev(B)
    if ldc_pad:
        buf = torch.full((M, N + ldc_pad), float("nan"), device="cuda:0")
        dC = buf[:, :N]
    else:
        dC = torch.empty((M, N), device="cuda:0")
    b.gemm(dA, dB, dC, variant=variant, config=config)
    if ldc_pad:
        assert bool(torch.isnan(buf[:, N:]).all()), "write outside C's columns"
    return to_host(dC)


# --------------------------------------------------------------------------
# the worked example of the pages, on every kernel configuration
# --------------------------------------------------------------------------

@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_worked_example(v, c, name):
    log(f"worked example on {name}")
    g = oracle_pins.read_golden()
    C = run(g["A"], g["B"], v, c)
    assert_exact(C[:2, :2], g["final_block00"], name)
    assert_exact(C, oracle.gemm(g["A"], g["B"]), name)


# --------------------------------------------------------------------------
# every configuration: several tiles plus a ragged tail in every dimension
# --------------------------------------------------------------------------

@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_ragged_uniform(v, c, name):
    M, N, K = 300, 277, 129
    log(f"ragged uniform {M}x{N}x{K} on {name}")
    A, B = make_inputs(M, N, K, "uniform", seed=5)
    C = run(A, B, v, c)
    _, ref64 = oracle.gemm(A, B, return_f64=True)
    assert_close(C, ref64, K, name)


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_integer_bit_exact(v, c, name):
    M, N, K = 257, 263, 131
    log(f"int4 {M}x{N}x{K} on {name}")
    A, B = make_inputs(M, N, K, "int4", seed=6)
    assert_exact(run(A, B, v, c), oracle.gemm(A, B), name)


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_identity_and_permutation(v, c, name):
    # bit-exact for any float data; on the matrix cores this also pins the
    # lane-to-element mapping of operands and accumulators
    log(f"identity/permutation on {name}")
    rng = np.random.default_rng(7)
    A = rng.standard_normal((96, 80), dtype=np.float32)
    assert_exact(run(A, np.eye(80, dtype=np.float32), v, c), A, name + " A.I")
    n = 72
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0
    Bm = rng.standard_normal((n, 100), dtype=np.float32)
    assert_exact(run(P, Bm, v, c), Bm[perm], name + " P.B")
    expect = np.empty((40, n), np.float32)
    Am = rng.standard_normal((40, n), dtype=np.float32)
    expect[:, perm] = Am
    assert_exact(run(Am, P, v, c), expect, name + " A.P")


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_full_tiles(v, c, name):
    """Shapes that are whole tiles of every configuration: the unguarded
    path, with direct global-to-LDS loads where a configuration has them."""
    M, N, K = 512, 512, 96
    log(f"full tiles {M}x{N}x{K} on {name}")
    A, B = make_inputs(M, N, K, "int4", seed=13)
    assert_exact(run(A, B, v, c), oracle.gemm(A, B), name + " int4")
    A, B = make_inputs(M, N, K, "uniform", seed=14)
    _, ref64 = oracle.gemm(A, B, return_f64=True)
    assert_close(run(A, B, v, c), ref64, K, name + " uniform")
    rng = np.random.default_rng(15)
    X = rng.standard_normal((M, 512), dtype=np.float32)
    assert_exact(run(X, np.eye(512, dtype=np.float32), v, c), X, name + " A.I")
    perm = rng.permutation(512)
    P = np.zeros((512, 512), dtype=np.float32)
    P[np.arange(512), perm] = 1.0
    Y = rng.standard_normal((512, N), dtype=np.float32)
    assert_exact(run(P, Y, v, c), Y[perm], name + " P.B")
    # C rows at an odd stride inside a NaN guard band: whole tiles, but no
    # vector stores of C
    A, B = make_inputs(M, N, K, "int4", seed=16)
    assert_exact(run(A, B, v, c, ldc_pad=1), oracle.gemm(A, B), name + " int4 odd ldc")


EDGE_CASES = [  # M, N, K, padding of B's rows
    (520, 776, 96, 0),   # M and N edges, whole K-steps
    (520, 774, 96, 2),   # N not a multiple of 4 (B rows padded to 16 bytes)
    (3, 8, 64, 0),       # almost every row and column of a tile clamped
    (512, 512, 72, 0),   # whole tiles, partial last K-step
    (520, 776, 100, 0),  # edges and a partial last K-step
    (256, 256, 20, 0),   # K shorter than one K-step
]


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_edge_tiles_and_k_tail(v, c, name):
    """16-byte-aligned rows with M or N not whole tiles and/or K not whole
    K-steps.  The direct-load configurations keep direct loads: loads past M
    or N are clamped into the operands (the stores are guarded) and a partial
    last K-step is staged through registers with zero fill.  N = 774 is not a
    multiple of 4, so there the edge tiles fall back to register staging."""
    import torch

    for M, N, K, bpad in EDGE_CASES:
        log(f"edge tiles {M}x{N}x{K} (B padding {bpad}) on {name}")
        A, B = make_inputs(M, N, K, "int4", seed=17)
        dB = torch.full((K, N + bpad), float("nan"), device="cuda:0")
        dB[:, :N] = to_dev(B)
        buf = torch.full((M, N + 4), float("nan"), device="cuda:0")
        b.gemm(to_dev(A), dB[:, :N], buf[:, :N], variant=v, config=c)
        assert bool(torch.isnan(buf[:, N:]).all()), "write outside C's columns"
        assert_exact(to_host(buf[:, :N]), oracle.gemm(A, B), f"{name} int4 {M}x{N}x{K}")
        A, B = make_inputs(M, N, K, "uniform", seed=18)
        dB[:, :N] = to_dev(B)
        _, ref64 = oracle.gemm(A, B, return_f64=True)
        out = torch.empty((M, N), device="cuda:0")
        b.gemm(to_dev(A), dB[:, :N], out, variant=v, config=c)
        assert_close(to_host(out), ref64, K, f"{name} uniform {M}x{N}x{K}")


DEEP_PIPELINES = [(v, c, n) for v, c, n in ALL_CONFIGS
                  if v == 3 and n.split("_")[0] in ("mfma3d", "mfma4d")]


@pytest.mark.parametrize("v,c,name", DEEP_PIPELINES, ids=[n for _, _, n in DEEP_PIPELINES])
def test_deep_pipeline_short_k(v, c, name):
    """Three- and four-buffer direct-load loops hold the loads of one or two
    later tiles in flight across each barrier, and wait for fewer of them in
    the last K-steps.  Every trip count from 1 to 6 K-steps, with and without
    a partial last step, with 16-byte-aligned rows (16-byte direct loads) and
    without (4-byte direct loads, B's rows one float longer)."""
    import torch

    bk = int(name.split("_")[1].split("x")[2])
    M, N = 256, 256  # whole tiles of every configuration: the unguarded loop
    for steps in range(1, 7):
        for K in (steps * bk, steps * bk + 8):
            for bpad in (0, 1):
                log(f"{name}: K={K} ({steps} K-steps), B padding {bpad}")
                A, B = make_inputs(M, N, K, "int4", seed=50 + steps)
                dB = torch.zeros((K, N + bpad), device="cuda:0")
                dB[:, :N] = to_dev(B)
                out = torch.empty((M, N), device="cuda:0")
                b.gemm(to_dev(A), dB[:, :N], out, variant=v, config=c)
                assert_exact(to_host(out), oracle.gemm(A, B), f"{name} K={K} pad={bpad}")


@pytest.fixture(scope="module")
def huge_strided():
    """Operands whose rows lie more than 2^31 floats apart from the start:
    A has 3 rows lda = 2^30 + 64 floats apart, B 64 rows ldb = 2^25 + 4
    floats apart (about 21 GB of device memory, only the used rows written)."""
    import torch

    M, N, K = 3, 8, 64
    lda, ldb = (1 << 30) + 64, (1 << 25) + 4
    A, B = make_inputs(M, N, K, "int4", seed=41)
    bufA = torch.empty((M - 1) * lda + K, dtype=torch.float32, device="cuda:0")
    bufB = torch.empty((K - 1) * ldb + N, dtype=torch.float32, device="cuda:0")
    dA = bufA.as_strided((M, K), (lda, 1))
    dB = bufB.as_strided((K, N), (ldb, 1))
    dA.copy_(to_dev(A))
    dB.copy_(to_dev(B))
    yield A, B, dA, dB
    del dA, dB, bufA, bufB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_offsets_beyond_2_31(v, c, name, huge_strided):
    """Element offsets above 2^31 in A and in B: 64-bit row offsets in every
    kernel."""
    import torch

    A, B, dA, dB = huge_strided
    log(f"offsets beyond 2^31 on {name}")
    out = torch.full((A.shape[0], B.shape[1]), float("nan"), device="cuda:0")
    b.gemm(dA, dB, out, variant=v, config=c)
    assert_exact(to_host(out), oracle.gemm(A, B), name)


@pytest.fixture(scope="module")
def huge_unaligned():
    """Operands whose rows are not 16-byte aligned and lie so far apart that
    a tile's offsets pass 2^29 floats (the range of 4-byte buffer loads):
    A has 5 rows lda = 2^27 + 3 floats apart, B 67 rows ldb = 2^22 + 1
    floats apart (about 3.2 GB of device memory)."""
    import torch

    M, N, K = 5, 9, 67
    lda, ldb = (1 << 27) + 3, (1 << 22) + 1
    A, B = make_inputs(M, N, K, "int4", seed=43)
    bufA = torch.empty((M - 1) * lda + K, dtype=torch.float32, device="cuda:0")
    bufB = torch.empty((K - 1) * ldb + N, dtype=torch.float32, device="cuda:0")
    dA = bufA.as_strided((M, K), (lda, 1))
    dB = bufB.as_strided((K, N), (ldb, 1))
    dA.copy_(to_dev(A))
    dB.copy_(to_dev(B))
    yield A, B, dA, dB
    del dA, dB, bufA, bufB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_unaligned_rows_register_staging(v, c, name, huge_unaligned):
    """Rows not 16-byte aligned beyond the 4-byte direct loads' range: the
    register-staged loads, 16 bytes at 4-byte alignment where four floats
    are in range, zero fill per element at the edges of M, N and K."""
    import torch

    A, B, dA, dB = huge_unaligned
    log(f"unaligned rows beyond 2^29 floats on {name}")
    out = torch.full((A.shape[0], B.shape[1]), float("nan"), device="cuda:0")
    b.gemm(dA, dB, out, variant=v, config=c)
    assert_exact(to_host(out), oracle.gemm(A, B), name)


CLAMP_CASES = [  # M, N, K, lda, ldb: row lengths under 4 with rows 4 floats apart, odd strides
    (5, 3, 37, 37, 4), (70, 2, 33, 35, 4), (3, 65, 20, 21, 66), (257, 259, 47, 49, 261),
    (1, 4, 17, 17, 4), (33, 7, 16, 16, 7)]


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_clamped_edges_exact_storage(v, c, name):
    """Edge tiles of register-staged kernels load clamped: rows past M or N
    read the last row, 4-column groups past N the row's last group, and a
    group that starts inside the row reads past its end (never in the last
    k row, which the zero-filled tail stages).  Every operand is allocated to
    exactly its last element; A transposed covers the k-major flavour of A."""
    import torch

    ops_list = ["NN", "TN"] if v == 3 and name in TRANS_CAPABLE else ["NN"]
    for M, N, K, lda, ldb in CLAMP_CASES:
        for ops in ops_list:
            log(f"clamped edges {ops} {M}x{N}x{K} lda={lda} ldb={ldb} on {name}")
            A, B = make_inputs(M, N, K, "int4", seed=61)
            if ops[0] == "T":  # A stored K x M, rows lda' apart
                lda_t = max(M, 4) if M < 4 else M + 1
                bufA = torch.empty((K - 1) * lda_t + M, device="cuda:0")
                stored = bufA.as_strided((K, M), (lda_t, 1))
                stored.copy_(to_dev(np.ascontiguousarray(A.T)))
                dA = stored.t()
            else:
                bufA = torch.empty((M - 1) * lda + K, device="cuda:0")
                dA = bufA.as_strided((M, K), (lda, 1))
                dA.copy_(to_dev(A))
            bufB = torch.empty((K - 1) * ldb + N, device="cuda:0")
            dB = bufB.as_strided((K, N), (ldb, 1))
            dB.copy_(to_dev(B))
            out = torch.full((M, N), float("nan"), device="cuda:0")
            b.gemm(dA, dB, out, variant=v, config=c)
            assert_exact(to_host(out), oracle.gemm(A, B), f"{name} {ops} {M}x{N}x{K}")


# --------------------------------------------------------------------------
# the small workloads in full, library choice and every MFMA configuration
# --------------------------------------------------------------------------

SMALL = ["square256", "square256_int4", "ragged", "ragged_int4"]
MFMA_CONFIGS = [(3, c, n) for v, c, n in ALL_CONFIGS if v == 3]


@pytest.mark.parametrize("wname", SMALL)
@pytest.mark.parametrize("kernel", [None] + MFMA_CONFIGS + [(0, -1, "naive"), (1, -1, "lds"),
                                                            (2, -1, "regblock")],
                         ids=lambda k: "select" if k is None else k[2])
def test_small_workloads(wname, kernel):
    w = WORKLOADS[wname]
    log(f"{wname} on {'select' if kernel is None else kernel[2]}")
    A, B = workload_inputs(wname)
    C = run(A, B) if kernel is None else run(A, B, kernel[0], kernel[1])
    ref32, ref64 = oracle.gemm(A, B, return_f64=True)
    if w.dist == "int4":
        assert_exact(C, ref32, wname)
    else:
        assert_close(C, ref64, w.K, wname)


# --------------------------------------------------------------------------
# layout, edges and semantics
# --------------------------------------------------------------------------

@pytest.mark.parametrize("variant", [0, 1, 2, 3, None], ids=["naive", "lds", "regblock", "mfma", "select"])
def test_leading_dimensions_and_guard_band(variant):
    """Operands are sub-matrices of wider allocations (unaligned lda, offset
    start) and C sits in a NaN-filled buffer: only C's M x N region may
    change."""
    import torch

    log(f"leading dims on variant {variant}")
    rng = np.random.default_rng(8)
    M, N, K = 211, 190, 97
    Aw = rng.integers(-4, 5, size=(M, K + 5)).astype(np.float32)
    Bw = rng.integers(-4, 5, size=(K, N + 8)).astype(np.float32)
    dAw, dBw = to_dev(Aw), to_dev(Bw)
    dA = dAw[:, 1:1 + K]      # lda = K + 5, start offset by one float
    dB = dBw[:, :N]           # ldb = N + 8
    buf = torch.full((M + 2, N + 13), float("nan"), device="cuda:0")
    dC = buf[1:1 + M, 3:3 + N]  # ldc = N + 13, guard rows above and below
    b.gemm(dA, dB, dC, variant=variant)
    host = to_host(buf)
    inner = host[1:1 + M, 3:3 + N]
    assert_exact(inner, oracle.gemm(Aw[:, 1:1 + K], Bw[:, :N]), "leading dims")
    mask = np.ones_like(host, dtype=bool)
    mask[1:1 + M, 3:3 + N] = False
    assert np.isnan(host[mask]).all(), "a write landed outside C's region"


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_nan_padding_never_reaches_c(v, c, name):
    """The padding between the rows of A and B is NaN: kernels may read it
    (clamped edge loads do), but no such value may reach C."""
    import torch

    ops_list = ["NN", "TN"] if v == 3 and name in TRANS_CAPABLE else ["NN"]
    for M, N, K in [(300, 277, 129), (520, 774, 100), (257, 263, 131)]:
        for ops in ops_list:
            log(f"NaN padding {ops} {M}x{N}x{K} on {name}")
            A, B = make_inputs(M, N, K, "int4", seed=71)
            if ops[0] == "T":  # A stored K x M with 3 NaN columns per row
                bufA = torch.full((K, M + 3), float("nan"), device="cuda:0")
                bufA[:, :M] = to_dev(np.ascontiguousarray(A.T))
                dA = bufA[:, :M].t()
            else:
                bufA = torch.full((M, K + 3), float("nan"), device="cuda:0")
                bufA[:, :K] = to_dev(A)
                dA = bufA[:, :K]
            bufB = torch.full((K, N + 5), float("nan"), device="cuda:0")
            bufB[:, :N] = to_dev(B)
            out = torch.empty((M, N), device="cuda:0")
            b.gemm(dA, bufB[:, :N], out, variant=v, config=c)
            assert_exact(to_host(out), oracle.gemm(A, B), f"{name} {ops} {M}x{N}x{K}")


@pytest.mark.parametrize("v,c,name", ALL_CONFIGS, ids=CONFIG_IDS)
def test_deterministic(v, c, name):
    log(f"determinism on {name}")
    A, B = make_inputs(320, 288, 300, "uniform", seed=9)
    C1 = run(A, B, v, c)
    C2 = run(A, B, v, c)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), name


def test_naive_tiled_regblock_identical():
    """The naive, LDS-tiled and register-blocked kernels add each cell's
    products in ascending k with fused multiply-adds, so they agree to the
    bit ("Tiled Matrix Multiplication in CUDA", section 8)."""
    log("naive == tiled == register-blocked")
    A, B = make_inputs(300, 277, 129, "uniform", seed=10)
    base = run(A, B, 0, 0)
    for v in (0, 1, 2):
        for c in range(b.gemm_f32_config_count(v)):
            assert_exact(run(A, B, v, c), base, b.gemm_f32_config_name(v, c))


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_k_zero_gives_zeros(variant):
    import torch

    log(f"K = 0 on variant {variant}")
    dA = torch.empty((7, 0), device="cuda:0")
    dB = torch.empty((0, 9), device="cuda:0")
    buf = torch.full((7, 12), float("nan"), device="cuda:0")
    b.gemm(dA, dB, buf[:, :9], variant=variant)
    host = to_host(buf)
    assert (host[:, :9] == 0).all()
    assert np.isnan(host[:, 9:]).all()


def test_empty_m_leaves_output():
    import torch

    dA = torch.empty((0, 5), device="cuda:0")
    dB = torch.ones((5, 4), device="cuda:0")
    out = torch.empty((0, 4), device="cuda:0")
    b.gemm(dA, dB, out)
    assert out.shape == (0, 4)


def test_runs_on_callers_stream():
    import torch

    log("non-default stream")
    A, B = make_inputs(512, 512, 512, "int4", seed=11)
    dA, dB = to_dev(A), to_dev(B)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dC = torch.empty((512, 512), device="cuda:0")
        b.gemm(dA, dB, dC)
    s.synchronize()
    assert_exact(dC.cpu().numpy(), oracle.gemm(A, B), "stream")


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 300, 70), (300, 1, 70), (33, 65, 1),
                                   (64, 64, 777), (1000, 8, 8), (2, 3000, 5)])
def test_degenerate_shapes(shape):
    M, N, K = shape
    log(f"degenerate {shape}")
    A, B = make_inputs(M, N, K, "uniform", seed=12)
    _, ref64 = oracle.gemm(A, B, return_f64=True)
    for v in (None, 0, 1, 2, 3):
        assert_close(run(A, B, v), ref64, K, f"{shape} variant {v}")


# --------------------------------------------------------------------------
# strided batches
# --------------------------------------------------------------------------

BATCH_KERNELS = [(None, -1, "select"), (0, 0, "naive_64x4"), (1, 1, "lds_t32"),
                 (2, 0, "regblock_128x128x8_t8x8_pad4")] + [
    (3, c, n) for v, c, n in ALL_CONFIGS if v == 3 and n in (
        "mfma_64x64x32_w2x2_pa4_pb0", "mfma_256x256x16_w2x4_pa4_pb0", "mfma3_256x256x16_w4x4_swz_pb0",
        "mfma2p_256x256x32_w4x4_swz_pb0", "mfma3d_128x256x16_w2x4_swz", "mfma2d_256x256x32_w4x4_swz_g4",
        "mfma2d_256x256x32_w2x4_swz_g4_il", "mfma2d_256x256x32_w4x4_swz_g4_il",
        "mfma2d_64x64x128_w2x2_k4_swz", "mfma2d_64x64x64_w2x2_k4_swz",
        "mfma3_256x256x16_w4x4_swz_g4_il", "mfma2_64x64x64_w2x2_k4_swz",
        "mfmag_64x64x64_w1x1_k4_d3", "mfmag_128x128x64_w1x1_k4_d2")]


def _run_batched(A3, B3, M, N, K, nb, sa, sb, sc, lda, ldb, ldc, kernel):
    """Runs one strided-batched call on flat device buffers laid out with the
    given strides; returns the whole C buffer (NaN outside the products)."""
    import torch

    dA = to_dev(A3)
    dB = to_dev(B3)
    csize = (nb - 1) * sc + (M - 1) * ldc + N + 17
    dC = torch.full((csize,), float("nan"), device="cuda:0")
    v, c, name = kernel
    if v is None:
        rc = b.gemm_f32_strided_batched(nb, M, N, K, dA.data_ptr(), lda, sa, dB.data_ptr(), ldb,
                                        sb, dC.data_ptr(), ldc, sc, None)
    else:
        rc = b.gemm_f32_strided_batched_variant(v, c, nb, M, N, K, dA.data_ptr(), lda, sa,
                                                dB.data_ptr(), ldb, sb, dC.data_ptr(), ldc, sc,
                                                None)
    assert rc == 0, b.gemm_f32_last_error()
    return to_host(dC)


def _layout(rng, nb, rows, cols, ld, stride, dist):
    """A flat buffer holding nb matrices rows x cols (leading dimension ld,
    stride floats apart; stride 0 = one shared matrix), padding NaN-free."""
    n = (max(nb - 1, 0) * stride + (rows - 1) * ld + cols) if rows and cols else 1
    if dist == "int4":
        flat = rng.integers(-4, 5, size=n).astype(np.float32)
    else:
        flat = (2 * rng.random(n, dtype=np.float32) - 1).astype(np.float32)
    mats = [flat[i * stride: i * stride + (rows - 1) * ld + cols] for i in range(nb)]
    mats = [np.lib.stride_tricks.as_strided(m, shape=(rows, cols), strides=(4 * ld, 4))
            for m in mats]
    return flat, [np.ascontiguousarray(m) for m in mats]


@pytest.mark.parametrize("kernel", BATCH_KERNELS, ids=[k[2] for k in BATCH_KERNELS])
@pytest.mark.parametrize("dist", ["int4", "uniform"])
def test_strided_batched(kernel, dist):
    log(f"batched {dist} on {kernel[2]}")
    rng = np.random.default_rng(21)
    nb, M, N, K = 3, 130, 70, 50
    lda, ldb, ldc = K + 3, N + 1, N + 5
    sa = M * lda + 37            # gaps between the A matrices
    sb = 0                       # one B shared by every product
    sc = M * ldc + 11
    A_flat, As = _layout(rng, nb, M, K, lda, sa, dist)
    B_flat, Bs = _layout(rng, 1, K, N, ldb, 0, dist)
    Bs = Bs * nb
    C_all = _run_batched(A_flat, B_flat, M, N, K, nb, sa, sb, sc, lda, ldb, ldc, kernel)
    written = np.zeros(C_all.shape, dtype=bool)
    for i in range(nb):
        view = np.lib.stride_tricks.as_strided(C_all[i * sc:], shape=(M, N), strides=(4 * ldc, 4))
        ref32, ref64 = oracle.gemm(As[i], Bs[i], return_f64=True)
        if dist == "int4":
            assert_exact(np.array(view), ref32, f"{kernel[2]} product {i}")
        else:
            assert_close(np.array(view), ref64, K, f"{kernel[2]} product {i}")
        for r in range(M):
            written[i * sc + r * ldc: i * sc + r * ldc + N] = True
    assert np.isnan(C_all[~written]).all(), "a write landed outside the products' C regions"


@pytest.mark.parametrize("kernel", BATCH_KERNELS, ids=[k[2] for k in BATCH_KERNELS])
@pytest.mark.parametrize("shape", [(512, 256, 64), (520, 264, 64), (520, 264, 84)],
                         ids=["whole", "edge", "edge_ktail"])
def test_strided_batched_full_tiles(kernel, shape):
    """Whole tiles in every product (the unguarded and direct-load paths),
    and ragged M and N with whole K-steps (direct interior, guarded edges)."""
    import torch

    log(f"batched {shape} on {kernel[2]}")
    nb = 2
    M, N, K = shape
    A, B = make_inputs(nb * M, N, K, "int4", seed=22)
    A3 = A.reshape(nb, M, K)
    B3 = np.stack([B, (B[::-1] * -1).copy()])
    out = torch.empty((nb, M, N), device="cuda:0")
    v, c, _ = kernel
    b.gemm_batched(to_dev(A3), to_dev(B3), out, variant=v, config=c)
    got = to_host(out)
    for i in range(nb):
        assert_exact(got[i], oracle.gemm(A3[i], B3[i]), f"{kernel[2]} product {i}")


# --------------------------------------------------------------------------
# transposed operands
# --------------------------------------------------------------------------

TRANS_CAPABLE = ["mfma2d_256x256x32_w4x4_swz", "mfma3d_256x128x32_w4x2_swz",
                 "mfma3d_128x256x16_w2x4_swz", "mfma3_64x64x16_w2x2_swz_pb0",
                 "mfma3_128x128x16_w2x2_swz_pb0", "mfma2p_256x256x32_w4x4_swz_pb0",
                 "mfma2d_256x256x32_w4x4_swz_g4_il", "mfma2d_256x256x32_w4x2_swz_g4_il",
                 "mfma2d_256x256x32_w2x4_swz_g4_il", "mfma3d_256x128x32_w4x2_swz_il",
                 "mfma3d_128x256x16_w2x4_swz_il", "mfma3_64x128x16_w2x2_swz_il",
                 "mfma2d_256x256x32_w2x4_swz_g8_il", "mfma2d_256x256x32_w4x4_swz_g8_il",
                 "mfma2d_64x64x128_w2x2_k4_swz", "mfma2d_64x64x64_w2x2_k4_swz",
                 "mfma3d_64x64x64_w2x2_k4_swz", "mfma4d_64x64x64_w2x2_k4_swz",
                 "mfma3_256x256x16_w4x4_swz_g4_il", "mfma2_64x64x64_w2x2_k4_swz",
                 "mfma2d_128x128x32_w2x2_swz_il", "mfma2r_64x64x64_w2x2_k4_swz",
                 "mfmag_64x64x64_w1x1_k4_d3", "mfmag_128x128x64_w1x1_k4_d2",
                 "mfmag_128x128x64_w1x1_k4_d2_p", "mfmag_96x128x64_w1x1_k4_d2_p",
                 "mfmag_16x16x64_w1x1_k4_d2"] + [
    n for n in CONFIG_IDS if "_m16" in n]  # every 16x16x4 configuration takes them
TRANS_KERNELS = [(None, -1, "select"), (0, 0, "naive_64x4")] + [
    (3, c, n) for v, c, n in ALL_CONFIGS if v == 3 and n in TRANS_CAPABLE]
OPS = ["NN", "NT", "TN", "TT"]


def _stored(X: np.ndarray, op: str):
    """Device operand for op(X) = X: the tensor itself, or a transposed view
    of its transpose stored row-major."""
    if op == "N":
        return to_dev(X)
    return to_dev(np.ascontiguousarray(X.T)).T


@pytest.mark.parametrize("kernel", TRANS_KERNELS, ids=[k[2] for k in TRANS_KERNELS])
@pytest.mark.parametrize("ops", OPS)
@pytest.mark.parametrize("shape", [(300, 277, 129), (512, 512, 96), (520, 776, 96),
                                   (520, 776, 100)],
                         ids=["ragged", "full", "edge", "edge_ktail"])
def test_transposed_operands(kernel, ops, shape):
    import torch

    M, N, K = shape
    log(f"{ops} {shape} on {kernel[2]}")
    v, c, name = kernel
    A, B = make_inputs(M, N, K, "int4", seed=31)
    out = torch.empty((M, N), device="cuda:0")
    b.gemm(_stored(A, ops[0]), _stored(B, ops[1]), out, variant=v, config=c)
    assert_exact(to_host(out), oracle.gemm(A, B), f"{name} {ops} int4")
    A, B = make_inputs(M, N, K, "uniform", seed=32)
    b.gemm(_stored(A, ops[0]), _stored(B, ops[1]), out, variant=v, config=c)
    _, ref64 = oracle.gemm(A, B, return_f64=True)
    assert_close(to_host(out), ref64, K, f"{name} {ops} uniform")


@pytest.mark.parametrize("ops", ["NT", "TN", "TT"])
def test_transposed_batched(ops):
    import torch

    log(f"batched {ops}")
    nb, M, N, K = 3, 256, 192, 80
    A, B = make_inputs(M * nb, N * nb, K, "int4", seed=33)
    A3 = A.reshape(nb, M, K)
    B3 = np.stack([B[:, i * N:(i + 1) * N] for i in range(nb)])
    dA = to_dev(A3) if ops[0] == "N" else to_dev(np.ascontiguousarray(A3.transpose(0, 2, 1))).transpose(1, 2)
    dB = to_dev(B3) if ops[1] == "N" else to_dev(np.ascontiguousarray(B3.transpose(0, 2, 1))).transpose(1, 2)
    out = torch.empty((nb, M, N), device="cuda:0")
    b.gemm_batched(dA, dB, out)
    got = to_host(out)
    for i in range(nb):
        assert_exact(got[i], oracle.gemm(A3[i], B3[i]), f"batched {ops} product {i}")


def test_transposed_rejected_where_unsupported():
    """Configurations without transposed operands reject them with
    ENOKERNEL."""
    import torch

    A = torch.ones((64, 64), device="cuda:0")
    for v, c, name in ALL_CONFIGS:
        if v in (1, 2) or (v == 3 and name not in TRANS_CAPABLE):
            for X, Y in ((A.T, A), (A, A.T)):
                with pytest.raises(b.GemmError) as e:
                    b.gemm(X, Y, variant=v, config=c)
                assert e.value.code == b.GEMM_F32_ENOKERNEL, name


# --------------------------------------------------------------------------
# split-K
# --------------------------------------------------------------------------

SPLITK_KERNELS = [(None, -1, "select"), (0, 0, "naive_64x4"), (1, 1, "lds_t32"),
                  (2, 0, "regblock_128x128x8_t8x8_pad4")] + [
    (3, c, n) for v, c, n in ALL_CONFIGS if v == 3 and n in (
        "mfma_64x64x32_w2x2_pa4_pb0", "mfma3_64x64x16_w2x2_swz_pb0", "mfma3_128x128x16_w2x2_swz_pb0",
        "mfma3d_128x256x16_w2x4_swz", "mfma2d_256x256x32_w4x4_swz", "mfma2d_64x64x64_w2x2_k4_swz",
        "mfma2d_64x64x128_w2x2_k4_swz", "mfmag_64x64x64_w1x1_k4_d3", "mfmag_128x128x64_w1x1_k4_d2",
        "mfmag_128x128x64_w1x1_k4_d2_p", "mfmag_96x128x64_w1x1_k4_d2_p")]


@pytest.mark.parametrize("kernel", SPLITK_KERNELS, ids=[k[2] for k in SPLITK_KERNELS])
@pytest.mark.parametrize("splits", [2, 3, 7, 0])
def test_splitk(kernel, splits):
    import torch

    M, N, K = 300, 277, 1029
    v, c, name = kernel
    log(f"split-K {splits} on {name}")
    A, B = make_inputs(M, N, K, "int4", seed=41)
    dA, dB = to_dev(A), to_dev(B)
    buf = torch.full((M, N + 3), float("nan"), device="cuda:0")
    b.gemm_splitk(dA, dB, splits, buf[:, :N], variant=v, config=c)
    host = to_host(buf)
    assert_exact(host[:, :N], oracle.gemm(A, B), f"{name} splits={splits} int4")
    assert np.isnan(host[:, N:]).all()
    A, B = make_inputs(M, N, K, "uniform", seed=42)
    dA, dB = to_dev(A), to_dev(B)
    out1 = b.gemm_splitk(dA, dB, splits, variant=v, config=c)
    out2 = b.gemm_splitk(dA, dB, splits, variant=v, config=c)
    _, ref64 = oracle.gemm(A, B, return_f64=True)
    C1 = to_host(out1)
    assert_close(C1, ref64, K, f"{name} splits={splits} uniform")
    assert np.array_equal(C1.view(np.uint32), to_host(out2).view(np.uint32)), "not reproducible"


@pytest.mark.parametrize("kernel", SPLITK_KERNELS, ids=[k[2] for k in SPLITK_KERNELS])
def test_splitk_full_tiles(kernel):
    """Whole tiles and whole splits: the unguarded and direct-load paths."""
    v, c, name = kernel
    log(f"split-K full tiles on {name}")
    M, N, K = 512, 512, 1024
    A, B = make_inputs(M, N, K, "int4", seed=43)
    out = b.gemm_splitk(to_dev(A), to_dev(B), 4, variant=v, config=c)
    assert_exact(to_host(out), oracle.gemm(A, B), f"{name} full tiles")


# (M, N, K, splits): slices of equal length, which the persistent tiles run as
# a batch of products (whole tiles, and the edge form)
SPLITK_EQUAL = [(512, 512, 1024, 4), (300, 260, 1024, 4), (384, 256, 2048, 8), (1024, 1024, 8192, 0)]


@pytest.mark.parametrize("kernel", [k for k in SPLITK_KERNELS if k[2] == "select" or k[2].endswith("_p")],
                         ids=[k[2] for k in SPLITK_KERNELS if k[2] == "select" or k[2].endswith("_p")])
@pytest.mark.parametrize("shape", SPLITK_EQUAL, ids=["x".join(map(str, s)) for s in SPLITK_EQUAL])
def test_splitk_equal_slices(kernel, shape):
    """Split-K whose slices all have the same length: the persistent tiles
    take the partial products as one batched launch of products over K /
    splits each.  Exact on integers, C inside a NaN guard band."""
    import torch

    M, N, K, splits = shape
    v, c, name = kernel
    log(f"split-K equal slices {M}x{N}x{K} / {splits} on {name}")
    A, B = make_inputs(M, N, K, "int4", seed=47)
    buf = torch.full((M, N + 3), float("nan"), device="cuda:0")
    b.gemm_splitk(to_dev(A), to_dev(B), splits, buf[:, :N], variant=v, config=c)
    host = to_host(buf)
    assert_exact(host[:, :N], oracle.gemm(A, B), f"{name} {shape}")
    assert np.isnan(host[:, N:]).all()


SPLITK_WHOLE_K = [(None, -1, "select")] + [
    (3, c, n) for v, c, n in ALL_CONFIGS if v == 3 and n in (
        "mfma2_64x64x64_w2x2_k4_swz", "mfma2d_64x64x64_w2x2_k4_swz", "mfma2d_64x64x128_w2x2_k4_swz",
        "mfma4d_64x64x64_w2x2_k4_swz", "mfma2d_256x256x32_w4x4_swz_g4_il",
        "mfmag_64x64x64_w1x1_k4_d3", "mfmag_128x128x64_w1x1_k4_d2", "mfmag_128x128x64_w1x1_k4_d2_p",
        "mfmag_96x128x64_w1x1_k4_d2_p")]


@pytest.mark.parametrize("kernel", SPLITK_WHOLE_K, ids=[k[2] for k in SPLITK_WHOLE_K])
@pytest.mark.parametrize("lda_pad", [0, 1], ids=["aligned", "lda+1"])
def test_splitk_slices_not_whole_k_steps(kernel, lda_pad):
    """K = 4160 is whole 64-k steps but its four 1056-k slices are not: the
    kernels with a 64- or 128-k step must take their K-checked path on every
    slice (rows 16-byte aligned, and rows one float longer), so that no
    slice adds k of the next one and the last reads nothing past K."""
    import torch

    M, N, K = 256, 256, 4160
    v, c, name = kernel
    log(f"split-K 4 x 1056 of K={K} on {name}, lda pad {lda_pad}")
    A, B = make_inputs(M, N, K, "int4", seed=46)
    Ab = np.zeros((M, K + lda_pad), np.float32)
    Ab[:, :K] = A
    dA = to_dev(Ab)[:, :K]
    out = torch.full((M, N), float("nan"), device="cuda:0")
    b.gemm_splitk(dA, to_dev(B), 4, out, variant=v, config=c)
    assert_exact(to_host(out), oracle.gemm(A, B), f"{name} lda pad {lda_pad}")


PERSISTENT = [(3, c, n) for v, c, n in ALL_CONFIGS if v == 3 and n.startswith("mfmag") and n.endswith("_p")]
# (kernel, operand forms): configurations without transposed operands run NN only
PERSISTENT_OPS = [(k, ops) for k in PERSISTENT for ops in (OPS if k[2] in TRANS_CAPABLE else ["NN"])]
PERSISTENT_OPS_IDS = [f"{k[2]}-{ops}" for k, ops in PERSISTENT_OPS]
PERSISTENT_SHAPES = [(256, 256, 384), (2048, 2304, 384), (1280, 4096, 768)]


@pytest.mark.parametrize("kernel,ops", PERSISTENT_OPS, ids=PERSISTENT_OPS_IDS)
def test_persistent_register_direct(kernel, ops):
    """The persistent register-direct kernel runs whole tiles with K a
    multiple of 128 (16 k x 4 groups x 2 chunks in flight), every operand
    form: one workgroup per CU walks one to five tiles, and the last chunks
    of each tile load the next tile's first ones.  Fewer tiles than CUs, and
    rounds with part of the workgroups idle.  Exact on integers."""
    import torch

    v, c, name = kernel
    for M, N, K in PERSISTENT_SHAPES:
        log(f"persistent {ops} {M}x{N}x{K} on {name}")
        A, B = make_inputs(M, N, K, "int4", seed=71)
        out = torch.full((M, N), float("nan"), device="cuda:0")
        b.gemm(_stored(A, ops[0]), _stored(B, ops[1]), out, variant=v, config=c)
        assert_exact(to_host(out), oracle.gemm(A, B), f"{name} {ops} {M}x{N}x{K}")


# edge tiles and K past whole rounds (K and k-major row lengths multiples of
# 4; M odd where A is a row operand), K below one chunk, one tile
PERSISTENT_EDGE_SHAPES = [(300, 260, 132), (301, 1020, 776), (2000, 2052, 388), (128, 132, 4),
                          (4, 4, 1000), (1028, 128, 128)]


@pytest.mark.parametrize("kernel,ops", PERSISTENT_OPS, ids=PERSISTENT_OPS_IDS)
def test_persistent_register_direct_edges(kernel, ops):
    """The persistent kernel's edge form: rows past M or N and k past K load
    as zeros (out-of-range buffer offsets), K rounds up to whole rounds of
    chunks, stores past M or N are skipped.  Shapes whose transposed operand
    has a row length that is not a multiple of 4 take the one-launch
    kernel.  NaN fill around C checks the skipped stores.  Exact on
    integers."""
    import torch

    v, c, name = kernel
    for M, N, K in PERSISTENT_EDGE_SHAPES:
        log(f"persistent edges {ops} {M}x{N}x{K} on {name}")
        A, B = make_inputs(M, N, K, "int4", seed=74)
        big = torch.full((M + 2, N + 3), float("nan"), device="cuda:0")
        out = big[1:M + 1, 1:N + 1]
        b.gemm(_stored(A, ops[0]), _stored(B, ops[1]), out, variant=v, config=c)
        got = to_host(big)
        assert_exact(np.ascontiguousarray(got[1:M + 1, 1:N + 1]), oracle.gemm(A, B), f"{name} {ops} {M}x{N}x{K}")
        rest = got.copy()
        rest[1:M + 1, 1:N + 1] = np.nan
        assert np.isnan(rest).all(), f"{name} {ops} {M}x{N}x{K}: a store outside C"


# (operand, leading dimension): just inside the buffer-offset limit of the
# persistent kernel (a chunk's byte offsets below 2^31) and just past it,
# where the launcher takes the one-launch kernel instead
PERSISTENT_FAR = [("A", 1 << 21), ("A", (1 << 21) + (1 << 17)), ("AT", (1 << 24)),
                  ("B", 1 << 24), ("B", (1 << 24) + (1 << 21)), ("BT", 1 << 21)]


PERSISTENT_FAR_CASES = [(k, o, ld) for k in PERSISTENT for o, ld in PERSISTENT_FAR
                        if k[2] in TRANS_CAPABLE or o in ("A", "B")]


@pytest.mark.parametrize("kernel,operand,ld", PERSISTENT_FAR_CASES,
                         ids=[f"{k[2]}-{o}_ld{ld}" for k, o, ld in PERSISTENT_FAR_CASES])
def test_persistent_register_direct_far_rows(kernel, operand, ld):
    """Whole 128 x 128 x 256 products with one operand's rows (or k rows)
    far apart: byte offsets within a chunk near 2^30 on the buffer-load
    path, and past the limit on the fallback.  Exact on integers."""
    import torch

    v, c, name = kernel
    M, N, K = 128, 128, 256
    A, B = make_inputs(M, N, K, "int4", seed=73)
    X = {"A": A, "AT": A.T, "B": B, "BT": B.T}[operand]
    rows, cols = X.shape
    log(f"persistent far rows {operand} ld {ld} on {name}")
    buf = torch.empty((rows - 1) * ld + cols, dtype=torch.float32, device="cuda:0")
    dX = buf.as_strided((rows, cols), (ld, 1))
    dX.copy_(to_dev(np.ascontiguousarray(X)))
    dA = dX if operand == "A" else dX.T if operand == "AT" else to_dev(A)
    dB = dX if operand == "B" else dX.T if operand == "BT" else to_dev(B)
    out = torch.full((M, N), float("nan"), device="cuda:0")
    b.gemm(dA, dB, out, variant=v, config=c)
    got = to_host(out)
    del dX, buf, dA, dB
    torch.cuda.empty_cache()
    assert_exact(got, oracle.gemm(A, B), f"{name} {operand} ld {ld}")


@pytest.mark.parametrize("kernel", PERSISTENT, ids=[k[2] for k in PERSISTENT])
@pytest.mark.parametrize("shape", [(512, 640, 384), (300, 260, 132)], ids=["whole", "edges"])
@pytest.mark.parametrize("cpad", [3, 0], ids=["rows_padded", "odd_batch_stride"])
def test_persistent_register_direct_batched(kernel, shape, cpad):
    """Three products in one persistent launch (tiles of all products on one
    walk), whole tiles or the edge form, B shared (stride 0), and C either
    with rows padded to an odd length or with aligned rows whose batch
    stride is odd (the second and third products' C is then not 16-byte
    aligned, which decides per product between vector and scalar stores)."""
    (M, N, K), nb = shape, 3
    rng = np.random.default_rng(72)
    lda, ldb, ldc = K, N, N + cpad
    sa, sb, sc = M * lda + 5, 0, M * ldc + 7
    A3, As = _layout(rng, nb, M, K, lda, sa, "int4")
    B3, Bs = _layout(rng, 1, K, N, ldb, 0, "int4")
    log(f"persistent batched {nb} x {M}x{N}x{K} on {kernel[2]}")
    Cflat = _run_batched(A3, B3, M, N, K, nb, sa, sb, sc, lda, ldb, ldc, kernel)
    for q in range(nb):
        got = np.lib.stride_tricks.as_strided(Cflat[q * sc:], shape=(M, N), strides=(4 * ldc, 4))
        assert_exact(np.ascontiguousarray(got), oracle.gemm(As[q], Bs[0]), f"{kernel[2]} product {q}")


def test_splitk_deep_k_full():
    """The deep-K workload in the launch configuration the benchmark times
    (library's choice of kernel and of splits), every cell against the
    oracle."""
    w = WORKLOADS["deepk"]
    log(f"split-K full size {w.name}")
    A, B = workload_inputs(w.name)
    C = to_host(b.gemm_splitk(to_dev(A), to_dev(B), 0))
    _, ref64 = oracle.gemm(A, B, return_f64=True)
    assert_close(C, ref64, w.K, "deepk")


def test_prepared_call_matches_gemm():
    """binding.prepare (arguments built once, for launch loops) enqueues the
    same call as gemm / gemm_batched, for row-major, transposed and batched
    operands, and keeps working on repeated launches."""
    import torch

    A, B = make_inputs(130, 70, 50, "uniform", seed=45)
    dA, dB = to_dev(A), to_dev(B)
    for a, b_, name in ((dA, dB, "NN"), (to_dev(np.ascontiguousarray(A.T)).T, dB, "TN")):
        ref = to_host(b.gemm(a, b_))
        out = torch.full((130, 70), float("nan"), device="cuda:0")
        launch = b.prepare(a, b_, out)
        for _ in range(3):
            launch()
        assert np.array_equal(to_host(out).view(np.uint32), ref.view(np.uint32)), name
    d3 = to_dev(np.stack([A, A[::-1].copy()]))
    dB3 = dB.expand(2, -1, -1)
    for kw in ({}, {"variant": "mfma", "config": "mfma2d_64x64x64_w2x2_k4_swz"}):
        ref = to_host(b.gemm_batched(d3, dB3, **kw))
        out = torch.empty((2, 130, 70), device="cuda:0")
        b.prepare(d3, dB3, out, batched=True, **kw)()
        assert np.array_equal(to_host(out).view(np.uint32), ref.view(np.uint32)), kw


@pytest.mark.parametrize("case", ["select", "k4", "splitk", "persistent", "persistent_edge"])
def test_graph_capture_replays(case):
    """A library call captured in a HIP graph (torch.cuda.CUDAGraph on a side
    stream) replays correctly: three replays, with eager work between them
    that changes A in place, each checked bit for bit against an eager call
    on the same inputs, and the last against the oracle.  The shape has no
    16-byte-aligned rows (4-byte direct loads) and ragged tiles; the
    persistent register-direct tile runs whole tiles and its edge form."""
    import torch

    M, N, K = {"persistent": (512, 640, 384), "persistent_edge": (300, 260, 132)}.get(case, (300, 277, 1029))
    A, B = make_inputs(M, N, K, "int4", seed=60)
    dA, dB = to_dev(A), to_dev(B)
    out = torch.full((M, N), float("nan"), device="cuda:0")
    ref = torch.empty((M, N), device="cuda:0")
    kw = {"variant": "mfma", "config": "mfma4d_64x64x64_w2x2_k4_swz"} if case == "k4" else {}
    if case.startswith("persistent"):
        kw = {"variant": "mfma", "config": "mfmag_128x128x64_w1x1_k4_d2_p"}
    if case == "splitk":
        need = b.gemm_f32_splitk_workspace_size(M, N, K, 3)
        work = torch.empty(need // 4, device="cuda:0")
        work_eager = torch.empty(need // 4, device="cuda:0")
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        if case == "splitk":
            b.gemm_splitk(dA, dB, 3, out, work, stream=cap)
        else:
            b.prepare(dA, dB, out, stream=cap, **kw)()
    scale = 1.0
    for r in range(3):
        f = -1.0 if r % 2 else 2.0  # exact in FP32 for these integers
        dA.mul_(f)
        scale *= f
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        if case == "splitk":
            b.gemm_splitk(dA, dB, 3, ref, work_eager)
        else:
            b.gemm(dA, dB, ref, **kw)
        torch.cuda.synchronize()
        got = to_host(out)
        assert np.array_equal(got.view(np.uint32), to_host(ref).view(np.uint32)), \
            f"{case}: replay {r} differs from the eager call"
    assert_exact(got, oracle.gemm((A * np.float32(scale)).astype(np.float32), B), f"{case} oracle")


def test_concurrent_calls_from_threads():
    """Calls are reentrant: four host threads, each on its own stream, run ten
    calls each on different shapes (some split in two launches by the
    library, some with rows that are not 16-byte aligned); every result is
    exact against the oracle on integer inputs."""
    import threading

    import torch

    shapes = [(300, 277, 129), (3584, 3584, 1024), (1000, 1023, 777), (2048, 5632, 1024)]
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = make_inputs(M, N, K, "int4", seed=80 + i)
        data.append((A, B, to_dev(A), to_dev(B), oracle.gemm(A, B)))
    errors = []

    def worker(i):
        try:
            A, B, dA, dB, ref = data[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(10):
                    out = b.gemm(dA, dB, stream=stream)
                    stream.synchronize()
                    if not np.array_equal(to_host(out), ref):
                        errors.append(f"thread {i}: wrong result")
                        return
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


def test_splitk_one_split_is_plain_product():
    A, B = make_inputs(200, 100, 64, "uniform", seed=44)
    dA, dB = to_dev(A), to_dev(B)
    one = to_host(b.gemm_splitk(dA, dB, 1))
    plain = to_host(b.gemm(dA, dB))
    assert np.array_equal(one.view(np.uint32), plain.view(np.uint32))


# --------------------------------------------------------------------------
# full-size workloads in the benchmark's launch configuration
# --------------------------------------------------------------------------

SPLIT_SHAPES = [(3584, 3584, 3584), (3300, 3300, 1000), (4607, 4609, 1001), (1800, 9000, 1024)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=["x".join(map(str, s)) for s in SPLIT_SHAPES])
@pytest.mark.parametrize("ops", ["NN", "TN", "NT"])
def test_split_products(shape, ops):
    """Products that gemm_f32 runs as two launches on complementary parts of
    C (rows or columns, see gemm_f32_plan), with operands stored as given
    and transposed, and with rows that are not 16-byte aligned (4607 x 4609
    x 1001): every cell exact against the oracle on integer inputs, and C
    inside a NaN guard band."""
    import torch

    M, N, K = shape
    plan = b.gemm_f32_plan(M, N, K, K, N, N)
    if ops == "NN":
        assert plan["parts"] == 2, plan
    log(f"split product {M}x{N}x{K} {ops}: plan {plan}")
    A, B = make_inputs(M, N, K, "int4", seed=70)
    buf = torch.full((M, N + 3), float("nan"), device="cuda:0")
    b.gemm(_stored(A, ops[0]), _stored(B, ops[1]), buf[:, :N])
    assert bool(torch.isnan(buf[:, N:]).all()), "write outside C's columns"
    C = to_host(buf[:, :N])
    assert_exact(C, oracle.gemm(A, B), f"{shape} {ops}")


SPLIT_BATCHES = [(2, 3840, 3840, 1024), (2, 3328, 3328, 1024), (2, 3584, 3584, 1024)]


@pytest.mark.parametrize("shape", SPLIT_BATCHES, ids=["x".join(map(str, s)) for s in SPLIT_BATCHES])
def test_split_batches(shape):
    """Strided batches whose products the library splits in two parts (rows
    for 3584^2 x 1024, columns for 3328^2 x 1024 and 3840^2 x 1024):
    every cell of every product exact against the oracle on integer inputs,
    and every C inside a NaN guard band."""
    import torch

    nb, M, N, K = shape
    log(f"split batch {shape}")
    A, B = make_inputs(nb * M, N, K, "int4", seed=71)
    A3 = A.reshape(nb, M, K)
    B3 = np.stack([B, (B[::-1] * -1).copy()])
    buf = torch.full((nb, M, N + 3), float("nan"), device="cuda:0")
    b.gemm_batched(to_dev(A3), to_dev(B3), buf[:, :, :N])
    assert bool(torch.isnan(buf[:, :, N:]).all()), "write outside C's columns"
    got = to_host(buf[:, :, :N])
    for i in range(nb):
        assert_exact(got[i], oracle.gemm(A3[i], B3[i]), f"{shape} product {i}")


def _random_case(rng):
    """One seeded random problem: sizes, leading-dimension padding, operand
    forms, batch and kernel (the library's choice or a random MFMA
    configuration that takes the operand forms)."""
    M, N, K = (int(x) for x in rng.integers(1, 700, size=3))
    ops = str(rng.choice(["NN", "NT", "TN", "TT"]))
    nb = int(rng.integers(1, 4))
    pads = [int(x) for x in rng.integers(0, 6, size=3)]
    if rng.random() < 0.4:
        kernel = (None, -1, "select")
    else:
        pool = [k for k in MFMA_CONFIGS if ops == "NN" or k[2] in TRANS_CAPABLE]
        kernel = pool[int(rng.integers(0, len(pool)))]
    return M, N, K, ops, nb, pads, kernel


def _stored_batch(X3: np.ndarray, op: str, pad: int):
    """Device batch holding op(X_b) = X_b: each matrix stored as given (or as
    its transpose) with `pad` extra floats per row, as a strided view."""
    import torch

    S = X3 if op == "N" else np.ascontiguousarray(np.swapaxes(X3, 1, 2))
    nb, r, c = S.shape
    buf = np.zeros((nb, r, c + pad), dtype=np.float32)
    buf[:, :, :c] = S
    dev = torch.from_numpy(buf).to("cuda:0")[:, :, :c]
    return dev if op == "N" else dev.transpose(1, 2)


def test_random_problems_exact():
    """200 seeded random problems (sizes up to 700, padded rows, all operand
    forms, batches of 1 to 3, the library's choice or a random MFMA
    configuration, a quarter of the single row-major products as split-K)
    on integer inputs: every product exact against the oracle, and C's
    padding untouched.  GEMM_F32_RANDOM_CASES and GEMM_F32_RANDOM_SEED set
    another count or seed for a longer run."""
    import os

    import torch

    rng = np.random.default_rng(int(os.environ.get("GEMM_F32_RANDOM_SEED", "2024")))
    for case in range(int(os.environ.get("GEMM_F32_RANDOM_CASES", "200"))):
        M, N, K, ops, nb, pads, (v, c, name) = _random_case(rng)
        log(f"random case {case}: {nb} x {M}x{N}x{K} {ops} pads {pads} on {name}")
        A = rng.integers(-4, 5, size=(nb, M, K)).astype(np.float32)
        B = rng.integers(-4, 5, size=(nb, K, N)).astype(np.float32)
        dA, dB = _stored_batch(A, ops[0], pads[0]), _stored_batch(B, ops[1], pads[1])
        buf = torch.full((nb, M, N + pads[2]), float("nan"), device="cuda:0")
        out = buf[:, :, :N]
        if nb == 1 and ops == "NN" and rng.random() < 0.25:  # split-K with 2 to 7 splits
            splits = int(rng.integers(2, 8))
            log(f"  as split-K with {splits} splits")
            b.gemm_splitk(dA[0], dB[0], splits, out[0], variant=v, config=c)
        elif nb == 1:
            b.gemm(dA[0], dB[0], out[0], variant=v, config=c)
        else:
            b.gemm_batched(dA, dB, out, variant=v, config=c)
        got = to_host(buf)
        assert np.isnan(got[:, :, N:]).all(), f"case {case}: write outside C's columns"
        for i in range(nb):
            assert_exact(got[i, :, :N], oracle.gemm(A[i], B[i]), f"case {case} product {i} on {name}")


def test_random_large_problems():
    """10 seeded random products large enough for the library to split some
    of them in two launches (M, N 2000-6000, K 500-3000, all operand forms,
    padded rows), library's choice, integer inputs: every cell exact against
    the oracle."""
    import torch

    rng = np.random.default_rng(77)
    splits = 0
    for case in range(10):
        M, N = (int(x) for x in rng.integers(2000, 6001, size=2))
        K = int(rng.integers(500, 3001))
        ops = str(rng.choice(["NN", "NT", "TN", "TT"]))
        pads = [int(x) for x in rng.integers(0, 5, size=3)]
        plan = b.gemm_f32_plan(M, N, K, K + pads[0], N + pads[1], N + pads[2])
        splits += plan["parts"] == 2
        log(f"large random case {case}: {M}x{N}x{K} {ops} pads {pads} plan {plan}")
        A = rng.integers(-4, 5, size=(1, M, K)).astype(np.float32)
        B = rng.integers(-4, 5, size=(1, K, N)).astype(np.float32)
        dA, dB = _stored_batch(A, ops[0], pads[0])[0], _stored_batch(B, ops[1], pads[1])[0]
        buf = torch.full((M, N + pads[2]), float("nan"), device="cuda:0")
        b.gemm(dA, dB, buf[:, :N])
        got = to_host(buf)
        assert np.isnan(got[:, N:]).all(), f"case {case}: write outside C's columns"
        assert_exact(got[:, :N], oracle.gemm(A[0], B[0]), f"large case {case}")
        del dA, dB, buf
    log(f"{splits} of 10 large random products were split (row-major plan)")


FULL_FLOAT = ["square4096", "square8192", "ffn", "square8000", "square8191", "ktail8100"]


@pytest.mark.parametrize("wname", FULL_FLOAT)
def test_full_size_every_cell(wname):
    """The full-size float workloads in the benchmark's launch
    configuration: every cell within the tolerance of the oracle's FP64
    sums (the oracle takes about 10-12 s for the 8192 shapes on 16 cores)."""
    import torch

    w = WORKLOADS[wname]
    log(f"full size {wname} {w.M}x{w.N}x{w.K}")
    A, B = workload_inputs(wname)
    dA, dB = to_dev(A), to_dev(B)
    dC = torch.empty((w.M, w.N), device="cuda:0")
    b.gemm(dA, dB, dC)
    C = to_host(dC)
    del dA, dB, dC
    _, ref64 = oracle.gemm(A, B, return_f64=True)
    stats = assert_close(C, ref64, w.K, wname)
    log(f"{wname}: every cell: max err {stats['max_err']:.3e} relF {stats['rel_fro']:.3e}")


@pytest.mark.parametrize("wname", ["square8192_int4", "ffn_int4"])
def test_full_size_integer_bit_exact(wname):
    """The headline shape (and the FFN shape) on integer inputs in [-4, 4]:
    every partial sum is an integer below 16 K <= 2^17, exact in FP32 in any
    order, so every cell must equal the oracle's bit for bit."""
    import torch

    w = WORKLOADS[wname]
    log(f"full size {wname} {w.M}x{w.N}x{w.K}")
    A, B = workload_inputs(wname)
    dA, dB = to_dev(A), to_dev(B)
    dC = torch.empty((w.M, w.N), device="cuda:0")
    b.gemm(dA, dB, dC)
    C = to_host(dC)
    del dA, dB, dC
    assert_exact(C, oracle.gemm(A, B), wname)


def test_full_size_batched_every_cell():
    import torch

    w = WORKLOADS["batched64_1024"]
    log(f"full size {w.name}: {w.batch} x {w.M}x{w.N}x{w.K}")
    A, B = workload_inputs(w.name)
    dC = torch.empty((w.batch, w.M, w.N), device="cuda:0")
    b.gemm_batched(to_dev(A), to_dev(B), dC)
    C = to_host(dC)
    for i in range(w.batch):
        _, ref64 = oracle.gemm(A[i], B[i], return_f64=True)
        assert_close(C[i], ref64, w.K, f"{w.name} product {i}")
