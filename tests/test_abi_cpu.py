"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects invalid arguments before touching the device (no compute call
reaches HIP here)."""

import ctypes
import json
import os
import re

import pytest

from dense_fp32_gemm_row_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f32.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_f32\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.LIBRARY):
        import __graft_entry__

        __graft_entry__.build()
    return b.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"gemm_f32", "gemm_f32_variant", "gemm_f32_strerror"} <= set(names)
    raw = ctypes.CDLL(b.LIBRARY)
    for name in names:
        assert hasattr(raw, name), f"{name} declared in gemm_f32.h but not exported"


def test_abi_version(lib):
    assert b.gemm_f32_abi_version() == 3


def test_strerror(lib):
    assert b.gemm_f32_strerror(0) == "success"
    assert b.gemm_f32_strerror(-1) == "invalid argument"
    assert b.gemm_f32_strerror(-2) == "HIP runtime error"
    assert b.gemm_f32_strerror(-3).startswith("no such kernel")
    assert b.gemm_f32_strerror(12345) == "unknown error code"


def test_config_registry(lib):
    for v in range(4):
        n = b.gemm_f32_config_count(v)
        assert n >= 1
        names = b.config_names(v)
        assert len(set(names)) == n and all(names)
        assert b.gemm_f32_config_name(v, n) is None
        assert b.gemm_f32_config_name(v, -1) is None
    assert b.gemm_f32_config_count(4) == b.GEMM_F32_ENOKERNEL
    assert b.config_names(0)[0].startswith("naive")
    assert all(n.startswith("mfma") for n in b.config_names(3))


@pytest.mark.parametrize("shape", [(8192, 8192, 8192), (4096, 4096, 4096), (8192, 14336, 4096),
                                   (1000, 1023, 777), (256, 256, 256), (1, 1, 1)])
def test_select_returns_valid_config(lib, shape):
    M, N, K = shape
    v, c = b.gemm_f32_select(M, N, K, K, N, N)
    assert v == b.VARIANT_MFMA
    assert 0 <= c < b.gemm_f32_config_count(v)


# Arguments that must be rejected before anything reaches the device.  Fake
# addresses are never dereferenced: validation is pure arithmetic.
BAD = [
    ("negative M", (-1, 4, 4, 0x1000, 4, 0x2000, 4, 0x3000, 4), "negative"),
    ("negative K", (4, 4, -2, 0x1000, 4, 0x2000, 4, 0x3000, 4), "negative"),
    ("M too large", (1 << 31, 4, 4, 0x1000, 4, 0x2000, 4, 0x3000, 4), "2^31"),
    ("lda < K", (4, 4, 5, 0x1000, 4, 0x2000, 4, 0x3000, 4), "lda"),
    ("ldb < N", (4, 6, 4, 0x1000, 4, 0x2000, 5, 0x3000, 6), "ldb"),
    ("ldc < N", (4, 6, 4, 0x1000, 4, 0x2000, 6, 0x3000, 5), "ldc"),
    ("ld zero", (0, 0, 0, 0, 0, 0, 1, 0, 1), "lda"),
    ("C NULL", (4, 4, 4, 0x1000, 4, 0x2000, 4, 0, 4), "C is NULL"),
    ("A NULL", (4, 4, 4, 0, 4, 0x2000, 4, 0x3000, 4), "A is NULL"),
    ("B NULL", (4, 4, 4, 0x1000, 4, 0, 4, 0x3000, 4), "B is NULL"),
    ("A misaligned", (4, 4, 4, 0x1002, 4, 0x2000, 4, 0x3000, 4), "aligned"),
    ("C misaligned", (4, 4, 4, 0x1000, 4, 0x2000, 4, 0x3001, 4), "aligned"),
    ("C overlaps A", (4, 4, 4, 0x1000, 4, 0x2000, 4, 0x1000 + 60, 4), "overlaps A"),
    ("C overlaps B", (4, 4, 4, 0x1000, 4, 0x2000, 4, 0x2000 - 4, 4), "overlaps B"),
    ("C inside B's padding span", (2, 2, 2, 0x1000, 2, 0x2000, 64, 0x2000 + 16, 2), "overlaps B"),
]


@pytest.mark.parametrize("args,detail", [(a, d) for _, a, d in BAD], ids=[n for n, _, _ in BAD])
def test_invalid_arguments(lib, args, detail):
    assert b.gemm_f32(*args, None) == b.GEMM_F32_EINVAL
    assert detail in b.gemm_f32_last_error()
    for v in range(4):
        assert b.gemm_f32_variant(v, 0, *args, None) == b.GEMM_F32_EINVAL
    assert b.gemm_f32_variant(3, -1, *args, None) == b.GEMM_F32_EINVAL


def test_empty_products_enqueue_nothing(lib):
    # M == 0 or N == 0: success without any launch, NULL pointers allowed.
    assert b.gemm_f32(0, 5, 7, 0, 7, 0, 5, 0, 5, None) == b.GEMM_F32_OK
    assert b.gemm_f32(5, 0, 7, 0, 7, 0, 1, 0, 1, None) == b.GEMM_F32_OK
    assert b.gemm_f32_last_error() == ""
    for v in range(4):
        assert b.gemm_f32_variant(v, -1, 0, 0, 0, 0, 1, 0, 1, 0, 1, None) == b.GEMM_F32_OK


def test_unknown_kernels(lib):
    args = (4, 4, 4, 0x1000, 4, 0x2000, 4, 0x3000, 4, None)
    assert b.gemm_f32_variant(4, 0, *args) == b.GEMM_F32_ENOKERNEL
    assert b.gemm_f32_variant(-1, 0, *args) == b.GEMM_F32_ENOKERNEL
    n = b.gemm_f32_config_count(3)
    assert b.gemm_f32_variant(3, n, *args) == b.GEMM_F32_ENOKERNEL
    assert b.gemm_f32_variant(3, -2, *args) == b.GEMM_F32_ENOKERNEL
    assert "configuration" in b.gemm_f32_last_error()


def test_select_rejects_invalid(lib):
    with pytest.raises(b.GemmError):
        b.gemm_f32_select(4, 4, 5, 4, 4, 4)


def test_tensor_wrapper_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    A = torch.zeros(3, 4)
    B = torch.zeros(4, 5)
    with pytest.raises(TypeError):
        b.gemm(A, B)


def test_tuning_table_names_compiled_configs(lib):
    import json

    table = json.load(open(os.path.join(ROOT, "dense_fp32_gemm_row_amd", "tune", "table.json")))
    names = {n for v in range(4) for n in b.config_names(v)}
    for c in table["model"]["candidates"]:
        assert c["config"] in names, f"model candidate names unknown configuration {c['config']}"
        assert c["config"].startswith("mfma")
        assert 1 <= len(c["gflops_per_cu"]) <= 4 and 0 < c["unaligned"] <= 1
    for e in table["entries"]:
        assert e["config"] in names, f"table entry {e} names an unknown configuration"
        v, c = b.gemm_f32_select(e["M"], e["N"], e["K"], e["K"], e["N"], e["N"])
        assert b.gemm_f32_config_name(v, c) == e["config"]


def test_cost_model_choices(lib):
    """The cost model's choice on shapes not in the table: small products
    get small tiles, a product that fills the chip many times over the
    largest tile, and wave quantisation is accounted for (3072^3: 144 tiles
    of 256^2 would leave 112 CUs idle, 576 of 128^2 a quarter-full round;
    96 x 128 tiles make three whole rounds, 64^2 nine)."""
    def pick(M, N, K, lda=None, ldb=None):
        v, c = b.gemm_f32_select(M, N, K, lda or K, ldb or N, N)
        return b.gemm_f32_config_name(v, c)

    def tile(name):
        bm, bn = (int(x) for x in name.split("_")[1].split("x")[:2])
        return bm * bn

    assert tile(pick(512, 512, 512)) <= 64 * 64      # 16 x 64 tiles (16x16x4 instructions)
    # one of the two fastest tiles on large products (within 0.5% of each
    # other at 8192^3): 256 x 256 LDS-staged, or the persistent 128 x 128
    # register-direct tile
    assert pick(8192, 8192, 8192 + 64) in {"mfma2d_256x256x32_w4x4_swz_g4_il",
                                           "mfmag_128x128x64_w1x1_k4_d2_p"}
    bm, bn = (int(x) for x in pick(3072, 3072, 3072).split("_")[1].split("x")[:2])
    assert ((3072 // bm) * (3072 // bn)) % 256 == 0
    # 8192 x 1024: a tile that fills whole waves of the 256 CUs (256 tiles of
    # 256 x 128 or 128 x 256, or 512 of 128 x 128), none with a part-empty wave
    bm, bn = (int(x) for x in pick(8192, 1024, 4096).split("_")[1].split("x")[:2])
    assert bm * bn >= 128 * 128 and ((8192 // bm) * (1024 // bn)) % 256 == 0
    # the same shape with rows that are not 16-byte aligned may choose differently,
    # but always a compiled configuration
    assert pick(4096, 4096, 4095, 4095, 4096) in {n for n in b.config_names(3)}


def test_generated_table_matches_json():
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "gen_table", os.path.join(ROOT, "dense_fp32_gemm_row_amd", "tune", "gen_table.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    import json

    with open(gen.TABLE) as f:
        expect = gen.render(json.load(f))
    with open(gen.OUT) as f:
        assert f.read() == expect, "csrc/tune_table.inc is stale: rebuild"


# (batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC) rejected before any HIP call
BAD_BATCH = [
    ("negative batch", (-1, 4, 4, 4, 0x1000, 4, 16, 0x2000, 4, 16, 0x3000, 4, 16), "negative batch"),
    ("batch too large", (1 << 31, 4, 4, 4, 0x1000, 4, 16, 0x2000, 4, 16, 0x3000, 4, 16), "batch"),
    ("negative stride", (2, 4, 4, 4, 0x1000, 4, -16, 0x2000, 4, 16, 0x30000, 4, 16), "negative batch stride"),
    ("C products overlap", (2, 4, 4, 4, 0x1000, 4, 16, 0x2000, 4, 16, 0x30000, 4, 15), "strideC"),
    ("C batch reaches A", (3, 4, 4, 4, 0x1000, 4, 16, 0x8000, 4, 16, 0x1000 - 64, 4, 16), "overlaps A"),
    ("C batch reaches B", (3, 4, 4, 4, 0x1000, 4, 16, 0x8000, 4, 0, 0x8000 - 96, 4, 16), "overlaps B"),
    ("span too large", (1 << 20, 4, 4, 4, 0x1000, 4, 1 << 40, 0x2000, 4, 16, 0x3000, 4, 16), "2^58"),
    ("lda < K", (2, 4, 4, 5, 0x1000, 4, 32, 0x2000, 4, 32, 0x3000, 4, 32), "lda"),
]


@pytest.mark.parametrize("args,detail", [(a, d) for _, a, d in BAD_BATCH],
                         ids=[n for n, _, _ in BAD_BATCH])
def test_invalid_batched_arguments(lib, args, detail):
    assert b.gemm_f32_strided_batched(*args, None) == b.GEMM_F32_EINVAL
    assert detail in b.gemm_f32_last_error()
    for v in range(4):
        assert b.gemm_f32_strided_batched_variant(v, 0, *args, None) == b.GEMM_F32_EINVAL


def test_empty_batches_enqueue_nothing(lib):
    assert b.gemm_f32_strided_batched(0, 4, 4, 4, 0, 4, 16, 0, 4, 16, 0, 4, 16, None) == 0
    assert b.gemm_f32_strided_batched(5, 0, 4, 4, 0, 4, 16, 0, 4, 16, 0, 4, 16, None) == 0
    # a single product ignores strideC's lower bound
    assert b.gemm_f32_strided_batched(0, 4, 4, 4, 0, 4, 0, 0, 4, 0, 0, 4, 0, None) == 0


def test_gemm_ex_validation(lib):
    args = (1, 4, 6, 5, 0x1000, 5, 0, 0x2000, 6, 0, 0x3000, 6, 0, None)
    # unknown operand forms
    assert b.gemm_f32_ex(-1, -1, 2, 0, *args) == b.GEMM_F32_EINVAL
    assert b.gemm_f32_ex(-1, -1, 0, -1, *args) == b.GEMM_F32_EINVAL
    assert "opA/opB" in b.gemm_f32_last_error()
    # unknown variant
    assert b.gemm_f32_ex(-2, 0, 0, 0, *args) == b.GEMM_F32_ENOKERNEL
    assert b.gemm_f32_ex(7, 0, 0, 0, *args) == b.GEMM_F32_ENOKERNEL
    # transposed A is stored K x M: its rows hold M floats (M = 4 here)
    bad = (1, 4, 6, 5, 0x1000, 3, 0, 0x2000, 6, 0, 0x3000, 6, 0, None)
    assert b.gemm_f32_ex(-1, -1, b.OP_T, b.OP_N, *bad) == b.GEMM_F32_EINVAL
    assert "lda=3 < max(1, M=4)" in b.gemm_f32_last_error()
    # transposed B is stored N x K: its rows hold K floats (K = 5)
    bad = (1, 4, 6, 5, 0x1000, 5, 0, 0x2000, 4, 0, 0x3000, 6, 0, None)
    assert b.gemm_f32_ex(-1, -1, b.OP_N, b.OP_T, *bad) == b.GEMM_F32_EINVAL
    assert "ldb=4 < max(1, K=5)" in b.gemm_f32_last_error()
    # overlap is checked on the stored (transposed) extents: A^T stored 5 x 4
    # at 0x1000 spans 80 bytes
    ov = (1, 4, 6, 5, 0x1000, 4, 0, 0x2000, 6, 0, 0x1000 + 76, 6, 0, None)
    assert b.gemm_f32_ex(-1, -1, b.OP_T, b.OP_N, *ov) == b.GEMM_F32_EINVAL
    assert "overlaps A" in b.gemm_f32_last_error()
    # empty products succeed without touching the device
    assert b.gemm_f32_ex(-1, -1, b.OP_T, b.OP_T, 1, 0, 6, 5, 0, 1, 0, 0, 5, 0, 0, 6, 0, None) == 0


def test_splitk_workspace_size(lib):
    f = b.gemm_f32_splitk_workspace_size
    # K = 1000 in 4 splits: length ceil(250 / 32) * 32 = 256, 4 slices
    assert f(100, 30, 1000, 4) == 4 * 100 * 30 * 4
    # 7 splits of K = 100: length 32, only 4 slices are used
    assert f(10, 10, 100, 7) == 4 * 10 * 10 * 4
    # one slice: no workspace
    assert f(10, 10, 32, 8) == 0
    assert f(10, 10, 100, 1) == 0
    assert f(0, 10, 100, 4) == 0 and f(-1, 10, 100, 4) == 0 and f(10, 10, 100, -1) == 0
    # library choice (splits = 0): 64 tiles of 128 x 128 -> 4 splits when K allows
    assert f(1024, 1024, 65536, 0) == 4 * 1024 * 1024 * 4
    assert f(512, 512, 65536, 0) == 16 * 512 * 512 * 4      # 16 tiles -> 16 splits
    assert f(256, 128, 8192, 0) == 8 * 256 * 128 * 4        # 2 tiles, 8 by K
    assert f(1024, 1024, 4096, 0) == 4 * 1024 * 1024 * 4   # at least 1024 k per split
    assert f(1000, 1023, 777, 0) == 0                      # too little K: one slice


def test_splitk_validation(lib):
    base = dict(M=100, N=30, K=1000, A=0x100000, lda=1000, B=0x200000, ldb=30, C=0x300000, ldc=30)
    need = b.gemm_f32_splitk_workspace_size(100, 30, 1000, 4)

    def call(splits=4, ws=0x400000, wbytes=need, **kw):
        a = dict(base, **kw)
        return b.gemm_f32_splitk(-1, -1, splits, a["M"], a["N"], a["K"], a["A"], a["lda"], a["B"],
                                 a["ldb"], a["C"], a["ldc"], ws, wbytes, None)

    assert call(splits=-1) == b.GEMM_F32_EINVAL and "splits" in b.gemm_f32_last_error()
    assert call(splits=70000) == b.GEMM_F32_EINVAL
    assert call(ws=None) == b.GEMM_F32_EINVAL and "workspace" in b.gemm_f32_last_error()
    assert call(wbytes=need - 4) == b.GEMM_F32_EINVAL and "needed" in b.gemm_f32_last_error()
    assert call(ws=0x400002) == b.GEMM_F32_EINVAL
    assert call(ws=0x300000 + 400) == b.GEMM_F32_EINVAL and "overlaps" in b.gemm_f32_last_error()
    assert call(lda=999) == b.GEMM_F32_EINVAL and "lda" in b.gemm_f32_last_error()
    assert b.gemm_f32_splitk(-2, 0, 4, 1, 1, 1, 0x1000, 1, 0x2000, 1, 0x3000, 1, 0x4000, 64,
                             None) == b.GEMM_F32_ENOKERNEL
    # empty products need nothing
    assert call(M=0) == b.GEMM_F32_OK


def test_splitk_noalloc_validation(lib):
    """The no-allocation split-K rejects, before any device call, invalid
    arguments and partial products larger than the library's static
    scratch."""
    assert b.SPLITK_SCRATCH_BYTES == 32 << 20

    def call(splits, M, N, K, lda=None):
        return b.gemm_f32_splitk_noalloc(-1, -1, splits, M, N, K, 1 << 40, lda or K, 2 << 40,
                                         N, 3 << 40, N, None)

    assert call(-1, 100, 30, 1000) == b.GEMM_F32_EINVAL and "splits" in b.gemm_f32_last_error()
    assert call(4, 100, 30, 1000, lda=999) == b.GEMM_F32_EINVAL
    # 16 slices of 1024 x 1024 need 64 MiB: above the 32 MiB scratch
    assert b.gemm_f32_splitk_workspace_size(1024, 1024, 65536, 16) > b.SPLITK_SCRATCH_BYTES
    assert call(16, 1024, 1024, 65536) == b.GEMM_F32_EINVAL
    assert "static scratch" in b.gemm_f32_last_error()
    assert b.gemm_f32_splitk_noalloc(-2, 0, 4, 1, 1, 1, 0x1000, 1, 0x2000, 1, 0x3000, 1,
                                     None) == b.GEMM_F32_ENOKERNEL
    assert call(4, 0, 30, 1000) == b.GEMM_F32_OK  # empty: nothing to do


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "gemm_f32.h"

int main(void) {
    /* every entry point, by address: the header declares them as C functions */
    void (*fns[])(void) = {
%(fns)s
    };
    int v, c, n = 0;
    for (v = 0; v < GEMM_F32_NUM_VARIANTS; ++v) {
        int count = gemm_f32_config_count(v);
        if (count <= 0 || gemm_f32_config_name(v, 0) == NULL) return 1;
        n += count;
    }
    if (gemm_f32_config_count(GEMM_F32_NUM_VARIANTS) != GEMM_F32_ENOKERNEL) return 2;
    if (gemm_f32_select(8192, 8192, 8192, 8192, 8192, 8192, &v, &c) != GEMM_F32_OK) return 3;
    /* invalid arguments are rejected on the host, before any device work */
    if (gemm_f32(-1, 1, 1, NULL, 1, NULL, 1, NULL, 1, NULL) != GEMM_F32_EINVAL) return 4;
    if (strlen(gemm_f32_last_error()) == 0) return 5;
    if (gemm_f32(0, 5, 5, NULL, 5, NULL, 5, NULL, 5, NULL) != GEMM_F32_OK) return 6;
    if (gemm_f32_splitk_workspace_size(1024, 1024, 65536, 0) <= 0) return 7;
    printf("abi %%d configs %%d select %%s %%d\n", gemm_f32_abi_version(), n,
           gemm_f32_config_name(v, c), (int)(sizeof fns / sizeof fns[0]));
    return 0;
}
"""


def test_header_serves_a_c_caller(lib, tmp_path):
    """A plain C99 program includes the header (warnings are errors), takes
    the address of every declared entry point, links against the library and
    runs the calls that need no GPU: the ABI is usable without Python."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    names = declared_functions()
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER % {"fns": "\n".join(f"        (void (*)(void))&{n}," for n in names)})
    exe = tmp_path / "caller"
    libdir = os.path.dirname(b.LIBRARY)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lgemm_f32",
           f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    with open(os.path.join(ROOT, "dense_fp32_gemm_row_amd", "tune", "table.json")) as f:
        tuned = {(e["M"], e["N"], e["K"]): e["config"] for e in json.load(f)["entries"]}
    assert f"select {tuned[(8192, 8192, 8192)]} {len(names)}" in run.stdout


def test_split_plans(lib):
    """gemm_f32 splits a product in two launches where the last wave of large
    tiles would be mostly empty, never for tuned shapes or shapes that fill
    whole waves, and the parts are whole tiles of the first part's
    configuration; gemm_f32_select reports the first part."""
    def plan(M, N, K):
        return b.gemm_f32_plan(M, N, K, max(K, 1), N, N)

    for M, N, K in [(3584, 3584, 3584), (5120, 5120, 5120), (7168, 7168, 7168), (2048, 5632, 8192)]:
        p = plan(M, N, K)
        assert p["parts"] == 2, (M, N, K, p)
        name = b.gemm_f32_config_name(*p["configs"][0])
        bm, bn = (int(x) for x in name.split("_")[1].split("x")[:2])
        extent, tile = (M, bm) if p["axis"] == 0 else (N, bn)
        assert 0 < p["split"] < extent and p["split"] % tile == 0, (name, p)
        assert b.gemm_f32_select(M, N, K, K, N, N) == p["configs"][0]
    for M, N, K in [(8192, 8192, 8192), (4096, 4096, 4096), (8192, 14336, 4096), (1000, 1023, 777),
                    (256, 256, 256), (4608, 4608, 0)]:
        p = plan(M, N, K)
        assert p["parts"] == 1 and len(p["configs"]) == 1, (M, N, K, p)
