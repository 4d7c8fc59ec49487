"""Code-generation checks of the MFMA kernels (CPU only: hipcc cross-compiles
gfx950 assembly without a GPU).

Two properties of the direct-load K loops are checked, both found by
measurement to matter: where the loop waits on global loads, and that it
advances its global addresses instead of recomputing them.

Direct global -> LDS loads of K-step t + 1 (or t + 2) land in a buffer that
step t does not read.  The compiler only knows that through the alias scopes
it gives each LDS array, and those scopes reach loads only a few address
offsets away from the array.  When they do not reach the fragment reads, the
compiler waits for all outstanding global loads before the first LDS read
of every K-step, which serialises the prefetch with the math (about 1.5% of
the headline throughput).  These tests keep the waits on global loads in
each K loop where they belong: right before the barrier that publishes the
next tile, and with three LDS buffers leaving the loads of the tile after it
in flight (a wait for every load there gives the third buffer nothing to
do).
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_fp32_gemm_row_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def mfma_build(tmp_path_factory):
    """gfx950 assembly of the MFMA kernels, and the compiler's resource
    remarks (registers, scratch) for every kernel."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from concurrent.futures import ThreadPoolExecutor

    tmp = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        out = tmp / (os.path.splitext(src)[0] + ".s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Rpass-analysis=kernel-resource-usage",
               "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert res.returncode == 0, res.stderr[-2000:]
        return out.read_text(), res.stderr

    with ThreadPoolExecutor(max_workers=3) as ex:
        parts = list(ex.map(compile_one, ["mfma.hip", "mfma16.hip", "mfma_regs.hip"]))
    return "\n".join(p[0] for p in parts), "\n".join(p[1] for p in parts)


@pytest.fixture(scope="module")
def mfma_asm(mfma_build):
    return mfma_build[0]


def test_no_kernel_spills_registers(mfma_build):
    """MFMA kernels keep their accumulators and fragments in registers: a
    kernel that spills to scratch memory runs at a fraction of its rate (a
    16-wavefront 256 x 256 tile of 16 x 16 blocks needs more than the 128
    registers per lane that four wavefronts per SIMD leave, spilled, and ran
    at 86 TFLOP/s at 8192^3).  Known exception: the register-staged variants
    of the two-buffer 256 x 256 x 32 tiles (their float4 staging registers on
    top of the fragments), which run only as the mfma2p stage configuration
    and as the fallback of the direct-load tiles for operands whose rows are
    not 16-byte aligned and that span more than 2^29 floats."""
    remarks = mfma_build[1]
    names = re.findall(r"Function Name: (\S+)", remarks)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", remarks)]
    assert len(names) == len(scratch) and len(names) > 100, (len(names), len(scratch))
    filt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    spilled = [n for n, s in zip(names, scratch) if s]
    dem = subprocess.run([filt], input="\n".join(spilled), capture_output=True,
                         text=True).stdout.splitlines() if spilled else []
    unexpected = []
    for d in dem:
        # <BM, BN, BK, WM, WN, PADA, PADB, STAGES, DIRECT, ...>
        args = [a.strip() for a in d[d.index("<") + 1:d.index(">")].split(",")]
        if not (args[:3] == ["256", "256", "32"] and args[7] == "2" and args[8] == "false"):
            unexpected.append(d)
    assert not unexpected, f"{len(unexpected)} kernels use scratch: {unexpected[:3]}"


def loops(body: str) -> list[str]:
    """The K loops of a kernel (a tile kernel with edge handling has two: one
    with direct loads, one with register staging), as layout ranges: every
    backward branch (to a label earlier in the code) closes a loop that spans
    from its target to itself, and overlapping spans are one loop.  The
    compiler's own loop comments are not used: a rotated loop whose entry
    block is also reached from before the loop is not marked as inside it."""
    lines = body.splitlines()
    label_at = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(\.LBB\S+):", line)
        if m:
            label_at[m.group(1)] = i
    spans = []
    for i, line in enumerate(lines):
        m = re.match(r"^\s*s_(?:c)?branch\S*\s+(\.LBB\S+)", line)
        if m and label_at.get(m.group(1), i + 1) < i:
            spans.append([label_at[m.group(1)], i])
    spans.sort()
    merged = []
    for a, b in spans:
        if merged and a <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], b)
        else:
            merged.append([a, b])
    assert merged, "no loop found"
    return ["\n".join(lines[a:b + 1]) for a, b in merged]


def ring_kernels(asm: str):
    """(template arguments, K loops) of every pipelined kernel."""
    names, bodies = [], []
    for m in re.finditer(r"^(_Z\S*gemm_mfma_ring_kernel\S*):[^\n]*\n(.*?)^\.Lfunc_end", asm,
                         re.S | re.M):
        names.append(m.group(1))
        bodies.append(m.group(2))
    filt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    assert filt, "c++filt not found"
    dem = subprocess.run([filt], input="\n".join(names), capture_output=True,
                         text=True).stdout.splitlines()
    for d, body in zip(dem, bodies):
        args = [a.strip() for a in d[d.index("<") + 1:d.index(">")].split(",")]
        yield args, loops(body)


def barrier_follows(lines: list[str], k: int) -> bool:
    """An s_barrier right after line k (comments and empty inline-asm
    markers between them do not count)."""
    for ln in lines[k + 1:k + 8]:
        if ln.startswith("s_barrier"):
            return True
        if ln and not ln.startswith((";", "//")):
            return False
    return False


def test_direct_load_kernels_wait_only_at_the_barrier(mfma_asm):
    checked = stages3 = 0
    for args, kloops in ring_kernels(mfma_asm):
        # <BM, BN, BK, WM, WN, PADA, PADB, STAGES, DIRECT, GUARD, VEC, TA, TB, IL, KG>
        if args[8] != "true":
            continue
        where = ", ".join(args)
        direct = [lp for lp in kloops
                  if "global_load_lds_dwordx4" in lp or re.search(r"buffer_load_dword .* lds", lp)]
        assert len(direct) == 1, f"<{where}>: {len(direct)} K loops with direct loads"
        lines = [ln.strip() for ln in direct[0].splitlines()]
        waits = [k for k, ln in enumerate(lines) if ln.startswith("s_waitcnt") and "vmcnt" in ln]
        for k in waits:
            assert barrier_follows(lines, k), \
                f"<{where}>: a wait on global loads that is not right before a barrier: {lines[k]}"
        counts = sorted(int(re.search(r"vmcnt\((\d+)\)", lines[k]).group(1)) for k in waits)
        if args[7] == "2":
            assert counts == [0], f"<{where}>: waits on global loads in the K loop: {counts}"
        else:
            # three (four) buffers: the loads of tile t + 2 (and t + 3) stay in
            # flight across the barrier (nonzero counts), except near the end
            nbuf = int(args[7])
            assert len(counts) == nbuf - 1 and counts[0] == 0 and \
                all(c == counts[1] * i for i, c in enumerate(counts)) and counts[1] > 0, \
                f"<{where}>: waits on global loads in the K loop: {counts}"
            stages3 += 1
        # the per-step global addresses advance by increments; a multiply per
        # K-step here cost the 16-wave kernels 11%
        muls = [ln for ln in lines if ln.startswith(("s_mul_i32", "s_mul_hi_u32"))]
        assert not muls, f"<{where}>: address multiplies in the K loop: {muls[:3]}"
        checked += 1
    assert checked >= 10 and stages3 >= 4, f"only {checked} direct-load kernels found ({stages3} with three buffers)"
