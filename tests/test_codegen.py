"""Code-generation checks of the MFMA kernels (CPU only: hipcc cross-compiles
gfx950 assembly without a GPU).

Direct global -> LDS loads of K-step t + 1 (or t + 2) land in a buffer that
step t does not read.  The compiler only knows that through the alias scopes
it gives each LDS array, and those scopes reach loads only a few address
offsets away from the array.  When they do not reach the fragment reads, the
compiler waits for all outstanding global loads before the first LDS read
of every K-step, which serialises the prefetch with the math (about 1.5% of
the headline throughput).  These tests keep the one wait on global loads in
each K loop where it belongs: right before the barrier that publishes the
next tile.
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
def mfma_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "mfma.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", os.path.join(CSRC, "mfma.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def loop_blocks(body: str) -> str:
    """The blocks of the (single, innermost) K loop of a kernel, in layout
    order: the block the compiler marks as loop header and every block it
    marks as inside that loop."""
    blocks, cur = [], []
    for line in body.splitlines():
        if re.match(r"^(\.LBB\S+:|; %bb\.\d+:)", line) and cur:
            blocks.append(cur)
            cur = []
        cur.append(line)
    blocks.append(cur)
    header = None
    for blk in blocks:
        m = re.match(r"^\.L(BB\S+):.*Loop Header", blk[0])
        if m:
            header = m.group(1)
    assert header, "no loop header found"
    keep = [blk for blk in blocks
            if blk[0].startswith(f".L{header}:") or f"Header={header} " in blk[0]]
    return "\n".join(line for blk in keep for line in blk)


def ring_kernels(asm: str):
    """(template arguments, K-loop blocks) of every pipelined kernel."""
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
        yield args, loop_blocks(body)


def test_direct_load_kernels_wait_only_at_the_barrier(mfma_asm):
    checked = 0
    for args, loop in ring_kernels(mfma_asm):
        # <BM, BN, BK, WM, WN, PADA, PADB, STAGES, DIRECT, GUARD, VEC, TA, TB, IL>
        if args[8] != "true":
            continue
        lines = [ln.strip() for ln in loop.splitlines()]
        waits = [k for k, ln in enumerate(lines) if ln.startswith("s_waitcnt") and "vmcnt" in ln]
        where = ", ".join(args)
        assert len(waits) == 1, f"<{where}>: {len(waits)} waits on global loads in the K loop"
        k = waits[0]
        assert any(ln.startswith("s_barrier") for ln in lines[k + 1:k + 3]), \
            f"<{where}>: the wait on global loads is not right before the barrier"
        checked += 1
    assert checked >= 10, f"only {checked} direct-load kernels found"
