"""Host-side logic of bench.py (no GPU needed)."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _copy_sources(tmp_path):
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    return str(tmp_path)


def test_fingerprint_ignores_comments_not_code(tmp_path):
    root = _copy_sources(tmp_path)
    name = "some_config"
    base = bench.kernel_fingerprint(name, root)
    assert base == bench.kernel_fingerprint(name, ROOT)
    src = tmp_path / bench.KERNEL_SOURCES[0]
    text = src.read_text()
    src.write_text("// a new comment line\n" + text.replace("\n", "\n  ", 3) + "\n/* block\n comment */\n")
    assert bench.kernel_fingerprint(name, root) == base
    src.write_text(text + "\nstatic int extra_symbol = 1;\n")
    assert bench.kernel_fingerprint(name, root) != base
    assert bench.kernel_fingerprint("other_config", ROOT) != base


def test_traffic_record_is_ignored_when_stale(tmp_path, monkeypatch):
    name, wl = "cfg_x", "square8192"
    prof = tmp_path / "profiles"
    prof.mkdir()
    fp = bench.kernel_fingerprint(name)
    (prof / f"traffic_{name}_{wl}.md").write_text(
        f"kernel_fingerprint: {fp}\nhbm_bytes_per_launch: 1.5e+09\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES",
                        [os.path.join(ROOT, r) for r in bench.KERNEL_SOURCES])
    assert bench.read_traffic(wl, name) == 1.5e9
    (prof / f"traffic_{name}_{wl}.md").write_text(
        "kernel_fingerprint: 0000000000000000\nhbm_bytes_per_launch: 1.5e+09\n")
    assert bench.read_traffic(wl, name) is None
    assert bench.read_traffic(wl, "no_such_config") is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_oracle_rows_plan():
    assert bench.oracle_rows_plan(8192, 12.0 / 8192, 90.0, 15.0) is None
    rows = bench.oracle_rows_plan(8192, 1.0, 90.0, 15.0)
    assert len(rows) == 512 and rows[0] == 0 and rows[-1] == 8191
    rows = bench.oracle_rows_plan(100000, 0.01, 90.0, 15.0)
    assert len(rows) == 1500 and rows[0] == 0 and rows[-1] == 99999


def test_oracle_leg_checks_every_cell_and_times_the_run():
    """With a whole-product budget the leg checks every cell: one wrong cell
    anywhere fails it; the baseline reports the rows it ran."""
    import numpy as np

    import oracle
    from dense_fp32_gemm_row_amd.workloads import make_inputs

    A, B = make_inputs(300, 200, 100, "uniform", seed=3)
    C = oracle.gemm(A, B)
    par, cpu = bench.oracle_leg(A, B, C, 90.0, 15.0, check=True, baseline=True)
    assert par["ok"] and par["cells_checked"] == 300 * 200 and "freivalds" not in par
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and "all 300 output rows" in cpu["sample"]
    bad = C.copy()
    bad[217, 133] += np.float32(0.05)
    par, _ = bench.oracle_leg(A, B, bad, 90.0, 15.0, check=True, baseline=False)
    assert not par["ok"]
    bad = C.copy()
    bad[5, 7] = np.nan
    par, _ = bench.oracle_leg(A, B, bad, 90.0, 15.0, check=True, baseline=False)
    assert not par["ok"]


def test_cpu_model_reads_the_first_processor(tmp_path):
    info = tmp_path / "cpuinfo"
    info.write_text("processor\t: 0\nvendor_id\t: AuthenticAMD\ncpu family\t: 26\nmodel\t\t: 2\n"
                    "model name\t: AMD EPYC\n\nprocessor\t: 1\ncpu family\t: 25\nmodel\t\t: 17\n"
                    "model name\t: Other\n")
    assert bench.cpu_model(str(info)) == "AMD EPYC (family 26, model 2)"
    info.write_text("processor\t: 0\nmodel name\t: Some CPU\n")
    assert bench.cpu_model(str(info)) == "Some CPU"
    assert bench.cpu_model(str(tmp_path / "missing")) is None
