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
