"""Planted mistakes in copies of the CPU oracle must fail its pins (no GPU).

Each mutant is a textual edit of ``oracle/gemm_oracle.c`` compiled into a
temporary library (the real oracle source is never modified).  The pins run
in a child process, so a mutant that reads out of bounds and crashes counts
as caught rather than taking the test runner down.  The unmodified source,
built the same way, must pass: that shows the harness itself is sound.
"""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, replacement): one plausible slip each
MUTANTS = [
    ("first_term_dropped", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 1; k < K; ++k)"),
    ("last_term_dropped", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k < K - 1; ++k)"),
    ("sign_flipped", "acc[j] += a_ik", "acc[j] -= a_ik"),
    ("float_accumulator", "acc[j] += a_ik * (double)b_row[j];",
     "acc[j] = (float)(acc[j] + (float)(a_ik * (double)b_row[j]));"),
    ("lda_ignored", "A + i * lda", "A + i * K"),
    ("ldb_ignored", "B + k * ldb", "B + k * N"),
    ("b_rows_reversed", "B + k * ldb", "B + (K - 1 - k) * ldb"),
    ("b_columns_mirrored", "(double)b_row[j]", "(double)b_row[N - 1 - j]"),
    ("a_row_reversed", "(double)a_row[k]", "(double)a_row[K - 1 - k]"),
    ("accumulator_not_reset", "acc[j] = 0.0;", "(void)0;"),
    ("row_selection_ignored", "const int64_t i = rows ? rows[t] : t;", "const int64_t i = t;"),
    ("fp64_sums_not_stored", "c64[j] = acc[j];", "c64[j] = (double)(float)acc[j];"),
    # B read as if transposed (B[j][k]); the modulo keeps the read in bounds
    ("b_transposed", "(double)b_row[j]", "(double)B[(j % K) * ldb + (k % N)]"),
]


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"lib{name}.so"
    oracle.build(str(src), str(lib))
    return lib


def _run_pins(lib):
    env = dict(os.environ, PYTHONPATH=ROOT, OMP_NUM_THREADS="2")
    return subprocess.run(
        [sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), "--lib", str(lib)],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_unmodified_copy_passes(tmp_path):
    with open(oracle.SOURCE) as f:
        text = f.read()
    res = _run_pins(_build(tmp_path, "control", text))
    assert res.returncode == 0, res.stdout + res.stderr


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(oracle.SOURCE) as f:
        text = f.read()
    assert old in text, f"mutation site for {name} not found"
    res = _run_pins(_build(tmp_path, name, text.replace(old, new, 1)))
    assert res.returncode != 0, f"mutant {name} passed every pin:\n{res.stdout}"
