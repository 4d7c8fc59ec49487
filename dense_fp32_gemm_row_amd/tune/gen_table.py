"""Writes csrc/tune_table.inc from tune/table.json (run by the build)."""

from __future__ import annotations

import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "table.json")
OUT = os.path.join(os.path.dirname(HERE), "csrc", "tune_table.inc")

# configuration names start with their variant's name
VARIANTS = {"naive": 0, "lds": 1, "regblock": 2, "mfma": 3}


def variant_of(config: str) -> int:
    for prefix, v in VARIANTS.items():
        if config.startswith(prefix):
            return v
    raise ValueError(f"configuration {config!r} names no variant")


def render(table: dict) -> str:
    lines = [
        "// Generated from tune/table.json by tune/gen_table.py; edit the JSON.",
        "#pragma once",
        "#include <cstdint>",
        "namespace gemm_f32_impl {",
        "struct TuneEntry {",
        "    int64_t M, N, K;",
        "    int variant;",
        "    const char *config;",
        "};",
        "// Exact shapes; the final entry (M = -1) matches nothing.",
        "constexpr TuneEntry kTuneTable[] = {",
    ]
    for e in table["entries"]:
        variant = variant_of(e["config"])
        lines.append(
            f'    {{{int(e["M"])}, {int(e["N"])}, {int(e["K"])}, {variant}, "{e["config"]}"}},'
        )
    lines += [
        '    {-1, -1, -1, 3, ""},',
        "};",
        "// Cost model for shapes not listed (see tune/table.json): per-CU",
        "// throughput of each candidate with 1, 2, ... of its tiles on a CU, and",
        "// a tile's fixed cost as k0 more k.",
        "struct ModelCandidate {",
        "    const char *config;",
        "    int bm, bn, nrates;",
        "    float gflops_per_cu[4];",
        "    float unaligned;",
        "    float k0;",
        "    float trans;  // rate factor with a transposed operand",
        "    int whole_k;  // > 0: a persistent kernel, whose K runs in rounds of whole_k, no split-K",
        "    float edge;   // its rate factor on edge tiles or K past whole rounds",
        "};",
        f'constexpr int kModelCUs = {int(table["model"]["cus"])};',
        "constexpr ModelCandidate kModel[] = {",
    ]
    for c in table["model"]["candidates"]:
        rates = [float(x) for x in c["gflops_per_cu"]]
        if not 1 <= len(rates) <= 4:
            raise ValueError(f"{c['config']}: 1 to 4 rates")
        padded = ", ".join(f"{x:.1f}f" for x in rates + [rates[-1]] * (4 - len(rates)))
        lines.append(f'    {{"{c["config"]}", {int(c["bm"])}, {int(c["bn"])}, {len(rates)}, '
                     f'{{{padded}}}, {float(c["unaligned"]):.3f}f, {float(c.get("k0", 0.0)):.1f}f, '
                     f'{float(c.get("trans", 1.0)):.3f}f, {int(c.get("whole_k", 0))}, '
                     f'{float(c.get("edge", 1.0)):.3f}f}},')
    lines += [
        "};",
        "}  // namespace gemm_f32_impl",
        "",
    ]
    return "\n".join(lines)


def main() -> str:
    with open(TABLE) as f:
        text = render(json.load(f))
    old = open(OUT).read() if os.path.exists(OUT) else None
    if old != text:
        with open(OUT, "w") as f:
            f.write(text)
    return OUT


if __name__ == "__main__":
    print(main())
