"""Per-shape tile autotuning ("Tiling and Blocking for Reuse", "choosing the
tile size": tile size trades reuse against occupancy and tail waste, and is
settled by measurement).

Times every compiled configuration of the chosen variants on each workload
shape through gemm_f32_variant, on the GPU, and writes the fastest
configuration per shape into a table in the format of tune/table.json.
The build turns that table into the dispatch table of gemm_f32.

    python -m dense_fp32_gemm_row_amd.tune.autotune --out tuned.json

Correctness of every configuration is established separately by the parity
tests; this script only measures.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_SHAPES = [
    # (name, M, N, K)
    ("square256", 256, 256, 256),
    ("ragged", 1000, 1023, 777),
    ("square4096", 4096, 4096, 4096),
    ("square8192", 8192, 8192, 8192),
    ("ffn", 8192, 14336, 4096),
    # one eighth of the 8192 rows: a row shard of the headline product
    ("square8192_rowshard8", 1024, 8192, 8192),
    # few output tiles, long K: the split-K shape
    ("deepk", 1024, 1024, 65536),
    # one tiny product: the floor of one timed launch
    ("tiny", 1, 1, 1),
]


def time_config(binding, v, c, dA, dB, dC, reps, warmup):
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        binding.gemm(dA, dB, dC, variant=v, config=c)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s, e in ev:
        s.record(stream)
        binding.gemm(dA, dB, dC, variant=v, config=c)
        e.record(stream)
    torch.cuda.synchronize()
    times = sorted(s.elapsed_time(e) for s, e in ev)
    return times[len(times) // 2]


def time_fn(fn, budget_ms: float) -> float:
    """Median milliseconds of fn() over enough launches to fill ~budget_ms."""
    import torch

    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    probe = []
    for _ in range(3):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        torch.cuda.synchronize()
        probe.append(s.elapsed_time(e))
    reps = int(max(5, min(500, budget_ms / max(min(probe), 1e-3))))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    times = sorted(s.elapsed_time(e) for s, e in ev)
    return times[len(times) // 2]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True, help="where to write the tuned table (JSON)")
    ap.add_argument("--base", default=os.path.join(HERE, "table.json"),
                    help="table whose defaults are kept")
    ap.add_argument("--variants", default="mfma")
    ap.add_argument("--shapes", default=",".join(s[0] for s in DEFAULT_SHAPES))
    ap.add_argument("--budget-ms", type=float, default=400.0,
                    help="approximate timed milliseconds per configuration")
    ap.add_argument("--splits", default="",
                    help="comma-separated split counts: also time gemm_f32_splitk with each "
                         "(reported, not written to the table)")
    args = ap.parse_args()

    import torch

    from dense_fp32_gemm_row_amd import binding

    binding.load()
    shapes = [s for s in DEFAULT_SHAPES if s[0] in args.shapes.split(",")]
    variants = [binding.VARIANTS[v] for v in args.variants.split(",")]
    with open(args.base) as f:
        table = json.load(f)
    entries = {(e["M"], e["N"], e["K"]): e for e in table.get("entries", [])}
    report = []
    for name, M, N, K in shapes:
        g = torch.Generator(device="cuda").manual_seed(0)
        dA = torch.rand((M, K), device="cuda", generator=g) * 2 - 1
        dB = torch.rand((K, N), device="cuda", generator=g) * 2 - 1
        dC = torch.empty((M, N), device="cuda")
        flops = 2.0 * M * N * K
        results = []
        for v in variants:
            for c in range(binding.gemm_f32_config_count(v)):
                cname = binding.gemm_f32_config_name(v, c)
                probe = time_config(binding, v, c, dA, dB, dC, reps=3, warmup=1)
                reps = int(max(5, min(500, args.budget_ms / max(probe, 1e-3))))
                ms = time_config(binding, v, c, dA, dB, dC, reps=reps, warmup=2)
                results.append((ms, cname))
                print(json.dumps({"shape": name, "M": M, "N": N, "K": K, "config": cname,
                                  "median_ms": round(ms, 5),
                                  "tflops": round(flops / ms / 1e9, 3)}), flush=True)
        for splits in [int(x) for x in args.splits.split(",") if x]:
            need = binding.gemm_f32_splitk_workspace_size(M, N, K, splits)
            work = torch.empty(max(need // 4, 1), device="cuda")
            for v in variants:
                for c in range(binding.gemm_f32_config_count(v)):
                    cname = binding.gemm_f32_config_name(v, c)

                    def split_call(v=v, c=c):
                        binding.gemm_splitk(dA, dB, splits, dC, work, variant=v, config=c)

                    ms = time_fn(split_call, args.budget_ms)
                    print(json.dumps({"shape": name, "M": M, "N": N, "K": K, "config": cname,
                                      "splitk": splits, "median_ms": round(ms, 5),
                                      "tflops": round(flops / ms / 1e9, 3)}), flush=True)
        results.sort()
        best_ms, best = results[0]
        entries[(M, N, K)] = {"M": M, "N": N, "K": K, "config": best, "shape": name,
                              "median_ms": round(best_ms, 5),
                              "tflops": round(flops / best_ms / 1e9, 3)}
        report.append(entries[(M, N, K)])
        del dA, dB, dC
        torch.cuda.empty_cache()
    table["entries"] = sorted(entries.values(), key=lambda e: (e["M"], e["N"], e["K"]))
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump(table, f, indent=2)
        f.write("\n")
    print(json.dumps({"best": report}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
