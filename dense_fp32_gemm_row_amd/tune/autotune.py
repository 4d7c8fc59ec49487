"""Per-shape tile autotuning ("Tiling and Blocking for Reuse", "choosing the
tile size": tile size trades reuse against occupancy and tail waste, and is
settled by measurement).

Times every compiled configuration of the chosen variants on each workload
shape through gemm_f32_variant, on the GPU, and writes the fastest
configuration per shape into a table in the format of tune/table.json.
The build turns that table into the dispatch table of gemm_f32.

    python -m dense_fp32_gemm_row_amd.tune.autotune --out tuned.json

With --calibrate it also measures the cost model that gemm_f32 uses for
shapes not in the table: every candidate of the table's "model" section runs
on the calibration shapes below, and for each shape a CU's share is
n = ceil(tiles / cus) tiles; the per-CU rate 2 * bm * bn * K * n /
(time - launch floor) is collected at level min(n, len(gflops_per_cu)), and
each entry of gflops_per_cu becomes the median of its level.  A tile also
has a fixed cost, its prologue and the stores of C that no other
workgroup's math hides, counted as k0 more k: on the short-K shapes below
k0 is the median of what the time needs beyond K at those rates, and the
rates are then fitted again with K + k0.  The number of
levels per candidate is set in the table (at least its occupancy, and two
for a candidate that fits one tile per CU, since one tile per CU runs
faster per CU than several in turn).  `unaligned` is the median ratio of
the rate on shapes whose rows are not 16-byte aligned to the aligned rate
at the same level, and `trans` the same ratio for operands stored transposed
(A as K x M and / or B as N x K) on a few squares.  A candidate with
`whole_k` (a persistent kernel) is fitted only on the shapes it runs in that
form: whole tiles, K a multiple of whole_k; its `edge` factor is the median
ratio of its rate on edge tiles and K past whole rounds (with K rounded up to
whole rounds) to the rate at the same level.

    python -m dense_fp32_gemm_row_amd.tune.autotune --out tuned.json --calibrate

Timing: every timed loop runs behind a long launch (two 8192^3 products),
so that the host has enqueued all timed launches before the first one runs
and the events around each launch time the GPU, not the host's launch cost
(which exceeds the kernel on small products).  The launch floor subtracted
above is then the GPU's own cost of a 1 x 1 x 1 launch of the candidate.

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


# calibration shapes of the cost model: every one runs long enough (K up to
# 8192 for the small tile counts) that the host-side launch floor, 7 to 20 us
# depending on the host, stays a small correction; squares over the sizes
# where the candidates trade places, a few rectangular products, and shapes
# whose rows are not 16-byte aligned (K or N not a multiple of 4)
CAL_SHAPES = ([(n, n, 8192) for n in (512, 768, 1024, 1280, 1536, 1792)] +
              [(n, n, n) for n in (2048, 2560, 3072, 3584, 4096, 5120, 6144, 8192)] +
              [(1024, 8192, 8192), (8192, 1024, 4096), (2048, 2048, 8192), (4096, 2048, 1024),
               (3000, 3000, 3000)])
CAL_UNALIGNED = [(1000, 1023, 7777), (2049, 2049, 2049), (3001, 3001, 3001), (4096, 4096, 4095),
                 (8192, 8192, 2047)]
# short K and many output tiles: where a tile's fixed cost (its prologue, and
# the stores of C that no other workgroup's math hides) shows
CAL_SHORTK = [(8192, 8192, 64), (8192, 8192, 128), (16384, 16384, 128), (16384, 16384, 256),
              (6144, 8192, 128)]
# transposed operands (A stored K x M and/or B stored N x K) on shapes of
# CAL_SHAPES, for the candidates that take them
CAL_TRANS = [(2048, 2048, 8192), (4096, 4096, 4096), (6144, 6144, 6144), (8192, 8192, 8192)]
TRANS_OPS = ("NT", "TN", "TT")
# edge tiles and K past whole rounds, for persistent candidates (whole_k)
CAL_EDGE = [(8000, 8000, 8000), (6000, 6000, 6000), (4000, 4000, 4000), (8192, 8192, 8100),
            (2000, 2000, 6000)]


def calibrate_model(binding, model: dict, budget_ms: float, blocker=None) -> dict:
    """Measured per-CU rates of the model's candidates (see the module doc)."""
    import math
    import statistics

    import torch

    cus = int(model["cus"])
    times: dict[tuple, float] = {}
    for M, N, K in CAL_SHAPES + CAL_UNALIGNED + CAL_SHORTK + [(1, 1, 1)]:
        g = torch.Generator(device="cuda").manual_seed(0)
        dA = torch.rand((M, K), device="cuda", generator=g)
        dB = torch.rand((K, N), device="cuda", generator=g)
        dC = torch.empty((M, N), device="cuda")
        for cand in model["candidates"]:
            cfg = cand["config"]

            def call(cfg=cfg):
                binding.gemm(dA, dB, dC, variant="mfma", config=cfg)

            times[(cfg, M, N, K)] = time_fn(call, budget_ms, blocker)
            print(json.dumps({"calibrate": cfg, "M": M, "N": N, "K": K,
                              "median_ms": round(times[(cfg, M, N, K)], 5)}), flush=True)
        del dA, dB, dC
        torch.cuda.empty_cache()
    for M, N, K in CAL_TRANS:
        g = torch.Generator(device="cuda").manual_seed(0)
        for ops in TRANS_OPS:
            dA = (torch.rand((K, M), device="cuda", generator=g).t() if ops[0] == "T"
                  else torch.rand((M, K), device="cuda", generator=g))
            dB = (torch.rand((N, K), device="cuda", generator=g).t() if ops[1] == "T"
                  else torch.rand((K, N), device="cuda", generator=g))
            dC = torch.empty((M, N), device="cuda")
            for cand in model["candidates"]:
                cfg = cand["config"]

                def call(cfg=cfg):
                    binding.gemm(dA, dB, dC, variant="mfma", config=cfg)

                try:
                    call()
                except binding.GemmError:  # the configuration takes row-major operands only
                    continue
                times[(cfg, ops, M, N, K)] = time_fn(call, budget_ms, blocker)
                print(json.dumps({"calibrate": cfg, "ops": ops, "M": M, "N": N, "K": K,
                                  "median_ms": round(times[(cfg, ops, M, N, K)], 5)}), flush=True)
            del dA, dB, dC
        torch.cuda.empty_cache()
    for M, N, K in CAL_EDGE:
        g = torch.Generator(device="cuda").manual_seed(0)
        dA = torch.rand((M, K), device="cuda", generator=g)
        dB = torch.rand((K, N), device="cuda", generator=g)
        dC = torch.empty((M, N), device="cuda")
        for cand in model["candidates"]:
            if not int(cand.get("whole_k", 0)):
                continue
            cfg = cand["config"]

            def call(cfg=cfg):
                binding.gemm(dA, dB, dC, variant="mfma", config=cfg)

            times[(cfg, "edge", M, N, K)] = time_fn(call, budget_ms, blocker)
            print(json.dumps({"calibrate": cfg, "edge": True, "M": M, "N": N, "K": K,
                              "median_ms": round(times[(cfg, "edge", M, N, K)], 5)}), flush=True)
        del dA, dB, dC
        torch.cuda.empty_cache()
    out = {"cus": cus, "candidates": []}
    for cand in model["candidates"]:
        cfg, bm, bn = cand["config"], int(cand["bm"]), int(cand["bn"])
        levels = len(cand["gflops_per_cu"])
        floor = times[(cfg, 1, 1, 1)]
        whole_k = int(cand.get("whole_k", 0))

        def rated(M, N, K):
            """Shapes the model rates this candidate on: all, or for a
            persistent candidate those it runs in that form."""
            return whole_k == 0 or (M % bm == 0 and N % bn == 0 and K % whole_k == 0)

        def share(M, N):
            n = math.ceil(math.ceil(M / bm) * math.ceil(N / bn) / cus)
            return n, min(n, levels)

        def fit_rates(k0):
            groups: dict[int, list[float]] = {}
            for M, N, K in CAL_SHAPES:
                if not rated(M, N, K):
                    continue
                n, level = share(M, N)
                ms = max(times[(cfg, M, N, K)] - floor, 1e-6)
                groups.setdefault(level, []).append(2.0 * bm * bn * (K + k0) * n / (ms * 1e-3) / 1e9)
            rates = []
            for level in range(1, levels + 1):  # a level with no shape inherits the one below
                rates.append(statistics.median(groups[level]) if level in groups else rates[-1])
            return rates

        def fit_k0(rates):
            extra = []
            for M, N, K in CAL_SHORTK:
                if not rated(M, N, K):
                    continue
                n, level = share(M, N)
                ms = max(times[(cfg, M, N, K)] - floor, 1e-6)
                extra.append(ms * 1e-3 * rates[level - 1] * 1e9 / (n * 2.0 * bm * bn) - K)
            return max(0.0, statistics.median(extra)) if extra else float(cand.get("k0", 0.0))

        k0 = fit_k0(fit_rates(0.0))
        rates = fit_rates(k0)
        k0 = fit_k0(rates)
        ratios = []
        for M, N, K in CAL_UNALIGNED:
            if not rated(M, N, K):
                continue
            n, level = share(M, N)
            ms = max(times[(cfg, M, N, K)] - floor, 1e-6)
            ratios.append(2.0 * bm * bn * (K + k0) * n / (ms * 1e-3) / 1e9 / rates[level - 1])
        # transposed operands: the median ratio of the rate to the row-major
        # rate at the same level (1 for candidates that do not take them)
        tratios = []
        for M, N, K in CAL_TRANS:
            n, level = share(M, N)
            for ops in TRANS_OPS:
                if (cfg, ops, M, N, K) in times and rated(M, N, K):
                    ms = max(times[(cfg, ops, M, N, K)] - floor, 1e-6)
                    tratios.append(2.0 * bm * bn * (K + k0) * n / (ms * 1e-3) / 1e9 / rates[level - 1])
        # a persistent candidate's edge form (edge tiles, K rounded up to whole
        # rounds of whole_k): the median ratio of its rate to the rate at the
        # same level
        eratios = []
        for M, N, K in CAL_EDGE:
            if (cfg, "edge", M, N, K) in times:
                n, level = share(M, N)
                kr = -(-K // whole_k) * whole_k
                ms = max(times[(cfg, "edge", M, N, K)] - floor, 1e-6)
                eratios.append(2.0 * bm * bn * (kr + k0) * n / (ms * 1e-3) / 1e9 / rates[level - 1])
        entry = {**cand, "gflops_per_cu": [round(r, 1) for r in rates], "k0": round(k0, 1),
                 "unaligned": round(min(1.0, statistics.median(ratios)), 3) if ratios else 1.0,
                 "trans": round(statistics.median(tratios), 3) if tratios else 1.0}
        if whole_k:
            entry["edge"] = round(min(1.0, statistics.median(eratios)), 3) if eratios else 1.0
        out["candidates"].append(entry)
    return out


def make_blocker(binding):
    """A launch of about 15 ms (two 8192^3 products).  Enqueued before a
    timed loop, it keeps the GPU busy while the host enqueues every timed
    launch, so that the events around each launch time the GPU's work (and
    its gap between kernels) rather than the host's launch cost, which
    exceeds the kernel time of small products."""
    import torch

    n = 8192
    bA = torch.zeros((n, n), device="cuda")
    bB = torch.zeros((n, n), device="cuda")
    bC = torch.empty((n, n), device="cuda")
    fn = binding.prepare(bA, bB, bC)

    def block():
        fn()
        fn()

    # prepare() keeps raw device addresses: the tensors must outlive every
    # call of the blocker (freed, their memory could be reused or unmapped)
    block.operands = (bA, bB, bC)
    return block


def time_config(binding, v, c, dA, dB, dC, reps, warmup, blocker=None):
    import torch

    stream = torch.cuda.current_stream()
    launch = binding.prepare(dA, dB, dC, variant=v, config=c)
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    if blocker is not None:
        blocker()
    for s, e in ev:
        s.record(stream)
        launch()
        e.record(stream)
    torch.cuda.synchronize()
    times = sorted(s.elapsed_time(e) for s, e in ev)
    return times[len(times) // 2]


def time_fn(fn, budget_ms: float, blocker=None) -> float:
    """Median milliseconds of fn() over enough launches to fill ~budget_ms
    (behind `blocker`, a long launch, when given: see make_blocker)."""
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
    if blocker is not None:
        blocker()
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
    ap.add_argument("--extra", default="",
                    help="comma-separated further shapes MxNxK to time (reported; written to "
                         "the table only with --keep-extra)")
    ap.add_argument("--keep-extra", action="store_true")
    ap.add_argument("--budget-ms", type=float, default=400.0,
                    help="approximate timed milliseconds per configuration")
    ap.add_argument("--calibrate", action="store_true",
                    help="also re-measure the cost model's per-CU rates (written to --out)")
    ap.add_argument("--configs", default="",
                    help="comma-separated configuration names to time (default: all)")
    ap.add_argument("--no-queue-ahead", action="store_true",
                    help="time launches without a long launch ahead of them (the events then "
                         "include the host's launch cost on small products)")
    ap.add_argument("--splits", default="",
                    help="comma-separated split counts: also time gemm_f32_splitk with each "
                         "(reported, not written to the table)")
    args = ap.parse_args()

    import torch

    from dense_fp32_gemm_row_amd import binding

    binding.load()
    shapes = [s for s in DEFAULT_SHAPES if s[0] in args.shapes.split(",")]
    extra = []
    for x in (x for x in args.extra.split(",") if x):
        M, N, K = (int(v) for v in x.split("x"))
        extra.append((x, M, N, K))
    shapes += extra
    variants = [binding.VARIANTS[v] for v in args.variants.split(",")]
    with open(args.base) as f:
        table = json.load(f)
    entries = {(e["M"], e["N"], e["K"]): e for e in table.get("entries", [])}
    report = []
    blocker = None if args.no_queue_ahead else make_blocker(binding)
    only = set(x for x in args.configs.split(",") if x)
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
                if only and cname not in only:
                    continue
                probe = time_config(binding, v, c, dA, dB, dC, reps=3, warmup=1, blocker=blocker)
                reps = int(max(5, min(500, args.budget_ms / max(probe, 1e-3))))
                ms = time_config(binding, v, c, dA, dB, dC, reps=reps, warmup=2, blocker=blocker)
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
        best_entry = {"M": M, "N": N, "K": K, "config": best, "shape": name,
                      "median_ms": round(best_ms, 5), "tflops": round(flops / best_ms / 1e9, 3)}
        if (name, M, N, K) not in extra or args.keep_extra:
            entries[(M, N, K)] = best_entry
        report.append(best_entry)
        del dA, dB, dC
        torch.cuda.empty_cache()
    table["entries"] = sorted(entries.values(), key=lambda e: (e["M"], e["N"], e["K"]))
    if args.calibrate:
        table["model"] = calibrate_model(binding, table["model"], min(args.budget_ms, 200.0),
                                         blocker)
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump(table, f, indent=2)
        f.write("\n")
    print(json.dumps({"best": report}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
