#!/usr/bin/env python3
"""FP32 GEMM throughput on one MI355X, through the C ABI.

One step is one call of gemm_f32 (C = A x B, row-major FP32) on the
workload's operands, which are resident in HBM before timing starts.  The
default workload is M = N = K = 8192 with uniform[-1, 1) inputs from seed 0.

Prints ONE JSON line with the throughput (TFLOP/s = 2 M N K / time), the
dominant kernel's roofline position (measured live with HIP events on the
stream the kernel runs on), the oracle timed on the host's cores, and a parity
check of the timed output against that oracle run: every row of the product
when the oracle finishes it within --full-oracle-seconds, else a bounded
sample of rows plus a Freivalds projection.
Each step is its own launch with an event pair around it; with --graph the
steps are captured into one HIP graph and timed as one replay, which removes
the host's cost per launch (it bounds the small workloads).

Other modes (results on stderr / in a file, not the contract line):
  --stages   time every kernel stage (naive, LDS-tiled, register-blocked,
             MFMA) on the workload
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_MATRIX_TFLOPS = 157.3  # MI355X: 256 CU x 4 SIMD x 64 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "FP32 GEMM TFLOP/s at M=N=K=8192 on 1 MI355X; % of FP32 matrix peak"
KERNEL_SOURCES = ["dense_fp32_gemm_row_amd/csrc/mfma_kernels.h",
                  "dense_fp32_gemm_row_amd/csrc/mfma.hip",
                  "dense_fp32_gemm_row_amd/csrc/mfma16.hip",
                  "dense_fp32_gemm_row_amd/csrc/mfma_regs.hip",
                  "dense_fp32_gemm_row_amd/csrc/gemm_internal.h"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_fingerprint(config_name: str, root: str = ROOT) -> str:
    """Hash of the configuration name and of the MFMA kernel sources with
    comments and whitespace removed: it changes when the compiled code can,
    not when a comment does."""
    h = hashlib.sha256(config_name.encode())
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, config_name: str) -> float | None:
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled against a copy kernel of known size), as recorded in
    profiles/; None when no record exists or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config_name}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fp = re.search(r"kernel_fingerprint:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not fp or not val or fp.group(1) != kernel_fingerprint(config_name):
        return None
    return float(val.group(1))


def cpu_model(path: str = "/proc/cpuinfo") -> str | None:
    """The first CPU's model name, with its family and model numbers (a
    virtualised host may report only a generic name)."""
    fields = {}
    try:
        with open(path) as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block only
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    except OSError:
        return None
    name = fields.get("model name")
    if name and "cpu family" in fields and "model" in fields:
        return f"{name} (family {fields['cpu family']}, model {fields['model']})"
    return name


def device_info(dev) -> dict:
    """Compute units and maximum engine clock of the device, and the FP32
    matrix peak they imply (CUs x 4 SIMDs x 64 FLOP per clock x clock).  The
    clock comes from rocminfo, run as a child process; None when unavailable."""
    import subprocess

    import torch

    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": p.gcnArchName, "cus": p.multi_processor_count,
            "max_sclk_mhz": None, "peak_from_clock_tflops": None}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return info
    arch = p.gcnArchName.split(":")[0]
    for agent in out.split("Agent ")[1:]:
        if re.search(rf"Name:\s+{re.escape(arch)}\b", agent) is None:
            continue
        clk = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        cus = re.search(r"Compute Unit:\s+(\d+)", agent)
        if clk and cus:
            info["max_sclk_mhz"] = int(clk.group(1))
            info["peak_from_clock_tflops"] = round(
                int(cus.group(1)) * 4 * 64 * int(clk.group(1)) * 1e6 / 1e12, 1)
        break
    return info


def time_launches(fn, steps: int, warmup: int, stream):
    """Runs fn() warmup times, then `steps` times with an event pair around
    each launch on `stream`.  Returns (total_ms, per-launch ms list)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    total = starts[0].elapsed_time(ends[-1])
    return total, per


def time_graph(make_fn, steps: int, warmup: int, stream):
    """Runs make_fn(stream)() warmup times, then captures `steps` launches of
    make_fn(capture stream) into one HIP graph (torch.cuda.CUDAGraph) and times
    a replay on `stream` with one event pair (after an untimed replay that
    uploads the graph).  Returns (total_ms, [total_ms / steps])."""
    import torch

    eager = make_fn(stream)
    for _ in range(warmup):
        eager()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        fn = make_fn(cap)
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        graph.replay()
        end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    return total, [total / steps]


def oracle_rows_plan(M: int, per_row_s: float, full_limit_s: float, target_s: float):
    """Rows the oracle computes: all of them when that takes at most
    full_limit_s, else enough evenly spaced rows (at least 512, the first and
    last included) for about target_s.  None stands for every row."""
    if per_row_s * M <= full_limit_s:
        return None
    n = int(min(M, max(512, target_s / max(per_row_s, 1e-9))))
    import numpy as np

    return sorted(set(np.linspace(0, M - 1, n).astype(np.int64).tolist()))


def oracle_leg(A, B, C, full_limit_s: float, target_s: float, check: bool, baseline: bool):
    """The oracle, as it stands, with the host's default OpenMP thread count,
    on the timed output's product: every row when the whole product takes at
    most full_limit_s on this host (8192^3 takes about 12 s on 16 cores),
    else a bounded sample of evenly spaced rows.  The one run gives both the
    CPU baseline (its rate, scaled per FLOP) and the parity check of every
    computed cell against the oracle's FP64 sums; a sampled check adds a
    Freivalds projection of the whole product.  Returns (parity, baseline)."""
    import numpy as np

    import oracle

    M, K = A.shape
    N = B.shape[1]
    threads = oracle.default_threads()
    probe = list(range(min(M, threads)))
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=probe, threads=threads)
    per_row = (time.perf_counter() - t0) / len(probe)
    rows = oracle_rows_plan(M, per_row, full_limit_s, target_s)
    t0 = time.perf_counter()
    _, ref = oracle.gemm(A, B, rows=rows, threads=threads, return_f64=True)
    t = time.perf_counter() - t0
    nrows = M if rows is None else len(rows)
    parity = cpu = None
    if check:
        got = (C if rows is None else C[rows]).astype(np.float64)
        err = np.abs(got - ref)
        max_err = float(err.max()) if err.size else 0.0
        norm = float(np.linalg.norm(ref))
        rel = float(np.linalg.norm(got - ref) / norm) if norm > 0 else 0.0
        del got, err
        tol_max, tol_rel = 1e-4 * math.sqrt(max(K, 1)), 1e-5
        ok = (not np.isnan(C).any()) and max_err <= tol_max and rel <= tol_rel
        parity = {"cells_checked": nrows * N, "cells": M * N, "max_abs_err": max_err,
                  "rel_fro": rel, "tol_max": tol_max, "tol_rel": tol_rel}
        if rows is not None:
            rng = np.random.default_rng(1)
            x = rng.choice([-1.0, 1.0], size=N)
            fr_ref = A.astype(np.float64) @ (B.astype(np.float64) @ x)
            fr = float(np.linalg.norm(C.astype(np.float64) @ x - fr_ref) / np.linalg.norm(fr_ref))
            parity["freivalds"] = fr
            ok = ok and fr <= tol_rel
        parity["ok"] = bool(ok)
    if baseline:
        what = (f"all {M} output rows" if rows is None else
                f"{nrows} of {M} output rows (evenly spaced)")
        cpu = {
            "value": round(2.0 * nrows * N * K / t / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": threads,
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{what} of the {M}x{N}x{K} product, each a full {K}x{N} sweep; "
                      f"{t:.1f} s wall, FP64 accumulation",
        }
    return parity, cpu


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square8192")
    ap.add_argument("--variant", default=None, help="naive|lds|regblock|mfma (default: library choice)")
    ap.add_argument("--config", default=None, help="configuration name of the variant")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time budget when the whole product would take longer than "
                         "--full-oracle-seconds (then a sample of rows is computed)")
    ap.add_argument("--full-oracle-seconds", type=float, default=90.0,
                    help="the oracle computes every row of the product when its estimate is "
                         "at most this")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--ops", default="NN", choices=["NN", "NT", "TN", "TT"],
                    help="store A and/or B transposed (the product is the same)")
    ap.add_argument("--splitk", type=int, default=None, metavar="S",
                    help="time gemm_f32_splitk with S splits (partial products + reduction); "
                         "0 = the library's choice of splits")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as one captured HIP graph instead of one launch each "
                         "(removes the host's launch cost; per-launch time is the replay / steps)")
    ap.add_argument("--stages", action="store_true")
    ap.add_argument("--stage-variants", default="naive,lds,regblock,mfma",
                    help="variants that --stages times")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes "
                         "(reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from dense_fp32_gemm_row_amd import binding
    from dense_fp32_gemm_row_amd.workloads import WORKLOADS, workload_inputs

    if args.ops != "NN" and args.stages:
        print("--ops does not apply to --stages", file=sys.stderr)
        return 2
    if args.splitk is not None and (args.ops != "NN" or args.stages):
        print("--splitk takes row-major operands and no --stages", file=sys.stderr)
        return 2

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps)
    binding.load()
    w = WORKLOADS[args.workload]
    M, N, K = w.M, w.N, w.K
    log(f"workload {w.name}: M={M} N={N} K={K} dist={w.dist}")
    A, B = workload_inputs(w.name)
    dev = torch.device("cuda:0")
    def stored(X, op):  # op(X) = X, kept as stored (N) or as a view of X^T (T)
        if op == "N":
            return torch.from_numpy(X).to(dev)
        return torch.from_numpy(np.ascontiguousarray(np.swapaxes(X, -1, -2))).to(dev).transpose(-1, -2)

    dA = stored(A, args.ops[0])
    dB = stored(B, args.ops[1])
    nb = w.batch
    dC = torch.empty((nb, M, N) if nb > 1 else (M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = 2.0 * nb * M * N * K

    if args.stages:
        return run_stages(args, w, A, B, dA, dB, dC, stream, flops)

    plan = None
    if args.variant is None:
        v, c = None, None
        if nb == 1 and args.ops == "NN":
            plan = binding.gemm_f32_plan(M, N, K, K, N, N)
            v, c = plan["configs"][0]
    else:
        v = binding.VARIANTS[args.variant]
        if args.config:
            c = binding.config_id(v, args.config)
        elif v == binding.VARIANT_MFMA:
            c = binding.gemm_f32_select(M, N, K, K, N, N)[1]
        else:
            c = 0
    cname = (binding.gemm_f32_config_name(v, c) if v is not None
             else f"library choice ({'batched ' if nb > 1 else ''}{args.ops})")
    if plan is not None and plan["parts"] == 2:  # two launches on complementary parts of C
        part = "rows" if plan["axis"] == 0 else "columns"
        cname = (f"{cname} (first {plan['split']} {part}) + "
                 f"{binding.gemm_f32_config_name(*plan['configs'][1])}")
    log(f"kernel {cname}")

    if args.splitk is not None:
        if nb > 1:
            print("--splitk takes a single product", file=sys.stderr)
            return 2
        need = binding.gemm_f32_splitk_workspace_size(M, N, K, args.splitk)
        work = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
        sv, sc = (None, -1) if args.variant is None else (v, c)

        def make_fn(s):
            return lambda: binding.gemm_splitk(dA, dB, args.splitk, dC, work, variant=sv,
                                               config=sc, stream=s)
        splits = args.splitk or "library choice of"
        cname = (f"{cname if args.variant is not None else 'library choice'}, "
                 f"split-K ({splits} splits)")
    else:  # gemm_f32 / gemm_f32_strided_batched (or the explicit kernel), arguments built once
        kw = {} if args.variant is None else {"variant": v, "config": c}

        def make_fn(s):
            return binding.prepare(dA, dB, dC, stream=s, batched=nb > 1, **kw)

    dinfo = device_info(dev)
    if args.graph:
        total_ms, per = time_graph(make_fn, args.steps, args.warmup, stream)
    else:
        total_ms, per = time_launches(make_fn(stream), args.steps, args.warmup, stream)
    ms_step = total_ms / args.steps
    avg_launch_ms = sum(per) / len(per)
    value = flops * args.steps / (total_ms / 1e3) / 1e12
    achieved = flops / (avg_launch_ms / 1e3) / 1e12
    log(f"{args.steps} steps: {ms_step:.3f} ms/step, {value:.2f} TFLOP/s "
        f"(avg launch {avg_launch_ms:.3f} ms, min {min(per):.3f}, max {max(per):.3f})")

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_FP32_MATRIX_TFLOPS, 2),
        "config": {"workload": w.name, "batch": nb, "M": M, "N": N, "K": K, "dist": w.dist,
                   "seed": w.seed, "ops": args.ops, "splitk": args.splitk,
                   "layout": "row-major C; A, B row-major, stored transposed where ops says T",
                   "kernel": cname, "parallelism": "none",
                   "timing": "one HIP graph of the steps" if args.graph else "one launch per step"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_MATRIX_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_MATRIX_TFLOPS, 4),
            "traffic": read_traffic(w.name, cname),
            "kernel": cname,
            "avg_launch_ms": round(avg_launch_ms, 4),
            "launch_ms": {"median": round(sorted(per)[len(per) // 2], 4),
                          "min": round(min(per), 4), "max": round(max(per), 4)},
            "flops_per_launch": flops,
        },
        "device": dinfo,
    }

    rc = 0
    if not (args.no_check and args.no_cpu_baseline):
        C = dC.cpu().numpy()
        products = [0, nb - 1] if nb > 1 else [None]
        checks = []
        for i in products:
            Ai, Bi, Ci = (A, B, C) if i is None else (A[i], B[i], C[i])
            par, cpu = oracle_leg(Ai, Bi, Ci, args.full_oracle_seconds, args.cpu_seconds,
                                  check=not args.no_check,
                                  baseline=not args.no_cpu_baseline and i in (None, 0))
            if par is not None:
                checks.append(par)
            if cpu is not None:
                result["cpu_baseline"] = cpu
                log(f"cpu baseline {cpu}")
        if checks:
            result["parity"] = max(checks, key=lambda r: r["rel_fro"])
            result["parity"]["ok"] = all(r["ok"] for r in checks)
            if nb > 1:
                result["parity"]["products_checked"] = products
            log(f"parity {result['parity']}")
            if not result["parity"]["ok"]:
                rc = 1
        del C
    print(json.dumps(result), flush=True)
    return rc


def run_stages(args, w, A, B, dA, dB, dC, stream, flops) -> int:
    """Per-stage timing: every compiled configuration of every variant."""
    from dense_fp32_gemm_row_amd import binding

    out = []
    wanted = [binding.VARIANTS[x] for x in args.stage_variants.split(",")]
    for v in wanted:
        for c in range(binding.gemm_f32_config_count(v)):
            name = binding.gemm_f32_config_name(v, c)
            steps = args.steps if v >= 2 else max(2, min(args.steps, 3))
            fn = binding.prepare(dA, dB, dC, variant=v, config=c, stream=stream,
                                 batched=w.batch > 1)
            total, per = time_launches(fn, steps, 1, stream)
            avg = sum(per) / len(per)
            tf = flops / (avg / 1e3) / 1e12
            rec = {"workload": w.name, "variant": v, "config": name, "avg_ms": round(avg, 4),
                   "min_ms": round(min(per), 4), "tflops": round(tf, 3),
                   "pct_peak": round(100 * tf / PEAK_FP32_MATRIX_TFLOPS, 2)}
            out.append(rec)
            log(json.dumps(rec))
    print(json.dumps({"stages": out}), flush=True)
    return 0


def copy_calibration(mib: int, steps: int) -> int:
    """A plain copy of `mib` MiB between two device buffers, `steps` times:
    each launch reads and writes exactly mib MiB of HBM, the reference that
    scales the HBM byte counters."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.rand(n, device="cuda:0")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    total, per = time_launches(lambda: dst.copy_(src), steps, 1, stream)
    avg = sum(per) / len(per)
    print(json.dumps({"copy_mib": mib, "avg_ms": round(avg, 4),
                      "gbs": round(2 * mib * (1 << 20) / (avg / 1e3) / 1e9, 1)}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
