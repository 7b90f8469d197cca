#!/usr/bin/env python3
"""Benchmark of the MI355X dense bf16 GEMM, C = A . B^T (bf16 in/out, fp32 sums).

One step is one GEMM call on one batch of synthetic input that is already
resident in HBM.  The default workload is the 4096^3 square GEMM with
N(0,1) inputs; ``--workload`` selects any other shape of
``synthetic_inputs.WORKLOADS`` (prefill, decode, ragged) for measurements
beyond the headline line, and ``--dtype f16`` measures the fp16-operand
entry point on the same shapes.

Printed: ONE JSON line with the contract fields, a ``roofline`` object for
the GEMM kernel (achieved rate from HIP events on the launch stream against
MI355X's published peak), and a ``cpu_baseline`` object (the oracle, timed on
this host's cores on a bounded sample of the same workload).

Memory-bound shapes (arithmetic intensity below the ridge point) rotate
through enough input sets to exceed the 256 MB Infinity Cache, so B is read
from HBM and not from cache ("cold" timing); compute-bound shapes reuse one
set.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("bf16 GEMM TFLOP/s (and % MFMA peak / % HBM BW) at 4096³, "
          "prefill & decode shapes")
PEAK_TFLOPS = 2500.0      # MI355X dense MFMA, bf16 and fp16 alike
PEAK_GBPS = 8000.0        # MI355X HBM3E
RIDGE = PEAK_TFLOPS * 1e12 / (PEAK_GBPS * 1e9)  # FLOP per byte
CACHE_BYTES = 256 << 20   # Infinity Cache (MALL)


def gemm_flops(M: int, N: int, K: int) -> int:
    """Algorithmic floating-point operations of one GEMM: 2MNK."""
    return 2 * M * N * K


def gemm_bytes(M: int, N: int, K: int, out_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one GEMM: A and B read once (bf16), C written
    once."""
    return 2 * M * K + 2 * N * K + out_bytes * M * N


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "dense_gemm_bf16_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, config: str):
    """HBM bytes per launch from committed rocprofv3 PMC counters, only if
    they were taken on the current kernel sources and the same config.  The
    key is the workload name, with "/f16" appended for fp16 operands."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(workload)
    if not rec or rec.get("kernel_src_hash") != kernel_source_hash():
        return None
    if rec.get("config") != config:
        return None
    return int(rec["hbm_bytes_per_launch"])


def cpu_baseline(w, A, B, target_s: float, fmt: str = "bf16"):
    """The oracle (as it stands) on the first R rows of this workload: the
    whole workload if it fits the time target, else as many rows as do."""
    import oracle

    threads = oracle.max_threads()
    rows = min(w.M, 64)
    t0 = time.perf_counter()
    oracle.gemm(A[:rows], B, K=w.K, want_f64=False, fmt=fmt)
    per_row = (time.perf_counter() - t0) / rows
    R = int(max(1, min(w.M, target_s / max(per_row, 1e-9))))
    t0 = time.perf_counter()
    oracle.gemm(A[:R], B, K=w.K, want_f64=False, fmt=fmt)
    dt = time.perf_counter() - t0
    what = "all" if R == w.M else f"first {R} of {w.M}"
    return {
        "value": round(gemm_flops(R, w.N, w.K) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{what} rows of A: {R}x{w.N}x{w.K} GEMM, fp64 sums, "
                  f"{dt:.1f} s on {threads} OpenMP threads ({os.cpu_count()} logical CPUs)",
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # Untimed warm-up: from an idle GPU the shader clock takes tens of ms to
    # ramp up; 500 launches (~65 ms at 4096^3) reach the steady state that
    # sustained runs of 1000+ launches also show.
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="square4096_normal")
    ap.add_argument("--config", default=None, help="force a kernel configuration")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default="bf16",
                    help="operand type (f16: the gemm_f16 entry point)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target length of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--context", action="store_true",
                    help="also time torch.matmul on the same tensors (context only)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (for counter "
                         "calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus "
              f"{args.gpus}); nothing was run.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_gemm_bf16_amd as g
    from synthetic_inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()

    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(5):
                dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": 5}))
        return 0

    w = WORKLOADS[args.workload]
    M, N, K = w.M, w.N, w.K
    half = args.dtype == "f16"
    A, B = w.make(fmt=args.dtype)
    flops = gemm_flops(M, N, K)
    nbytes = gemm_bytes(M, N, K)
    ai = flops / nbytes
    bound = "mfma" if ai >= RIDGE else "hbm"
    # rotate input sets for memory-bound shapes so B cannot stay in cache
    sets = 1 if bound == "mfma" else max(2, -(-4 * CACHE_BYTES // (2 * N * K)))
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dBs = [torch.from_numpy(B.view(np.int16)).cuda()]
    for i in range(1, sets):
        dBs.append(dBs[0].roll(i, dims=0).contiguous())  # same values, new addresses
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    cfg = args.config or g.config_name(M, N, K)
    ws = g.workspace_size(M, N, K) if args.config is None else 1 << 30
    if ws:
        g.reserve_workspace(ws, stream)
    torch.cuda.synchronize()

    entry = g.gemm_f16_ex if half else g.gemm_bf16_ex

    def step(i):
        entry(args.config, M, N, K, dA, K, dBs[i % sets], K, dC, N, False, stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1) / args.steps

    t = ms * 1e-3
    tflops = flops / t / 1e12
    gbps = nbytes / t / 1e9
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_GBPS,
                "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 4)}
    roof["traffic"] = measured_traffic(args.workload + ("/f16" if half else ""), cfg)
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = nbytes

    metric = METRIC if not half else METRIC.replace("bf16 GEMM", "fp16-operand GEMM", 1)
    out = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "kernel_config": cfg, "input_sets": sets,
                   "pct_mfma_peak": round(100 * tflops / PEAK_TFLOPS, 2),
                   "pct_hbm_bw": round(100 * gbps / PEAK_GBPS, 2),
                   "wall_s_timed": round(wall, 4)},
        "roofline": roof,
    }
    if args.context:
        tdt = torch.float16 if half else torch.bfloat16
        a = dA.view(tdt)
        b = dBs[0].view(tdt)
        with torch.cuda.stream(stream):
            for _ in range(5):
                torch.matmul(a, b.t())
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                torch.matmul(a, b.t())
            e1.record(stream)
        torch.cuda.synchronize()
        out["context"] = {"torch_matmul_tflops": round(flops / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e12, 2)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_seconds, args.dtype)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
