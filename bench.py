#!/usr/bin/env python3
"""Benchmark of the MI355X dense bf16 GEMM, C = A . B^T (bf16 in/out, fp32 sums).

One step is one GEMM call on one batch of synthetic input that is already
resident in HBM.  The headline workload is the 4096^3 square GEMM with
N(0,1) inputs (``--workload`` selects another shape of
``synthetic_inputs.WORKLOADS``; ``--dtype f16`` measures the fp16-operand
entry point).  The line also carries a ``workloads`` object: the M = 8192
prefill and M = 256 decode linear layers timed the same way (same steps and
warm-up), each with its roofline fraction.  ``--shapes MxNxK,...`` times
further shapes the same way (N(0,1) activations, weights scaled by
1/sqrt(K), as the workloads) under ``shapes``; with ``--context`` every
timed shape also carries the vendor library's time on the same tensors.

Timing, per workload:
  * clock ramp: the GEMM runs untimed for ``--ramp-s`` seconds first, because
    from an idle GPU the shader clock needs tens of milliseconds to reach
    the level sustained GEMM work settles at (timed at 10 launches after
    idle, 4096^3 ran 10-30 % slower than at steady state);
  * ``--warmup`` untimed launches, then exactly ``--steps`` launches between
    two HIP events recorded on the launch stream (``value``, ``us``); the GPU
    is kept busy from the end of the ramp to the timed region (no
    synchronisation or host-side metrics read with it idle in between);
  * ``--repeats`` further timings of ``--steps`` launches each, reported as
    min / median / max, so run-to-run noise is visible;
  * clocks: shader (per XCD) and memory clock sampled through amdsmi while
    the same GEMM keeps running untimed right after the timed region.
Memory-bound shapes (arithmetic intensity below the ridge point) rotate
through enough copies of B to exceed the 256 MB Infinity Cache, so B is read
from HBM ("cold"); compute-bound shapes reuse one set.

Printed: ONE JSON line with the contract fields, a ``roofline`` object for
the headline kernel (algorithmic work / HIP-event time against MI355X's
published peak), ``workloads``, ``clocks`` and a ``cpu_baseline`` object
(the oracle, timed on this host's cores on a bounded sample of the headline
workload, plus its one-core rate extrapolated from a few rows).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
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

# The prefill and decode linear layers reported next to the headline.
REPORTED = ("prefill_attn_out", "prefill_mlp_up", "decode_attn_out", "decode_qkv",
            "decode_mlp_up", "decode_mlp_down")

TRAFFIC_COUNTS = ("L2-to-fabric bytes per launch: rocprofv3 FETCH_SIZE x 2.000 + WRITE_SIZE "
                  "x 1.000 (factors from a 1 GiB copy); Infinity Cache hits are included, so "
                  "this bounds HBM traffic from above")


def gemm_flops(M: int, N: int, K: int) -> int:
    """Algorithmic floating-point operations of one GEMM: 2MNK."""
    return 2 * M * N * K


def gemm_bytes(M: int, N: int, K: int, out_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one GEMM: A and B read once (bf16), C written
    once."""
    return 2 * M * K + 2 * N * K + out_bytes * M * N


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_bf16_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "**", "*"), recursive=True)):
        if not os.path.isfile(p):
            continue
        with open(p, "rb") as f:
            h.update(os.path.relpath(p, csrc).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, config: str):
    """L2-to-fabric bytes per launch from committed rocprofv3 counters, only
    if they were taken on the current kernel sources and the same plan.  The
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
    return int(rec["l2_fabric_bytes_per_launch"])


def cpu_model() -> dict:
    info = {"model": None, "sockets": None, "logical_cpus": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            phys = set()
            for line in f:
                if line.startswith("model name") and info["model"] is None:
                    info["model"] = line.split(":", 1)[1].strip()
                elif line.startswith("physical id"):
                    phys.add(line.split(":", 1)[1].strip())
            info["sockets"] = len(phys) or None
    except OSError:
        pass
    return info


def cpu_baseline(w, A, B, target_s: float, fmt: str = "bf16"):
    """The oracle (as it stands) on the first R rows of this workload on
    every host thread: the whole workload if it fits the time target, else
    as many rows as do.  Then one thread on the first min(M, 8) rows,
    extrapolated linearly to the whole workload."""
    import oracle

    threads = oracle.max_threads()
    rows = min(w.M, 64)
    t0 = time.perf_counter()
    oracle.gemm(A[:rows], B, K=w.K, want_f64=False, threads=threads, fmt=fmt)
    per_row = (time.perf_counter() - t0) / rows
    R = int(max(1, min(w.M, target_s / max(per_row, 1e-9))))
    t0 = time.perf_counter()
    oracle.gemm(A[:R], B, K=w.K, want_f64=False, threads=threads, fmt=fmt)
    dt = time.perf_counter() - t0
    r1 = min(w.M, 8)
    t0 = time.perf_counter()
    oracle.gemm(A[:r1], B, K=w.K, want_f64=False, threads=1, fmt=fmt)
    dt1 = time.perf_counter() - t0
    what = "all" if R == w.M else f"first {R} of {w.M}"
    cpu = cpu_model()
    return {
        "value": round(gemm_flops(R, w.N, w.K) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{what} rows of A: {R}x{w.N}x{w.K} GEMM, fp64 sums, "
                  f"{dt:.1f} s on {threads} OpenMP threads",
        "cpu_model": cpu["model"],
        "sockets": cpu["sockets"],
        "logical_cpus": cpu["logical_cpus"],
        "one_core": {
            "value": round(gemm_flops(r1, w.N, w.K) / dt1 / 1e12, 6),
            "unit": "TFLOP/s",
            "extrapolated": True,
            "sample": f"first {r1} rows of A on 1 thread ({dt1:.2f} s), "
                      f"whole workload extrapolated: {dt1 * w.M / r1:.0f} s",
        },
    }


class ClockReader:
    """Shader and memory clocks of the GPU through amdsmi (None when amdsmi
    or its metrics are not available).  The GPU metrics refresh about once a
    second (their system_clock_counter steps by ~1 s), so a value is used
    only if it was refreshed after the timed region began."""

    def __init__(self, torch):
        self.h = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            self.smi = amdsmi
            handles = amdsmi.amdsmi_get_processor_handles()
            want = None
            try:
                p = torch.cuda.get_device_properties(0)
                want = (int(p.pci_domain_id), int(p.pci_bus_id), int(p.pci_device_id))
            except Exception:
                pass
            for h in handles:
                if want is None:
                    break
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.h = h
            if self.h is None and len(handles) == 1:
                self.h = handles[0]
        except Exception:
            self.h = None

    def sample(self):
        if self.h is None:
            return None
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
        except Exception:
            return None

        def num(v):
            return v if isinstance(v, (int, float)) and 0 < v < 100000 else None

        xcd = [num(v) for v in (m.get("current_gfxclks") or [])]
        xcd = [v for v in xcd if v is not None]
        t = m.get("system_clock_counter")
        return {"t": t if isinstance(t, int) else None,
                "gfx": xcd or ([num(m.get("current_gfxclk"))] if num(m.get("current_gfxclk"))
                               else []),
                "mem": num(m.get("current_uclk"))}

    def stamp(self):
        s = self.sample()
        return None if s is None else s["t"]


def summarize_clocks(samples):
    gfx = [v for s in samples if s for v in s["gfx"]]
    mem = [s["mem"] for s in samples if s and s["mem"]]
    if not gfx:
        return None
    return {"sclk_mhz_median": round(statistics.median(gfx)), "sclk_mhz_min": min(gfx),
            "sclk_mhz_max": max(gfx),
            "mclk_mhz_median": round(statistics.median(mem)) if mem else None,
            "samples": len(samples), "per_xcd": True}


def time_workload(g, torch, np, w, args, stream, clocks, config=None):
    """Time one workload as the module docstring describes.  Returns a dict of
    results (plus the host arrays, for the CPU baseline).  With --context the
    vendor library (torch.matmul) is timed the same way on the same tensors,
    after the library, under the key "vendor"."""
    M, N, K = w.M, w.N, w.K
    half = args.dtype == "f16"
    A, B = w.make(fmt=args.dtype)
    flops = gemm_flops(M, N, K)
    nbytes = gemm_bytes(M, N, K)
    bound = "mfma" if flops / nbytes >= RIDGE else "hbm"
    sets = 1 if bound == "mfma" or args.hot else max(2, -(-4 * CACHE_BYTES // (2 * N * K)))
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dBs = [torch.from_numpy(B.view(np.int16)).cuda()]
    for i in range(1, sets):
        dBs.append(dBs[0].roll(i, dims=0).contiguous())  # same values, new addresses
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    plan = config or g.config_name(M, N, K)
    ws = g.workspace_size(M, N, K) if config is None else 1 << 30
    if ws:
        g.reserve_workspace(ws, stream)
    torch.cuda.synchronize()
    entry = g.gemm_f16_ex if half else g.gemm_bf16_ex

    def step(i):
        entry(config, M, N, K, dA, K, dBs[i % sets], K, dC, N, False, stream)

    res = {"M": M, "N": N, "K": K, "plan": plan, "bound": bound}
    res.update(_measure(torch, step, flops, nbytes, bound, args, stream, clocks))
    res["b_sets"] = sets
    res["b_read"] = "cold" if sets > 1 else "hot"
    if args.context:
        tdt = torch.float16 if half else torch.bfloat16
        a, c = dA.view(tdt), dC.view(tdt)
        bts = [d.view(tdt).t() for d in dBs]

        def vendor_step(i):
            torch.matmul(a, bts[i % sets], out=c)

        v = _measure(torch, vendor_step, flops, nbytes, bound, args, stream, clocks)
        v["library"] = "torch.matmul"
        v["us_ratio_library_over_vendor"] = round(res["us"] / v["us"], 4)
        res["vendor"] = v
    return res, (A, B, dA, dBs, dC, stream)


def _measure(torch, step, flops, nbytes, bound, args, stream, clocks):
    """Clock ramp, warm-up, the timed launches, the repeats and the clocks
    of the module docstring, for one launch function."""

    def timed(n):
        # No synchronisation before the first event: the launches queued
        # before it (warm-up, or the previous timing) keep the GPU busy up to
        # the timed region, so its clock does not dip in an idle gap.
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(n):
                step(i)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3, time.perf_counter() - w0  # us per launch

    # clock ramp, then the warm-up launches.  The clock stamp (a read of the
    # GPU metrics, ~ms on the host) is taken while queued launches run: taken
    # with the GPU idle, the first timed launches ran ~2 % slower than the
    # repeats after them.
    ramp_launches = 0
    t0 = time.perf_counter()
    t_end = t0 + args.ramp_s
    with torch.cuda.stream(stream):
        while time.perf_counter() < t_end:
            for i in range(20):
                step(ramp_launches + i)
            ramp_launches += 20
            torch.cuda.synchronize()
        # a last batch of ramp launches, ~10 ms of GPU work, queued before the
        # stamp so that the GPU is still busy while it is read
        per_launch = (time.perf_counter() - t0) / max(ramp_launches, 1)
        bridge = int(min(2000, max(20, 0.01 / max(per_launch, 1e-6))))
        for i in range(bridge):
            step(ramp_launches + i)
        ramp_launches += bridge
        t_begin = clocks.stamp() if clocks is not None else None
        for i in range(args.warmup):
            step(i)
    us, wall = timed(args.steps)
    reps = [timed(args.steps)[0] for _ in range(args.repeats)]

    # clocks: the same launches keep running, untimed, until the GPU metrics
    # have been refreshed after the timed region began (at most --clock-s)
    samples = []
    if clocks is not None and t_begin is not None:
        batch = int(min(2000, max(1, 0.02 * 1e6 / max(us, 1.0))))  # ~20 ms of launches
        t_stop = time.perf_counter() + args.clock_s
        with torch.cuda.stream(stream):
            while time.perf_counter() < t_stop:
                s = clocks.sample()
                if s is not None and s["t"] is not None and s["t"] > t_begin:
                    samples.append(s)
                    break
                for i in range(batch):
                    step(i)
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    t = us * 1e-6
    tflops = flops / t / 1e12
    gbps = nbytes / t / 1e9
    return {
        "us": round(us, 2), "tflops": round(tflops, 1), "tbps": round(gbps / 1e3, 3),
        "pct_mfma_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "pct_hbm_bw": round(100 * gbps / PEAK_GBPS, 2),
        "frac": round((tflops / PEAK_TFLOPS) if bound == "mfma" else (gbps / PEAK_GBPS), 4),
        "repeats_us": {"n": len(reps), "min": round(min(reps), 2),
                       "median": round(statistics.median(reps), 2),
                       "max": round(max(reps), 2)} if reps else None,
        "clock_ramp": {"s": args.ramp_s, "launches": ramp_launches},
        "clocks": summarize_clocks(samples),
        "wall_s_timed": round(wall, 4),
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ramp-s", type=float, default=0.3,
                    help="seconds of untimed launches before the warm-up (clock ramp)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="extra timings of --steps launches (min / median / max)")
    ap.add_argument("--clock-s", type=float, default=1.5,
                    help="at most this many seconds of untimed launches while waiting for "
                         "a refresh of the GPU clock metrics")
    ap.add_argument("--workload", default="square4096_normal")
    ap.add_argument("--workloads", default="default",
                    help="the shapes of the 'workloads' object: 'default' (the prefill and "
                         "decode layers), 'none', or a comma list of workload names")
    ap.add_argument("--shapes", default="",
                    help="extra shapes MxNxK,MxNxK timed like the workloads, under 'shapes'")
    ap.add_argument("--config", default=None, help="force a kernel configuration")
    ap.add_argument("--hot", action="store_true",
                    help="reuse one B for memory-bound shapes too (B may stay in cache)")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default="bf16",
                    help="operand type (f16: the gemm_f16 entry point)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target length of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--context", action="store_true",
                    help="also time the vendor library (torch.matmul) on the same tensors, "
                         "the same way, for every timed shape (context only; never the value)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (for counter "
                         "calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus "
              f"{args.gpus}); nothing was run.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_gemm_bf16_amd as g
    from synthetic_inputs import WORKLOADS, Workload

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

    clocks = ClockReader(torch)
    w = WORKLOADS[args.workload]
    head, (A, B, dA, dBs, dC, _) = time_workload(g, torch, np, w, args, stream, clocks,
                                                   args.config)
    M, N, K = w.M, w.N, w.K
    half = args.dtype == "f16"
    flops, nbytes = gemm_flops(M, N, K), gemm_bytes(M, N, K)
    us = head["us"]
    tflops = flops / (us * 1e-6) / 1e12
    gbps = nbytes / (us * 1e-6) / 1e9
    if head["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_GBPS,
                "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 4)}
    roof["traffic"] = measured_traffic(args.workload + ("/f16" if half else ""), head["plan"])
    roof["traffic_counts"] = TRAFFIC_COUNTS
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
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "kernel_config": head["plan"], "input_sets": head["b_sets"],
                   "pct_mfma_peak": head["pct_mfma_peak"], "pct_hbm_bw": head["pct_hbm_bw"],
                   "wall_s_timed": head["wall_s_timed"]},
        "roofline": roof,
        "repeats_us": head["repeats_us"],
        "clock_ramp": head["clock_ramp"],
        "clocks": head["clocks"],
    }
    del dA, dBs, dC

    names = {"default": list(REPORTED), "none": []}.get(args.workloads)
    if names is None:
        names = [n for n in args.workloads.split(",") if n]
    if names:
        wl = {}
        for name in names:
            if name == args.workload:
                continue
            res, keep = time_workload(g, torch, np, WORKLOADS[name], args, stream, clocks)
            del keep
            torch.cuda.empty_cache()
            wl[name] = res
        out["workloads"] = wl

    if args.shapes:
        sh = {}
        for spec in (x for x in args.shapes.split(",") if x):
            Ms, Ns, Ks = (int(v) for v in spec.split("x"))
            ws = Workload(spec, Ms, Ns, Ks, "normal", True, 0x5A01, 0x5B01)
            res, keep = time_workload(g, torch, np, ws, args, stream, clocks)
            del keep
            torch.cuda.empty_cache()
            sh[spec] = res
        out["shapes"] = sh

    if args.context:
        out["context"] = {"vendor": head["vendor"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_seconds, args.dtype)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
