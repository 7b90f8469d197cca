"""Offline tuning sweep: time candidate launch plans for given GEMM shapes on
the GPU and write the fastest into the shape -> configuration table that
the library's plan choice consults first (``csrc/gemm_tuned.inc``).

A plan is a configuration name of the library (``gemm_bf16_config_at``)
plus the K split count, raster grouping and K-step rotation
(``<tile>_k<S>_g<G>[_r<R>][_n1][_h<S>|_m<1|2>]``), exactly the names ``gemm_bf16_ex``
accepts.
For each shape the sweep

1. enumerates candidates (every tile built for the operand type, except
   the LDS-layout ablation tiles; split counts that keep at least four
   K-steps per slice and at most ~4 workgroups per CU; GROUP_M 4 and 8;
   rotation off and on; with one row of tiles, non-temporal B loads off and
   on where the tile is built with them; with more than one pass of tiles
   over the CUs and the last one partial, the hybrid plans "_h2" .. "_h4"
   and, on the 256 x 256 tile, the mixed plans "_m1" and "_m2"),
2. times every candidate briefly (HIP events on one stream, after a warm-up
   long enough for the clock to settle; memory-bound shapes cycle through
   copies of B larger than the 256 MB Infinity Cache, as ``bench.py`` does),
3. re-times the best few for longer, alternating between them so that a
   drift of the clock does not favour one, and keeps the fastest by median.

Usage (on a machine with the GPU):

    python -m dense_gemm_bf16_amd.tune --workloads all --out dense_gemm_bf16_amd/csrc/gemm_tuned.inc

then rebuild the library.  Only exact (M, N, K) matches use the table; every
other shape falls back to the static rules in ``gemm_api.hip``.  The
sweep's measurements are written next to the table as JSON
(``--json``), so a table entry can be traced to its numbers.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import statistics
import sys
import time

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)

CACHE_BYTES = 256 << 20  # Infinity Cache
RIDGE = 2500e12 / 8000e9  # FLOP per byte at the published peaks
ABLATION_TILES = ("_x0_", "_x1_")  # LDS layouts kept only to measure conflicts


def parse_tile(name: str):
    """(BM, BN, BK) of a tile configuration name ``t{BM}x{BN}x{BK}_...``."""
    dims = name[1:].split("_")[0].split("x")
    return int(dims[0]), int(dims[1]), int(dims[2])


def candidates(M: int, N: int, K: int, tiles: list[str], cus: int = 256,
               stream_tiles: frozenset = frozenset()) -> list[str]:
    """Plan names worth timing for one shape (no GPU needed).  For the tiles
    in ``stream_tiles`` (built with non-temporal B loads) and a single row of
    tiles, every plan is also tried with "_n1"."""
    out = []
    for tile in tiles:
        if any(a in tile for a in ABLATION_TILES):
            continue
        bm, bn, bk = parse_tile(tile)
        n_tiles = -(-M // bm) * -(-N // bn)
        k_tiles = -(-K // bk)
        # zero-padding work beyond 4x the useful work is never worth it
        if bm > 4 * M and bm > 32:
            continue
        for s in (1, 2, 3, 4, 6, 8):
            if s > 1 and (k_tiles // s < 4 or n_tiles * s > 4 * cus):
                continue
            if s > 1 and n_tiles >= cus:
                continue  # the tiles alone fill the chip
            # GROUP_M orders tile rows; with one row of tiles every value
            # gives the same launch, so time only one
            one_row = -(-M // bm) == 1
            # more than one pass of tiles, the last one partial: also the
            # hybrid plans (whole passes unsplit, the columns left over with
            # K split h ways)
            hybrid = s == 1 and n_tiles > cus and n_tiles % cus != 0
            for g in ((4, 8) if not one_row else (4,)):
                for r in (0, 1):
                    name = f"{tile}_k{s}_g{g}" + (f"_r{r}" if r else "")
                    out.append(name)
                    if one_row and tile in stream_tiles:
                        out.append(name + "_n1")
                    if hybrid:
                        out += [f"{name}_h{h}" for h in (2, 3, 4) if k_tiles // h >= 4]
                        if tile == MIXED_TILE:
                            out += [f"{name}_m1", f"{name}_m2"]
    return out


# the tile whose plans take a mixed tail ("_m1": 256 x 128 tiles, "_m2":
# 128 x 128 tiles for the columns past the whole passes)
MIXED_TILE = "t256x256x64_w2x2_s2_x3_p10"


def stream_tiles(g, tiles: list[str]) -> frozenset:
    """The tiles whose plans accept "_n1" (asked of the library with M = 0,
    so nothing is launched)."""
    import ctypes

    fake = ctypes.c_void_p(0x10000)
    ok = set()
    for t in tiles:
        rc = g._lib.gemm_bf16_ex((t + "_k1_g4_n1").encode(), 0, 64, 64, fake, 64, fake, 64,
                                 fake, 64, 0, None)
        if rc == g.GEMM_OK:
            ok.add(t)
    return frozenset(ok)


def _time_plans(lib_call, plans, n, sets, reps=1):
    """Median microseconds per launch of each plan (HIP events)."""
    import torch

    stream = torch.cuda.current_stream()
    res = {p: [] for p in plans}
    for _ in range(reps):
        for p in plans:
            for i in range(3):
                lib_call(p, i % sets)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                lib_call(p, i % sets)
            e1.record(stream)
            torch.cuda.synchronize()
            res[p].append(e0.elapsed_time(e1) / n * 1e3)
    return {p: statistics.median(v) for p, v in res.items()}


def tune_shape(M: int, N: int, K: int, half: bool = False, keep: int = 6,
               log=print) -> dict:
    """Time the candidates of one shape; returns {"best": name, "us": t,
    "auto": (rule-based name, its us), "timings": {name: us}}."""
    import torch

    import dense_gemm_bf16_amd as g

    tiles = g.f16_config_names() if half else g.config_names()
    plans = candidates(M, N, K, tiles, stream_tiles=stream_tiles(g, tiles))
    auto = g.config_name(M, N, K)
    if auto not in plans:
        plans.append(auto)
    dt = torch.float16 if half else torch.bfloat16
    gen = torch.Generator(device="cpu").manual_seed(M * 131 + N * 7 + K)
    A = torch.randn(M, K, generator=gen).to(dt).cuda()
    B0 = torch.randn(N, K, generator=gen).to(dt).cuda()
    flops = 2 * M * N * K
    nbytes = 2 * (M * K + N * K + M * N)
    memory_bound = flops / nbytes < RIDGE
    sets = max(2, -(-4 * CACHE_BYTES // (2 * N * K))) if memory_bound else 1
    Bs = [B0] + [B0.roll(i, 0).contiguous() for i in range(1, sets)]
    C = torch.empty(M, N, dtype=dt, device="cuda")
    g.reserve_workspace(max(g.workspace_size(M, N, K), 8 * M * ((N + 7) // 8 * 8) * 4),
                        torch.cuda.current_stream())
    entry = g.gemm_f16_ex if half else g.gemm_bf16_ex

    def call(plan, i):
        entry(plan, M, N, K, A, K, Bs[i], K, C, N)

    t_one = max(flops / 1.2e15, 2e-6)
    # warm the clock up: ~0.3 s of launches
    for i in range(int(min(2000, max(50, 0.3 / t_one)))):
        call(auto, i % sets)
    torch.cuda.synchronize()
    n_short = int(min(50, max(5, 2e-3 / t_one)))
    first = _time_plans(call, plans, n_short, sets)
    best = sorted(first, key=first.get)[:keep]
    if auto not in best:
        best.append(auto)
    n_long = int(min(200, max(10, 5e-3 / t_one)))
    second = _time_plans(call, best, n_long, sets, reps=5)
    win = min(second, key=second.get)
    log(f"{M}x{N}x{K}{' f16' if half else ''}: {len(plans)} candidates; best {win} "
        f"{second[win]:.2f} us; rules {auto} {second[auto]:.2f} us")
    return {"best": win, "us": round(second[win], 3), "auto": [auto, round(second[auto], 3)],
            "timings": {p: round(t, 3) for p, t in sorted(second.items(), key=lambda x: x[1])},
            "first_pass": {p: round(t, 3) for p, t in sorted(first.items(), key=lambda x: x[1])[:20]}}


def read_table(path: str) -> dict[tuple[int, int, int], str]:
    """The entries of a table written by write_table (empty if none)."""
    out = {}
    try:
        text = open(path).read()
    except OSError:
        return out
    for line in text.splitlines():
        m = re.match(r'^\{(\d+), (\d+), (\d+), "([^"]+)"\},$', line.strip())
        if m:
            out[(int(m.group(1)), int(m.group(2)), int(m.group(3)))] = m.group(4)
    return out


def choose_entries(results: dict, old: dict, min_gain: float) -> list[tuple[int, int, int, str]]:
    """Table rows from a sweep's results.  The sweep times the plan the
    library currently picks ("auto"), which for a shape already in the table
    is that table entry, not the static rules.  So: a shape gets the sweep's
    best plan if it beats the current choice by more than min_gain; else a
    shape already in the table keeps its entry (still within min_gain of the
    best); else the automatic choice (cost model or rules) stays in charge.
    Rows of shapes this sweep did not time are kept as they are, after the
    swept ones."""
    entries = []
    swept = set()
    for key, r in results.items():
        M, N, K = (int(v) for v in key.split("x"))
        swept.add((M, N, K))
        auto, auto_us = r["auto"]
        if r["best"] != auto and r["us"] < auto_us * (1 - min_gain):
            entries.append((M, N, K, r["best"]))
        elif (M, N, K) in old:
            entries.append((M, N, K, old[(M, N, K)]))
    entries += [(M, N, K, plan) for (M, N, K), plan in old.items() if (M, N, K) not in swept]
    return entries


def write_table(entries: list[tuple[int, int, int, str]], path: str, note: str) -> None:
    """Write the C include the plan choice reads: one {M, N, K, "plan"} row
    per shape."""
    lines = [
        "// Shape -> launch plan table written by dense_gemm_bf16_amd/tune.py.",
        f"// {note}.",
        "// Exact (M, N, K) matches only; other shapes use the automatic choice",
        "// in gemm_api.hip (cost model, rules).  Regenerate with the tuning sweep,",
        "// do not edit by hand.",
    ]
    for M, N, K, plan in entries:
        lines.append(f'{{{M}, {N}, {K}, "{plan}"}},')
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workloads", default="all",
                    help="comma-separated names from synthetic_inputs.WORKLOADS, 'all' or 'none'")
    ap.add_argument("--shapes", default="", help="extra shapes MxNxK,MxNxK")
    ap.add_argument("--out", default=os.path.join(_HERE, "csrc", "gemm_tuned.inc"))
    ap.add_argument("--json", default=os.path.join(_HERE, "csrc", "gemm_tuned.json"))
    ap.add_argument("--min-gain", type=float, default=0.02,
                    help="keep a table entry only if it beats the rules by this fraction")
    ap.add_argument("--from-json", default="",
                    help="rebuild the table from a saved sweep (no GPU) instead of sweeping")
    args = ap.parse_args(argv)
    old = read_table(args.out)

    if args.from_json:
        with open(args.from_json) as f:
            saved = json.load(f)
        entries = choose_entries(saved["results"], old, args.min_gain)
        n_swept = sum(f"{M}x{N}x{K}" in saved["results"] for M, N, K, _ in entries)
        note = (f"{len(entries)} rows, {n_swept} of them from the {len(saved['results'])} shapes of "
                f"{os.path.basename(args.from_json)} (min gain {args.min_gain * 100:g}%)")
        write_table(entries, args.out, note)
        print(note)
        return 0

    import torch

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from synthetic_inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("tune: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    names = list(WORKLOADS) if args.workloads == "all" else [
        w for w in args.workloads.split(",") if w and w != "none"]
    shapes = []
    for n in names:
        w = WORKLOADS[n]
        if (w.M, w.N, w.K) not in shapes:
            shapes.append((w.M, w.N, w.K))
    for s in args.shapes.split(","):
        if s:
            M, N, K = (int(v) for v in s.split("x"))
            shapes.append((M, N, K))
    results = {}
    t0 = time.time()
    for (M, N, K) in shapes:
        results[f"{M}x{N}x{K}"] = tune_shape(M, N, K)
    entries = choose_entries(results, old, args.min_gain)
    n_swept = sum(f"{M}x{N}x{K}" in results for M, N, K, _ in entries)
    note = (f"{len(entries)} rows, {n_swept} of them from the {len(shapes)} swept shapes (min gain "
            f"{args.min_gain * 100:g}%); sweep took {time.time() - t0:.0f} s")
    write_table(entries, args.out, note)
    with open(args.json, "w") as f:
        json.dump({"note": note, "results": results}, f, indent=1)
    print(note)
    return 0


if __name__ == "__main__":
    sys.exit(main())
