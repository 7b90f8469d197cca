"""The launch-time model behind the automatic plan choice for M > 256.

``choose_plan`` (``csrc/gemm_api.hip``, ``model_plan``) picks, for M > 256,
the plan with the lowest estimated time among the three direct-to-LDS tiles
(256 x 256, 256 x 128, 128 x 128), K split 1, 2, 3, 4, 6 or 8 ways, the
hybrid plans and the mixed plans.  This module holds the same model in Python, the sweep that
measures plans on the GPU, and the fit of the model's ten constants to
those measurements, so the constants compiled into the library can be
re-derived and checked.

Model of one launch (times in microseconds).  ``tiles * S`` workgroups run
one per CU at a time; every full pass over the 256 CUs costs one unit's
time, ``steps * step_us[tile] + tile_us[tile]`` (``steps`` = K-steps per
slice, ``tile_us`` the first loads and the epilogue); a last pass with a
fraction f of the CUs busy costs ``partial + (1 - partial) * f`` of a full
one; every launch adds ``launch_us``; a split adds ``split_us`` plus
``split_us_per_mb`` per MB of fp32 partial slices (S * M * roundup8(N) * 4
bytes).  A hybrid plan is two launches: the whole passes' tile columns
unsplit, and the remaining columns with K split; with two or more whole
passes it must beat the other plans by HYBRID_MARGIN.  A mixed plan
(``_m1`` / ``_m2``, 256 x 256 tiles only) is the same two launches with the
remaining columns unsplit on 256 x 128 / 128 x 128 tiles, under the same
margin.

Usage::

    python -m dense_gemm_bf16_amd.plan_model sweep --out timings.json   # GPU
    python -m dense_gemm_bf16_amd.plan_model fit                        # CPU

``fit`` reads ``plan_model_data/fit_shapes.json`` (77 shapes, 1,000 plan
timings on MI355X) and reports the choice quality on
``plan_model_data/holdout_shapes.json`` (42 other shapes) and
``plan_model_data/multipass_shapes.json`` (30 shapes of up to 8.75 passes
of 256 x 256 tiles over the CUs) and ``plan_model_data/irregular_shapes.json``
(20 shapes with M, N and K off the tile sizes, rows off 128-byte lines),
both swept with this module.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
DATA = os.path.join(_HERE, "plan_model_data")
CUS = 256
SCRATCH_BYTES = 64 << 20  # GEMM_NOALLOC_SCRATCH_BYTES: the model never needs more

# name -> (BM, BN, index into the per-tile constants)
TILES = {
    "t256x256x64_w2x2_s2_x3_p10": (256, 256, 0),
    "t256x128x64_w2x2_s3_x3_p10": (256, 128, 1),
    "t128x128x64_w2x2_s4_x3_p10": (128, 128, 2),
}
BK = 64
PLAN = re.compile(r"^(t\d+x\d+x64_w2x2_s\d_x3_p10)_k(\d+)_g\d+(_r\d+)?(_h(\d+))?(_n1)?(_m[12])?$")
BIG, MID, M128 = ("t256x256x64_w2x2_s2_x3_p10", "t256x128x64_w2x2_s3_x3_p10",
                  "t128x128x64_w2x2_s4_x3_p10")
# constant order: step_us[3], tile_us[3], partial, split_us, split_us_per_mb, launch_us
NAMES = ["step_us_256x256", "step_us_256x128", "step_us_128x128", "tile_us_256x256",
         "tile_us_256x128", "tile_us_128x128", "partial", "split_us", "split_us_per_mb",
         "launch_us"]
START = [1.45, 0.80, 0.50, 3, 3, 3, 0.7, 2, 0.18, 2]


def even_splits(s: int, k_tiles: int) -> int:
    """K splits as the library equalises them (ceil(k_tiles / S) steps a slice)."""
    s = min(s, k_tiles)
    if s <= 1:
        return 1
    per = -(-k_tiles // s)
    return -(-k_tiles // per)


def launches(plan: str, M: int, N: int, K: int):
    """The launches a plan name runs: (tile index, tiles, S, K-steps, M, N) each,
    or None for a plan outside the model (another tile)."""
    m = PLAN.match(plan)
    if not m or m.group(1) not in TILES:
        return None
    bm, bn, ti = TILES[m.group(1)]
    kt = -(-K // BK)
    tm, tn = -(-M // bm), -(-N // bn)
    S = even_splits(int(m.group(2)), kt)
    h = int(m.group(5) or 0)
    if m.group(7) and S == 1 and not h and m.group(1) == BIG:
        # mixed: the whole passes' columns on 256 x 256 tiles, the rest
        # unsplit on 256 x 128 (_m1) or 128 x 128 (_m2) tiles
        head_cols = (tm * tn // CUS) * CUS // tm
        if 0 < head_cols < tn:
            n1 = head_cols * bn
            mbm, mbn, mti = TILES[MID if m.group(7) == "_m1" else M128]
            return [(ti, tm * head_cols, 1, kt, M, n1),
                    (mti, -(-M // mbm) * -(-(N - n1) // mbn), 1, kt, M, N - n1)]
    if h and S == 1:
        head_cols = (tm * tn // CUS) * CUS // tm
        hs = even_splits(h, kt)
        if 0 < head_cols < tn and hs > 1:
            n1 = head_cols * bn
            return [(ti, tm * head_cols, 1, kt, M, n1),
                    (ti, tm * (tn - head_cols), hs, -(-kt // hs), M, N - n1)]
    return [(ti, tm * tn, S, -(-kt // S), M, N)]


def cost(p, launch_list) -> float:
    """Estimated microseconds of a plan's launches under constants p."""
    t = 0.0
    for ti, tiles, S, steps, M, N in launch_list:
        units = tiles * S
        full, rem = divmod(units, CUS)
        passes = full + ((p[6] + (1 - p[6]) * rem / CUS) if rem else 0.0)
        t += (steps * p[ti] + p[3 + ti]) * passes + p[9]
        if S > 1:
            t += p[7] + p[8] * S * M * (-(-N // 8) * 8) * 4 / 1e6
    return t


# A hybrid whose unsplit part makes two or more whole passes is chosen only
# if its estimate is this much below the others': with whole passes before
# it, a partial last pass runs faster than the model's partial-pass term
# says (the plain plan's cost is overestimated), which on the multi-pass
# sweep made the model prefer hybrids that were up to 4.7 % slower.
HYBRID_MARGIN = 0.03


def choice_cost(p, launch_list) -> float:
    """The cost the choice compares: the estimate, with HYBRID_MARGIN added
    to a hybrid whose unsplit part makes two or more whole passes."""
    t = cost(p, launch_list)
    if len(launch_list) == 2 and launch_list[0][1] // CUS >= 2:
        t *= 1 + HYBRID_MARGIN
    return t


def candidates(M: int, N: int, K: int) -> list[str]:
    """The plans the library's model chooses among, as names."""
    out = []
    kt = -(-K // BK)
    for name, (bm, bn, _) in TILES.items():
        tm, tn = -(-M // bm), -(-N // bn)
        tiles = tm * tn
        for S in (1, 2, 3, 4, 6, 8):
            if S > 1 and (kt // S < 8 or tiles * S > 4 * CUS):
                continue
            s = even_splits(S, kt)
            if S > 1 and s <= 1:
                continue
            if s > 1 and s * M * (-(-N // 8) * 8) * 4 > SCRATCH_BYTES:
                continue
            out.append(f"{name}_k{s}_g4")
        if tiles > CUS and tiles % CUS:
            head_cols = (tiles // CUS) * CUS // tm
            if not 0 < head_cols < tn:
                continue
            n1 = head_cols * bn
            for h in (2, 3, 4, 6, 8):
                hs = even_splits(h, kt)
                if hs <= 1 or hs * M * (-(-(N - n1) // 8) * 8) * 4 > SCRATCH_BYTES:
                    continue
                out.append(f"{name}_k1_g4_h{hs}")
            if name == BIG:
                out += [f"{name}_k1_g4_m1", f"{name}_k1_g4_m2"]
    return list(dict.fromkeys(out))


def choose(p, M: int, N: int, K: int) -> str:
    """The cheapest candidate under constants p (first one on ties, in the
    order the library considers them)."""
    best, best_t = None, None
    for c in candidates(M, N, K):
        t = choice_cost(p, launches(c, M, N, K))
        if best is None or t < best_t:
            best, best_t = c, t
    return best


def rows_of(data: dict):
    """(shape, plan, measured us, launches) for every timing the model covers."""
    rows = []
    for shape, rec in data.items():
        M, N, K = (int(x) for x in shape.split("x"))
        for plan, us in rec["times"].items():
            L = launches(plan, M, N, K)
            if L:
                rows.append((shape, plan, us, L))
    return rows


def fit(data: dict):
    """Least squares on log time (Nelder-Mead from START); returns the
    constants and the RMS log error."""
    import numpy as np
    from scipy.optimize import minimize

    rows = rows_of(data)

    def loss(p):
        if np.any(p < 0):
            return 1e9
        return sum((math.log(cost(p, L)) - math.log(us)) ** 2 for _, _, us, L in rows)

    r = minimize(loss, np.array(START, dtype=float), method="Nelder-Mead",
                 options={"maxiter": 20000, "maxfev": 20000, "xatol": 1e-4, "fatol": 1e-6})
    return list(r.x), math.sqrt(r.fun / len(rows))


def choice_quality(p, data: dict):
    """Per shape: measured time of the plan the model picks among the timed
    plans, over the fastest timed plan; and the same for the plan recorded
    as the library's choice when the sweep ran ("auto")."""
    by = {}
    for shape, plan, us, L in rows_of(data):
        by.setdefault(shape, []).append((plan, us, choice_cost(p, L)))
    out = {}
    for shape, lst in by.items():
        best = min(u for _, u, _ in lst)
        pick = min(lst, key=lambda x: x[2])
        rec = data[shape]
        out[shape] = (pick[1] / best, rec["times"][rec["auto"]] / best)
    return out


def geomean(xs):
    xs = list(xs)
    return math.exp(sum(math.log(x) for x in xs) / len(xs))


def sweep(Ms, NKs, out_path: str) -> None:
    """Time every model candidate (and the library's current choice) of each
    shape on the GPU, one plan after another with HIP events, best of two."""
    import ctypes
    import time

    import torch

    if _HERE not in sys.path:
        sys.path.insert(0, os.path.dirname(_HERE))
    import dense_gemm_bf16_amd as g

    torch.cuda.set_device(0)
    s = torch.cuda.current_stream()
    g.reserve_workspace(1 << 30, s)
    def ld(x):  # row strides are multiples of 8 elements
        return -(-x // 8) * 8

    maxM, maxN, maxK = max(Ms), ld(max(n for n, _ in NKs)), ld(max(k for _, k in NKs))
    A = torch.randn(maxM * maxK, device="cuda").to(torch.bfloat16)
    B = torch.randn(maxN * maxK, device="cuda").to(torch.bfloat16)
    C = torch.empty(maxM * maxN, device="cuda", dtype=torch.bfloat16)
    out = {}
    for N, K in NKs:
        for M in Ms:
            def run(plan):
                rc = g._lib.gemm_bf16_ex(plan.encode(), M, N, K, A.data_ptr(), ld(K),
                                         B.data_ptr(), ld(K), C.data_ptr(), ld(N), 0,
                                         ctypes.c_void_p(s.cuda_stream))
                if rc:
                    raise RuntimeError(f"{plan}: status {rc}")
            auto = g.config_name(M, N, K)
            plans = list(dict.fromkeys([auto] + candidates(M, N, K)))
            n = int(min(50, max(3, 0.02 / (2 * M * N * K / 1.2e15))))
            t_end = time.perf_counter() + 0.3
            while time.perf_counter() < t_end:
                run(auto)
                torch.cuda.synchronize()
            times = {}
            for _ in range(2):
                for p in plans:
                    run(p)
                    run(p)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(n):
                        run(p)
                    e1.record()
                    torch.cuda.synchronize()
                    times[p] = min(times.get(p, 1e30), e0.elapsed_time(e1) / n * 1e3)
            out[f"{M}x{N}x{K}"] = {"auto": auto, "times": times}
            print(f"{M}x{N}x{K}: {len(plans)} plans, auto {times[auto]:.1f} us, "
                  f"best {min(times.values()):.1f} us", flush=True)
            with open(out_path, "w") as f:
                json.dump(out, f)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    sw = sub.add_parser("sweep", help="time the model's candidate plans on the GPU")
    sw.add_argument("--ms", default="320,384,512,640,768,1024,1536,2048,3072,4096,6144")
    sw.add_argument("--nks", default="4096x4096,14336x4096,4096x14336,8192x8192,"
                                     "10240x8192,5376x5376,28672x8192")
    sw.add_argument("--out", required=True)
    ft = sub.add_parser("fit", help="fit the constants and report the choice quality")
    ft.add_argument("--data", default=os.path.join(DATA, "fit_shapes.json"))
    ft.add_argument("--holdout", default=",".join(
        os.path.join(DATA, f) for f in ("holdout_shapes.json", "multipass_shapes.json",
                                        "irregular_shapes.json")),
        help="comma list of sweeps to report the choice quality on")
    args = ap.parse_args(argv)
    if args.cmd == "sweep":
        Ms = [int(x) for x in args.ms.split(",")]
        NKs = [tuple(int(v) for v in x.split("x")) for x in args.nks.split(",")]
        sweep(Ms, NKs, args.out)
        return 0
    with open(args.data) as f:
        data = json.load(f)
    p, rms = fit(data)
    print(f"{len(rows_of(data))} timings of {len(data)} shapes; RMS log error {rms:.4f}")
    for name, v in zip(NAMES, p):
        print(f"  {name:18s} {v:.4f}")
    for label, path in [("fit shapes", args.data)] + [
            (f"held out ({os.path.basename(h)})", h) for h in args.holdout.split(",") if h]:
        with open(path) as f:
            q = choice_quality(p, json.load(f))
        print(f"{label}: model's pick / fastest timed {geomean(v[0] for v in q.values()):.4f} "
              f"(worst {max(v[0] for v in q.values()):.3f}); the library's choice when swept "
              f"{geomean(v[1] for v in q.values()):.4f} (worst {max(v[1] for v in q.values()):.3f})")
    return 0


if __name__ == "__main__":
    sys.exit(main())
