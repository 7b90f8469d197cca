"""Build the HIP library ``libgemm_bf16.so`` in-tree for gfx950.

Each ``csrc/*.hip`` file is compiled to an object in parallel with hipcc,
then linked into a shared library next to this file.  Build products live in
``_build/`` (ignored by git) and the package directory.

The default build holds the product configurations (those the plan choice
-- tuned table, cost model, rules -- can pick).  ``build(ablation=True)``, or the environment
variable ``GEMM_BUILD_ABLATION=1``, also compiles ``csrc/ablation/``: the
kernel families and LDS layouts the product choices were measured against,
selectable by name through ``gemm_bf16_ex`` for ablations and sweeps.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgemm_bf16.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # hipcc may form packed fp32 ops from plain float code; keep them off.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _compile(src: str, defines: tuple = ()) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *defines, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


# Files that take longest to compile start first (the direct-to-LDS tiles
# split over four files each), so the build takes about as long as the
# slowest file.
_SLOW_FIRST = ("gemm_inst_mid", "gemm_inst_big", "gemm_inst_mid128")


def _order(src: str):
    base = os.path.basename(src)
    for i, p in enumerate(_SLOW_FIRST):
        if base.startswith(p):
            return (i, base)
    return (len(_SLOW_FIRST), base)


def sources(ablation: bool = False) -> list[str]:
    srcs = glob.glob(os.path.join(CSRC, "*.hip"))
    if ablation:
        srcs += glob.glob(os.path.join(CSRC, "ablation", "*.hip"))
    return sorted(srcs, key=_order)


def build(jobs: int | None = None, ablation: bool | None = None) -> str:
    """Compile the HIP sources and link ``libgemm_bf16.so``.  Returns its path."""
    if ablation is None:
        ablation = os.environ.get("GEMM_BUILD_ABLATION", "") not in ("", "0")
    if os.path.isdir(BUILD):
        shutil.rmtree(BUILD)  # objects of the other build set must not be linked
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources(ablation)
    defines = ("-DGEMM_WITH_ABLATION",) if ablation else ()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, defines), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    print(build())
