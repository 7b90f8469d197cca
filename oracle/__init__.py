"""Oracle for the dense GEMM C[M,N] = A[M,K] . B[N,K]^T over bf16 (and fp16)
operands (CPU, fp64 sums).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow definition that
the GPU library is checked against.  Only ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product
package ``dense_gemm_bf16_amd`` never imports it and shares no code with it;
the only thing both sides consume is the seeded input bytes from
``synthetic_inputs``.

The arithmetic lives in ``oracle_gemm.c`` (plain C + OpenMP over rows).  What
it follows, from the pages:

* "Matrix Multiplication on NVIDIA's Blackwell: A Four-Part Deep Dive",
  definition section: C is M x N inner products over K, a triple loop; and
  the naive-kernel section: the second operand is read as b[col, k] (stored
  N x K), bf16 in and out, the sum carried wider than bf16.
* "Hand-writing a Blackwell GEMM: from 164 to 1400 TFLOP/s", Step 1: a C
  tile is the sum of A_k B_k^T over K-slices starting from zero.

* The fp16 variant: the same page runs its comparisons on fp16 tensors; the
  same sum over fp16 operands, rounded once to fp16 (IEEE binary16).

Readings where the pages are silent (each also pinned by a test): the sum is
carried in fp64 in natural k order; the fp64 sum is rounded once, directly,
to the output format with round-to-nearest-even; K = 0 gives zeros.

Everything here takes and returns numpy arrays of raw 16-bit patterns
(``uint16``; ``fmt`` = "bf16" or "f16" says which format) and fp64 sums.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")

_lib = None
_FORMATS = ("bf16", "f16")


def _check_fmt(fmt):
    if fmt not in _FORMATS:
        raise ValueError(f"fmt must be one of {_FORMATS}, not {fmt!r}")


def build(force: bool = True) -> str:
    """Compile ``oracle_gemm.c`` with gcc into ``liboracle_gemm.so``.

    No fast-math and no FP contraction: the loop must add in the order it is
    written.
    """
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_round_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_round_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_f64_to_f16.restype = ctypes.c_uint16
    lib.oracle_round_f64_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_f16_bits_to_f64.restype = ctypes.c_double
    lib.oracle_f16_bits_to_f64.argtypes = [ctypes.c_uint16]
    for fmt in _FORMATS:
        f = getattr(lib, f"oracle_gemm_{fmt}")
        f.restype = ctypes.c_int
        f.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, ctypes.c_int]
        f = getattr(lib, f"oracle_gemm_{fmt}_entries")
        f.restype = ctypes.c_int
        f.argtypes = [i64, i64, i64, p, i64, p, i64, i64, p, p, p, p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_u16_2d(x, name):
    x = np.asarray(x)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 array of 16-bit patterns")
    if x.size == 0 or x.shape[0] == 1:
        return np.ascontiguousarray(x)
    if x.strides[1] != 2:
        raise ValueError(f"{name} rows must be contiguous")
    return x


def _ld(x):
    """Row stride in elements (at least the row length, at least 1)."""
    if x.size == 0 or x.shape[0] == 1:
        return max(x.shape[1], 1)
    return x.strides[0] // 2


def round_to_bf16(x: float) -> int:
    """One fp64 value rounded to bf16 (RNE), as its 16-bit pattern."""
    return int(_load().oracle_round_f64_to_bf16(float(x)))


def round_to_f16(x: float) -> int:
    """One fp64 value rounded to fp16 (RNE), as its 16-bit pattern."""
    return int(_load().oracle_round_f64_to_f16(float(x)))


def f16_to_f64(bits: int) -> float:
    """The value of one fp16 bit pattern."""
    return float(_load().oracle_f16_bits_to_f64(int(bits)))


def gemm(A: np.ndarray, B: np.ndarray, K: int | None = None,
         want_bf16: bool = True, want_f64: bool = True, threads: int = 0,
         fmt: str = "bf16"):
    """C = A . B^T for 16-bit arrays A (M x >=K) and B (N x >=K) of format
    ``fmt`` ("bf16" or "f16").

    ``K`` defaults to A's column count; row strides are taken from the arrays,
    so padded (lda > K) views are allowed.  Returns ``(C16, S_f64)``: the
    RNE-rounded bits in the operands' format (``want_bf16`` asks for them
    whatever the format) and the exact-order fp64 sums (either may be None).
    """
    _check_fmt(fmt)
    A = _as_u16_2d(A, "A")
    B = _as_u16_2d(B, "B")
    M, N = A.shape[0], B.shape[0]
    if K is None:
        K = A.shape[1]
    if A.shape[1] < K or B.shape[1] < K:
        raise ValueError("K exceeds an operand's column count")
    lda, ldb = _ld(A), _ld(B)
    C = np.empty((M, N), np.uint16) if want_bf16 else None
    S = np.empty((M, N), np.float64) if want_f64 else None
    fn = getattr(_load(), f"oracle_gemm_{fmt}")
    rc = fn(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), N, _ptr(S), N, threads)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return C, S


def gemm_entries(A: np.ndarray, B: np.ndarray, ms, ns, K: int | None = None,
                 threads: int = 0, fmt: str = "bf16"):
    """Elements (ms[i], ns[i]) of A . B^T only.  Returns (16-bit patterns in
    the operands' format, fp64 sums)."""
    _check_fmt(fmt)
    A = _as_u16_2d(A, "A")
    B = _as_u16_2d(B, "B")
    if K is None:
        K = A.shape[1]
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D and of equal length")
    cnt = ms.shape[0]
    out16 = np.empty(cnt, np.uint16)
    out64 = np.empty(cnt, np.float64)
    rc = getattr(_load(), f"oracle_gemm_{fmt}_entries")(
        A.shape[0], B.shape[0], K, _ptr(A), _ld(A), _ptr(B), _ld(B), cnt, _ptr(ms), _ptr(ns), _ptr(out16), _ptr(out64),
        threads)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out16, out64


def max_threads() -> int:
    """Threads the oracle's OpenMP loop uses by default."""
    return int(_load().oracle_max_threads())
