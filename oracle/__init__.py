"""Oracle for the dense bf16 GEMM C[M,N] = A[M,K] . B[N,K]^T (CPU, fp64 sums).

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

Readings where the pages are silent (each also pinned by a test): the sum is
carried in fp64 in natural k order; the fp64 sum is rounded once, directly,
to bf16 with round-to-nearest-even; K = 0 gives zeros.

Everything here takes and returns numpy arrays of raw bf16 bit patterns
(``uint16``) and fp64 sums.
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
    lib.oracle_gemm_bf16.restype = ctypes.c_int
    lib.oracle_gemm_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64,
                                     p, i64, ctypes.c_int]
    lib.oracle_gemm_bf16_entries.restype = ctypes.c_int
    lib.oracle_gemm_bf16_entries.argtypes = [i64, i64, i64, p, i64, p, i64,
                                             i64, p, p, p, p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_u16_2d(x, name):
    x = np.asarray(x)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 array of bf16 bits")
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


def gemm(A: np.ndarray, B: np.ndarray, K: int | None = None,
         want_bf16: bool = True, want_f64: bool = True, threads: int = 0):
    """C = A . B^T for bf16-bit arrays A (M x >=K) and B (N x >=K).

    ``K`` defaults to A's column count; row strides are taken from the arrays,
    so padded (lda > K) views are allowed.  Returns ``(C_bf16, S_f64)``: the
    RNE-rounded bf16 bits and the exact-order fp64 sums (either may be None).
    """
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
    rc = _load().oracle_gemm_bf16(M, N, K, _ptr(A), lda, _ptr(B), ldb,
                                  _ptr(C), N, _ptr(S), N, threads)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return C, S


def gemm_entries(A: np.ndarray, B: np.ndarray, ms, ns, K: int | None = None,
                 threads: int = 0):
    """Elements (ms[i], ns[i]) of A . B^T only.  Returns (bf16 bits, fp64)."""
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
    rc = _load().oracle_gemm_bf16_entries(
        A.shape[0], B.shape[0], K, _ptr(A), _ld(A), _ptr(B), _ld(B), cnt, _ptr(ms), _ptr(ns), _ptr(out16), _ptr(out64),
        threads)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out16, out64


def max_threads() -> int:
    """Threads the oracle's OpenMP loop uses by default."""
    return int(_load().oracle_max_threads())
