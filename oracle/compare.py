"""Parity criteria between a GPU result and the oracle.

TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package).

Criteria (the pages fix bf16 in/out with a wider accumulator but no
tolerance; the readings below are stated in the design notes):

* Integer-valued inputs: every partial sum is an integer below 2^24, exact in
  fp32 in any order, so the bf16 (or fp16) result must equal the oracle's bit
  for bit and the fp32 debug output must equal the fp64 sum exactly.
* Real-valued inputs: a correct fp32 accumulation may round differently from
  the exact sum, so an element passes if its bf16 value is within 1 ulp of
  the oracle's rounded result, or (near zero, where one bf16 ulp is finer
  than fp32 accumulation error) within an absolute floor of
  1e-4 * sqrt(K) * sigma_A * sigma_B of the exact sum.  The fp16 variant is
  held to the same rule in fp16 ulps (both formats are sign-magnitude, so
  adjacent values of either differ by one in the ordering key below).
* fp32 debug output: |C32 - s| <= 1e-4 * sqrt(K) * sigma_A * sigma_B.

The floor relaxes "within 1 ulp" for the elements near zero only; reports
carry ``max_ulp`` and ``n_floor`` (elements beyond 1 ulp that passed by the
floor), so how many needed it is always visible.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return b.view(np.float16).astype(np.float64)


_DECODE = {"bf16": bf16_bits_to_f64, "f16": f16_bits_to_f64}


def ulp_key(bits: np.ndarray) -> np.ndarray:
    """Map bf16 (or fp16) patterns to integers ordered like the values they
    encode.

    +0 and -0 both map to 0; adjacent bf16 values differ by 1."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_dist(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(ulp_key(a_bits) - ulp_key(b_bits))


def abs_floor(K: int, sigma_a: float = 1.0, sigma_b: float = 1.0) -> float:
    return 1e-4 * np.sqrt(max(K, 1)) * sigma_a * sigma_b


def check_bf16(got_bits, ref_bits, ref_sum, K, sigma_a=1.0, sigma_b=1.0,
               exact=False, fmt="bf16") -> dict:
    """Compare GPU 16-bit results (bf16, or fp16 with ``fmt="f16"``) with the
    oracle.  Returns a report dict whose ``ok`` field is the outcome."""
    got_bits = np.asarray(got_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    d = ulp_dist(got_bits, ref_bits)
    n = d.size
    rep = {"n": int(n), "max_ulp": int(d.max()) if n else 0,
           "n_ulp_gt0": int((d > 0).sum())}
    if exact:
        rep["ok"] = bool(n == 0 or rep["max_ulp"] == 0)
        rep["n_fail"] = int((d != 0).sum())
        return rep
    floor = abs_floor(K, sigma_a, sigma_b)
    err = np.abs(_DECODE[fmt](got_bits) - np.asarray(ref_sum, np.float64))
    need_floor = d > 1
    fail = need_floor & ~(err <= floor)
    rep.update({"n_floor": int(need_floor.sum()), "n_fail": int(fail.sum()),
                "floor": floor, "ok": bool(not fail.any())})
    return rep


def check_f32(got, ref_sum, K, sigma_a=1.0, sigma_b=1.0, exact=False) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref_sum, np.float64)
    err = got - ref
    n = err.size
    tol = 0.0 if exact else abs_floor(K, sigma_a, sigma_b)
    rep = {"n": int(n),
           "max_abs_err": float(np.abs(err).max()) if n else 0.0,
           "rms_err": float(np.sqrt((err ** 2).mean())) if n else 0.0,
           "mean_err": float(err.mean()) if n else 0.0,
           "tol": tol}
    rep["ok"] = bool(n == 0 or rep["max_abs_err"] <= tol)
    return rep
