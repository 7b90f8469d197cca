"""Seeded synthetic inputs for the dense bf16 (and fp16) GEMM workloads.

This module only draws random numbers and stores them as bf16 or fp16 bit
patterns;
it holds none of the GEMM's arithmetic.  The GPU library's tests, the
benchmark and the oracle all consume the same bytes from here.

Workload shapes follow the pages:

* "Hand-writing a Blackwell GEMM: from 164 to 1400 TFLOP/s", section "two
  workloads, not one": the 4096^3 reference shape, prefill at M = 8192 with
  the attention out-projection (N = K = 8192) and the MLP up-projection
  (N = 28672, K = 8192) of a 70B-class transformer, and decode at M = 256
  with attention out, fused QKV (N = 10240), MLP up and MLP down
  (N = 8192, K = 28672).  The same section notes that real decode batches
  are often 1 to 64 rows, which the ragged-M cases cover.
* "Matrix Multiplication on NVIDIA's Blackwell: A Four-Part Deep Dive",
  results list: the 512 x 8192 x 5376 projection of a 27B-class model.

Distributions (the pages give none, so these are stated readings):
activations and the square cases are N(0, 1); weights are N(0, 1) scaled by
1/sqrt(K) (standard deviation 1/sqrt(K)); the exact-result sets are integers
drawn uniformly from {-4, ..., 4} (or {-16, ..., 16} for the wide set, whose
sums of typical size 2000 exercise fp16 rounding of integers above 2048).
Each fp32 sample is rounded to bf16 or fp16 by torch's CPU conversion (round
to nearest even); the fp16 inputs of a workload are the same fp32 samples as
its bf16 inputs.  The generator is numpy's PCG64 with the fixed seeds below.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), rounded by torch (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> fp16 bit patterns (uint16), rounded by torch (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)


_TO_BITS = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits}
NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00}


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rows: int, cols: int, seed: int, std: float = 1.0,
                fmt: str = "bf16") -> np.ndarray:
    """rows x cols bits of N(0, std^2) samples (fp32 sample, then RNE to
    ``fmt``, "bf16" or "f16")."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _TO_BITS[fmt](x)


def int_bf16(rows: int, cols: int, seed: int, lo: int = -4, hi: int = 4,
             fmt: str = "bf16") -> np.ndarray:
    """rows x cols bits of integers uniform on {lo, ..., hi} (exact in both
    formats for |v| <= 256)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.integers(lo, hi + 1, size=(rows, cols), dtype=np.int32).astype(np.float32)
    return _TO_BITS[fmt](x)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str          # "int" (both operands) or "normal"
    weight_scaled: bool  # B ~ N(0, 1/K) instead of N(0, 1)
    seed_a: int
    seed_b: int
    int_range: int = 4   # "int" sets draw from {-int_range, ..., int_range}

    @property
    def sigma_a(self) -> float:
        return 1.0

    @property
    def sigma_b(self) -> float:
        return float(1.0 / np.sqrt(self.K)) if self.weight_scaled else 1.0

    def make(self, lda: int | None = None, ldb: int | None = None, fmt: str = "bf16"):
        """Return (A, B) as uint16 arrays of shape (M, lda) and (N, ldb), in
        format ``fmt`` ("bf16" or "f16").

        The first K columns hold the data; padding columns (if any) hold
        NaN so that any read of them shows up in the result."""
        lda = self.K if lda is None else lda
        ldb = self.K if ldb is None else ldb
        if self.dist == "int":
            r = self.int_range
            a = int_bf16(self.M, self.K, self.seed_a, -r, r, fmt=fmt)
            b = int_bf16(self.N, self.K, self.seed_b, -r, r, fmt=fmt)
        else:
            a = normal_bf16(self.M, self.K, self.seed_a, fmt=fmt)
            b = normal_bf16(self.N, self.K, self.seed_b, self.sigma_b, fmt=fmt)
        return _pad(a, lda, NAN_BITS[fmt]), _pad(b, ldb, NAN_BITS[fmt])


def _pad(x: np.ndarray, ld: int, nan_bits: int = 0x7FC0) -> np.ndarray:
    if ld == x.shape[1]:
        return x
    out = np.full((x.shape[0], ld), nan_bits, np.uint16)
    out[:, : x.shape[1]] = x
    return out


def _w(name, M, N, K, dist, scaled, sa, sb, int_range=4):
    return Workload(name, M, N, K, dist, scaled, sa, sb, int_range)


WORKLOADS = {w.name: w for w in [
    # 512^3: exact integer set and N(0,1) set
    _w("square512_int", 512, 512, 512, "int", False, 0x1A01, 0x1B01),
    _w("square512_normal", 512, 512, 512, "normal", False, 0x1A02, 0x1B02),
    _w("square512_int_wide", 512, 512, 512, "int", False, 0x1A03, 0x1B03, 16),
    # 4096^3: the headline shape
    _w("square4096_normal", 4096, 4096, 4096, "normal", False, 0x2A01, 0x2B01),
    _w("square4096_int", 4096, 4096, 4096, "int", False, 0x2A02, 0x2B02),
    # prefill, M = 8192 tokens
    _w("prefill_attn_out", 8192, 8192, 8192, "normal", True, 0x3A01, 0x3B01),
    _w("prefill_mlp_up", 8192, 28672, 8192, "normal", True, 0x3A02, 0x3B02),
    # decode, M = 256
    _w("decode_attn_out", 256, 8192, 8192, "normal", True, 0x4A01, 0x4B01),
    _w("decode_qkv", 256, 10240, 8192, "normal", True, 0x4A02, 0x4B02),
    _w("decode_mlp_up", 256, 28672, 8192, "normal", True, 0x4A03, 0x4B03),
    _w("decode_mlp_down", 256, 8192, 28672, "normal", True, 0x4A04, 0x4B04),
    # irregular
    _w("proj_512x8192x5376", 512, 8192, 5376, "normal", True, 0x5A01, 0x5B01),
    _w("ragged_m1", 1, 8192, 8192, "normal", True, 0x5A11, 0x5B11),
    _w("ragged_m17", 17, 8192, 8192, "normal", True, 0x5A12, 0x5B12),
    _w("ragged_m64", 64, 8192, 8192, "normal", True, 0x5A13, 0x5B13),
    _w("ragged_m200", 200, 8192, 8192, "normal", True, 0x5A14, 0x5B14),
]}
