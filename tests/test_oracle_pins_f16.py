"""Pins for the oracle's fp16 variant, checked against things other than the
oracle itself.

CPU only.  The fp16 decode and the direct fp64 -> fp16 rounding are tied to
numpy's float16 type (a library routine with its own conversion code) and to
exact rational arithmetic written here; the fp16 GEMM is tied to exact
rational sums, to int64 matmul and to the bf16 variant on inputs both
formats hold exactly.  A plausible slip -- a wrong exponent bias, a dropped
implicit bit, 10 or 12 significant bits instead of 11, round-half-up, a
detour through fp32, a missed overflow -- fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from synthetic_inputs import WORKLOADS, f32_to_f16_bits, int_bf16, normal_bf16

MAX_F16 = Fraction(65504)  # (2 - 2^-10) * 2^15


def exact_rne_f16_bits(s: Fraction) -> int:
    """Exact rational -> fp16 bits, round half to even, written independently
    of the oracle (integer arithmetic on Fractions, then numpy to encode the
    exact value)."""
    if s == 0:
        return 0
    sign = 0x8000 if s < 0 else 0
    a = abs(s)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    while Fraction(2) ** e <= a:
        e += 1
    q = max(e - 11, -24)
    n = a / Fraction(2) ** q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * Fraction(2) ** q
    if val > MAX_F16:
        return sign | 0x7C00
    bits = int(np.array([float(val)], np.float16).view(np.uint16)[0])
    return sign | bits


def f16_value(b) -> float:
    return float(np.array([b], np.uint16).view(np.float16)[0])


def torch_rne_f16_from_f32(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(
        torch.float16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------- decode and round

def test_decode_every_pattern_against_numpy(oracle_lib):
    """All 65536 fp16 patterns decode to numpy's float16 value (NaN to NaN,
    -0 keeps its sign)."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.f16_to_f64(int(p)) for p in pats])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_round_every_finite_pair(oracle_lib):
    """Every finite fp16 pair (x, next(x)): both map to themselves, the
    midpoint goes to the even pattern, points just off it go to the nearer
    one.  Both signs."""
    rnd = oracle_lib.round_to_f16
    pos = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = pos.view(np.float16).astype(np.float64)
    nxt = np.append(vals[1:], 65536.0)  # the first value past the range
    for i in range(0, len(pos), 3):
        x, y = vals[i], nxt[i]
        mid = (x + y) / 2
        bx, by = int(pos[i]), int(pos[i]) + 1
        assert rnd(x) == bx
        assert rnd(-x) == (0x8000 | bx)
        even = bx if bx % 2 == 0 else by
        if by == 0x7C00:          # the tie above 65504 rounds to infinity
            even = 0x7C00
        assert rnd(mid) == even
        assert rnd(mid - (y - x) / 4096) == bx
        assert rnd(mid + (y - x) / 4096) == (by if by < 0x7C00 else 0x7C00)


def test_round_random_doubles_against_numpy(oracle_lib):
    """numpy converts float64 to float16 directly (one rounding, ties to
    even); over twelve decades of magnitude, subnormals and overflow, the
    oracle agrees."""
    rng = np.random.default_rng(77)
    x = rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5.2, 20000)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle_lib.round_to_f16(v) for v in x], np.uint16)
    assert np.array_equal(got, want)


def test_round_is_direct_not_via_fp32(oracle_lib):
    """Just above the tie between 1 and 1 + 2^-10: direct rounding goes up,
    fp32 first would land on the tie and go to even (down)."""
    x = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert oracle_lib.round_to_f16(x) == 0x3C01
    assert torch_rne_f16_from_f32(np.array([x], np.float32))[0] == 0x3C00


def test_round_special_values(oracle_lib):
    rnd = oracle_lib.round_to_f16
    assert rnd(65504.0) == 0x7BFF
    assert rnd(65519.99) == 0x7BFF            # below the tie: finite
    assert rnd(65520.0) == 0x7C00             # tie with 2^16 (even): overflow
    assert rnd(-70000.0) == 0xFC00
    assert rnd(2.0 ** -24) == 0x0001          # smallest subnormal
    assert rnd(2.0 ** -25) == 0x0000          # tie with 0 -> even
    assert rnd(1.5 * 2.0 ** -25) == 0x0001
    assert rnd(2.0 ** -14) == 0x0400          # smallest normal
    assert rnd(2.0 ** -14 - 2.0 ** -24) == 0x03FF
    assert rnd(2049.0) == 0x6800              # 2048 (tie, even)
    assert rnd(2051.0) == 0x6802              # 2052 (tie, even)
    assert rnd(-0.0) == 0x8000
    assert rnd(float("inf")) == 0x7C00


# --------------------------------------------------------------- the product

@pytest.mark.parametrize("seed", range(10))
def test_brute_force_tiny_random_f16(oracle_lib, seed):
    """Exact rational sums of random fp16 products for M, N, K <= 6."""
    rng = np.random.default_rng(2000 + seed)
    M, N, K = (int(v) for v in rng.integers(1, 7, size=3))
    A = f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32) * 3)
    B = f32_to_f16_bits(rng.standard_normal((N, K)).astype(np.float32) * 3)
    C, S = oracle_lib.gemm(A, B, fmt="f16")
    for m in range(M):
        for n in range(N):
            s = sum(Fraction(f16_value(A[m, k])) * Fraction(f16_value(B[n, k]))
                    for k in range(K))
            assert Fraction(S[m, n]) == s
            assert int(C[m, n]) == exact_rne_f16_bits(s)


def test_wide_integer_set_against_int64_matmul(oracle_lib):
    """Integers in [-16, 16], K = 512: sums pass 2048, where fp16 starts to
    round integers.  int64 matmul is exact; torch rounds the (exact) fp32
    value to fp16."""
    A = int_bf16(40, 512, seed=7, lo=-16, hi=16, fmt="f16")
    B = int_bf16(33, 512, seed=8, lo=-16, hi=16, fmt="f16")
    a = A.view(np.float16).astype(np.int64)
    b = B.view(np.float16).astype(np.int64)
    want = a @ b.T
    assert (np.abs(want) > 2048).mean() > 0.2
    C, S = oracle_lib.gemm(A, B, fmt="f16")
    assert np.array_equal(S, want.astype(np.float64))
    assert np.array_equal(C, torch_rne_f16_from_f32(want.astype(np.float32)))


def test_same_sums_as_bf16_on_common_values(oracle_lib):
    """Inputs both formats hold exactly (small integers) give the same fp64
    sums through either decode; a wrong fp16 decode would not."""
    w = WORKLOADS["square512_int"]
    A16, B16 = w.make(fmt="f16")
    Ab, Bb = w.make(fmt="bf16")
    _, S16 = oracle_lib.gemm(A16[:64], B16[:48], fmt="f16")
    _, Sb = oracle_lib.gemm(Ab[:64], Bb[:48], fmt="bf16")
    assert np.array_equal(S16, Sb)


def test_numpy_float64_matmul_cross_check_f16(oracle_lib):
    A = normal_bf16(96, 384, seed=41, fmt="f16")
    B = normal_bf16(80, 384, seed=42, fmt="f16")
    a = A.view(np.float16).astype(np.float64)
    b = B.view(np.float16).astype(np.float64)
    ref = a @ b.T
    C, S = oracle_lib.gemm(A, B, fmt="f16")
    assert np.max(np.abs(S - ref)) <= 1e-12 * np.max(np.abs(ref))
    rb = ref.ravel()[:2000].astype(np.float16).view(np.uint16)
    assert np.array_equal(C.ravel()[:2000], rb)


def test_identity_and_orientation_f16(oracle_lib):
    """A = I: C = B^T bit-exact; a non-square integer case fixes which
    operand is transposed."""
    K, N = 20, 13
    A = f32_to_f16_bits(np.eye(K, dtype=np.float32))
    B = normal_bf16(N, K, seed=43, fmt="f16")
    C, _ = oracle_lib.gemm(A, B, fmt="f16")
    assert np.array_equal(C, B.T)
    A = int_bf16(5, 7, seed=44, fmt="f16")
    B = int_bf16(3, 7, seed=45, fmt="f16")
    a = A.view(np.float16).astype(np.int64)
    b = B.view(np.float16).astype(np.int64)
    _, S = oracle_lib.gemm(A, B, fmt="f16")
    assert S.shape == (5, 3)
    assert np.array_equal(S, (a @ b.T).astype(np.float64))


def test_overflow_to_infinity_f16(oracle_lib):
    """Sums of 255 * 256 = 65280 stay finite, 256 * 256 = 65536 overflow."""
    K = 256
    A = f32_to_f16_bits(np.full((2, K), 16.0, np.float32))
    B = f32_to_f16_bits(np.stack([np.full(K, 16.0, np.float32),
                                  np.r_[np.full(K - 1, 16.0), 0.0].astype(np.float32),
                                  np.full(K, -16.0, np.float32)]))
    C, S = oracle_lib.gemm(A, B, fmt="f16")
    assert list(S[0]) == [65536.0, 65280.0, -65536.0]
    assert list(C[0]) == [0x7C00, 0x7BF8, 0xFC00]


def test_entries_match_full_f16(oracle_lib):
    A = normal_bf16(40, 72, seed=46, fmt="f16")
    B = normal_bf16(50, 72, seed=47, fmt="f16")
    C, S = oracle_lib.gemm(A, B, fmt="f16")
    rng = np.random.default_rng(5)
    ms = rng.integers(0, 40, 150)
    ns = rng.integers(0, 50, 150)
    c16, c64 = oracle_lib.gemm_entries(A, B, ms, ns, fmt="f16")
    assert np.array_equal(c16, C[ms, ns]) and np.array_equal(c64, S[ms, ns])


def test_fmt_is_checked(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.gemm(np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16), fmt="fp8")
