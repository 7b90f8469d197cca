"""Pins for the oracle, checked against things other than the oracle itself.

CPU only.  Each test ties one part of the oracle (the sum, the indexing and
layout, the rounding) to an independent fact: exact rational arithmetic in
Python, a textbook special case, a closed form, or a library routine (numpy
float64 matmul, torch's fp32->bf16 conversion).  A plausible slip in the
oracle -- a dropped or doubled term, a sign, a swapped index, a transposed
operand, round-half-up instead of half-even, a detour through fp32 -- fails
at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from synthetic_inputs import bf16_bits_to_f32, f32_to_bf16_bits, int_bf16, normal_bf16

MAX_BF16 = Fraction((2 ** 8 - 1) * 2 ** 120)  # (2 - 2^-7) * 2^127


def exact_rne_bf16_bits(s: Fraction) -> int:
    """Exact rational -> bf16 bits, round half to even, written independently
    of the oracle (integer arithmetic on Fractions only)."""
    if s == 0:
        return 0
    sign = 0x8000 if s < 0 else 0
    a = abs(s)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    while Fraction(2) ** e <= a:
        e += 1
    q = max(e - 8, -133)
    n = a / Fraction(2) ** q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * Fraction(2) ** q
    if val > MAX_BF16:
        return sign | 0x7F80
    bits = int(np.array([float(val)], np.float32).view(np.uint32)[0] >> 16)
    return sign | bits


def frac_of_bits(b) -> Fraction:
    return Fraction(float(bf16_bits_to_f32(np.array([b], np.uint16))[0]))


def torch_rne_from_f32(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- P1: the sum

@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny_random_bf16(oracle_lib, seed):
    """Exact rational sums of random bf16 products for M,N,K <= 6."""
    rng = np.random.default_rng(1000 + seed)
    M, N, K = (int(v) for v in rng.integers(1, 7, size=3))
    A = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * 3)
    B = f32_to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * 3)
    C, S = oracle_lib.gemm(A, B)
    for m in range(M):
        for n in range(N):
            s = sum(frac_of_bits(A[m, k]) * frac_of_bits(B[n, k]) for k in range(K))
            assert Fraction(S[m, n]) == s
            assert int(C[m, n]) == exact_rne_bf16_bits(s)


def test_brute_force_exhaustive_small_ints(oracle_lib):
    """Every 2x2 pair of A rows from {-2..2}, K = 2, against Python ints."""
    vals = np.arange(-2, 3, dtype=np.float32)
    grid = np.array(np.meshgrid(vals, vals)).reshape(2, -1).T  # 25 x 2
    A = f32_to_bf16_bits(grid)
    B = f32_to_bf16_bits(grid)
    C, S = oracle_lib.gemm(A, B)
    want = grid.astype(np.int64) @ grid.astype(np.int64).T
    assert np.array_equal(S, want.astype(np.float64))
    assert np.array_equal(C, torch_rne_from_f32(want.astype(np.float32)))


def test_integer_set_against_int64_matmul(oracle_lib):
    """Integer inputs in [-4, 4]: int64 matmul is exact; rounding by torch."""
    A = int_bf16(37, 300, seed=5)
    B = int_bf16(41, 300, seed=6)
    a = bf16_bits_to_f32(A).astype(np.int64)
    b = bf16_bits_to_f32(B).astype(np.int64)
    want = a @ b.T
    C, S = oracle_lib.gemm(A, B)
    assert np.array_equal(S, want.astype(np.float64))
    assert np.array_equal(C, torch_rne_from_f32(want.astype(np.float32)))


def test_numpy_float64_matmul_cross_check(oracle_lib):
    """A library routine with another summation order agrees to ~1e-13."""
    A = normal_bf16(128, 512, seed=11)
    B = normal_bf16(96, 512, seed=12)
    a = bf16_bits_to_f32(A).astype(np.float64)
    b = bf16_bits_to_f32(B).astype(np.float64)
    ref = a @ b.T
    C, S = oracle_lib.gemm(A, B)
    assert np.max(np.abs(S - ref)) <= 1e-12 * np.max(np.abs(ref))
    # rounding the library's sums gives the same bf16 except at exact ties,
    # which random real data does not hit
    rb = np.array([exact_rne_bf16_bits(Fraction(x)) for x in ref.ravel()[:2000]],
                  np.uint16)
    assert np.array_equal(C.ravel()[:2000], rb)


def test_k_zero_is_empty_sum(oracle_lib):
    A = np.zeros((3, 0), np.uint16)
    B = np.zeros((5, 0), np.uint16)
    C, S = oracle_lib.gemm(A, B)
    assert C.shape == (3, 5) and not C.any() and not S.any()


def test_empty_m_or_n(oracle_lib):
    C, S = oracle_lib.gemm(np.zeros((0, 4), np.uint16), np.zeros((2, 4), np.uint16))
    assert C.shape == (0, 2)
    C, S = oracle_lib.gemm(np.zeros((3, 4), np.uint16), np.zeros((0, 4), np.uint16))
    assert C.shape == (3, 0)


# ------------------------------------------------- P2: indexing and layout

def test_identity_left_gives_b_transpose(oracle_lib):
    """A = I_K: C[m,n] = B[n,m], bit-exact for any bf16 B (sums of zeros)."""
    K, N = 24, 17
    A = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    B = normal_bf16(N, K, seed=21)
    C, _ = oracle_lib.gemm(A, B)
    assert np.array_equal(C, B.T)


def test_identity_right_gives_a(oracle_lib):
    """B = I_K: C = A, bit-exact."""
    M, K = 19, 32
    A = normal_bf16(M, K, seed=22)
    B = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    C, _ = oracle_lib.gemm(A, B)
    assert np.array_equal(C, A)


def test_permutation(oracle_lib):
    """A = P (a permutation): C[m,n] = B[n, pi(m)]."""
    K, N = 33, 9
    pi = np.random.default_rng(3).permutation(K)
    P = np.zeros((K, K), np.float32)
    P[np.arange(K), pi] = 1.0
    B = normal_bf16(N, K, seed=23)
    C, _ = oracle_lib.gemm(f32_to_bf16_bits(P), B)
    assert np.array_equal(C, B[:, pi].T)


def test_transpose_identity(oracle_lib):
    """(A.B^T)^T = B.A^T exactly (same products, same k order)."""
    A = normal_bf16(13, 70, seed=24)
    B = normal_bf16(29, 70, seed=25)
    _, S1 = oracle_lib.gemm(A, B)
    _, S2 = oracle_lib.gemm(B, A)
    assert np.array_equal(S1.T, S2)


def test_padded_leading_dimensions_ignore_padding(oracle_lib):
    """lda, ldb > K with NaN in the padding: same result as contiguous."""
    A = normal_bf16(21, 40, seed=26)
    B = normal_bf16(23, 40, seed=27)
    Ap = np.full((21, 48), 0x7FC0, np.uint16)
    Bp = np.full((23, 56), 0x7FC0, np.uint16)
    Ap[:, :40] = A
    Bp[:, :40] = B
    C1, S1 = oracle_lib.gemm(A, B)
    C2, S2 = oracle_lib.gemm(Ap, Bp, K=40)
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)


def test_nonsquare_shapes_and_orientation(oracle_lib):
    """M != N != K: a transposed operand or swapped index cannot match."""
    A = int_bf16(5, 7, seed=28)
    B = int_bf16(3, 7, seed=29)
    a = bf16_bits_to_f32(A).astype(np.int64)
    b = bf16_bits_to_f32(B).astype(np.int64)
    _, S = oracle_lib.gemm(A, B)
    assert S.shape == (5, 3)
    for m in range(5):
        for n in range(3):
            assert S[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(7))


def test_entries_match_full(oracle_lib):
    A = normal_bf16(50, 64, seed=30)
    B = normal_bf16(60, 64, seed=31)
    C, S = oracle_lib.gemm(A, B)
    rng = np.random.default_rng(4)
    ms = rng.integers(0, 50, 200)
    ns = rng.integers(0, 60, 200)
    c16, c64 = oracle_lib.gemm_entries(A, B, ms, ns)
    assert np.array_equal(c16, C[ms, ns]) and np.array_equal(c64, S[ms, ns])


# ------------------------------------------------------------ P3: rounding

def test_rounding_exhaustive_ties_and_neighbours(oracle_lib):
    """Every finite bf16 pair (x, next(x)): x and next map to themselves,
    the midpoint goes to the even pattern, points just off it go to the
    nearer one.  Both signs."""
    rnd = oracle_lib.round_to_bf16
    pos = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    vals = bf16_bits_to_f32(pos).astype(np.float64)
    nxt = np.append(vals[1:], 2.0 ** 128)
    for i in range(0, len(pos), 7):  # stride keeps the test quick
        x, y = vals[i], nxt[i]
        mid = (x + y) / 2
        bx, by = int(pos[i]), int(pos[i]) + 1
        assert rnd(x) == bx
        even = bx if bx % 2 == 0 else by
        assert rnd(mid) == even
        assert rnd(-mid) == (0x8000 | even)
        assert rnd(mid - (y - x) / 1024) == bx
        assert rnd(mid + (y - x) / 1024) == by


def test_rounding_integer_ties(oracle_lib):
    """Integers 256..65536 are exact fp32 values; torch's fp32->bf16 is RNE.
    Covers the ties 257 -> 256, 259 -> 260, 514 -> 512, 518 -> 520."""
    ints = np.arange(256, 65537, dtype=np.float64)
    got = np.array([oracle_lib.round_to_bf16(v) for v in ints], np.uint16)
    assert np.array_equal(got, torch_rne_from_f32(ints.astype(np.float32)))
    f = lambda v: float(bf16_bits_to_f32(np.array([oracle_lib.round_to_bf16(v)], np.uint16))[0])
    assert (f(257), f(259), f(514), f(518)) == (256, 260, 512, 520)


def test_rounding_is_direct_not_via_fp32(oracle_lib):
    """A value just above a bf16 tie that fp32 would round onto the tie:
    direct rounding goes up, fp32-then-bf16 would go to even (down)."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40   # tie between 1 and 1+2^-7, nudged up
    assert oracle_lib.round_to_bf16(x) == 0x3F81
    assert torch_rne_from_f32(np.array([x], np.float32))[0] == 0x3F80


def test_rounding_overflow_and_subnormal(oracle_lib):
    rnd = oracle_lib.round_to_bf16
    assert rnd(3.4e38) == 0x7F80 and rnd(-3.4e38) == 0xFF80
    assert rnd(3.0e38) == 0x7F62            # finite: below the largest bf16
    assert rnd(float(MAX_BF16)) == 0x7F7F
    assert rnd(2.0 ** -133) == 0x0001
    assert rnd(2.0 ** -134) == 0x0000           # tie with 0 -> even (0)
    assert rnd(1.5 * 2.0 ** -134) == 0x0001
    assert rnd(-0.0) == 0x8000


def test_k1_outer_product_against_torch(oracle_lib):
    """K = 1: C = RNE(a*b) of one exact product (exact in fp32), any bf16."""
    A = normal_bf16(64, 1, seed=32)
    B = normal_bf16(48, 1, seed=33)
    a = bf16_bits_to_f32(A)[:, 0]
    b = bf16_bits_to_f32(B)[:, 0]
    prod = np.outer(a, b).astype(np.float32)   # exact: 8-bit x 8-bit
    C, S = oracle_lib.gemm(A, B)
    assert np.array_equal(S, prod.astype(np.float64))
    assert np.array_equal(C, torch_rne_from_f32(prod))


def test_all_ones_and_rank_one(oracle_lib):
    K = 300
    ones = f32_to_bf16_bits(np.ones((4, K), np.float32))
    C, S = oracle_lib.gemm(ones, ones)
    assert np.all(S == K)
    assert np.all(C == exact_rne_bf16_bits(Fraction(K)))  # 300 -> 300 (exact)
    u = np.array([1, -2, 3, 0.5], np.float32)
    v = np.array([4, -0.25, 2], np.float32)
    A = f32_to_bf16_bits(np.repeat(u[:, None], K, 1))
    B = f32_to_bf16_bits(np.repeat(v[:, None], K, 1))
    _, S = oracle_lib.gemm(A, B)
    assert np.array_equal(S, K * np.outer(u, v).astype(np.float64))


# ----------------------------------------------------------- P4: linearity

def test_linearity_in_a(oracle_lib):
    """gemm(2*A1 - 3*A2, B) = 2*gemm(A1,B) - 3*gemm(A2,B), exact on ints."""
    A1 = bf16_bits_to_f32(int_bf16(20, 64, seed=34))
    A2 = bf16_bits_to_f32(int_bf16(20, 64, seed=35))
    B = int_bf16(15, 64, seed=36)
    Acomb = f32_to_bf16_bits(2 * A1 - 3 * A2)
    _, S = oracle_lib.gemm(Acomb, B)
    _, S1 = oracle_lib.gemm(f32_to_bf16_bits(A1), B)
    _, S2 = oracle_lib.gemm(f32_to_bf16_bits(A2), B)
    assert np.array_equal(S, 2 * S1 - 3 * S2)


def test_thread_count_does_not_change_result(oracle_lib):
    A = normal_bf16(70, 200, seed=37)
    B = normal_bf16(30, 200, seed=38)
    C1, S1 = oracle_lib.gemm(A, B, threads=1)
    C4, S4 = oracle_lib.gemm(A, B, threads=4)
    assert np.array_equal(C1, C4) and np.array_equal(S1, S4)
