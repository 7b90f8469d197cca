"""GPU parity of the fp16-operand entry points against the oracle's fp16
variant, element by element.

The gates are those of the bf16 path, in fp16 terms: integer-valued inputs
bit-exact (the fp32 sums are exact, and one round-to-nearest-even to fp16
must match the oracle's direct rounding, also above 2048 where fp16 stops
holding every integer, and at the overflow threshold); N(0,1)-type inputs
within 1 fp16 ulp, or within 1e-4 * sqrt(K) * sigma_A * sigma_B near zero;
fp32 debug output within the same absolute bound (exact on integers).

Every call goes through the C ABI (``gemm_f16_ex``).
"""
import numpy as np
import pytest

from oracle.compare import check_bf16, check_f32
from synthetic_inputs import WORKLOADS, f32_to_f16_bits, int_bf16, normal_bf16
from tests.gpu_util import run_gemm

pytestmark = pytest.mark.gpu
F16 = "f16"


def _oracle():
    import oracle

    return oracle


def _check_full(w, A, B, exact, f32=True):
    o = _oracle()
    ref16, ref64 = o.gemm(A, B, K=w.K, fmt=F16)
    got = run_gemm(A, B, K=w.K, fmt=F16)
    rep = check_bf16(got, ref16, ref64, w.K, w.sigma_a, w.sigma_b, exact=exact, fmt=F16)
    print(w.name, "f16", rep, flush=True)
    assert rep["ok"], rep
    if f32:
        got32 = run_gemm(A, B, K=w.K, out_f32=True, fmt=F16)
        rep32 = check_f32(got32, ref64, w.K, w.sigma_a, w.sigma_b, exact=exact)
        print(w.name, "f16->f32", rep32, flush=True)
        assert rep32["ok"], rep32


@pytest.mark.parametrize("name", ["square512_int", "square512_int_wide", "square512_normal",
                                  "square4096_int", "square4096_normal"])
def test_square_f16(name):
    w = WORKLOADS[name]
    A, B = w.make(fmt=F16)
    _check_full(w, A, B, exact=(w.dist == "int"))


@pytest.mark.parametrize("name", ["decode_attn_out", "decode_mlp_down", "proj_512x8192x5376",
                                  "ragged_m1", "ragged_m17", "ragged_m64", "ragged_m200"])
def test_decode_and_irregular_f16(name):
    """fp16 and fp32 output on every element: split-K plans (attention-out,
    MLP-down, M = 64 and 200) take the reduction's fp32 branch, M = 1 and
    17 the small-M kernel's fp32 store."""
    w = WORKLOADS[name]
    A, B = w.make(fmt=F16)
    _check_full(w, A, B, exact=False, f32=True)


def test_prefill_sampled_f16():
    """M = 8192 prefill (attention out-projection): full rows and columns at
    both edges and spread through the middle."""
    w = WORKLOADS["prefill_attn_out"]
    A, B = w.make(fmt=F16)
    got = run_gemm(A, B, fmt=F16)
    o = _oracle()
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(w.M - 16, w.M),
                                     rng.choice(w.M, 16, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(w.N - 16, w.N),
                                     rng.choice(w.N, 16, replace=False)]))
    r16, r64 = o.gemm(np.ascontiguousarray(A[rows]), B, K=w.K, fmt=F16)
    rep = check_bf16(got[rows], r16, r64, w.K, w.sigma_a, w.sigma_b, fmt=F16)
    assert rep["ok"], rep
    c16, c64 = o.gemm(A, np.ascontiguousarray(B[cols]), K=w.K, fmt=F16)
    rep = check_bf16(got[:, cols], c16, c64, w.K, w.sigma_a, w.sigma_b, fmt=F16)
    assert rep["ok"], rep


def test_every_f16_config_bit_exact_on_ragged_shape():
    """Each configuration built for fp16, plain, split K (through the
    reduction kernel's fp16 rounding) and split with K-step rotation, on a
    shape ragged in M, N and K with integers in [-16, 16]: sums of typical
    size 2000, so the fp16 rounding of integers is exercised; bit-exact."""
    import dense_gemm_bf16_amd as g

    M, N, K = 300, 520, 456
    A = int_bf16(M, K, seed=111, lo=-16, hi=16, fmt=F16)
    B = int_bf16(N, K, seed=112, lo=-16, hi=16, fmt=F16)
    ref16, ref64 = _oracle().gemm(A, B, fmt=F16)
    assert (np.abs(ref64) > 2048).mean() > 0.1
    names = g.f16_config_names()
    assert "t256x256x64_w2x2_s2_x3_p10" in names
    for cfg in names:
        for suffix in ("_k1", "_k3", "_k2_g4_r1"):
            name = cfg + suffix
            got = run_gemm(A, B, config=name, fmt=F16)
            rep = check_bf16(got, ref16, None, K, exact=True, fmt=F16)
            print(name, rep, flush=True)
            assert rep["ok"], (name, rep)
        for suffix in ("_k1", "_k3"):
            name = cfg + suffix
            got32 = run_gemm(A, B, config=name, out_f32=True, fmt=F16)
            rep = check_f32(got32, ref64, K, exact=True)
            print(name, "f32", rep, flush=True)
            assert rep["ok"], (name, rep)


@pytest.mark.parametrize("K", [1, 7, 65, 200])
def test_ragged_k_f16(K):
    M, N = 70, 90
    lda = ldb = ((K + 7) // 8) * 8 + 8
    A = np.full((M, lda), 0x7E00, np.uint16)
    B = np.full((N, ldb), 0x7E00, np.uint16)
    A[:, :K] = int_bf16(M, K, seed=210 + K, fmt=F16)
    B[:, :K] = int_bf16(N, K, seed=310 + K, fmt=F16)
    ref16, ref64 = _oracle().gemm(A, B, K=K, fmt=F16)
    got = run_gemm(A, B, K=K, fmt=F16)
    assert check_bf16(got, ref16, None, K, exact=True, fmt=F16)["ok"]
    got32 = run_gemm(A, B, K=K, out_f32=True, fmt=F16)
    assert check_f32(got32, ref64, K, exact=True)["ok"]


@pytest.mark.parametrize("config", [None, "t256x128x64_w2x2_s3_x3_p10_k3",
                                    "t32x128x64_w1x4_s6_x2_p0_k1"])
def test_overflow_threshold_f16(config):
    """Sums 65504 (largest finite), 65519 (rounds down to it), 65520 (the
    tie with 2^16: overflows to infinity) and -65520, exact in fp32; each
    epilogue (direct store and the split-K reduction) must round them as
    the oracle does."""
    K = 256
    a = np.full(K, 16.0, np.float32)
    a[-1] = 1.0
    base = np.full(K, 16.0, np.float32)
    rows_b = []
    for last in (224.0, 239.0, 240.0):   # 65280 + last
        r = base.copy()
        r[-1] = last
        rows_b.append(r)
    rows_b.append(-rows_b[-1])
    A = f32_to_f16_bits(np.tile(a, (40, 1)))
    B = f32_to_f16_bits(np.tile(np.stack(rows_b), (10, 1)))  # N = 40
    ref16, ref64 = _oracle().gemm(A, B, fmt=F16)
    assert list(ref16[0, :4]) == [0x7BFF, 0x7BFF, 0x7C00, 0xFC00]
    got = run_gemm(A, B, config=config, fmt=F16)
    assert np.array_equal(got, ref16), (got[0, :4], ref16[0, :4])


def test_torch_matmul_form_f16():
    """The torch convenience form on float16 tensors, including a single-row
    A whose row stride is not a multiple of 8."""
    import torch

    import dense_gemm_bf16_amd as g

    A = normal_bf16(33, 136, seed=801, fmt=F16)
    B = normal_bf16(72, 136, seed=802, fmt=F16)
    ref16, ref64 = _oracle().gemm(A, B, fmt=F16)
    tA = torch.from_numpy(A.view(np.float16)).cuda()
    tB = torch.from_numpy(B.view(np.float16)).cuda()
    C = g.matmul(tA, tB)
    torch.cuda.synchronize()
    assert C.dtype == torch.float16
    got = C.cpu().numpy().view(np.uint16)
    assert check_bf16(got, ref16, ref64, 136, fmt=F16)["ok"]
    C1 = g.matmul(tA[:1, :130], tB[:, :130])
    torch.cuda.synchronize()
    r1, s1 = _oracle().gemm(np.ascontiguousarray(A[:1, :130]),
                            np.ascontiguousarray(B[:, :130]), fmt=F16)
    assert check_bf16(C1.cpu().numpy().view(np.uint16), r1, s1, 130, fmt=F16)["ok"]


def test_same_bits_as_bf16_path_on_common_integers():
    """Small integers are exact in both formats and the fp32 sums are exact,
    so the fp16 and bf16 paths' fp32 outputs agree exactly."""
    w = WORKLOADS["square512_int"]
    A16, B16 = w.make(fmt=F16)
    Ab, Bb = w.make(fmt="bf16")
    f = run_gemm(A16, B16, out_f32=True, fmt=F16)
    b = run_gemm(Ab, Bb, out_f32=True)
    assert np.array_equal(f, b)
