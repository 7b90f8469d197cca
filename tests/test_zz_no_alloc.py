"""The no-allocation entry point, gemm_bf16_ex_noalloc, through the C ABI,
against the existing gemm_bf16_ex on the same inputs: same plan and
summation order, so the same bits (bf16 and fp32 output), on two calls in a
row whose second is smaller (the static scratch keeps the first call's
partials, which the second must not read), and both against the oracle.
A plan whose partials exceed the scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest

from oracle.compare import check_bf16, check_f32
from synthetic_inputs import WORKLOADS, int_bf16

pytestmark = pytest.mark.gpu


def _call(fn, config, A, B, K, out_f32):
    import torch

    M, N = A.shape[0], B.shape[0]
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    dC = torch.full((M, N), -1, dtype=torch.float32 if out_f32 else torch.int16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    cfg = None if config is None else config.encode()
    rc = fn(cfg, M, N, K, ctypes.c_void_p(dA.data_ptr()), A.shape[1],
            ctypes.c_void_p(dB.data_ptr()), B.shape[1], ctypes.c_void_p(dC.data_ptr()), N,
            1 if out_f32 else 0, ctypes.c_void_p(s))
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    return rc, (out if out_f32 else out.view(np.uint16))


def test_noalloc_matches_gemm_bf16_ex_on_two_calls():
    import dense_gemm_bf16_amd as g
    import oracle

    so = g._lib
    # call 1: decode attention-out, split K (32 MiB of partials)
    w = WORKLOADS["decode_attn_out"]
    A, B = w.make()
    plan = g.config_name(w.M, w.N, w.K)
    assert "_k1_" not in plan, plan
    print("call 1", (w.M, w.N, w.K), plan, flush=True)
    rc, got = _call(so.gemm_bf16_ex_noalloc, None, A, B, w.K, False)
    assert rc == g.GEMM_OK, g.status_string(rc)
    rc, ref = _call(so.gemm_bf16_ex, None, A, B, w.K, False)
    assert rc == g.GEMM_OK
    assert np.array_equal(got, ref)
    r16, r64 = oracle.gemm(A, B)
    rep = check_bf16(got, r16, r64, w.K, w.sigma_a, w.sigma_b)
    print("call 1 vs oracle", rep, flush=True)
    assert rep["ok"], rep

    # call 2: smaller, split K again, integer inputs (exact), fp32 and bf16
    M, N, K = 200, 4096, 2048
    A2 = int_bf16(M, K, seed=1201)
    B2 = int_bf16(N, K, seed=1202)
    plan2 = g.config_name(M, N, K)
    assert "_k1_" not in plan2, plan2
    print("call 2", (M, N, K), plan2, flush=True)
    r16, r64 = oracle.gemm(A2, B2)
    for out_f32 in (True, False):
        rc, got = _call(so.gemm_bf16_ex_noalloc, None, A2, B2, K, out_f32)
        assert rc == g.GEMM_OK, g.status_string(rc)
        rc, ref = _call(so.gemm_bf16_ex, None, A2, B2, K, out_f32)
        assert rc == g.GEMM_OK
        assert np.array_equal(got, ref), out_f32
        if out_f32:
            assert check_f32(got, r64, K, exact=True)["ok"]
        else:
            assert check_bf16(got, r16, None, K, exact=True)["ok"]

    # a forced plan that fits, and one whose partials do not
    cfg = "t256x128x64_w2x2_s3_x3_p10_k8"
    rc, got = _call(so.gemm_bf16_ex_noalloc, cfg, A2, B2, K, False)
    assert rc == g.GEMM_OK
    assert check_bf16(got, r16, None, K, exact=True)["ok"]
    big = "t256x128x64_w2x2_s3_x3_p10_k16"
    A3 = int_bf16(256, 8192, seed=1203)
    B3 = int_bf16(8192, 8192, seed=1204)
    rc, got = _call(so.gemm_bf16_ex_noalloc, big, A3, B3, 8192, False)
    assert rc == g.GEMM_ERR_SCRATCH
    assert np.all(got == 0xFFFF)  # nothing was written
