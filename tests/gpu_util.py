"""Helpers for the GPU tests: move bf16 (or fp16) bit arrays to the device,
call the library through its C ABI, bring results back.  Not collected by
pytest."""
from __future__ import annotations

import numpy as np


def dev_u16(x: np.ndarray):
    """uint16 bf16-bit array -> int16 device tensor with the same bytes."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
    return t.to("cuda", non_blocking=False)


NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00}


def _pad8(x: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """Pad rows to a multiple of 8 elements (the library's stride rule),
    filling the padding with NaN so any read of it shows."""
    ld = x.shape[1]
    if ld % 8 == 0 and ld > 0:
        return x
    ld8 = max(8, (ld + 7) // 8 * 8)
    out = np.full((x.shape[0], ld8), NAN_BITS[fmt], np.uint16)
    out[:, :ld] = x
    return out


def run_gemm(A: np.ndarray, B: np.ndarray, K: int | None = None, out_f32=False,
             config=None, ldc: int | None = None, canary=None, fmt: str = "bf16"):
    """C = A . B^T on the GPU via gemm_bf16_ex (gemm_f16_ex for
    fmt="f16").  A: M x lda, B: N x ldb (uint16 bit patterns, first K
    columns used).  Returns C as uint16 bits (or float32) of shape (M, ldc)
    when ldc/canary are given, else (M, N)."""
    import torch

    import dense_gemm_bf16_amd as g

    K = A.shape[1] if K is None else K
    A, B = _pad8(A, fmt), _pad8(B, fmt)
    M, lda = A.shape
    N, ldb = B.shape
    ldc_eff = N if ldc is None else ldc
    ldc_eff = max(8, (ldc_eff + 7) // 8 * 8)
    dA, dB = dev_u16(A), dev_u16(B)
    dtype = torch.float32 if out_f32 else torch.int16
    rows = M + (2 if canary is not None else 0)
    dC = torch.empty((max(rows, 1), ldc_eff), dtype=dtype, device="cuda")
    if canary is not None:
        dC.fill_(canary)
        c_view = dC[1:]
    else:
        c_view = dC
    fn = {"bf16": g.gemm_bf16_ex, "f16": g.gemm_f16_ex}[fmt]
    fn(config, M, N, K, dA, lda, dB, ldb, c_view, ldc_eff, out_f32)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    if not out_f32:
        out = out.view(np.uint16)
    if canary is not None or ldc is not None:
        return out
    return out[:M, :N]
