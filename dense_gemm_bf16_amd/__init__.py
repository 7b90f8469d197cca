"""Python binding of ``libgemm_bf16.so``, the MI355X dense bf16 GEMM.

    C[M,N] = A[M,K] . B[N,K]^T     bf16 in, fp32 accumulate, bf16 out
                                   (gemm_f16*: the same over fp16)

The functions here only marshal arguments (sizes, device pointers, a HIP
stream) to the C entry points of the same names declared in
``include/gemm_bf16.h``; every step of the product runs in the library's HIP
kernels.  PyTorch is used for device memory and streams only.  Importing
this package fails loudly if the library has not been built; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_bf16.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = 1
GEMM_ERR_MISALIGNED = 2
GEMM_ERR_UNSUPPORTED = 3
GEMM_ERR_HIP = 4
GEMM_ERR_CAPTURE = 5
GEMM_ERR_SCRATCH = 6
GEMM_NOALLOC_SCRATCH_BYTES = 64 << 20

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with dense_gemm_bf16_amd.build.build() "
        "(hipcc, gfx950).  There is no CPU fallback.")

# PyTorch ships its own copy of the HIP runtime (same soname).  If this
# library were loaded first, the process would end up with two HIP runtimes
# (ours resolved from /opt/rocm, torch's from its own directory), and device
# pointers and streams from one would be unknown to the other.  Loading torch
# first makes the dynamic loader reuse its runtime for this library too.
try:
    import torch  # noqa: F401
except ImportError:  # plain C-ABI use without torch: /opt/rocm's runtime
    pass

_lib = ctypes.CDLL(LIB_PATH)
_i64, _p = ctypes.c_int64, ctypes.c_void_p
_lib.gemm_bf16.restype = ctypes.c_int
_lib.gemm_bf16.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.gemm_bf16_f32out.restype = ctypes.c_int
_lib.gemm_bf16_f32out.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.gemm_bf16_ex.restype = ctypes.c_int
_lib.gemm_bf16_ex.argtypes = [ctypes.c_char_p, _i64, _i64, _i64, _p, _i64, _p, _i64,
                              _p, _i64, ctypes.c_int, _p]
_lib.gemm_bf16_config_name.restype = ctypes.c_char_p
_lib.gemm_bf16_config_name.argtypes = [_i64, _i64, _i64]
_lib.gemm_bf16_config_at.restype = ctypes.c_char_p
_lib.gemm_bf16_config_at.argtypes = [ctypes.c_int]
_lib.gemm_bf16_status_string.restype = ctypes.c_char_p
_lib.gemm_bf16_status_string.argtypes = [ctypes.c_int]
_lib.gemm_bf16_last_hip_error.restype = ctypes.c_int
_lib.gemm_bf16_last_hip_error.argtypes = []
_lib.gemm_bf16_reserve_workspace.restype = ctypes.c_int
_lib.gemm_bf16_reserve_workspace.argtypes = [ctypes.c_size_t, _p]
_lib.gemm_bf16_workspace_size.restype = ctypes.c_size_t
_lib.gemm_bf16_workspace_size.argtypes = [_i64, _i64, _i64]
_lib.gemm_bf16_release_workspace.restype = ctypes.c_int
_lib.gemm_bf16_release_workspace.argtypes = []
_lib.gemm_f16.restype = ctypes.c_int
_lib.gemm_f16.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.gemm_f16_f32out.restype = ctypes.c_int
_lib.gemm_f16_f32out.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.gemm_f16_ex.restype = ctypes.c_int
_lib.gemm_f16_ex.argtypes = [ctypes.c_char_p, _i64, _i64, _i64, _p, _i64, _p, _i64,
                             _p, _i64, ctypes.c_int, _p]
_lib.gemm_f16_config_at.restype = ctypes.c_char_p
_lib.gemm_f16_config_at.argtypes = [ctypes.c_int]
_lib.gemm_bf16_ex_noalloc.restype = ctypes.c_int
_lib.gemm_bf16_ex_noalloc.argtypes = [ctypes.c_char_p, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                      _p, _i64, ctypes.c_int, _p]


class GemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = status_string(status)
        if status == GEMM_ERR_HIP:
            msg += f" (hipError {last_hip_error()})"
        super().__init__(f"gemm_bf16 status {status}: {msg}")


def _ptr(x):
    """Device pointer of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    """hipStream_t of a torch stream (default: torch's current stream)."""
    if s is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int) -> None:
    if rc != GEMM_OK:
        raise GemmError(rc)


def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = A . B^T, bf16 output.  A, B, C: device tensors or addresses."""
    _check(_lib.gemm_bf16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                          _stream(stream)))


def gemm_bf16_f32out(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """Same product, fp32 sums stored unrounded in C (float32)."""
    _check(_lib.gemm_bf16_f32out(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                                 _stream(stream)))


def gemm_bf16_ex(config, M, N, K, A, lda, B, ldb, C, ldc, out_f32=False,
                 stream=None) -> None:
    """As gemm_bf16 with the kernel configuration named (None = automatic)."""
    cfg = None if config is None else config.encode()
    _check(_lib.gemm_bf16_ex(cfg, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                             1 if out_f32 else 0, _stream(stream)))


def gemm_f16(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = A . B^T over fp16 operands, fp16 output."""
    _check(_lib.gemm_f16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                         _stream(stream)))


def gemm_f16_f32out(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """fp16 operands, fp32 sums stored unrounded in C (float32)."""
    _check(_lib.gemm_f16_f32out(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                                _stream(stream)))


def gemm_f16_ex(config, M, N, K, A, lda, B, ldb, C, ldc, out_f32=False,
                stream=None) -> None:
    """As gemm_f16 with the kernel configuration named (None = automatic)."""
    cfg = None if config is None else config.encode()
    _check(_lib.gemm_f16_ex(cfg, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                            1 if out_f32 else 0, _stream(stream)))


def gemm_bf16_ex_noalloc(config, M, N, K, A, lda, B, ldb, C, ldc, out_f32=False,
                         stream=None) -> None:
    """As gemm_bf16_ex, with the split-K partials in the library's static
    scratch array instead of an allocated workspace (nothing is allocated)."""
    cfg = None if config is None else config.encode()
    _check(_lib.gemm_bf16_ex_noalloc(cfg, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                                     1 if out_f32 else 0, _stream(stream)))


def gemm_bf16_status(M, N, K, A, lda, B, ldb, C, ldc, stream=0, out_f32=False,
                     config=None, half=False) -> int:
    """Raw status code of one call (for tests of argument checking);
    ``half`` calls gemm_f16_ex instead of gemm_bf16_ex."""
    cfg = None if config is None else config.encode()
    fn = _lib.gemm_f16_ex if half else _lib.gemm_bf16_ex
    return int(fn(cfg, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                  1 if out_f32 else 0, stream))


def config_name(M, N, K) -> str:
    return _lib.gemm_bf16_config_name(M, N, K).decode()


def config_at(i: int):
    """The i-th built configuration name, or None past the end."""
    n = _lib.gemm_bf16_config_at(i)
    return None if n is None else n.decode()


def config_names() -> list[str]:
    out = []
    while (n := config_at(len(out))) is not None:
        out.append(n)
    return out


def f16_config_at(i: int):
    """The i-th configuration built for fp16 operands, or None past the end."""
    n = _lib.gemm_f16_config_at(i)
    return None if n is None else n.decode()


def f16_config_names() -> list[str]:
    out = []
    while (n := f16_config_at(len(out))) is not None:
        out.append(n)
    return out


def status_string(status: int) -> str:
    return _lib.gemm_bf16_status_string(status).decode()


def last_hip_error() -> int:
    return int(_lib.gemm_bf16_last_hip_error())


def reserve_workspace(nbytes: int, stream=None) -> None:
    _check(_lib.gemm_bf16_reserve_workspace(nbytes, _stream(stream)))


def workspace_size(M, N, K) -> int:
    return int(_lib.gemm_bf16_workspace_size(M, N, K))


def release_workspace() -> None:
    _check(_lib.gemm_bf16_release_workspace())


# The C names, for callers who prefer them.
gemm_bf16_config_name = config_name
gemm_bf16_config_at = config_at
gemm_bf16_status_string = status_string
gemm_bf16_last_hip_error = last_hip_error
gemm_bf16_reserve_workspace = reserve_workspace
gemm_bf16_workspace_size = workspace_size
gemm_bf16_release_workspace = release_workspace
gemm_f16_config_at = f16_config_at


def _row_stride(t, rows, cols):
    """Leading dimension to pass for a 2-D tensor: its row stride, or for a
    single row (whose stride is never used) the row length rounded up to 8."""
    return t.stride(0) if rows > 1 else max(8, (cols + 7) // 8 * 8)


def matmul(A, B, out=None, out_f32=False, config=None, stream=None):
    """Convenience form on torch tensors: A (M x K, rows contiguous), B (N x K,
    rows contiguous), both bfloat16 or both float16 on the GPU; returns C
    (M x N) of the same type, or float32 with ``out_f32``."""
    import torch

    if A.dtype != B.dtype or A.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("A and B must both be torch.bfloat16 or both torch.float16")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("need A (M x K) and B (N x K)")
    if A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("rows of A and B must be contiguous")
    M, K = A.shape
    N = B.shape[0]
    out_dtype = torch.float32 if out_f32 else A.dtype
    if out is None:
        out = torch.empty((M, N), device=A.device, dtype=out_dtype)
    if out.dtype != out_dtype or out.dim() != 2 or tuple(out.shape) != (M, N):
        raise ValueError(f"out must be a {M} x {N} {out_dtype} tensor")
    if out.stride(1) != 1:
        raise ValueError("rows of C must be contiguous")
    lda = _row_stride(A, M, K)
    ldb = _row_stride(B, N, K)
    ldc = _row_stride(out, M, N)
    fn = gemm_f16_ex if A.dtype == torch.float16 else gemm_bf16_ex
    fn(config, M, N, K, A, lda, B, ldb, out, ldc, out_f32, stream)
    return out
