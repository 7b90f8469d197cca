// Split-K reduction:  C[m][n] = sum_{s=0}^{S-1} P_s[m][n], added in the fixed
// order s = 0, 1, ..., S-1 in fp32, then rounded once to bf16 or fp16
// (round to nearest even) or stored as fp32.  P_s are the unrounded partial products
// of the K-slices written by the GEMM kernel; because the order never
// changes, the result is bitwise reproducible and independent of which
// slice finished first.
//
// Memory-bound and elementwise: each thread owns 8 consecutive columns of
// one row (two 16-byte loads per slice, one 16-byte 16-bit store), so every
// access is a coalesced 16-byte vector access.
#include "gemm_internal.h"

namespace gemm {
namespace {

template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P,
                                                            int64_t ldp, int64_t slice_stride,
                                                            int S, void* __restrict__ C,
                                                            int64_t ldc, int M, int N) {
  const int chunks = (N + 7) >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * chunks) return;
  const int m = (int)(idx / chunks);
  const int n = (int)(idx - (int64_t)m * chunks) * 8;
  const float* p = P + (int64_t)m * ldp + n;
  float v[8];
  if (n + 8 <= N) {
    f32x4 lo = *(const f32x4*)p, hi = *(const f32x4*)(p + 4);
    for (int s = 1; s < S; ++s) {
      const float* q = p + (int64_t)s * slice_stride;
      lo += *(const f32x4*)q;
      hi += *(const f32x4*)(q + 4);
    }
    for (int j = 0; j < 4; ++j) {
      v[j] = lo[j];
      v[4 + j] = hi[j];
    }
  } else {
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    for (int j = 0; j < 8 && n + j < N; ++j) {
      float acc = p[j];
      for (int s = 1; s < S; ++s) acc += p[(int64_t)s * slice_stride + j];
      v[j] = acc;
    }
  }
  if constexpr (OUT == kStoreF32) {
    float* c = (float*)C + (int64_t)m * ldc + n;
    if (n + 8 <= N) {
      *(f32x4*)c = (f32x4){v[0], v[1], v[2], v[3]};
      *(f32x4*)(c + 4) = (f32x4){v[4], v[5], v[6], v[7]};
    } else {
      for (int j = 0; j < 8 && n + j < N; ++j) c[j] = v[j];
    }
  } else {
    // T: __bf16 or _Float16; the conversion rounds to nearest even
    using T = std::conditional_t<OUT == kStoreF16, _Float16, __bf16>;
    typedef T t2 __attribute__((ext_vector_type(2)));
    typedef T t8 __attribute__((ext_vector_type(8)));
    T* c = (T*)C + (int64_t)m * ldc + n;
    t2 r[4];
    for (int j = 0; j < 4; ++j)
      r[j] = __builtin_convertvector((f32x2){v[2 * j], v[2 * j + 1]}, t2);
    if (n + 8 <= N) {
      *(t8*)c = (t8){r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    } else {
      for (int j = 0; j < 8 && n + j < N; ++j) c[j] = r[j >> 1][j & 1];
    }
  }
}

}  // namespace

hipError_t launch_splitk_reduce(const float* P, int64_t ldp, int64_t slice_stride, int S,
                                void* C, int64_t ldc, int M, int N, int out_kind,
                                hipStream_t stream) {
  const int64_t items = (int64_t)M * ((N + 7) / 8);
  const int64_t blocks = (items + 255) / 256;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  switch (out_kind) {
    case kStoreF32:
      hipLaunchKernelGGL(splitk_reduce_kernel<kStoreF32>, grid, block, 0, stream, P, ldp,
                         slice_stride, S, C, ldc, M, N);
      break;
    case kStoreF16:
      hipLaunchKernelGGL(splitk_reduce_kernel<kStoreF16>, grid, block, 0, stream, P, ldp,
                         slice_stride, S, C, ldc, M, N);
      break;
    case kStoreBf16:
      hipLaunchKernelGGL(splitk_reduce_kernel<kStoreBf16>, grid, block, 0, stream, P, ldp,
                         slice_stride, S, C, ldc, M, N);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gemm
