// Launcher template for one tile configuration: maps the run-time variant
// flags (kOutF32 | kSplitK | kRaggedK | kF16 | kPartialK | kPersistent |
// kStreamB) to the instantiated kernels.  Each
// gemm_inst_*.hip file instantiates it for its configurations, so the
// configurations compile in parallel.
#pragma once

#include "gemm_dtl.hpp"
#include "gemm_kernel.hpp"
#include "gemm_wavek.hpp"
#ifdef GEMM_WITH_ABLATION
#include "ablation/gemm_pingpong.hpp"
#include "ablation/gemm_regstage.hpp"
#endif

namespace gemm {

// PIPE 0 / 1 / 3 / 4: gemm_bf16_kernel with burst / spread load issue;
// PIPE 2 / 5: gemm_bf16_pingpong_kernel (8 waves as 2 x 4) with the
// thread-strided / wave-contiguous dealing of loads;
// PIPE 6: gemm_bf16_regstage_kernel (loads staged through ST register
// buffers, two LDS slots);
// PIPE 8 / 10: gemm_bf16_dtl_kernel (LDS-DMA straight into an ST-slot ring)
// with 32x32x16 / 16x16x32 MFMAs; PIPE 11 / 12: PIPE 10 with B loaded 1 / 2
// K-steps ahead of A in 1 / 2 more B slots;
// PIPE 9: gemm_bf16_wavek_kernel (small M: four waves split each K-step of
// one BM x 32 block; WM = WN = 1 name the block, 256 threads run it).
template <int BM, int BN, int BK, int WM, int WN, int ST, int SWZ, int PIPE, int FLAGS>
hipError_t launch_one(const KernelArgs& a, int grid, hipStream_t s) {
#ifdef GEMM_WITH_ABLATION
  if constexpr (PIPE == 2 || PIPE == 5) {
    static_assert(WM == 2 && WN == 4, "ping-pong runs 2 x 4 waves");
    hipLaunchKernelGGL((gemm_bf16_pingpong_kernel<BM, BN, BK, ST, SWZ, FLAGS, PIPE == 5>),
                       dim3(grid), dim3(512), 0, s, a);
  } else if constexpr (PIPE == 6) {
    hipLaunchKernelGGL((gemm_bf16_regstage_kernel<BM, BN, BK, WM, WN, ST, SWZ, FLAGS>),
                       dim3(grid), dim3(WM * WN * 64), 0, s, a);
  } else
#endif
  if constexpr (PIPE == 8 || PIPE == 10 || PIPE == 11 || PIPE == 12) {
    hipLaunchKernelGGL((gemm_bf16_dtl_kernel<BM, BN, BK, WM, WN, ST, SWZ, FLAGS,
                                             PIPE == 8 ? 32 : 16, PIPE >= 11 ? PIPE - 10 : 0>),
                       dim3(grid), dim3(WM * WN * 64), 0, s, a);
  } else if constexpr (PIPE == 9) {
    static_assert(WM == 1 && WN == 1, "one block per workgroup");
    hipLaunchKernelGGL((gemm_bf16_wavek_kernel<BM, BN, BK, ST, SWZ, FLAGS>), dim3(grid), dim3(256),
                       0, s, a);
  } else {
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, ST, SWZ, PIPE, FLAGS>), dim3(grid),
                       dim3(WM * WN * 64), 0, s, a);
  }
  return hipGetLastError();
}

// LDS bytes a configuration's kernel allocates.
template <int BM, int BN, int BK, int WM, int WN, int ST, int SWZ, int PIPE>
constexpr int lds_bytes_of() {
  using C = TileCfg<BM, BN, BK, WM, WN, PIPE == 6 ? 2 : ST, SWZ>;
  return C::kLdsBytes + (PIPE >= 11 ? (PIPE - 10) * C::kBBytes : 0);
}

// Kernels with a separate K % BK != 0 variant: direct-to-LDS and small M.
constexpr bool has_partial_variant(int pipe) { return pipe >= 8 && pipe <= 12; }

// The (kOutF32, kSplitK, kRaggedK) combinations that occur, with the fixed
// bits E (kF16, kPartialK).
// A persistent grid has only the bf16-output kernels: it never splits K,
// and the fp32 debug output of a persistent plan comes from the ordinary
// kernel (same tiles, same per-tile K order, so the same sums).
template <int BM, int BN, int BK, int WM, int WN, int ST, int SWZ, int PIPE, int E>
hipError_t launch_variant(const KernelArgs& a, int grid, hipStream_t s, int flags) {
  if constexpr ((E & kPersistent) != 0) {
    switch (flags & 7) {
      case 0: return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 0>(a, grid, s);
      case 4:
        if constexpr ((E & kPartialK) != 0)
          return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 4>(a, grid, s);
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (flags & 7) {
      case 0: return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 0>(a, grid, s);
      case 1: return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 1>(a, grid, s);
      case 2: return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 2>(a, grid, s);
      default: break;
    }
    // K % 8 != 0 (the direct-to-LDS and small-M kernels handle it only in
    // their K % BK != 0 variant, which every such K selects)
    if constexpr (!has_partial_variant(PIPE) || (E & kPartialK) != 0) {
      switch (flags & 7) {
        case 4: return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 4>(a, grid, s);
        case 5: return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 5>(a, grid, s);
        default: return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | 6>(a, grid, s);
      }
    }
    return hipErrorInvalidValue;
  }
}

// Operand type E (0 or kF16, with kPersistent for a persistent grid) and,
// for the direct-to-LDS and small-M kernels, kPartialK.
template <int BM, int BN, int BK, int WM, int WN, int ST, int SWZ, int PIPE, int E>
hipError_t launch_partial(const KernelArgs& a, int grid, hipStream_t s, int flags) {
  if constexpr (has_partial_variant(PIPE)) {
    if (flags & (kPartialK | kRaggedK))
      return launch_variant<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | kPartialK>(a, grid, s, flags);
  }
  return launch_variant<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E>(a, grid, s, flags);
}

// What a configuration row builds beyond the bf16 kernels (its OPT mask).
enum : int {
  kOptF16 = 1,      // the fp16-operand kernels
  kOptPersist = 2,  // the persistent-grid kernels, bf16 operands (direct-to-LDS only)
  kOptStream = 4,   // kernels with non-temporal B loads (kStreamB): whole K-steps,
                    // 16-bit output, plain and split
};

// The kStreamB kernels of operand type E (0 or kF16): 16-bit output or split
// K (flags & 7 is 0 or kSplitK; the caller has checked).
template <int BM, int BN, int BK, int WM, int WN, int ST, int SWZ, int PIPE, int E>
hipError_t launch_stream(const KernelArgs& a, int grid, hipStream_t s, int flags) {
  if (flags & kSplitK)
    return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | kStreamB | kSplitK>(a, grid, s);
  return launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E | kStreamB>(a, grid, s);
}

template <int BM, int BN, int BK, int WM, int WN, int ST, int SWZ, int PIPE, int OPT>
hipError_t launch_cfg(const KernelArgs& a, int grid, hipStream_t s, int flags) {
  if (flags & kSplitK) flags &= ~kOutF32;  // split slices always write fp32 partials
  if (flags & kStreamB) {
    flags &= ~kStreamB;
    // Where no such kernel is built (fp32 output, a K that is not a whole
    // number of K-steps, a persistent grid, or a row without kOptStream)
    // the ordinary kernel runs: the loads' cache policy changes no result.
    if constexpr ((OPT & kOptStream) != 0) {
      if ((flags & (kOutF32 | kRaggedK | kPartialK | kPersistent)) == 0) {
        if ((flags & kF16) == 0)
          return launch_stream<BM, BN, BK, WM, WN, ST, SWZ, PIPE, 0>(a, grid, s, flags);
        if constexpr ((OPT & kOptF16) != 0)
          return launch_stream<BM, BN, BK, WM, WN, ST, SWZ, PIPE, kF16>(a, grid, s, flags);
      }
    }
  }
  if (flags & kPersistent) {
    if constexpr ((OPT & kOptPersist) != 0) {
      static_assert(PIPE == 8 || PIPE == 10, "only the direct-to-LDS kernel without B lead walks tiles");
      if ((flags & (kF16 | kSplitK | kOutF32)) == 0)
        return launch_partial<BM, BN, BK, WM, WN, ST, SWZ, PIPE, kPersistent>(a, grid, s, flags);
    }
    return hipErrorInvalidValue;
  }
  if (flags & kF16) {
    if constexpr ((OPT & kOptF16) != 0)
      return launch_partial<BM, BN, BK, WM, WN, ST, SWZ, PIPE, kF16>(a, grid, s, flags);
    else
      return hipErrorInvalidValue;
  }
  return launch_partial<BM, BN, BK, WM, WN, ST, SWZ, PIPE, 0>(a, grid, s, flags);
}

// Built configurations, one row each:
//   X(name, BM, BN, BK, WAVES_M, WAVES_N, STAGES, SWZ, PIPE, OPT, TU)
// where OPT is a mask of kOptF16 (also build the row for fp16 operands),
// kOptPersist (also build its persistent-grid kernels) and kOptStream (also
// build its kernels with non-temporal B loads), and TU names the
// gemm_inst_<TU>.hip file that instantiates it.  A row whose parameters
// are also needed elsewhere (the files that split its kernel variants over
// several translation units) takes them from a GEMM_*_PARAMS macro, through
// GEMM_ROW so the macro expands into separate arguments.
//
// The product set is every configuration the plan choice (tuned table,
// cost model, rules) can pick:
//   big     256 x 256 direct-to-LDS, 16x16x32 MFMAs (4096^3, prefill)
//   mid     256 x 128 direct-to-LDS, three ring slots (M = 256 decode)
//   mid128  128 x 128 direct-to-LDS, four ring slots (M = 512 class)
//   smallm  BM x 32 strips with the waves splitting K (M <= 48)
//   skinny  32 / 64 x 128 LDS-DMA burst tiles (other M <= 64)
#define GEMM_ROW(X, ...) X(__VA_ARGS__)
#define GEMM_BIG_PARAMS 256, 256, 64, 2, 2, 2, 3, 10
#define GEMM_MID_PARAMS 256, 128, 64, 2, 2, 3, 3, 10
#define GEMM_PRODUCT_CONFIGS(X)                                        \
  GEMM_ROW(X, t256x256x64_w2x2_s2_x3_p10, GEMM_BIG_PARAMS, 3, big)     \
  GEMM_ROW(X, t256x128x64_w2x2_s3_x3_p10, GEMM_MID_PARAMS, 5, mid)     \
  X(t128x128x64_w2x2_s4_x3_p10, 128, 128, 64, 2, 2, 4, 3, 10, 1, mid128) \
  X(t32x32x64_w1x1_s8_x2_p9, 32, 32, 64, 1, 1, 8, 2, 9, 5, smallm)     \
  X(t64x32x64_w1x1_s6_x2_p9, 64, 32, 64, 1, 1, 6, 2, 9, 5, smallm)     \
  X(t64x128x64_w1x4_s6_x2_p0, 64, 128, 64, 1, 4, 6, 2, 0, 5, skinny)   \
  X(t32x128x64_w1x4_s6_x2_p0, 32, 128, 64, 1, 4, 6, 2, 0, 5, skinny)

// The ablation set (built only with GEMM_WITH_ABLATION, by
// build(ablation=True)): the other kernel families and layouts that the
// measurements behind the product choices compared against -- LDS-DMA
// spread issue (PIPE 1, 3, 4), ping-pong (2, 5), register-staged (6), the
// 32x32x16 forms of the direct-to-LDS tiles (8), the unswizzled and
// row-mod-8 LDS layouts (x0, x1), the direct-to-LDS tiles on 8 waves (two
// per SIMD: 256 x 256 as 2 x 4 or 4 x 2 waves, 256 x 128 as 4 x 2), and the
// 256 x 128 tile with B one or two K-steps ahead of A (PIPE 11, 12).
#ifdef GEMM_WITH_ABLATION
#define GEMM_ABLATION_CONFIGS(X)                                  \
  X(t256x256x64_w2x2_s2_x2_p0, 256, 256, 64, 2, 2, 2, 2, 0, 0, a) \
  X(t256x256x64_w2x2_s2_x2_p3, 256, 256, 64, 2, 2, 2, 2, 3, 0, b) \
  X(t256x256x64_w2x2_s2_x2_p4, 256, 256, 64, 2, 2, 2, 2, 4, 0, c) \
  X(t256x256x64_w2x2_s2_x2_p1, 256, 256, 64, 2, 2, 2, 2, 1, 1, d) \
  X(t256x256x64_w2x4_s2_x2_p3, 256, 256, 64, 2, 4, 2, 2, 3, 0, e) \
  X(t256x256x64_w2x4_s2_x2_p1, 256, 256, 64, 2, 4, 2, 2, 1, 0, f) \
  X(t256x256x32_w2x4_s4_x2_p2, 256, 256, 32, 2, 4, 4, 2, 2, 0, g) \
  X(t256x256x32_w2x4_s4_x2_p5, 256, 256, 32, 2, 4, 4, 2, 5, 1, l) \
  X(t256x256x32_w2x2_s3_x2_p6, 256, 256, 32, 2, 2, 3, 2, 6, 0, m) \
  X(t256x256x32_w2x2_s4_x2_p6, 256, 256, 32, 2, 2, 4, 2, 6, 0, n) \
  X(t256x256x64_w2x2_s2_x2_p6, 256, 256, 64, 2, 2, 2, 2, 6, 1, o) \
  X(t256x128x64_w2x2_s3_x2_p1, 256, 128, 64, 2, 2, 3, 2, 1, 0, h) \
  X(t256x128x64_w2x2_s2_x2_p3, 256, 128, 64, 2, 2, 2, 2, 3, 0, k) \
  X(t128x128x64_w2x2_s4_x2_p1, 128, 128, 64, 2, 2, 4, 2, 1, 0, i) \
  X(t64x256x64_w1x4_s4_x2_p0, 64, 256, 64, 1, 4, 4, 2, 0, 0, p)   \
  X(t32x256x64_w1x4_s4_x2_p0, 32, 256, 64, 1, 4, 4, 2, 0, 0, p)   \
  X(t64x256x64_w1x4_s4_x2_p6, 64, 256, 64, 1, 4, 4, 2, 6, 0, r)   \
  X(t32x256x64_w1x4_s4_x2_p6, 32, 256, 64, 1, 4, 4, 2, 6, 0, r)   \
  X(t256x128x64_w2x2_s2_x2_p6, 256, 128, 64, 2, 2, 2, 2, 6, 1, s) \
  X(t128x256x64_w2x2_s2_x2_p6, 128, 256, 64, 2, 2, 2, 2, 6, 1, s) \
  X(t256x256x64_w2x2_s2_x2_p8, 256, 256, 64, 2, 2, 2, 2, 8, 1, t) \
  X(t256x128x64_w2x2_s3_x2_p8, 256, 128, 64, 2, 2, 3, 2, 8, 1, v) \
  X(t128x128x64_w2x2_s4_x2_p8, 128, 128, 64, 2, 2, 4, 2, 8, 1, w) \
  X(t256x256x64_w2x2_s2_x0_p0, 256, 256, 64, 2, 2, 2, 0, 0, 0, j) \
  X(t256x256x64_w2x2_s2_x1_p0, 256, 256, 64, 2, 2, 2, 1, 0, 0, j) \
  X(t256x256x64_w2x4_s2_x3_p10, 256, 256, 64, 2, 4, 2, 3, 10, 0, big8)   \
  X(t256x256x64_w4x2_s2_x3_p10, 256, 256, 64, 4, 2, 2, 3, 10, 0, big8b)  \
  X(t256x128x64_w4x2_s3_x3_p10, 256, 128, 64, 4, 2, 3, 3, 10, 0, mid8)   \
  X(t256x128x64_w2x2_s3_x3_p11, 256, 128, 64, 2, 2, 3, 3, 11, 0, midb1)   \
  X(t256x128x64_w2x2_s2_x3_p12, 256, 128, 64, 2, 2, 2, 3, 12, 0, midb2)
#else
#define GEMM_ABLATION_CONFIGS(X)
#endif

#define GEMM_TILE_CONFIGS(X) GEMM_PRODUCT_CONFIGS(X) GEMM_ABLATION_CONFIGS(X)

#define GEMM_DECLARE_LAUNCH(NAME, BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT, TU) \
  extern template hipError_t launch_cfg<BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT>(  \
      const KernelArgs&, int, hipStream_t, int);
GEMM_TILE_CONFIGS(GEMM_DECLARE_LAUNCH)
#undef GEMM_DECLARE_LAUNCH

}  // namespace gemm
