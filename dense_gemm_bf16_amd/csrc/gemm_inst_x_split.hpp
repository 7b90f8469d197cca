// The "x" configuration (256x256x64 tile, 2x2 waves, two ring slots, the
// direct-to-LDS kernel on 16x16x32 MFMAs) has the most kernel variants of
// any row of GEMM_TILE_CONFIGS: two operand types times the K % BK tail
// variant times up to six flag combinations.  Compiled in one file they take
// most of a full build, so each (operand type, K-tail) group is instantiated
// in a file of its own, named by GEMM_X_OWN = its kF16 | kPartialK bits:
// gemm_inst_x.hip (0) also holds the dispatch, gemm_inst_x1.hip (16),
// gemm_inst_x2.hip (8) and gemm_inst_x3.hip (24) the other three groups.
// Every other file sees all four as extern.  The parameters below must match
// the "x" row of GEMM_TILE_CONFIGS.
#pragma once

#include "gemm_launch.hpp"

#ifndef GEMM_X_OWN
#define GEMM_X_OWN (-1)
#endif

#define GEMM_X_VARIANT(E)                                                \
  template hipError_t launch_variant<256, 256, 64, 2, 2, 2, 3, 10, E>( \
      const KernelArgs&, int, hipStream_t, int);

namespace gemm {
static_assert(kF16 == 8 && kPartialK == 16, "GEMM_X_OWN numbers the groups by these bits");
#if GEMM_X_OWN == 0
GEMM_X_VARIANT(0)
#else
extern GEMM_X_VARIANT(0)
#endif
#if GEMM_X_OWN == 16
GEMM_X_VARIANT(16)
#else
extern GEMM_X_VARIANT(16)
#endif
#if GEMM_X_OWN == 8
GEMM_X_VARIANT(8)
#else
extern GEMM_X_VARIANT(8)
#endif
#if GEMM_X_OWN == 24
GEMM_X_VARIANT(24)
#else
extern GEMM_X_VARIANT(24)
#endif
}  // namespace gemm
