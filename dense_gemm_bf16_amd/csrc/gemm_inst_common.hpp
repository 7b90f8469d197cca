// Body of every gemm_inst_<tag>.hip file: instantiates launch_cfg for the
// rows of GEMM_TILE_CONFIGS (gemm_launch.hpp) whose TU tag is the including
// file's.  That file defines GEMM_INST_<tag> as GEMM_DO_INST before
// including this header; every other tag expands to nothing.
#pragma once

#include "gemm_launch.hpp"

#define GEMM_DO_INST(BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT)   \
  template hipError_t launch_cfg<BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT>( \
      const KernelArgs&, int, hipStream_t, int);
#define GEMM_NO_INST(BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT)

#ifndef GEMM_INST_big
#define GEMM_INST_big GEMM_NO_INST
#endif
#ifndef GEMM_INST_mid
#define GEMM_INST_mid GEMM_NO_INST
#endif
#ifndef GEMM_INST_mid128
#define GEMM_INST_mid128 GEMM_NO_INST
#endif
#ifndef GEMM_INST_smallm
#define GEMM_INST_smallm GEMM_NO_INST
#endif
#ifndef GEMM_INST_skinny
#define GEMM_INST_skinny GEMM_NO_INST
#endif
#ifndef GEMM_INST_midb1
#define GEMM_INST_midb1 GEMM_NO_INST
#endif
#ifndef GEMM_INST_midb2
#define GEMM_INST_midb2 GEMM_NO_INST
#endif
#ifndef GEMM_INST_big8
#define GEMM_INST_big8 GEMM_NO_INST
#endif
#ifndef GEMM_INST_big8b
#define GEMM_INST_big8b GEMM_NO_INST
#endif
#ifndef GEMM_INST_mid8
#define GEMM_INST_mid8 GEMM_NO_INST
#endif
#ifndef GEMM_INST_a
#define GEMM_INST_a GEMM_NO_INST
#endif
#ifndef GEMM_INST_b
#define GEMM_INST_b GEMM_NO_INST
#endif
#ifndef GEMM_INST_c
#define GEMM_INST_c GEMM_NO_INST
#endif
#ifndef GEMM_INST_d
#define GEMM_INST_d GEMM_NO_INST
#endif
#ifndef GEMM_INST_e
#define GEMM_INST_e GEMM_NO_INST
#endif
#ifndef GEMM_INST_f
#define GEMM_INST_f GEMM_NO_INST
#endif
#ifndef GEMM_INST_g
#define GEMM_INST_g GEMM_NO_INST
#endif
#ifndef GEMM_INST_h
#define GEMM_INST_h GEMM_NO_INST
#endif
#ifndef GEMM_INST_i
#define GEMM_INST_i GEMM_NO_INST
#endif
#ifndef GEMM_INST_j
#define GEMM_INST_j GEMM_NO_INST
#endif
#ifndef GEMM_INST_k
#define GEMM_INST_k GEMM_NO_INST
#endif
#ifndef GEMM_INST_l
#define GEMM_INST_l GEMM_NO_INST
#endif
#ifndef GEMM_INST_m
#define GEMM_INST_m GEMM_NO_INST
#endif
#ifndef GEMM_INST_n
#define GEMM_INST_n GEMM_NO_INST
#endif
#ifndef GEMM_INST_o
#define GEMM_INST_o GEMM_NO_INST
#endif
#ifndef GEMM_INST_p
#define GEMM_INST_p GEMM_NO_INST
#endif
#ifndef GEMM_INST_r
#define GEMM_INST_r GEMM_NO_INST
#endif
#ifndef GEMM_INST_s
#define GEMM_INST_s GEMM_NO_INST
#endif
#ifndef GEMM_INST_t
#define GEMM_INST_t GEMM_NO_INST
#endif
#ifndef GEMM_INST_v
#define GEMM_INST_v GEMM_NO_INST
#endif
#ifndef GEMM_INST_w
#define GEMM_INST_w GEMM_NO_INST
#endif

namespace gemm {
#define GEMM_INSTANTIATE(NAME, BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT, TU) \
  GEMM_INST_##TU(BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT)
GEMM_TILE_CONFIGS(GEMM_INSTANTIATE)
#undef GEMM_INSTANTIATE
}  // namespace gemm
