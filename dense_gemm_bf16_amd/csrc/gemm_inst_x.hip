// Kernel instantiations for the configurations tagged "x" in
// GEMM_TILE_CONFIGS (gemm_launch.hpp): the dispatch and the bf16 kernels
// with whole K-steps; the other variant groups are in gemm_inst_x1..x3.hip.
#define GEMM_X_OWN 0
#include "gemm_inst_x_split.hpp"
#define GEMM_INST_x GEMM_DO_INST
#include "gemm_inst_common.hpp"
