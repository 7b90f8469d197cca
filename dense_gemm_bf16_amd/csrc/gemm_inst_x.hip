// Kernel instantiations for the configurations tagged "x" in
// GEMM_TILE_CONFIGS (gemm_launch.hpp).
#define GEMM_INST_x GEMM_DO_INST
#include "gemm_inst_common.hpp"
