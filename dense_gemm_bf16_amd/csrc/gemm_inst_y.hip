// Kernel instantiations for the configurations tagged "y" in
// GEMM_TILE_CONFIGS (gemm_launch.hpp).
#define GEMM_INST_y GEMM_DO_INST
#include "gemm_inst_common.hpp"
