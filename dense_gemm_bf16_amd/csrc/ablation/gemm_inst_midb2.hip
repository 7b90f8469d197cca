// Ablation build only: kernel instantiations of the 256 x 128 direct-to-LDS tile with B two K-steps ahead ("midb2" in GEMM_TILE_CONFIGS).
#define GEMM_INST_midb2 GEMM_DO_INST
#include "gemm_inst_common.hpp"
