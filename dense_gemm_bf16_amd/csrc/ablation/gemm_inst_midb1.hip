// Ablation build only: kernel instantiations of the 256 x 128 direct-to-LDS tile with B one K-step ahead ("midb1" in GEMM_TILE_CONFIGS).
#define GEMM_INST_midb1 GEMM_DO_INST
#include "gemm_inst_common.hpp"
