// Ablation build only: kernel instantiations of the 256 x 256 direct-to-LDS tile on 8 waves (4 x 2) ("big8b" in GEMM_TILE_CONFIGS).
#define GEMM_INST_big8b GEMM_DO_INST
#include "gemm_inst_common.hpp"
