// Ablation build only: kernel instantiations of the 256 x 256 direct-to-LDS tile on 8 waves (2 x 4) ("big8" in GEMM_TILE_CONFIGS).
#define GEMM_INST_big8 GEMM_DO_INST
#include "gemm_inst_common.hpp"
