// Ablation build only: kernel instantiations of the 256 x 128 direct-to-LDS tile on 8 waves ("mid8" in GEMM_TILE_CONFIGS).
#define GEMM_INST_mid8 GEMM_DO_INST
#include "gemm_inst_common.hpp"
