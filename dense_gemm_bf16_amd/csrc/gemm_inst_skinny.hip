// Kernel instantiations of the 32 / 64 x 128 LDS-DMA burst tiles ("skinny" in GEMM_TILE_CONFIGS).
#define GEMM_INST_skinny GEMM_DO_INST
#include "gemm_inst_common.hpp"
