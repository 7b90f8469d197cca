// Kernel instantiations of the 128 x 128 direct-to-LDS tile ("mid128" in GEMM_TILE_CONFIGS).
#define GEMM_INST_mid128 GEMM_DO_INST
#include "gemm_inst_common.hpp"
