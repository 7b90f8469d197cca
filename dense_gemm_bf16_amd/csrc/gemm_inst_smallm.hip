// Kernel instantiations of the small-M strip kernels ("smallm" in GEMM_TILE_CONFIGS).
#define GEMM_INST_smallm GEMM_DO_INST
#include "gemm_inst_common.hpp"
