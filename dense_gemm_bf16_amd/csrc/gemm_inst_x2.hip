// The fp16 kernels with whole K-steps of the "x" configuration of
// GEMM_TILE_CONFIGS (split from gemm_inst_x.hip to shorten the build).
#define GEMM_X_OWN 8
#include "gemm_inst_x_split.hpp"
