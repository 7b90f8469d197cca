// The bf16 kernels for K % 64 != 0 of the "x" configuration of
// GEMM_TILE_CONFIGS (split from gemm_inst_x.hip to shorten the build).
#define GEMM_X_OWN 16
#include "gemm_inst_x_split.hpp"
