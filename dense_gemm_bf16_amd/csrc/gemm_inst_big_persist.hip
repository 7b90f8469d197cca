// Kernel instantiations of the 256 x 256 direct-to-LDS tile ("big" in GEMM_TILE_CONFIGS):
// the persistent-grid kernels, bf16 operands and output, whole K-steps.
#define GEMM_SPLIT_PARAMS GEMM_BIG_PARAMS
#define GEMM_SPLIT_RAGGED_APART
#define GEMM_SPLIT_PERSIST
#define GEMM_SPLIT_OWN 32
#include "gemm_inst_split.hpp"
