// Kernel instantiations of the 256 x 256 direct-to-LDS tile ("big" in GEMM_TILE_CONFIGS):
// fp16 operands, whole K-steps.
#define GEMM_SPLIT_PARAMS GEMM_BIG_PARAMS
#define GEMM_SPLIT_RAGGED_APART
#define GEMM_SPLIT_PERSIST
#define GEMM_SPLIT_OWN 8
#include "gemm_inst_split.hpp"
