// Kernel instantiations of the 256 x 256 direct-to-LDS tile ("big" in GEMM_TILE_CONFIGS):
// bf16 operands, whole K-steps; also the dispatch.
#define GEMM_SPLIT_PARAMS GEMM_BIG_PARAMS
#define GEMM_SPLIT_RAGGED_APART
#define GEMM_SPLIT_PERSIST
#define GEMM_SPLIT_OWN 0
#include "gemm_inst_split.hpp"
#define GEMM_INST_big GEMM_DO_INST
#include "gemm_inst_common.hpp"
