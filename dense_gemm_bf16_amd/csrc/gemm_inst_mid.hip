// Kernel instantiations of the 256 x 128 direct-to-LDS tile ("mid" in GEMM_TILE_CONFIGS):
// bf16 operands, whole K-steps; also the dispatch.
#define GEMM_SPLIT_PARAMS GEMM_MID_PARAMS
#define GEMM_SPLIT_STREAM
#define GEMM_SPLIT_OWN 0
#include "gemm_inst_split.hpp"
#define GEMM_INST_mid GEMM_DO_INST
#include "gemm_inst_common.hpp"
