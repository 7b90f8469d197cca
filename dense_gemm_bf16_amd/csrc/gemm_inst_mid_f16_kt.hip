// Kernel instantiations of the 256 x 128 direct-to-LDS tile ("mid" in GEMM_TILE_CONFIGS):
// fp16 operands, K % BK != 0.
#define GEMM_SPLIT_PARAMS GEMM_MID_PARAMS
#define GEMM_SPLIT_STREAM
#define GEMM_SPLIT_OWN 24
#include "gemm_inst_split.hpp"
