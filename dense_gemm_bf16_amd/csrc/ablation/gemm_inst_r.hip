// Ablation build only: kernel instantiations of the configurations tagged
// "r" in GEMM_ABLATION_CONFIGS (gemm_launch.hpp).
#define GEMM_INST_r GEMM_DO_INST
#include "gemm_inst_common.hpp"
