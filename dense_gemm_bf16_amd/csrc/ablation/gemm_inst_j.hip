// Ablation build only: kernel instantiations of the configurations tagged
// "j" in GEMM_ABLATION_CONFIGS (gemm_launch.hpp).
#define GEMM_INST_j GEMM_DO_INST
#include "gemm_inst_common.hpp"
