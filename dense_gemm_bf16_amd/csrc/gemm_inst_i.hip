// Kernel instantiations for the configurations tagged "i" in
// GEMM_TILE_CONFIGS (gemm_launch.hpp).
#include "gemm_launch.hpp"

namespace gemm {
#define GEMM_INSTANTIATE(NAME, BM, BN, BK, WM, WN, ST, SWZ, PIPE, TU) \
  GEMM_INST_##TU(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_i(BM, BN, BK, WM, WN, ST, SWZ, PIPE) \
  template hipError_t launch_cfg<BM, BN, BK, WM, WN, ST, SWZ, PIPE>(const KernelArgs&, int, hipStream_t, int);
#define GEMM_INST_a(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_b(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_c(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_d(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_e(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_f(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_g(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_h(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_j(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
#define GEMM_INST_k(BM, BN, BK, WM, WN, ST, SWZ, PIPE)
GEMM_TILE_CONFIGS(GEMM_INSTANTIATE)
}  // namespace gemm
