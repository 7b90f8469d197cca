// Instantiations of the GEMM kernel template and the table that names them.
#include <string.h>

#include "gemm_internal.h"

namespace gemm {
namespace {

template <int BM, int BN, int WM, int WN, int ST, int SWZ, int FLAGS>
hipError_t launch_one(const KernelArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, ST, SWZ, FLAGS>), dim3(grid),
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

// Dispatch the runtime variant flags to the instantiated kernels.
template <int BM, int BN, int WM, int WN, int ST, int SWZ>
hipError_t launch(const KernelArgs& a, int grid, hipStream_t s, int flags) {
  switch (flags & 7) {
    case 0: return launch_one<BM, BN, WM, WN, ST, SWZ, 0>(a, grid, s);
    case 1: return launch_one<BM, BN, WM, WN, ST, SWZ, 1>(a, grid, s);
    case 2: return launch_one<BM, BN, WM, WN, ST, SWZ, 2>(a, grid, s);
    case 3: return launch_one<BM, BN, WM, WN, ST, SWZ, 3>(a, grid, s);
    case 4: return launch_one<BM, BN, WM, WN, ST, SWZ, 4>(a, grid, s);
    case 5: return launch_one<BM, BN, WM, WN, ST, SWZ, 5>(a, grid, s);
    case 6: return launch_one<BM, BN, WM, WN, ST, SWZ, 6>(a, grid, s);
    default: return launch_one<BM, BN, WM, WN, ST, SWZ, 7>(a, grid, s);
  }
}

#define GEMM_CFG(NAME, BM, BN, WM, WN, ST, SWZ) \
  {NAME, BM, BN, WM * WN * 64, TileCfg<BM, BN, WM, WN, ST, SWZ>::kLdsBytes, &launch<BM, BN, WM, WN, ST, SWZ>}

}  // namespace

const TileConfig* tile_configs() {
  static const TileConfig table[] = {
      GEMM_CFG("t256x256_w2x2_s2_x1", 256, 256, 2, 2, 2, 1),
      GEMM_CFG("t256x256_w2x2_s2_x2", 256, 256, 2, 2, 2, 2),
      GEMM_CFG("t256x128_w2x2_s2_x1", 256, 128, 2, 2, 2, 1),
      GEMM_CFG("t128x128_w2x2_s3_x1", 128, 128, 2, 2, 3, 1),
      {nullptr, 0, 0, 0, 0, nullptr},
  };
  return table;
}

const TileConfig* find_tile_config(const char* name) {
  for (const TileConfig* c = tile_configs(); c->name; ++c)
    if (strcmp(c->name, name) == 0) return c;
  return nullptr;
}

}  // namespace gemm
