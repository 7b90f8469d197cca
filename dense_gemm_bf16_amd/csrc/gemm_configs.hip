// The table of built tile configurations (names and launchers).
#include <string.h>

#include "gemm_internal.h"
#include "gemm_launch.hpp"

namespace gemm {

const TileConfig* tile_configs() {
#define GEMM_TABLE_ROW(NAME, BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT, TU)                 \
  {#NAME, BM, BN, BK, PIPE == 9 ? 256 : WM * WN * 64,                                  \
   lds_bytes_of<BM, BN, BK, WM, WN, ST, SWZ, PIPE>(),                                     \
   (OPT & kOptF16) != 0, (OPT & kOptPersist) != 0, (OPT & kOptStream) != 0,              \
   &launch_cfg<BM, BN, BK, WM, WN, ST, SWZ, PIPE, OPT>},
  static const TileConfig table[] = {
      GEMM_TILE_CONFIGS(GEMM_TABLE_ROW){nullptr, 0, 0, 0, 0, 0, false, false, false, nullptr}};
#undef GEMM_TABLE_ROW
  return table;
}

const TileConfig* find_tile_config(const char* name) {
  for (const TileConfig* c = tile_configs(); c->name; ++c)
    if (strcmp(c->name, name) == 0) return c;
  return nullptr;
}

}  // namespace gemm
