// Host-side description of the kernel configurations the library is built
// with, shared between the launcher table and the C-ABI front end.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace gemm {

// One compiled tile configuration.  `launch` takes the variant flags
// (kOutF32 | kSplitK | kRaggedK | kF16 | kPartialK | kPersistent | kStreamB)
// and enqueues the matching kernel; kF16 only where `f16` is set.
struct TileConfig {
  const char* name;  // e.g. "t256x256x64_w2x2_s2_x2"
  int bm, bn;        // output tile
  int bk;            // K elements per ring slot
  int threads;       // workgroup size
  int lds_bytes;     // static LDS per workgroup
  bool f16;          // also built for fp16 operands
  bool persist;      // also built for a persistent grid (bf16 operands)
  bool stream;       // also built with non-temporal B loads (kStreamB)
  hipError_t (*launch)(const KernelArgs&, int grid, hipStream_t, int flags);
};

// Table of built configurations, terminated by an entry with name == NULL.
const TileConfig* tile_configs();

const TileConfig* find_tile_config(const char* name);

// A complete launch plan: tile config, split count and raster grouping.
struct Plan {
  const TileConfig* tile;
  int splits;
  int group_m;
  int k_rot;    // K-step rotation stride per tile, 0 = none
  int persist;  // persistent grid of this many workgroups (a multiple of 8), 0 = none
  int stream_b; // 1: B loads non-temporal (where the tile is built with it)
  // Hybrid: the tile columns that fill whole passes over the CUs run
  // unsplit, the columns from split_n on run as a second call with K split
  // tail_splits ways (0 / 0: not hybrid).
  int tail_splits;
  int64_t split_n;
  // Mixed: as the hybrid, but the columns from split_n on run unsplit on
  // this narrower tile (256 x 128 or 128 x 128 under 256 x 256), which fills
  // the CUs where the wide tile's last pass would be part empty (null: not
  // mixed).
  const TileConfig* tail_tile;
  char name[64];
};

// Fixed-order fp32 sum of S partial buffers P + s*slice_stride (rows of
// stride ldp) into C, rounded to bf16 or fp16 or stored as fp32 (out_kind is
// kStoreBf16, kStoreF16 or kStoreF32).
hipError_t launch_splitk_reduce(const float* P, int64_t ldp, int64_t slice_stride, int S,
                                void* C, int64_t ldc, int M, int N, int out_kind,
                                hipStream_t stream);

}  // namespace gemm
