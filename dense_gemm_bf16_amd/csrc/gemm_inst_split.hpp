// Splits the kernel variants of one configuration over four translation
// units.  The direct-to-LDS tiles have the most variants of any row of
// GEMM_TILE_CONFIGS (two operand types, times the K % BK != 0 variant, times
// up to six flag combinations); compiled in one file they take minutes, so
// each (operand type, K-tail) group is instantiated in a file of its own and
// the files compile side by side.
//
// The including file defines GEMM_SPLIT_PARAMS as the configuration's
// template parameters (one of the GEMM_*_PARAMS macros of gemm_launch.hpp,
// so they cannot drift from the table) and GEMM_SPLIT_OWN as the group it
// instantiates, numbered by its kF16 | kPartialK bits (0, 8, 16 or 24); the
// other three groups are declared extern.  The file owning group 0 also
// instantiates the configuration's launch_cfg (the dispatch).  With
// GEMM_SPLIT_RAGGED_APART defined, the three ragged-K kernels (K % 8 != 0)
// of each K-tail group go to one more file each, GEMM_SPLIT_OWN 20 (bf16)
// or 28 (fp16), as they would otherwise make the K-tail files the longest
// of the build.  With GEMM_SPLIT_PERSIST defined (rows built with
// kOptPersist), the persistent-grid groups (kPersistent, with and without
// kPartialK) are instantiated by the files with GEMM_SPLIT_OWN 32 and 48;
// with GEMM_SPLIT_STREAM defined (rows built with kOptStream), the kernels
// with non-temporal B loads by the files with GEMM_SPLIT_OWN 64 (bf16) and
// 72 (fp16).
#pragma once

#include "gemm_launch.hpp"

#if !defined(GEMM_SPLIT_PARAMS) || !defined(GEMM_SPLIT_OWN)
#error "define GEMM_SPLIT_PARAMS and GEMM_SPLIT_OWN before including gemm_inst_split.hpp"
#endif

#define GEMM_SPLIT_EXPAND(M, ...) M(__VA_ARGS__)
#define GEMM_SPLIT_VARIANT_(E, BM, BN, BK, WM, WN, ST, SWZ, PIPE)          \
  template hipError_t launch_variant<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E>( \
      const KernelArgs&, int, hipStream_t, int);
#define GEMM_SPLIT_VARIANT(E) GEMM_SPLIT_EXPAND(GEMM_SPLIT_VARIANT_, E, GEMM_SPLIT_PARAMS)
#define GEMM_SPLIT_STREAM_(E, BM, BN, BK, WM, WN, ST, SWZ, PIPE)          \
  template hipError_t launch_stream<BM, BN, BK, WM, WN, ST, SWZ, PIPE, E>( \
      const KernelArgs&, int, hipStream_t, int);
#define GEMM_SPLIT_STREAM_GROUP(E) GEMM_SPLIT_EXPAND(GEMM_SPLIT_STREAM_, E, GEMM_SPLIT_PARAMS)
#define GEMM_SPLIT_ONE_(F, BM, BN, BK, WM, WN, ST, SWZ, PIPE)          \
  template hipError_t launch_one<BM, BN, BK, WM, WN, ST, SWZ, PIPE, F>( \
      const KernelArgs&, int, hipStream_t);
#define GEMM_SPLIT_ONE(F) GEMM_SPLIT_EXPAND(GEMM_SPLIT_ONE_, F, GEMM_SPLIT_PARAMS)
// The ragged-K kernels of K-tail group G (flags G | kRaggedK, | kOutF32,
// | kSplitK).
#define GEMM_SPLIT_RAGGED(G) GEMM_SPLIT_ONE(G + 4) GEMM_SPLIT_ONE(G + 5) GEMM_SPLIT_ONE(G + 6)
#define GEMM_SPLIT_RAGGED_EXTERN(G) \
  extern GEMM_SPLIT_ONE(G + 4) extern GEMM_SPLIT_ONE(G + 5) extern GEMM_SPLIT_ONE(G + 6)

namespace gemm {
static_assert(kF16 == 8 && kPartialK == 16 && kRaggedK == 4,
              "GEMM_SPLIT_OWN numbers the groups by these bits");
static_assert(kPersistent == 32, "GEMM_SPLIT_OWN 32 and 48 name the persistent groups");
#ifdef GEMM_SPLIT_STREAM
static_assert(kStreamB == 64, "GEMM_SPLIT_OWN 64 and 72 name the stream-B groups");
#if GEMM_SPLIT_OWN == 64
GEMM_SPLIT_STREAM_GROUP(0)
#else
extern GEMM_SPLIT_STREAM_GROUP(0)
#endif
#if GEMM_SPLIT_OWN == 72
GEMM_SPLIT_STREAM_GROUP(8)
#else
extern GEMM_SPLIT_STREAM_GROUP(8)
#endif
#endif
#ifdef GEMM_SPLIT_PERSIST
#if GEMM_SPLIT_OWN == 32
GEMM_SPLIT_VARIANT(32)
#else
extern GEMM_SPLIT_VARIANT(32)
#endif
#if GEMM_SPLIT_OWN == 48
GEMM_SPLIT_VARIANT(48)
#else
extern GEMM_SPLIT_VARIANT(48)
#endif
#endif
#ifdef GEMM_SPLIT_RAGGED_APART
#if GEMM_SPLIT_OWN == 20
GEMM_SPLIT_RAGGED(16)
#else
GEMM_SPLIT_RAGGED_EXTERN(16)
#endif
#if GEMM_SPLIT_OWN == 28
GEMM_SPLIT_RAGGED(24)
#else
GEMM_SPLIT_RAGGED_EXTERN(24)
#endif
#endif
#if GEMM_SPLIT_OWN == 0
GEMM_SPLIT_VARIANT(0)
#else
extern GEMM_SPLIT_VARIANT(0)
#endif
#if GEMM_SPLIT_OWN == 16
GEMM_SPLIT_VARIANT(16)
#else
extern GEMM_SPLIT_VARIANT(16)
#endif
#if GEMM_SPLIT_OWN == 8
GEMM_SPLIT_VARIANT(8)
#else
extern GEMM_SPLIT_VARIANT(8)
#endif
#if GEMM_SPLIT_OWN == 24
GEMM_SPLIT_VARIANT(24)
#else
extern GEMM_SPLIT_VARIANT(24)
#endif
}  // namespace gemm
