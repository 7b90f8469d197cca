// Eight-wave "ping-pong" variant of the bf16 GEMM kernel for gfx950.
//
// Why a second schedule: on this chip a wave issues LDS-DMA loads
// (buffer_load ... lds, 1 KB each) only about one per 70-100 cycles, and
// while it waits to issue, its in-order instruction stream cannot issue
// MFMAs either.  A 256x256 tile needs 64 such loads per 64-wide K-step, so a
// single wave per SIMD loses a large part of every K-step to issue stalls.
//
// Here the workgroup has two groups of four waves, one wave of each group on
// every SIMD.  Group g computes rows [g*BM/2, (g+1)*BM/2) of the tile (each
// wave a (BM/2) x (BN/4) sub-tile).  Work alternates in phases separated by
// workgroup barriers: while one group runs the MFMAs of a K-step on
// fragments it already holds (C phase), the other group reads its fragments
// of the next K-step from LDS and issues its share of the LDS-DMA loads of a
// K-step STAGES-1 ahead (M phase).  Every SIMD therefore always has one wave
// feeding the MFMA pipe while the other wave's loads are being issued.
//
//   phase:      -1    0     1     2     3    ...  2s-1    2s
//   group 0:   M(0)  C(0)  M(1)  C(1)  M(2)      M(s)    C(s)
//   group 1:    -    M(0)  C(0)  M(1)  C(1)      C(s-1)  M(s)
//
// M(s) reads all fragments of step s (slot s % STAGES) and issues this
// wave's loads of step s+STAGES-1 into slot (s-1) % STAGES, which both
// groups finished reading before the barrier that ends phase 2s-2.  At the
// end of its M(s) every wave waits until its own loads of step s+1 have
// landed (its loads of steps s+2 .. s+STAGES-1 may stay in flight); the
// barrier that follows publishes step s+1 before group 0 reads it in phase
// 2s+1.  Both groups execute the same number of barriers: group 1 idles in
// phase -1, group 0 in the phase after its last C.
//
// The data path per step is the one of gemm_kernel.hpp: XOR-swizzled LDS
// rows filled by LDS-DMA through range-checked buffer resources, ds_read_b128
// fragments, v_mfma_f32_32x32x16_bf16 with the B tile as first operand, the
// same epilogue and split-K partial output.  (Page "Matrix Multiplication on
// NVIDIA's Blackwell", Kernel 6: overlapping loads with MMAs through a ring
// of stages and specialised warps; here the roles alternate between two
// wave groups instead of being fixed.)
#pragma once

#include "gemm_kernel.hpp"

namespace gemm {

// CONTIG selects how a step's LDS-DMA loads are dealt to the waves:
//   false: load i of thread t fills the 16-byte LDS slot i*512 + t, so a
//          wave's loads are 8 KB apart and each rewrites M0;
//   true:  the step's 1 KB loads are numbered through the stage (A's
//          first), and wave w issues loads w*L .. w*L+L-1 (L per wave): they
//          are adjacent in LDS, so up to four share one M0 value and differ
//          only in the instruction offset, which lets them issue faster.
template <int BM, int BN, int BK, int STAGES, int SWZ, int FLAGS, bool CONTIG>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void
gemm_bf16_pingpong_kernel(KernelArgs a) {
  using Cfg = TileCfg<BM, BN, BK, 2, 4, STAGES, SWZ>;
  constexpr int T = Cfg::kThreads;
  constexpr int CPR = Cfg::kCpr;
  constexpr int LPS = Cfg::kLoadsPerStage;
  constexpr int SUB = Cfg::kSub;
  constexpr int kStore = store_kind<FLAGS>();
  constexpr bool kHalf = (FLAGS & kF16) != 0;
  constexpr bool kSplit = (FLAGS & kSplitK) != 0;
  constexpr bool kRagged = (FLAGS & kRaggedK) != 0;
  static_assert(STAGES >= 3, "ping-pong refills a slot one step after it is read");
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[Cfg::kLdsBytes];
  lds_u8* const smem = (lds_u8*)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0 or 1: which half of the tile rows
  const int wm = grp, wn = wave & 3;

  // ---- which tile and which K-slice (same mapping as gemm_bf16_kernel) ---
  const int ntiles = a.tiles_m * a.tiles_n;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int split = kSplit ? logical / ntiles : 0;
  const int t = logical - split * ntiles;
  int tm, tn;
  {
    const int span = a.group_m * a.tiles_n;
    const int gid = t / span;
    const int first_m = gid * a.group_m;
    const int gsz = min(a.tiles_m - first_m, a.group_m);
    const int in = t - gid * span;
    tm = first_m + in % gsz;
    tn = in / gsz;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int kt_begin = split * a.k_tiles_per_split;
  const int kt_end = kSplit ? min(a.k_tiles, kt_begin + a.k_tiles_per_split) : a.k_tiles;
  const int n_iter = kt_end - kt_begin;
  const KOrder korder = make_korder(a, t, kt_begin, n_iter);
  const int full_tiles = a.K / BK;

  const int rows_a = min(BM, a.M - m0);
  const int rows_b = min(BN, a.N - n0);
  const u32x4 rsrc_a = make_rsrc(a.A + (int64_t)m0 * a.lda, (uint32_t)(rows_a * a.lda * 2));
  const u32x4 rsrc_b = make_rsrc(a.B + (int64_t)n0 * a.ldb, (uint32_t)(rows_b * a.ldb * 2));

  uint32_t voff_a[Cfg::kLoadsA], voff_b[Cfg::kLoadsB];
  int chunk_a[Cfg::kLoadsA], chunk_b[Cfg::kLoadsB];
  // wave-contiguous dealing: load i of this wave is stage load g = wave*LPS + i
  constexpr int kStageLoadsA = Cfg::kABytes / 1024;
  static_assert(Cfg::kABytes % 1024 == 0 && 8 * LPS * 1024 == Cfg::kStageBytes,
                "a step is 8 waves x LPS loads of 1 KB, A's first");
  uint32_t voff_c[LPS];
  int chunk_c[LPS];
  u32x4 rsrc_c[LPS];
  if constexpr (CONTIG) {
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int g = wave * LPS + i;
      const bool is_a = g < kStageLoadsA;
      const int s = (is_a ? g : g - kStageLoadsA) * 64 + lane;
      const int row = s / CPR, c = (s % CPR) ^ swz<SWZ, CPR>(row);
      chunk_c[i] = c;
      const int rows = is_a ? rows_a : rows_b;
      const int ld = is_a ? a.lda : a.ldb;
      voff_c[i] = row < rows ? (uint32_t)(row * ld * 2 + c * 16) : kOOB;
      const uint32_t back = (uint32_t)((i % 4) * 1024);
      rsrc_c[i] = is_a ? shifted_rsrc(a.A + (int64_t)m0 * a.lda, (uint32_t)(rows_a * a.lda * 2), back)
                       : shifted_rsrc(a.B + (int64_t)n0 * a.ldb, (uint32_t)(rows_b * a.ldb * 2), back);
    }
  } else {
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i) {
      const int s = i * T + tid, row = s / CPR, c = (s % CPR) ^ swz<SWZ, CPR>(row);
      chunk_a[i] = c;
      voff_a[i] = row < rows_a ? (uint32_t)(row * a.lda * 2 + c * 16) : kOOB;
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i) {
      const int s = i * T + tid, row = s / CPR, c = (s % CPR) ^ swz<SWZ, CPR>(row);
      chunk_b[i] = c;
      voff_b[i] = row < rows_b ? (uint32_t)(row * a.ldb * 2 + c * 16) : kOOB;
    }
  }

  // This wave's loads of step `it` (nothing if the step does not exist).
  auto issue_step = [&](int it) {
    if (it >= n_iter) return;
    const int kt = korder.kt(it);
    const uint32_t base = smem_addr + (it % STAGES) * Cfg::kStageBytes;
    if constexpr (CONTIG) {
      const uint32_t wbase = base + wave * LPS * 1024;
      const int k0 = kt * BK;
      if (kt < full_tiles) {
        // K offset in soffset: the per-lane offsets are used as they are
        constexpr_for<LPS>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          dma16_off<(i % 4) * 1024>(rsrc_c[i], wbase + (i / 4) * 4096, voff_c[i],
                                    (uint32_t)(k0 * 2));
        });
      } else {
        constexpr_for<LPS>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          const uint32_t v =
              (k0 + chunk_c[i] * 8) < a.K ? voff_c[i] + (uint32_t)(k0 * 2) : kOOB;
          dma16_off<(i % 4) * 1024>(rsrc_c[i], wbase + (i / 4) * 4096, v, 0u);
        });
      }
    } else if (kt < full_tiles) {
      issue_tile_loads<Cfg::kLoadsA, T>(rsrc_a, base, voff_a, kt * BK, wave);
      issue_tile_loads<Cfg::kLoadsB, T>(rsrc_b, base + Cfg::kABytes, voff_b, kt * BK, wave);
    } else {
      issue_tail_loads<Cfg::kLoadsA, T>(rsrc_a, base, voff_a, chunk_a, kt * BK, a.K, wave);
      issue_tail_loads<Cfg::kLoadsB, T>(rsrc_b, base + Cfg::kABytes, voff_b, chunk_b, kt * BK,
                                        a.K, wave);
    }
  };

  // Patch this wave's chunks of step `it` that straddle a ragged K (after
  // its loads of that step have landed).
  auto fix_step = [&](int it) {
    if constexpr (kRagged) {
      if (it < n_iter && korder.kt(it) == a.k_tiles - 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_u8* st = smem + (it % STAGES) * Cfg::kStageBytes;
        const int k0 = korder.kt(it) * BK;
        if constexpr (CONTIG) {
          fix_tail_chunks<LPS, 64>(st + wave * LPS * 1024, chunk_c, k0, a.K, lane);
        } else {
          fix_tail_chunks<Cfg::kLoadsA, T>(st, chunk_a, k0, a.K, tid);
          fix_tail_chunks<Cfg::kLoadsB, T>(st + Cfg::kABytes, chunk_b, k0, a.K, tid);
        }
      }
    }
  };

  f32x16 acc[Cfg::kFragM][Cfg::kFragN];
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  bf16x8 fa[SUB][Cfg::kFragM], fb[SUB][Cfg::kFragN];

  // ---- prologue: steps 0 .. STAGES-2 in flight, step 0 landed ----------
#pragma unroll
  for (int p = 0; p + 1 < STAGES; ++p) issue_step(p);
  fix_step(0);
  ring_wait_barrier_n<LPS, STAGES - 2>(max(0, min(STAGES - 2, n_iter - 1)));
  if (grp == 1) asm volatile("s_barrier" ::: "memory");  // group 1 idles in phase -1

  for (int s = 0; s < n_iter; ++s) {
    // ---- M(s): fragments of step s, loads of step s+STAGES-1 ---------------
    const lds_u8* sa = smem + (s % STAGES) * Cfg::kStageBytes;
    const lds_u8* sb = sa + Cfg::kABytes;
#pragma unroll
    for (int kk = 0; kk < SUB; ++kk) read_frags<Cfg, SWZ>(sa, sb, kk, wm, wn, lane, fa[kk], fb[kk]);
    issue_step(s + STAGES - 1);
    fix_step(s + 1);
    // own loads of step s+1 landed; steps s+2 .. min(s+STAGES-1, n-1) may
    // remain in flight
    ring_wait_barrier_n<LPS, STAGES - 2>(max(0, min(STAGES - 2, n_iter - 2 - s)));
    __builtin_amdgcn_sched_barrier(0);
    // ---- C(s): the MFMAs of step s -----------------------------------------
#pragma unroll
    for (int kk = 0; kk < SUB; ++kk) mfma_block<Cfg, kHalf>(acc, fa[kk], fb[kk]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
  }
  if (grp == 0) asm volatile("s_barrier" ::: "memory");  // group 0 idles in the last phase

  finish_tile<Cfg, kStore, kSplit>(a, smem, wave, m0, n0, acc, m0 + wm * Cfg::kWaveM,
                                   n0 + wn * Cfg::kWaveN, lane, split);
}

}  // namespace gemm
