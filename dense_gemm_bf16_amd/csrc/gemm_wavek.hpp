// Small-M kernel: one workgroup per BM x 32 block of C over the whole K
// range (or its K slice), its four waves splitting every K-step between
// them, so that a decode batch of M <= 64 rows and N = 8192 fills the 256
// CUs with 256 workgroups and needs no split-K pass and no reduction kernel.
//
// At M <= 64 the product is bound by streaming B from HBM.  Each K-step of
// BK = 64 brings BM + 32 rows of 128 bytes into an S-slot LDS ring with
// LDS-DMA loads (coalesced: 8 lanes per 128-byte row segment), and wave w
// multiplies 16-wide substep w of that step: kFragM MFMAs of 32 x 32 x 16.
// A deep ring (S = 8: seven steps in flight per CU) covers the HBM latency,
// and with kStreamB (one row of tiles, so no other workgroup reads this B)
// B's loads are non-temporal.
// At the end every wave holds the partial sums of its quarter of K; they
// meet in LDS and are added in the fixed order wave 0, 1, 2, 3, so the
// result does not depend on timing.
//
// Per K-step X: wait until step X has landed (vmcnt) and barrier; the slot
// of step X-1 is now free (every wave's fragment reads of it fed its MFMAs
// before the barrier), so issue the loads of step X+S-1 into it; read the
// wave's fragments of step X and multiply.  Load layout, K offsets, the
// step past K and the chunk that straddles K are handled as in the
// direct-to-LDS kernel.
#pragma once

#include "gemm_kernel.hpp"

namespace gemm {

template <int BM, int BN, int BK, int S, int SWZ, int FLAGS>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void gemm_bf16_wavek_kernel(
    KernelArgs a) {
  using Cfg = TileCfg<BM, BN, BK, 1, 1, S, SWZ>;  // one wave's view of the whole tile
  constexpr int T = 256;                          // four waves
  constexpr int CPR = Cfg::kCpr;
  constexpr int LA = Cfg::kABytes / (T * 16);
  constexpr int LB = Cfg::kBBytes / (T * 16);
  constexpr int L = LA + LB;  // loads per thread (and per wave) per step
  constexpr int kStore = store_kind<FLAGS>();
  constexpr bool kHalf = (FLAGS & kF16) != 0;
  constexpr bool kSplit = (FLAGS & kSplitK) != 0;
  constexpr bool kRagged = (FLAGS & kRaggedK) != 0;
  constexpr bool kStream = (FLAGS & kStreamB) != 0;  // B loads non-temporal
  constexpr bool kPartial = (FLAGS & kPartialK) != 0;
  static_assert(BN == 32 && BK == 64, "32 columns, four 16-wide substeps per step");
  static_assert(Cfg::kSub == 4, "one substep per wave");
  static_assert(Cfg::kABytes % (T * 16) == 0 && Cfg::kBBytes % (T * 16) == 0,
                "tiles split into whole loads");
  static_assert(!kRagged || kPartial, "K % 8 != 0 implies K % BK != 0");
  static_assert((S - 2) * L < 64, "vmcnt range");
  constexpr int kRedBytes = 4 * Cfg::kFragM * 64 * 64;  // four waves' partial sums
  static_assert(kRedBytes <= Cfg::kLdsBytes, "the reduction reuses the ring");

  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[Cfg::kLdsBytes];
  lds_u8* const smem = (lds_u8*)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which tile and which K-slice (as in the other kernels) -------------
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

  // Load i of thread tid fills LDS position i*T + tid of its operand region
  // (row (i*T + tid) / CPR, chunk slot tid % CPR holding logical chunk
  // slot ^ swz(row)); its per-lane offset is range checked, so rows past M
  // or N read zero.
  constexpr int RPI = T / CPR;
  const int r0 = tid / CPR, c0 = tid % CPR;
  int chunk[L];
  uint32_t voff[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool is_a = i < LA;
    const int ii = is_a ? i : i - LA;
    const int row = ii * RPI + r0;
    chunk[i] = c0 ^ swz<SWZ, CPR>(row);
    const int ld = (int)(is_a ? a.lda : a.ldb);
    voff[i] = row < (is_a ? rows_a : rows_b) ? (uint32_t)(row * ld * 2 + chunk[i] * 16) : kOOB;
  }

  auto issue_step = [&](int Y) __attribute__((always_inline)) {
    const int kt = korder.kt(Y);
    const uint32_t slot = smem_addr + (uint32_t)((Y % S) * Cfg::kStageBytes);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool is_a = i < LA;
      const uint32_t dst =
          slot + (uint32_t)((is_a ? 0 : Cfg::kABytes) + ((is_a ? i : i - LA) * T + wave * 64) * 16);
      const u32x4& rs = is_a ? rsrc_a : rsrc_b;
      uint32_t v = voff[i], so = (uint32_t)(kt * BK * 2);
      if (kPartial && kt >= full_tiles) {
        const int k0 = kt * BK;
        v = (k0 + chunk[i] * 8 < a.K) ? voff[i] + (uint32_t)(k0 * 2) : kOOB;
        so = 0u;
      }
      if (is_a)
        dma16(rs, dst, v, so);
      else
        dma16<kStream>(rs, dst, v, so);
    }
  };

  auto trim_tail = [&](int Y) __attribute__((always_inline)) {
    const int k0 = korder.kt(Y) * BK;
    lds_u8* slot = smem + (Y % S) * Cfg::kStageBytes;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool is_a = i < LA;
      const int keep = a.K - (k0 + chunk[i] * 8);
      if (keep > 0 && keep < 8) {
        lds_u32x4* p = (lds_u32x4*)(slot + (is_a ? 0 : Cfg::kABytes) +
                                    ((is_a ? i : i - LA) * T + tid) * 16);
        u32x4 v = *p;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e = 2 * w;
          v[w] &= (e + 1 < keep) ? 0xFFFFFFFFu : (e < keep ? 0x0000FFFFu : 0u);
        }
        *p = v;
      }
    }
  };

  f32x16 acc[Cfg::kFragM][1];
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][0][r] = 0.0f;
  bf16x8 fa[Cfg::kFragM], fb[1];

#pragma unroll
  for (int p = 0; p + 1 < S; ++p)
    if (p < n_iter) issue_step(p);

  for (int X = 0; X < n_iter; ++X) {
    if constexpr (kRagged) {
      if (korder.kt(X) == a.k_tiles - 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        trim_tail(X);
      }
    }
    // in flight after step X: steps X+1 .. min(X+S-2, n_iter-1)
    ring_wait_barrier_n<L, S - 2>(min(S - 2, n_iter - 1 - X));
    if (X + S - 1 < n_iter) issue_step(X + S - 1);
    const lds_u8* sa = smem + (X % S) * Cfg::kStageBytes;
    read_frags<Cfg, SWZ>(sa, sa + Cfg::kABytes, wave, 0, 0, lane, fa, fb);
    mfma_block<Cfg, kHalf>(acc, fa, fb);
  }

  // ---- the four waves' partial sums, added in a fixed order ---------------
  // Wave w's block fm, lane l: 16 floats at red + ((w*kFragM + fm)*64 + l)*64.
  // Afterwards wave w adds elements 4w .. 4w+3 of every lane's 16 over the
  // four waves (0, 1, 2, 3) and stores them: row m0 + fm*32 + l % 32,
  // columns n0 + 8w + 4(l / 32) .. +3 (the layout of store_block).
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm) {
    lds_u8* p = smem + ((wave * Cfg::kFragM + fm) * 64 + lane) * 64;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(__attribute__((address_space(3))) f32x4*)(p + q * 16) =
          (f32x4){acc[fm][0][4 * q], acc[fm][0][4 * q + 1], acc[fm][0][4 * q + 2],
                  acc[fm][0][4 * q + 3]};
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm) {
    typedef const __attribute__((address_space(3))) f32x4 lds_f32x4;
    f32x4 s = *(lds_f32x4*)(smem + (fm * 64 + lane) * 64 + wave * 16);
#pragma unroll
    for (int v = 1; v < 4; ++v)
      s += *(lds_f32x4*)(smem + ((v * Cfg::kFragM + fm) * 64 + lane) * 64 + wave * 16);
    const int m = m0 + fm * 32 + (lane & 31);
    const int n = n0 + 8 * wave + 4 * (lane >> 5);
    if (m < a.M) {
      if constexpr (kSplit)
        store_quad<kStoreF32>(a.part + (int64_t)split * a.part_stride, a.ldp, s, m, n, a.N);
      else
        store_quad<kStore>(a.C, a.ldc, s, m, n, a.N);
    }
  }
}

}  // namespace gemm
