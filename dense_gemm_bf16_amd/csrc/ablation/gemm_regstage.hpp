// Four-wave bf16 GEMM kernel for gfx950 with register-staged global loads.
//
// Why another load path: measured on MI355X, an ordinary buffer load into
// VGPRs placed between MFMAs costs the issuing wave little MFMA time (four
// 1 KB loads per 16 MFMAs: about 3 %), while an LDS-DMA load in the same
// place costs about four times as much, and any load issued in a burst
// blocks the wave for ~100 cycles.  So here every wave streams its share of
// the next tiles through registers: each K-step's loads are issued NBUF
// steps ahead into a ring of NBUF register buffers, and written to LDS
// (ds_write_b128 at the XOR-swizzled position) one step ahead of use, both
// spread one at a time between the MFMAs of the current step.  LDS holds
// two slots: the step being read and the step being written.
//
// Four waves (2 x 2), one per SIMD, each with a 128 x 128 sub-tile of a
// 256 x 256 workgroup tile: 256 accumulator registers per lane, and per
// K-step of 16 each wave reads (128 + 128) rows of fragments, two thirds of
// what eight waves with 128 x 64 sub-tiles read.
//
// Per K-step X (slot X % 2 holds it):
//   substeps 0 .. SUB-2: fragments of the next substep are read; between
//     the MFMAs go the loads of step X+NBUF (into buffer X % NBUF, whose data
//     went to LDS during step X-1) and the ds_writes of step X+1 (from buffer
//     (X+1) % NBUF into slot (X+1) % 2, free since the barrier of step X-1),
//     all writes before the barrier;
//   then every wave's LDS writes are waited for and the workgroup barriers,
//     which publishes step X+1 (slot X % 2 is no longer read: the last
//     substep's fragments are already in registers);
//   last substep: fragments of step X+1's first substep are read from the
//     new slot while this substep's MFMAs run.
// The compiler inserts the vmcnt waits that a ds_write needs for its loaded
// registers (loads return in order, so later steps' loads stay in flight).
//
// Edges: out-of-range rows and K-chunks read as zero through the buffer
// range check (the K test is per chunk for the K-steps at the end of K);
// when K % 8 != 0, the chunk that straddles K is masked in registers before
// it is written to LDS.  (Page "Matrix Multiplication on NVIDIA's
// Blackwell", Kernel 6, and page "Hand-writing a Blackwell GEMM", Step 2:
// overlapping the loads of later K-steps with the MMAs of the current one.)
#pragma once

#include "gemm_kernel.hpp"

namespace gemm {

// Zero the elements k >= K of one loaded 16-byte chunk holding k0 .. k0+7.
__device__ __forceinline__ u32x4 mask_tail_chunk(u32x4 v, int k0, int K) {
  const int keep = K - k0;
  if (keep > 0 && keep < 8) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e = 2 * w;
      const uint32_t m = (e + 1 < keep) ? 0xFFFFFFFFu : (e < keep ? 0x0000FFFFu : 0u);
      v[w] &= m;
    }
  }
  return v;
}

template <int BM, int BN, int BK, int WM, int WN, int NBUF, int SWZ, int FLAGS>
__global__ __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                          amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void
gemm_bf16_regstage_kernel(KernelArgs a) {
  using Cfg = TileCfg<BM, BN, BK, WM, WN, 2, SWZ>;  // two LDS slots
  constexpr int T = Cfg::kThreads;
  constexpr int CPR = Cfg::kCpr;
  constexpr int R = Cfg::kRowBytes;
  constexpr int SUB = Cfg::kSub;
  constexpr int LA = Cfg::kLoadsA;
  constexpr int L = Cfg::kLoadsPerStage;  // loads (and writes) per thread per step
  constexpr int kStore = store_kind<FLAGS>();
  constexpr bool kHalf = (FLAGS & kF16) != 0;
  constexpr bool kSplit = (FLAGS & kSplitK) != 0;
  constexpr bool kRagged = (FLAGS & kRaggedK) != 0;
  static_assert(T == 256 || T == 512, "one or two waves per SIMD");
  static_assert(SUB % 2 == 0, "fragment buffers alternate per substep, also across steps");
  static_assert(NBUF >= 2, "loads run at least one step ahead of their LDS writes");
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[Cfg::kLdsBytes];
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- which tile and which K-slice (as in gemm_bf16_kernel) -------------
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

  const int rows_a = min(BM, a.M - m0);
  const int rows_b = min(BN, a.N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.A + (int64_t)m0 * a.lda), (short)0, rows_a * (int)a.lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.B + (int64_t)n0 * a.ldb), (short)0, rows_b * (int)a.ldb * 2, 0x00020000);

  // Load i of this thread: 16-byte chunk s = i*T + tid of the operand (A
  // for i < LA, then B): row i*RPI + r0 with r0 = tid / CPR, logical chunk
  // c = tid % CPR (the same for every i), read from global row*ld + c*8 (+
  // the step's k0) and written to LDS position c ^ swz(row) of that row.
  // So a load's global offset is the lane's offset for i = 0 plus a
  // wave-uniform i*RPI*ld*2, and its LDS offset is one of two lane values
  // (swz depends on i only through its lowest bit) plus a constant.  Rows
  // past the operand's end fall outside the buffer range and read zero.
  constexpr int RPI = T / CPR;  // rows covered by one load of all threads
  static_assert(T % CPR == 0, "every load covers whole rows");
  const int r0 = tid / CPR, c0 = tid % CPR;
  const uint32_t voff_a0 = (uint32_t)(r0 * (int)a.lda * 2 + c0 * 16);
  const uint32_t voff_b0 = (uint32_t)(r0 * (int)a.ldb * 2 + c0 * 16);
  uint32_t lane_loff[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = p * RPI + r0;
    lane_loff[p] = (uint32_t)(r0 * R + ((c0 ^ swz<SWZ, CPR>(row)) << 4));
  }
  static_assert(swz_period_two<SWZ, CPR, RPI, L>(), "swz(i*RPI + r) depends on i only via i & 1");
  const int kc = c0 * 8;  // first k of this lane's chunks within a step
  u32x4 stg[NBUF][L];
  f32x16 acc[Cfg::kFragM][Cfg::kFragN];
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  bf16x8 fa[2][Cfg::kFragM], fb[2][Cfg::kFragN];

  // Load i of step `it` into buffer B.  Chunks at or past the end of this
  // workgroup's K range (K itself, or the end of its K slice) read as zero
  // without touching memory, so the loads of steps past the range cost
  // nothing; the K offset goes into the range-checked voffset.  (Keeping a
  // second, test-free variant for steps inside K doubled the code paths and
  // made the register allocator spill; the test is three VALU operations.)
  const int klim = min(a.K, kt_end * BK);
  auto load_one = [&](auto bc, auto ic, int it) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value, i = decltype(ic)::value;
    constexpr bool is_a = i < LA;
    constexpr int ii = is_a ? i : i - LA;  // load index within the operand
    // steps past the range (it >= n_iter) load nothing: k0 at the range end
    const int k0 = (it < n_iter ? korder.kt(it) : kt_end) * BK;
    const uint32_t rowoff = (uint32_t)(ii * RPI * (int)(is_a ? a.lda : a.ldb) * 2 + k0 * 2);
    const uint32_t v = (k0 + kc) < klim ? (is_a ? voff_a0 : voff_b0) + rowoff : kOOB;
    stg[B][i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(is_a ? rsrc_a : rsrc_b, (int)v, 0, 0));
  };

  // Write chunk i of step `it` from buffer B into its LDS slot.
  auto write_one = [&](auto bc, auto ic, int it) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value, i = decltype(ic)::value;
    constexpr bool is_a = i < LA;
    constexpr int ii = is_a ? i : i - LA;
    // swz of row ii*RPI + r0 equals that of row (ii & 1)*RPI + r0
    constexpr uint32_t kConst = (uint32_t)((is_a ? 0 : Cfg::kABytes) + ii * RPI * R);
    u32x4 v = stg[B][i];
    if constexpr (kRagged) {
      if (it < n_iter && korder.kt(it) == a.k_tiles - 1)
        v = mask_tail_chunk(v, korder.kt(it) * BK + kc, a.K);
    }
    *(lds_u32x4*)(smem + (it & 1) * Cfg::kStageBytes + lane_loff[ii & 1] + kConst) = v;
  };

  // ---- prologue: steps 0 .. NBUF-1 loading, step 0 in LDS -----------------
  constexpr_for<NBUF>([&](auto bc) {
    constexpr int B = decltype(bc)::value;
    if (B < n_iter) {
      constexpr_for<L>([&](auto ic) { load_one(bc, ic, B); });
    }
  });
  constexpr_for<L>([&](auto ic) { write_one(std::integral_constant<int, 0>{}, ic, 0); });
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  read_frags<Cfg, SWZ>(smem, smem + Cfg::kABytes, 0, wm, wn, lane, fa[0], fb[0]);

  // ---- one K-step X; B = X % NBUF ------------------------------------------
  auto step = [&](auto bc, int X) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    constexpr int WB = (B + 1) % NBUF;  // buffer holding step X+1
    constexpr int LOADS = L;
    const lds_u8* sa = smem + (X & 1) * Cfg::kStageBytes;
    const lds_u8* sb = sa + Cfg::kABytes;
    const lds_u8* na = smem + ((X + 1) & 1) * Cfg::kStageBytes;
    // Substep kk carries loads [llo, lhi) of step X+NBUF and writes
    // [wlo, whi) of step X+1.  With three or more register buffers, loads go
    // early in the step (first half of the substeps) and writes late (from
    // the middle up to the barrier), so a load has about NBUF - 0.75 steps
    // to return before its data is written to LDS.  With two buffers that
    // order would keep both buffers live at once (more registers than a
    // lane has), so the writes of step X+1 go first, freeing buffer
    // (X+1) % 2 register by register, and the loads follow, spread over the
    // whole step.
    constexpr_for<SUB>([&](auto kc_) __attribute__((always_inline)) {
      constexpr int kk = decltype(kc_)::value;
      constexpr bool kEarly = NBUF >= 3;
      constexpr int LS = kEarly ? SUB / 2 : SUB;                     // substeps with loads
      constexpr int WS0 = kEarly ? SUB / 2 - 1 : 0, WSN = SUB - 1 - WS0;  // with writes
      constexpr int llo = kk < LS ? kk * LOADS / LS : LOADS;
      constexpr int lhi = kk < LS ? (kk + 1) * LOADS / LS : LOADS;
      constexpr bool wsub = kk >= WS0 && kk < SUB - 1;
      constexpr int wlo = wsub ? (kk - WS0) * L / WSN : 0;
      constexpr int whi = wsub ? (kk - WS0 + 1) * L / WSN : 0;
      constexpr int G = (whi - wlo) + (lhi - llo);
      constexpr int cur = kk & 1, nxt = cur ^ 1;
      if constexpr (kk + 1 < SUB) {
        read_frags<Cfg, SWZ>(sa, sb, kk + 1, wm, wn, lane, fa[nxt], fb[nxt]);
      } else {
        // every wave's writes of step X+1 are done: publish it
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        read_frags<Cfg, SWZ>(na, na + Cfg::kABytes, 0, wm, wn, lane, fa[nxt], fb[nxt]);
      }
      mfma_interleave<Cfg, kHalf, G>(acc, fa[cur], fb[cur], [&](auto qc) __attribute__((always_inline)) {
        constexpr int Q = decltype(qc)::value;
        // NBUF >= 3: loads, then writes; NBUF == 2: writes, then loads
        constexpr int NL = lhi - llo, NW = whi - wlo;
        constexpr bool kLoad = NBUF >= 3 ? Q < NL : Q >= NW;
        if constexpr (kLoad) {
          load_one(bc, std::integral_constant<int, llo + (NBUF >= 3 ? Q : Q - NW)>{}, X + NBUF);
        } else {
          write_one(std::integral_constant<int, WB>{},
                    std::integral_constant<int, wlo + (NBUF >= 3 ? Q - NL : Q)>{}, X + 1);
        }
      });
    });
  };

  // Whole groups of NBUF steps without branches (so the compiler's
  // load-wait bookkeeping stays exact around the loop), then the rest.
  int X0 = 0;
  for (; X0 + NBUF <= n_iter; X0 += NBUF) {
    constexpr_for<NBUF>([&](auto bc) __attribute__((always_inline)) { step(bc, X0 + decltype(bc)::value); });
  }
  constexpr_for<NBUF - 1>([&](auto bc) __attribute__((always_inline)) {
    if (X0 + decltype(bc)::value < n_iter) step(bc, X0 + decltype(bc)::value);
  });

  finish_tile<Cfg, kStore, kSplit>(a, smem, wave, m0, n0, acc, m0 + wm * Cfg::kWaveM,
                                   n0 + wn * Cfg::kWaveN, lane, split);
}

}  // namespace gemm
