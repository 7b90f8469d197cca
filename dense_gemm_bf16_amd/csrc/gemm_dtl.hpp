// Direct-to-LDS GEMM kernel: operand tiles go from global memory straight
// into an S-slot LDS ring with LDS-DMA loads (`buffer_load_dwordx4 ... lds`,
// no VGPR staging and no ds_write), each wave computes a block of the tile
// from ds_read_b128 fragments with 32x32x16 MFMAs (MF = 32) or 16x16x32
// MFMAs (MF = 16; same work per cycle, and the chip holds a higher clock
// under its power limit with them).
//
// Why this shape of kernel, from measurements on MI355X:
//  * LDS writes through ds_write_b128 run at ~76-105 B/clk per CU, LDS reads
//    at ~216-270 B/clk; staging every operand byte through VGPRs and
//    ds_write (the register-staged kernel) keeps the LDS busy for a large
//    share of each step.  LDS-DMA fills LDS from the texture path instead.
//  * An LDS-DMA load with its addresses ready in registers costs its wave
//    only a few cycles of issue (an MFMA stream with one such load per four
//    32-cycle MFMAs stays ~95 % busy), so loads can sit between MFMAs.
//  * The per-CU load path delivers ~64 B/clk; a 256 x 256 tile needs 32 B per
//    MFMA-clock at full rate, so loads keep up.
//
// Per K-step X (SUB = BK/16 substeps of 32x32x16 MFMAs, or BK/32 of
// 16x16x32), in every wave:
//   substep kk < SUB-1:  MFMAs of kk with, between them, the ds_reads of
//                        substep kk+1's fragments and load group kk+1 of
//                        step X+S-1 (groups 1..F-1; F = 2 groups per step
//                        with two slots, SUB with three or more);
//   substep SUB-1:       wait for step X+1's loads, barrier (this also frees
//                        slot X % S: every wave has read its last fragments
//                        of step X), then the MFMAs of substep SUB-1 with the
//                        reads of step X+1's first fragments and group 0 of
//                        step X+S (into the slot just freed) between them.
//                        With two substeps (16x16x32, BK = 64) the first half
//                        of this substep's MFMAs runs before the barrier, so
//                        that it still sits three quarters into the step and
//                        the loads have as long to land as with four.
// So a load is issued S-2 steps and a few substeps before the barrier that
// needs it, and nothing waits on a load issued in the same step unless S = 2.
//
// The loads of a step: load i (A rows first, then B) of thread tid fills LDS
// position s = i*T + tid of its operand's region: row s / CPR, chunk slot
// tid % CPR, which holds logical 16-byte chunk (slot ^ swz(row)) of that row.
// Each load keeps its own per-lane offset register (row*ld*2 + chunk*16, or
// an out-of-range value for rows past M or N, which then read zero), so the
// issue of a load is one M0 update and the instruction; the K offset of the
// step goes in the (unchecked) scalar offset.  In the step that K ends in
// (compiled only when K % BK != 0) the lanes whose chunk starts at or past K
// take the out-of-range offset instead (a select, not a branch); a chunk
// that straddles K (K % 8 != 0) is trimmed in LDS once it has landed.
#pragma once

#include "gemm_kernel.hpp"

namespace gemm {

// DL (B lead): B runs DL K-steps ahead of A.  The ring then has S slots
// of A + B and DL more B-only slots; the loads of "stage" Y are A of step Y
// and B of step Y + DL (an out-of-range load that reads zero into a free B
// slot when Y + DL is past the end, so every stage issues the same loads and
// the wait counts stay those of DL = 0), and the prologue first issues B of
// steps 0 .. DL-1.  B comes from HBM in the memory-bound shapes while A
// (the activations, shared by every tile of a K range) mostly comes from L2,
// so this keeps more of B in flight per CU.
template <int BM, int BN, int BK, int WM, int WN, int S, int SWZ, int FLAGS, int MF, int DL = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                          amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void
gemm_bf16_dtl_kernel(KernelArgs a) {
  using Cfg = TileCfg<BM, BN, BK, WM, WN, S, SWZ, MF>;
  static_assert(DL >= 0, "B lead");
  constexpr int SB = S + DL;  // B slots
  constexpr int kRingBytes = S * Cfg::kStageBytes + DL * Cfg::kBBytes;
  static_assert(kRingBytes <= 160 * 1024, "LDS is 160 KB per CU");
  constexpr int T = Cfg::kThreads;
  constexpr int CPR = Cfg::kCpr;
  constexpr int SUB = Cfg::kSub;
  constexpr int LA = Cfg::kLoadsA;
  constexpr int L = Cfg::kLoadsPerStage;
  // Load groups per step.  With two slots a step's loads must land within
  // the step before it, so they go out in the first two substeps; with
  // three or more they have over a step to land and are spread over all
  // four, which keeps fewer loads between any two MFMAs.
  constexpr int F = (S >= 3 && Cfg::kLoadsPerStage % Cfg::kSub == 0) ? Cfg::kSub : 2;
  constexpr int kStore = store_kind<FLAGS>();
  constexpr bool kHalf = (FLAGS & kF16) != 0;
  constexpr bool kSplit = (FLAGS & kSplitK) != 0;
  constexpr bool kRagged = (FLAGS & kRaggedK) != 0;    // K % 8 != 0
  constexpr bool kStream = (FLAGS & kStreamB) != 0;    // B loads non-temporal
  constexpr bool kPartial = (FLAGS & kPartialK) != 0;  // K % BK != 0
  static_assert(!kRagged || kPartial, "K % 8 != 0 implies K % BK != 0");
  static_assert(SUB % 2 == 0, "fragment buffers alternate per substep, also across steps");
  static_assert(F <= SUB, "a step's load groups fit in the substeps before its barrier");
  static_assert(L % F == 0, "equal load groups");
  static_assert((S - 2) * L + L / F < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[kRingBytes];
  lds_u8* const smem = (lds_u8*)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- which tile and which K-slice (as in the other kernels) -------------
  // A work unit is one (tile, K-slice).  Each workgroup takes unit
  // blockIdx.x, and with a persistent grid also blockIdx.x + gridDim.x,
  // + 2 gridDim.x, ...: unit v runs on XCD v % 8 either way (the grid is a
  // multiple of 8), so xcd_remap gives the same tile order per XCD as a grid
  // of one workgroup per unit.
  constexpr bool kPersist = (FLAGS & kPersistent) != 0;
  static_assert(!(kPersist && kSplit), "a persistent grid does not split K");
  static_assert(!(kPersist && DL > 0), "a persistent grid has no B lead");
  const int ntiles = a.tiles_m * a.tiles_n;
  const int units = kSplit ? ntiles * a.splits : ntiles;
  const int full_tiles = a.K / BK;  // K-steps wholly inside K

  // Per-lane offsets of this thread's loads (see the header comment).
  constexpr int RPI = T / CPR;  // rows covered by one load of all threads
  static_assert(T % CPR == 0, "every load covers whole rows");
  static_assert(swz_period_two<SWZ, CPR, RPI, (LA > L - LA ? LA : L - LA)>(),
                "swz(i*RPI + r) depends on i only via i & 1");
  const int r0 = tid / CPR, c0 = tid % CPR;
  int chunk2[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) chunk2[p] = c0 ^ swz<SWZ, CPR>(p * RPI + r0);

  // The current unit's tile, K range and load addressing.
  int split = 0, m0 = 0, n0 = 0, n_iter = 0;
  KOrder korder{0, 0, 0};
  u32x4 rsrc_a, rsrc_b;
  uint32_t voff[L];
  auto setup = [&](int unit) __attribute__((always_inline)) {
    const int logical = xcd_remap(unit, units);
    split = kSplit ? logical / ntiles : 0;
    const int t = logical - split * ntiles;
    const int span = a.group_m * a.tiles_n;
    const int gid = t / span;
    const int first_m = gid * a.group_m;
    const int gsz = min(a.tiles_m - first_m, a.group_m);
    const int in = t - gid * span;
    m0 = (first_m + in % gsz) * BM;
    n0 = (in / gsz) * BN;
    const int kt_begin = split * a.k_tiles_per_split;
    const int kt_end = kSplit ? min(a.k_tiles, kt_begin + a.k_tiles_per_split) : a.k_tiles;
    n_iter = kt_end - kt_begin;
    korder = make_korder(a, t, kt_begin, n_iter);
    const int rows_a = min(BM, a.M - m0);
    const int rows_b = min(BN, a.N - n0);
    rsrc_a = make_rsrc(a.A + (int64_t)m0 * a.lda, (uint32_t)(rows_a * a.lda * 2));
    rsrc_b = make_rsrc(a.B + (int64_t)n0 * a.ldb, (uint32_t)(rows_b * a.ldb * 2));
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool is_a = i < LA;
      const int ii = is_a ? i : i - LA;
      const int row = ii * RPI + r0;
      const int ld = (int)(is_a ? a.lda : a.ldb);
      voff[i] = row < (is_a ? rows_a : rows_b) ? (uint32_t)(row * ld * 2 + chunk2[ii & 1] * 16)
                                               : kOOB;
    }
  };
  int unit = blockIdx.x;
  setup(unit);

  // Byte offset of the ring slot of K-step Y.  With a persistent grid, step
  // 0 of every unit goes to slot 1: slot 0 then stages the previous unit's C
  // while the next unit's first S-1 steps land in slots 1 .. S-1.
  auto slot_off = [](int Y) __attribute__((always_inline)) {
    return (uint32_t)(((kPersist ? Y + 1 : Y) % S) * Cfg::kStageBytes);
  };

  // Byte offset of the B tile of K-step Y: in its step's slot when DL = 0,
  // else in a ring of S + DL B slots (the first S inside the A + B slots).
  auto b_off = [&](int Y) __attribute__((always_inline)) {
    if constexpr (DL == 0) {
      return slot_off(Y) + (uint32_t)Cfg::kABytes;
    } else {
      const int j = Y % SB;
      return (uint32_t)(j < S ? j * Cfg::kStageBytes + Cfg::kABytes
                              : S * Cfg::kStageBytes + (j - S) * Cfg::kBBytes);
    }
  };

  // LDS byte offset (within its operand tile) of load i's 1 KB of this wave.
  auto lds_off = [&](int i) __attribute__((always_inline)) {
    return (uint32_t)(((i < LA ? i : i - LA) * T + wave * 64) * 16);
  };

  // Load i of stage Y (Y < n_iter): A of step Y, or B of step Y + DL.
  auto dma_one = [&](int Y, int i) __attribute__((always_inline)) {
    const bool is_a = i < LA;
    const int YS = is_a ? Y : Y + DL;  // the K-step this load belongs to
    const uint32_t dst = smem_addr + (is_a ? slot_off(Y) : b_off(YS)) + lds_off(i);
    const u32x4& rs = is_a ? rsrc_a : rsrc_b;
    // (i is a constant wherever this is called, so is_a picks the form at
    // compile time)
    auto load = [&](uint32_t v, uint32_t so) __attribute__((always_inline)) {
      if (is_a)
        dma16(rs, dst, v, so);
      else
        dma16<kStream>(rs, dst, v, so);
    };
    if constexpr (DL > 0) {
      if (YS >= n_iter) {  // past the end: keep the stage's load count
        load(kOOB, 0u);
        return;
      }
    }
    const int kt = korder.kt(YS);
    const uint32_t k2 = (uint32_t)(kt * BK * 2);
    if constexpr (kPartial) {
      // In the K-step that K ends in, a lane whose 16-byte chunk starts at
      // or past K reads nothing (an out-of-range offset: zeros); the other
      // lanes and steps read as usual.  A select on a per-lane predicate
      // that does not change in the loop, not a branch: a branch around
      // each load broke up the loop's MFMA schedule (calls with K % 64 != 0
      // ran 21 % slower than with K rounded up to 64).
      const bool tail = kt >= full_tiles;  // the same in every lane
      const bool past = full_tiles * BK + chunk2[(i < LA ? i : i - LA) & 1] * 8 >= a.K;
      load(tail && past ? kOOB : voff[i], k2);
      return;
    }
    load(voff[i], k2);
  };

  // Trim the chunk that straddles K in this thread's part of step Y's A and
  // B tiles (after their loads have landed).
  auto trim_tail = [&](int Y) __attribute__((always_inline)) {
    const int k0 = korder.kt(Y) * BK;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int ii = i < LA ? i : i - LA;
      const int keep = a.K - (k0 + chunk2[ii & 1] * 8);
      if (keep > 0 && keep < 8) {
        lds_u32x4* p = (lds_u32x4*)(smem + (i < LA ? slot_off(Y) : b_off(Y)) + (ii * T + tid) * 16);
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

  // With a B lead, the wait for step Y leaves the B loads of stage Y (B of
  // step Y + DL, the last LB loads that stage issues) in flight: loads land
  // in order, so the count still proves that A of step Y and everything
  // issued before it (B of step Y came with stage Y - DL) have landed.
  constexpr int kLeadSlack = DL > 0 ? L - LA : 0;
  static_assert((S - 2) * L + L / F + kLeadSlack < 64, "vmcnt range");

  // Wait until step Y's loads have landed in every wave and publish them;
  // `later` steps after Y (whole) may still be in flight.
  auto publish = [&](int Y, int later) __attribute__((always_inline)) {
    if constexpr (kRagged) {
      if (korder.kt(Y) == a.k_tiles - 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        trim_tail(Y);
      }
    }
    ring_wait_barrier_n_off<L, S - 2, kLeadSlack>(later);
  };

  typename Cfg::Acc acc[Cfg::kFragM][Cfg::kFragN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
        for (int r = 0; r < MF * MF / 64; ++r) acc[i][j][r] = 0.0f;
    if constexpr (MF == 16) mfma16_settle();
  };
  zero_acc();
  // B fragments alternate between two buffers per substep.  A fragments
  // too with 32 x 32 blocks; with 16 x 16 blocks (twice as many fragments)
  // there is one A buffer, and fragment fm of the next substep replaces
  // that of the current one as soon as its row of MFMAs has issued.
  constexpr int kABufs = MF == 16 ? 1 : 2;
  bf16x8 fa[kABufs][Cfg::kFragM], fb[2][Cfg::kFragN];

  // ---- prologue: steps 0..S-2 whole (head), group 0 of step S-1 (tail),
  // then wait for step 0 and read its first fragments --------------------
  constexpr int G = L / F;
  auto prologue_head = [&]() __attribute__((always_inline)) {
    if constexpr (DL > 0) {  // B of steps 0 .. DL-1 (later B comes with the stages)
#pragma unroll
      for (int p = 0; p < DL; ++p)
        if (p < n_iter)
#pragma unroll
          for (int i = LA; i < L; ++i) dma_one(p - DL, i);
    }
#pragma unroll
    for (int p = 0; p + 1 < S; ++p)
      if (p < n_iter)
#pragma unroll
        for (int i = 0; i < L; ++i) dma_one(p, i);
  };
  auto prologue_tail = [&]() __attribute__((always_inline)) {
    if (S - 1 < n_iter)
#pragma unroll
      for (int i = 0; i < G; ++i) dma_one(S - 1, i);
  };
  // In flight after step 0: steps 1 .. min(S-2, n_iter-1) whole and group 0
  // of step S-1 if it exists.  (With a persistent grid the previous unit's C
  // stores were issued between head and tail; loads land in order, so the
  // count below still proves that step 0 has landed.)
  auto prologue_wait = [&]() __attribute__((always_inline)) {
    if (n_iter > 0) {
      if constexpr (kRagged) {
        if (korder.kt(0) == a.k_tiles - 1) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          trim_tail(0);
        }
      }
      ring_wait_barrier_ng<L, S - 2, G, kLeadSlack>(min(S - 2, n_iter - 1), S - 1 < n_iter);
      read_frags<Cfg, SWZ>(smem + slot_off(0), smem + b_off(0), 0, wm, wn, lane, fa[0], fb[0]);
    }
  };
  prologue_head();
  prologue_tail();

  // ---- one K-step X.  V = 0: loads of steps X+S-1 (groups 1..F-1) and X+S
  // (group 0); V = 1: only those of step X+S-1; V = 2: none.
  auto step = [&](auto vc, int X) __attribute__((always_inline)) {
    constexpr int V = decltype(vc)::value;
    const lds_u8* sa = smem + slot_off(X);
    const lds_u8* sb = smem + b_off(X);
    constexpr_for<SUB>([&](auto kc_) __attribute__((always_inline)) {
      constexpr int kk = decltype(kc_)::value;
      constexpr int cur = kk & 1, nxt = cur ^ 1;
      // load group carried by this substep, and the step it belongs to
      constexpr bool kLast = kk == SUB - 1;
      constexpr int grp = kLast ? 0 : kk + 1;
      constexpr bool kLoads = kLast ? V == 0 : (V <= 1 && grp < F);
      const int Y = kLast ? X + S : X + S - 1;
      // fragments read during this substep: substep kk+1 of step X, or
      // substep 0 of step X+1 once it is published
      const lds_u8* read_a = kLast ? smem + slot_off(X + 1) : sa;
      const lds_u8* read_b = kLast ? smem + b_off(X + 1) : sb;
      constexpr int rkk = kLast ? 0 : kk + 1;
      const bool reads = !kLast || V <= 1 || X + 1 < n_iter;
      // MFMAs of this substep that run before the barrier (kLast only)
      constexpr int NM = Cfg::kFragM * Cfg::kFragN;
      constexpr int J0 = kLast && SUB == 2 ? NM / 2 : 0;
      constexpr int ca = MF == 16 ? 0 : cur, na = MF == 16 ? 0 : nxt;  // A buffers
      if constexpr (kLast) {
        if constexpr (J0 > 0) {
          if constexpr (MF == 16)
            mfma_each<Cfg, kHalf, 0, J0>(acc, fa[ca], fb[cur], [](auto) {});
          else
            mfma_range<Cfg, kHalf, 0, J0, 0>(acc, fa[ca], fb[cur], [](auto) {});
          // MFMAs touch no memory, so without this the scheduler would move
          // them past the barrier
          __builtin_amdgcn_sched_barrier(0);
        }
        // in flight after step X+1: steps X+2 .. min(X+S-1, n_iter-1)
        if (reads) publish(X + 1, V <= 1 ? S - 2 : min(S - 2, n_iter - 2 - X));
        if constexpr (J0 > 0) __builtin_amdgcn_sched_barrier(0);
      }
      constexpr int NL = kLoads ? G : 0;
      if constexpr (MF == 16) {
        // Where each operation goes (after which MFMA j of the substep; j
        // counts fm-major).  Substep 0 issues its loads (the group that
        // must land by this step's barrier) in its first half, i.e. the
        // first quarter of the step as with 32 x 32 blocks: at the clock
        // these MFMAs run at, a step is short enough that loads spread
        // further stall the barrier.  A fragment i of the next substep may
        // replace the current one only after MFMA i*FN + FN-1, the last of
        // row i.  Row 0 of the next substep needs A fragment 0 and every B
        // fragment, so those are read first: in substep 0 the B fragments
        // over its middle half, in the last substep (where reads wait for
        // the barrier, and the loads, a step ahead, are spread over the
        // rest) A0, B0 .. B(FN-1), A1, ... evenly over the MFMAs after it.
        constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN, NR = FM + FN, n = NM - J0;
        auto pos_a = [](int i) constexpr {
          const int row_end = i * FN + FN - 1;
          const int want = kLast ? J0 + ((i == 0 ? 0 : FN + i) * n) / NR : row_end;
          return want > row_end ? want : row_end;
        };
        auto pos_b = [](int i) constexpr {
          return kLast ? J0 + ((1 + i) * n) / NR : n / 4 + (i * n) / (2 * FN);
        };
        constexpr int load_span = kLast ? n : n / 2;
        mfma_each<Cfg, kHalf, J0, NM>(
            acc, fa[0], fb[cur], [&](auto jc) __attribute__((always_inline)) {
              constexpr int j = decltype(jc)::value;
              constexpr_for<NR>([&](auto rc) __attribute__((always_inline)) {
                constexpr int r = decltype(rc)::value;  // A fragments, then B
                constexpr int at = r < FM ? pos_a(r) : pos_b(r - FM);
                if constexpr ((at < NM - 1 ? at : NM - 1) == j) {
                  if (reads)
                    read_frag_one<Cfg, SWZ, r>(read_a, read_b, rkk, wm, wn, lane, fa[0],
                                               fb[nxt]);
                  __builtin_amdgcn_sched_barrier(0);
                }
              });
              constexpr_for<NL>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                if constexpr (J0 + ((2 * q + 1) * load_span) / (2 * NL) == j) {
                  dma_one(Y, grp * G + q);
                  __builtin_amdgcn_sched_barrier(0);
                }
              });
            });
      } else {
        // The reads (in the order the next substep needs them) and the loads
        // alternate between the MFMAs, evenly: issued back to back, the
        // reads of four waves leaving a barrier together queue in the LDS
        // ahead of their MFMAs, and a burst of loads fills the texture path.
        constexpr int NR = Cfg::kFragM + Cfg::kFragN;
        mfma_range<Cfg, kHalf, J0, NM, NR + NL>(
            acc, fa[ca], fb[cur], [&](auto qc) __attribute__((always_inline)) {
              constexpr int p = decltype(qc)::value;
              constexpr int rb = p * NR / (NR + NL), rn = (p + 1) * NR / (NR + NL);
              if constexpr (rn > rb) {
                if (reads)
                  read_frag_one<Cfg, SWZ, frag_need_order<Cfg>(rb)>(
                      read_a, read_b, rkk, wm, wn, lane, fa[na], fb[nxt]);
              } else {
                dma_one(Y, grp * G + (p - rb));
              }
            });
      }
    });
  };

  // The unit's main loop, from its first fragments to its last MFMA.
  auto run_unit = [&]() __attribute__((always_inline)) {
    prologue_wait();
    int X = 0;
    for (; X < n_iter - S; ++X) step(std::integral_constant<int, 0>{}, X);
    if (n_iter >= S) {
      step(std::integral_constant<int, 1>{}, X);
      ++X;
    }
    for (; X < n_iter; ++X) step(std::integral_constant<int, 2>{}, X);
    if constexpr (MF == 16) mfma16_settle();
  };

  if constexpr (!kPersist) {
    run_unit();
    finish_tile<Cfg, kStore, kSplit>(a, smem, wave, m0, n0, acc, m0 + wm * Cfg::kWaveM,
                                     n0 + wn * Cfg::kWaveN, lane, split);
  } else {
    for (;;) {
      run_unit();
      // C of this unit drains through slot 0 while the next unit's steps
      // 0 .. S-2 land in slots 1 .. S-1.
      const int em0 = m0, en0 = n0;
      const int next = unit + (int)gridDim.x;
      const bool more = next < units;
      // every wave is done with the ring (its last fragments are read)
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (more) {
        setup(next);
        prologue_head();
      }
      finish_tile<Cfg, kStore, false, Cfg::kStageBytes, false>(
          a, smem, wave, em0, en0, acc, em0 + wm * Cfg::kWaveM, en0 + wn * Cfg::kWaveN, lane, 0);
      if (!more) return;
      // every wave has read its staged rows back before slot 0 is refilled
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      prologue_tail();
      unit = next;
      zero_acc();
    }
  }
}

}  // namespace gemm
