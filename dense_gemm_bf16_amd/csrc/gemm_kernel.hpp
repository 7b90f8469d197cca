// Dense bf16 GEMM kernel for gfx950 (CDNA4):  C[M,N] = A[M,K] * B[N,K]^T.
//
// One workgroup computes one BM x BN tile of C over a range of K (the whole
// of K, or one slice when K is split).  The steps, and where the pages
// describe the idea they adapt:
//
//  1. Tile rasterisation.  Workgroup ids are dealt round-robin to the eight
//     XCDs, each with its own L2.  The id is first remapped so that every XCD
//     receives a contiguous run of logical tiles, and logical tiles are
//     ordered in groups of `group_m` tile rows, so tiles resident on one XCD
//     at the same time share A rows and B columns in that XCD's L2.  (Page
//     "Matrix Multiplication on NVIDIA's Blackwell", Kernel 9: thread-block
//     swizzle for L2 reuse; the XCD split is specific to this chip.)
//
//  2. Global -> LDS staging through an S-slot ring.  Each K-step of BK = 64
//     copies A[m0:m0+BM, k:k+64] and B[n0:n0+BN, k:k+64] (rows of 128 bytes)
//     into one ring slot with buffer_load ... lds (16 bytes per lane, straight
//     into LDS, no VGPR round trip).  Loads for step t+S-1 are in flight while
//     step t computes.  (Page "Hand-writing a Blackwell GEMM", Step 2: a
//     multi-stage shared-memory pipeline; page "Matrix Multiplication on
//     NVIDIA's Blackwell", Kernel 6: a ring of stages.)  Out-of-range rows
//     and K-chunks read as zero through the buffer resource's range check.
//
//  3. XOR swizzle.  Within each 128-byte LDS row the 16-byte chunk index is
//     XORed with a function of the row, a permutation inside the row, so the
//     reads of one 16-byte column across consecutive rows land in different
//     LDS banks.  (Page "Hand-writing a Blackwell GEMM", Step 4: 128B
//     swizzle; page "Matrix Multiplication on NVIDIA's Blackwell", appendix
//     on the swizzle functor: bits 7-9 of the byte offset XORed into bits
//     4-6.)  The LDS-DMA writes each lane's 16 bytes at a fixed position, so
//     the swizzle is applied by choosing which global chunk each lane fetches.
//
//  4. MFMA.  Each wave owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held as
//     32x32 fp32 blocks in registers, and per 16-wide K-step issues
//     v_mfma_f32_32x32x16_bf16 on fragments read from LDS with ds_read_b128.
//     The MFMA's first operand is taken from B and the second from A, so a
//     lane's accumulator holds four consecutive columns of one row of C,
//     which makes the output stores row-contiguous.  (Page "Hand-writing a
//     Blackwell GEMM", Step 1: C_tile = sum_k A_k B_k^T.)
//
//  5. Split-K (when K is sliced): each slice writes its fp32 partial tile to
//     a workspace, increments a per-tile counter, and the workgroup that
//     arrives last adds the partials in slice order 0..S-1 (a fixed order, so
//     results are reproducible) and runs the epilogue.  It then resets the
//     counter to zero for the next call.
//
//  6. Epilogue: fp32 -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32) and
//     predicated stores of 4 consecutive columns per lane (or fp32 for the
//     debug output).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kBK = 64;                 // K elements per ring slot (128 B rows)
constexpr uint32_t kOOB = 0x80000000u;  // voffset that fails the range check

struct KernelArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t lda, ldb, ldc;  // elements
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t k_tiles;            // ceil(K / kBK)
  int32_t splits;             // slices of K per tile (>= 1)
  int32_t k_tiles_per_split;  // every slice non-empty (host guarantees)
  int32_t group_m;            // raster group height in tiles
  float* partials;            // splits > 1: tiles * splits * BM * BN floats
  uint32_t* counters;         // splits > 1: one per tile, zero between calls
};

// Ring synchronisation: s_waitcnt vmcnt(N) lgkmcnt(0) then s_barrier.
// After it, this wave has at most N vector-memory ops outstanding (the later
// ring steps' loads) and no LDS op outstanding; after the barrier every wave
// of the workgroup has done the same.  Written as one asm statement with a
// memory clobber so that the compiler neither moves LDS accesses across it
// nor adds waits of its own for the LDS-DMA loads (which it cannot see).
template <int N>
__device__ __forceinline__ void ring_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 128-bit buffer resource (base, range in bytes) held in SGPRs.  Range
// checking is by offset against num_records (raw buffer, stride 0).
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
  r[3] = 0x00020000;  // 32-bit data format; raw (untyped) access
  return r;
}

// One LDS-DMA load: 16 bytes per lane from rsrc.base + voff + soff into LDS
// at lds_addr + 16*lane (M0 holds the wave's LDS base).  voff is range
// checked (out of range reads zero); soff is not.  The s_nop covers the
// M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds_addr, uint32_t voff,
                                      uint32_t soff) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds" ::"{m0}"(lds_addr),
      "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// Workgroup ids are dispatched round-robin over the 8 XCDs.  Remap so that
// XCD x handles logical ids [start_x, start_x + count_x), contiguous.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  constexpr int kXcd = 8;
  const int q = nwg / kXcd, r = nwg % kXcd;
  const int x = wg % kXcd, i = wg / kXcd;
  return x * q + (x < r ? x : r) + i;
}

// 16-byte chunk permutation inside a 128-byte LDS row.
template <int SWZ>
__device__ __forceinline__ int swz(int row) {
  if constexpr (SWZ == 0) return 0;                      // no swizzle
  else if constexpr (SWZ == 1) return row & 7;           // XOR with row mod 8
  else return (row ^ (row >> 3)) & 7;                    // also folds row/8
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int SWZ>
struct TileCfg {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kWaveM = BM / WAVES_M;
  static constexpr int kWaveN = BN / WAVES_N;
  static constexpr int kFragM = kWaveM / 32;
  static constexpr int kFragN = kWaveN / 32;
  static constexpr int kABytes = BM * kBK * 2;
  static constexpr int kBBytes = BN * kBK * 2;
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kLdsBytes = STAGES * kStageBytes;
  static constexpr int kLoadsA = kABytes / (kThreads * 16);
  static constexpr int kLoadsB = kBBytes / (kThreads * 16);
  static constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
  static constexpr int kRowsPerLoad = kThreads / 8;  // rows one load round covers
  static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile in 32-blocks");
  static_assert(kABytes % (kThreads * 16) == 0, "A tile splits into loads");
  static_assert(kBBytes % (kThreads * 16) == 0, "B tile splits into loads");
  static_assert(kLdsBytes <= 160 * 1024, "LDS is 160 KB per CU");
  static_assert(STAGES >= 2, "ring needs two slots");
  static_assert(kLoadsPerStage * (STAGES - 2) < 64, "vmcnt range");
};

// Issue the LDS-DMA loads of one operand tile (rows x 64 k) into LDS at
// byte address `dst`.  voff[i] holds row*ld*2 + chunk*16 (or kOOB for absent
// rows); the K offset goes in soffset, so this is only for K-steps that lie
// wholly inside K.
template <int NLOADS, int THREADS>
__device__ __forceinline__ void issue_tile_loads(const u32x4& rsrc, uint32_t dst,
                                                 const uint32_t (&voff)[NLOADS], int k0,
                                                 int wave) {
#pragma unroll
  for (int i = 0; i < NLOADS; ++i)
    dma16(rsrc, dst + (i * THREADS + wave * 64) * 16, voff[i], (uint32_t)(k0 * 2));
}

// The K-step that reaches past K: chunks starting at or beyond K are sent
// out of range (read as zero); the K offset moves into the range-checked
// voffset.
template <int NLOADS, int THREADS>
__device__ __forceinline__ void issue_tail_loads(const u32x4& rsrc, uint32_t dst,
                                                 const uint32_t (&voff)[NLOADS],
                                                 const int (&chunk)[NLOADS], int k0, int K,
                                                 int wave) {
#pragma unroll
  for (int i = 0; i < NLOADS; ++i) {
    const uint32_t v = (k0 + chunk[i] * 8) < K ? voff[i] + (uint32_t)(k0 * 2) : kOOB;
    dma16(rsrc, dst + (i * THREADS + wave * 64) * 16, v, 0u);
  }
}

// Zero the elements k >= K of this lane's own chunks of the tail K-step.
// Needed only when K is not a multiple of 8, where one 16-byte chunk
// straddles K.  Must run after this wave's loads of that step have landed.
template <int NLOADS, int THREADS>
__device__ __forceinline__ void fix_tail_chunks(lds_u8* dst, const int (&chunk)[NLOADS], int k0,
                                                int K, int tid) {
#pragma unroll
  for (int i = 0; i < NLOADS; ++i) {
    const int keep = K - (k0 + chunk[i] * 8);  // elements of this chunk below K
    if (keep > 0 && keep < 8) {
      __attribute__((address_space(3))) u32x4* p =
          (__attribute__((address_space(3))) u32x4*)(dst + (i * THREADS + tid) * 16);
      u32x4 v = *p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e = 2 * w;  // elements e, e+1 live in dword w
        const uint32_t m = (e + 1 < keep) ? 0xFFFFFFFFu : (e < keep ? 0x0000FFFFu : 0u);
        v[w] &= m;
      }
      *p = v;
    }
  }
}

// Variant flags of the kernel template.
enum : int {
  kOutF32 = 1,   // store the fp32 sums (debug output) instead of bf16
  kSplitK = 2,   // K is sliced across workgroups; reduce through the workspace
  kRaggedK = 4,  // K % 8 != 0: patch the 16-byte chunk that straddles K
};

template <typename Cfg, bool OUT_F32>
__device__ __forceinline__ void store_tile(const KernelArgs& a,
                                           const f32x16 (&acc)[Cfg::kFragM][Cfg::kFragN],
                                           int m_base, int n_base, int lane) {
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm) {
    const int m = m_base + fm * 32 + (lane & 31);
    if (m >= a.M) continue;
#pragma unroll
    for (int fn = 0; fn < Cfg::kFragN; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // lane holds C[m][n .. n+3] in acc[fm][fn][4g .. 4g+3]
        const int n = n_base + fn * 32 + 8 * g + 4 * (lane >> 5);
        const f32x4 v = {acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
                         acc[fm][fn][4 * g + 3]};
        if constexpr (OUT_F32) {
          float* c = (float*)a.C + (int64_t)m * a.ldc + n;
          if (n + 3 < a.N) {
            *(f32x4*)c = v;
          } else {
            for (int j = 0; j < 4; ++j)
              if (n + j < a.N) c[j] = v[j];
          }
        } else {
          const bf16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2);
          const bf16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2);
          __bf16* c = (__bf16*)a.C + (int64_t)m * a.ldc + n;
          if (n + 3 < a.N) {
            *(bf16x4*)c = (bf16x4){lo[0], lo[1], hi[0], hi[1]};
          } else {
            const __bf16 e[4] = {lo[0], lo[1], hi[0], hi[1]};
            for (int j = 0; j < 4; ++j)
              if (n + j < a.N) c[j] = e[j];
          }
        }
      }
    }
  }
}

// Read the MFMA fragments of one 16-wide K-substep from a ring slot.
// Lane l supplies 8 consecutive k of row (l % 32) at 16-byte chunk
// 2*kk + l/32 of that row's 128 bytes.
template <typename Cfg, int SWZ>
__device__ __forceinline__ void read_frags(const lds_u8* sa, const lds_u8* sb, int kk, int wm,
                                           int wn, int lane, bf16x8 (&fa)[Cfg::kFragM],
                                           bf16x8 (&fb)[Cfg::kFragN]) {
  typedef const __attribute__((address_space(3))) bf16x8 lds_frag;
  const int lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm) {
    const int row = wm * Cfg::kWaveM + fm * 32 + lrow;
    fa[fm] = *(lds_frag*)(sa + row * 128 + (((2 * kk + lhalf) ^ swz<SWZ>(row)) << 4));
  }
#pragma unroll
  for (int fn = 0; fn < Cfg::kFragN; ++fn) {
    const int row = wn * Cfg::kWaveN + fn * 32 + lrow;
    fb[fn] = *(lds_frag*)(sb + row * 128 + (((2 * kk + lhalf) ^ swz<SWZ>(row)) << 4));
  }
}

template <typename Cfg>
__device__ __forceinline__ void mfma_block(f32x16 (&acc)[Cfg::kFragM][Cfg::kFragN],
                                           const bf16x8 (&fa)[Cfg::kFragM],
                                           const bf16x8 (&fb)[Cfg::kFragN]) {
  // D[n][m] += sum_k B[n][k] * A[m][k]: first operand from B, second from A.
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Cfg::kFragN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fn], fa[fm], acc[fm][fn], 0, 0, 0);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int SWZ, int FLAGS>
__global__ __attribute__((amdgpu_flat_work_group_size(WAVES_M * WAVES_N * 64,
                                                      WAVES_M * WAVES_N * 64),
                          amdgpu_waves_per_eu(1, 1))) void
gemm_bf16_kernel(KernelArgs a) {
  using Cfg = TileCfg<BM, BN, WAVES_M, WAVES_N, STAGES, SWZ>;
  constexpr int T = Cfg::kThreads;
  constexpr bool kF32 = (FLAGS & kOutF32) != 0;
  constexpr bool kSplit = (FLAGS & kSplitK) != 0;
  constexpr bool kRagged = (FLAGS & kRaggedK) != 0;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[Cfg::kLdsBytes];
  lds_u8* const smem = (lds_u8*)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;  // LDS byte address

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---- which tile and which K-slice ------------------------------------
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
  const int full_tiles = a.K / kBK;  // k-tiles that need no K check

  // ---- buffer resources: tile-origin based, range = valid rows ----------
  const int rows_a = min(BM, a.M - m0);
  const int rows_b = min(BN, a.N - n0);
  const u32x4 rsrc_a = make_rsrc(a.A + (int64_t)m0 * a.lda, (uint32_t)(rows_a * a.lda * 2));
  const u32x4 rsrc_b = make_rsrc(a.B + (int64_t)n0 * a.ldb, (uint32_t)(rows_b * a.ldb * 2));

  // Per-lane load offsets.  Load i of this lane fills LDS slot
  // s = i*T + tid (16 B each): row s/8, position s%8, which holds logical
  // chunk (position ^ swz(row)) of that row.
  uint32_t voff_a[Cfg::kLoadsA], voff_b[Cfg::kLoadsB];
  int chunk_a[Cfg::kLoadsA], chunk_b[Cfg::kLoadsB];
#pragma unroll
  for (int i = 0; i < Cfg::kLoadsA; ++i) {
    const int s = i * T + tid, row = s >> 3, c = (s & 7) ^ swz<SWZ>(row);
    chunk_a[i] = c;
    voff_a[i] = row < rows_a ? (uint32_t)(row * a.lda * 2 + c * 16) : kOOB;
  }
#pragma unroll
  for (int i = 0; i < Cfg::kLoadsB; ++i) {
    const int s = i * T + tid, row = s >> 3, c = (s & 7) ^ swz<SWZ>(row);
    chunk_b[i] = c;
    voff_b[i] = row < rows_b ? (uint32_t)(row * a.ldb * 2 + c * 16) : kOOB;
  }

  auto issue_stage = [&](int it) {
    const int kt = kt_begin + it;
    const uint32_t base = smem_addr + (it % STAGES) * Cfg::kStageBytes;
    if (kt < full_tiles) {
      issue_tile_loads<Cfg::kLoadsA, T>(rsrc_a, base, voff_a, kt * kBK, wave);
      issue_tile_loads<Cfg::kLoadsB, T>(rsrc_b, base + Cfg::kABytes, voff_b, kt * kBK, wave);
    } else {
      issue_tail_loads<Cfg::kLoadsA, T>(rsrc_a, base, voff_a, chunk_a, kt * kBK, a.K, wave);
      issue_tail_loads<Cfg::kLoadsB, T>(rsrc_b, base + Cfg::kABytes, voff_b, chunk_b, kt * kBK,
                                        a.K, wave);
    }
  };

  f32x16 acc[Cfg::kFragM][Cfg::kFragN];
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- prologue: fill STAGES-1 slots ------------------------------------
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < n_iter) issue_stage(p);

  // ---- main loop ----------------------------------------------------------
  for (int it = 0; it < n_iter; ++it) {
    lds_u8* stage = smem + (it % STAGES) * Cfg::kStageBytes;
    if constexpr (kRagged) {
      if (kt_begin + it == a.k_tiles - 1) {
        // The last K-step: wait for all of this wave's loads, zero the part
        // of the chunk that straddles K, then publish with the barrier below.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        fix_tail_chunks<Cfg::kLoadsA, T>(stage, chunk_a, (kt_begin + it) * kBK, a.K, tid);
        fix_tail_chunks<Cfg::kLoadsB, T>(stage + Cfg::kABytes, chunk_b, (kt_begin + it) * kBK,
                                         a.K, tid);
      }
    }
    // This wave's loads for step `it` have landed once at most the later
    // steps' loads remain outstanding; its LDS accesses of the previous step
    // are done.  After the barrier the same holds for every wave, so slot
    // (it-1) % STAGES may be refilled.
    if (it + STAGES - 2 < n_iter) ring_wait_barrier<Cfg::kLoadsPerStage * (STAGES - 2)>();
    else ring_wait_barrier<0>();
    if (it + STAGES - 1 < n_iter) issue_stage(it + STAGES - 1);

    const lds_u8* sa = stage;
    const lds_u8* sb = stage + Cfg::kABytes;
    // Fragments are double-buffered across the four 16-wide substeps: the
    // reads for substep kk+1 are issued ahead of substep kk's MFMAs.
    constexpr int kReads = Cfg::kFragM + Cfg::kFragN;
    constexpr int kMfmas = Cfg::kFragM * Cfg::kFragN;
    bf16x8 fa[2][Cfg::kFragM], fb[2][Cfg::kFragN];
    read_frags<Cfg, SWZ>(sa, sb, 0, wm, wn, lane, fa[0], fb[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // DS reads
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      if (kk + 1 < kBK / 16) {
        read_frags<Cfg, SWZ>(sa, sb, kk + 1, wm, wn, lane, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
      }
      mfma_block<Cfg>(acc, fa[kk & 1], fb[kk & 1]);
      __builtin_amdgcn_sched_group_barrier(0x008, kMfmas, 0);  // MFMA
    }
  }

  const int m_base = m0 + wm * Cfg::kWaveM;
  const int n_base = n0 + wn * Cfg::kWaveN;

  if constexpr (kSplit) {
    // ---- split-K: publish the partial; the last arriver reduces ----------
    // Workspace layout: [tile][slice][q][thread] of float4, q = the lane's
    // float4 index (fm, fn, g), so every store and load is one contiguous
    // 16 B per lane.
    constexpr int Q = Cfg::kFragM * Cfg::kFragN * 4;
    f32x4* ws = (f32x4*)a.partials + (int64_t)t * a.splits * Q * T;
    {
      f32x4* mine = ws + (int64_t)split * Q * T;
#pragma unroll
      for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::kFragN; ++fn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int q = (fm * Cfg::kFragN + fn) * 4 + g;
            __builtin_nontemporal_store(
                (f32x4){acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
                        acc[fm][fn][4 * g + 3]},
                mine + q * T + tid);
          }
    }
    // Make this thread's partial visible device-wide before the count.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __shared__ uint32_t s_last;
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev =
          __hip_atomic_fetch_add(a.counters + t, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t last = (prev == (uint32_t)a.splits - 1) ? 1u : 0u;
      // every slice has counted: reset for the next call on this workspace
      if (last) __hip_atomic_store(a.counters + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // acc = p_0 + p_1 + ... + p_{S-1} in this order, whichever slice is last.
#pragma unroll
    for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
      for (int fn = 0; fn < Cfg::kFragN; ++fn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q = (fm * Cfg::kFragN + fn) * 4 + g;
          f32x4 sum = __builtin_nontemporal_load(ws + q * T + tid);
          for (int sl = 1; sl < a.splits; ++sl)
            sum += __builtin_nontemporal_load(ws + ((int64_t)sl * Q + q) * T + tid);
          acc[fm][fn][4 * g] = sum[0];
          acc[fm][fn][4 * g + 1] = sum[1];
          acc[fm][fn][4 * g + 2] = sum[2];
          acc[fm][fn][4 * g + 3] = sum[3];
        }
  }

  store_tile<Cfg, kF32>(a, acc, m_base, n_base, lane);
}

}  // namespace gemm
