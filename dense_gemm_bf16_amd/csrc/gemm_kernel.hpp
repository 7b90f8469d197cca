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
//  2. Global -> LDS staging through an S-slot ring.  Each K-step of BK
//     elements copies A[m0:m0+BM, k:k+BK] and B[n0:n0+BN, k:k+BK] (rows of
//     2*BK bytes) into one ring slot with buffer_load ... lds (16 bytes per
//     lane, straight into LDS, no VGPR round trip).  A slot is refilled as
//     soon as every wave has read its last fragments, so up to S-1 K-steps of
//     loads are in flight ahead of the MFMAs.  (Page "Hand-writing a
//     Blackwell GEMM", Step 2: a multi-stage shared-memory pipeline; page
//     "Matrix Multiplication on NVIDIA's Blackwell", Kernel 6: a ring of
//     stages.)  Out-of-range rows and K-chunks read as zero through the
//     buffer resource's range check.
//
//  3. XOR swizzle.  Within each LDS row the 16-byte chunk index is XORed
//     with a function of the row, a permutation inside the row, so the
//     ds_read_b128 fragment reads of one chunk column across 16 consecutive
//     rows (one LDS access phase of 16 lanes over 64 banks) land in 16
//     different 16-byte bank groups.  (Page "Hand-writing a Blackwell GEMM",
//     Step 4: 128B swizzle; page "Matrix Multiplication on NVIDIA's
//     Blackwell", appendix on the swizzle functor: high address bits XORed
//     into the 16-byte chunk bits.)  The LDS-DMA writes each lane's 16 bytes
//     at a fixed position, so the swizzle is applied by choosing which
//     global chunk each lane fetches.
//
//  4. MFMA.  Each wave owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held as
//     32x32 fp32 blocks in accumulator registers, and per 16-wide K substep
//     issues v_mfma_f32_32x32x16_bf16 on fragments read from LDS with
//     ds_read_b128.  The fragments of substep j+1 are read while substep j's
//     MFMAs run; across K-steps too, because the ring barrier sits before
//     the last substep.  The MFMA's first operand is taken from B and the
//     second from A, so a lane's accumulator holds four consecutive columns
//     of one row of C, which makes the output stores row-contiguous.  (Page
//     "Hand-writing a Blackwell GEMM", Step 1: C_tile = sum_k A_k B_k^T.)
//
//  5. Split-K (when the tiles alone cannot fill the chip): slice s of K
//     writes its fp32 partial tile, unrounded, to partial buffer s; a
//     separate reduction kernel (gemm_reduce.hip) then adds the slices in
//     the fixed order 0..S-1 and rounds once, so results are reproducible.
//
//  6. Epilogue: fp32 -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32) and
//     predicated stores of 4 consecutive columns per lane (or fp32 for the
//     debug output and the split-K partials).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr uint32_t kOOB = 0x80000000u;  // voffset that fails the range check

struct KernelArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;                 // output, or the fp32 partial buffers when K is split
  int64_t lda, ldb, ldc;   // elements
  float* part;             // split K: fp32 partial buffer of slice 0 (M x ldp)
  int64_t ldp;             // split K: row stride of the partial buffers (floats)
  int64_t part_stride;     // split K: floats between the partial buffers of two slices
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t k_tiles;            // ceil(K / BK)
  int32_t splits;             // slices of K per tile (>= 1)
  int32_t k_tiles_per_split;  // every slice non-empty (host guarantees)
  int32_t group_m;            // raster group height in tiles
  int32_t k_rot;              // K-step rotation stride per tile (0: none)
};

// Order of a workgroup's K-steps.  With rotation, the workgroup of tile t
// starts its K range at step (t * k_rot) mod n instead of 0 and wraps
// around, so that workgroups running at the same time read different
// K columns of the operands.  Rows of a power-of-two leading dimension would
// otherwise send them all to the same few memory channels.  Each workgroup
// still sums its steps in one fixed order, so results stay reproducible.
// (Plain values captured by copy: held as a struct captured by reference in
// the kernels' lambdas, the compiler once kept it in private memory and
// read it there without the initialising store.)
struct KOrder {
  int begin, n, rot;
  // global K-step of the workgroup's it-th step (0 <= it < n)
  __device__ __forceinline__ int kt(int it) const {
    const int j = it + rot;
    return begin + (j >= n ? j - n : j);
  }
};

__device__ __forceinline__ KOrder make_korder(const KernelArgs& a, int t, int kt_begin,
                                              int n_iter) {
  const int rot = a.k_rot > 0 && n_iter > 0 ? (int)(((int64_t)t * a.k_rot) % n_iter) : 0;
  return KOrder{kt_begin, n_iter, __builtin_amdgcn_readfirstlane(rot)};
}

// Variant flags of the kernel template.
enum : int {
  kOutF32 = 1,   // store the fp32 sums (debug output) instead of bf16
  kSplitK = 2,   // K is sliced across workgroups (fp32 partials, then a reduction)
  kRaggedK = 4,  // K % 8 != 0: patch the 16-byte chunk that straddles K
  kF16 = 8,      // operands (and the 16-bit output) are fp16 instead of bf16
  kPartialK = 16,  // K % BK != 0 (only the direct-to-LDS kernel has a variant for it)
  kPersistent = 32,  // persistent grid: each workgroup walks several tiles (direct-to-LDS)
  kStreamB = 64,     // B loads non-temporal (direct-to-LDS, small-M and burst kernels)
};

// What the epilogue writes.
enum : int { kStoreBf16 = 0, kStoreF16 = 1, kStoreF32 = 2 };

template <int FLAGS>
constexpr int store_kind() {
  return (FLAGS & kOutF32) ? kStoreF32 : (FLAGS & kF16) ? kStoreF16 : kStoreBf16;
}

// ---------------------------------------------------------------- primitives

// Wait until at most N vector-memory ops of this wave are outstanding and
// all its LDS ops are done, then barrier the workgroup.  One asm statement
// with a memory clobber, so that the compiler neither moves LDS accesses
// across it nor adds waits of its own for the LDS-DMA loads, which it does
// not see (they are issued from asm too).
template <int N>
__device__ __forceinline__ void ring_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ring_wait_barrier<STEP * n + OFF> for a run-time n in [0, MAXN].
template <int STEP, int MAXN, int OFF>
__device__ __forceinline__ void ring_wait_barrier_n_off(int n) {
  if constexpr (MAXN <= 0) {
    ring_wait_barrier<OFF>();
  } else {
    if (n >= MAXN) ring_wait_barrier<STEP * MAXN + OFF>();
    else ring_wait_barrier_n_off<STEP, MAXN - 1, OFF>(n);
  }
}

template <int STEP, int MAXN>
__device__ __forceinline__ void ring_wait_barrier_n(int n) {
  ring_wait_barrier_n_off<STEP, MAXN, 0>(n);
}

// ring_wait_barrier<STEP * n + (g ? G : 0) + OFF> for run-time n in
// [0, MAXN] and a run-time flag g.
template <int STEP, int MAXN, int G, int OFF = 0>
__device__ __forceinline__ void ring_wait_barrier_ng(int n, bool g) {
  if (g) ring_wait_barrier_n_off<STEP, MAXN, G + OFF>(n);
  else ring_wait_barrier_n_off<STEP, MAXN, OFF>(n);
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
// M0-write -> LDS-DMA hazard.  lds_addr and soff are the same in every lane;
// readfirstlane states that, so they are always given as scalar operands
// (the compiler's divergence analysis cannot always prove it).  NT marks the
// load non-temporal, for data that no other workgroup reads: with one row of
// tiles each element of B is read by exactly one workgroup, and streaming it
// past the L2 measured 12-15 % faster at M = 1 and 17 (B at 6.1 TB/s) and up
// to 6.5 % faster on M = 256 shapes, while loads that other workgroups
// share (A, or B with several rows of tiles) were much slower with it.
template <bool NT = false>
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds_addr, uint32_t voff,
                                      uint32_t soff) {
  if constexpr (NT)
    asm volatile(
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds" ::"{m0}"(
            __builtin_amdgcn_readfirstlane(lds_addr)),
        "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
  else
    asm volatile(
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds" ::"{m0}"(
            __builtin_amdgcn_readfirstlane(lds_addr)),
        "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
}

// LDS-DMA load with an instruction offset OFF (< 4096): 16 bytes per lane
// from rsrc.base + soff + voff + OFF into LDS at M0 + OFF + 16*lane.  The
// offset steps the LDS destination without rewriting M0, so consecutive
// loads that share M0 issue faster; `rsrc` must have its base moved back
// by OFF (see shifted_rsrc) so that the global address stays base + voff.
template <int OFF>
__device__ __forceinline__ void dma16_off(const u32x4& rsrc, uint32_t m0, uint32_t voff,
                                          uint32_t soff) {
  static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen offset:%4 lds" ::"{m0}"(
          __builtin_amdgcn_readfirstlane(m0)),
      "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "n"(OFF)
      : "memory");
}

// Buffer resource for dma16_off<back>: base moved back by `back` bytes and
// the range extended by as much, so voffset v addresses base + v and is in
// range exactly when v < num_bytes, whether or not the hardware counts the
// instruction offset in its range check.  (The host keeps num_bytes + back
// below 2^31, so kOOB stays out of range.)
__device__ __forceinline__ u32x4 shifted_rsrc(const void* base, uint32_t num_bytes,
                                              uint32_t back) {
  return make_rsrc((const uint8_t*)base - back, num_bytes + back);
}

// Workgroup ids are dispatched round-robin over the 8 XCDs.  Remap so that
// XCD x handles logical ids [start_x, start_x + count_x), contiguous.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  constexpr int kXcd = 8;
  const int q = nwg / kXcd, r = nwg % kXcd;
  const int x = wg % kXcd, i = wg / kXcd;
  return x * q + (x < r ? x : r) + i;
}

// 16-byte chunk permutation inside an LDS row of CPR chunks (CPR = BK / 8).
//   SWZ 0: none.
//   SWZ 1: XOR with row mod CPR.
//   SWZ 2: conflict-free for 16-lane phases over 64 four-byte banks: the
//          16 rows of a phase cover 16 distinct (row-in-256-bytes, chunk)
//          pairs.  128-byte rows: (row ^ row/8) mod 8; 64-byte rows:
//          (row / 4) mod 4.
//   SWZ 3: for 16 x 16 x 32 fragments, 128-byte rows: (row / 2) mod 8.
//          A fragment read takes 16 rows at two adjacent chunks in each
//          half-wave; counted on MI355X, the LDS serves 32 lanes (512
//          bytes) at a time, so rows 4 apart must land in different
//          chunk pairs, which SWZ 2 does not do for this pattern (bank
//          conflicts doubled the read time).  It repeats every 16 rows, so
//          all fragments of a wave see one pattern and their read
//          addresses differ by constants.
template <int SWZ, int CPR>
__host__ __device__ constexpr int swz(int row) {
  if constexpr (SWZ == 0) return 0;
  else if constexpr (SWZ == 1) return row & (CPR - 1);
  else if constexpr (CPR == 8 && SWZ == 3) return (row >> 1) & 7;
  else if constexpr (CPR == 8) return (row ^ (row >> 3)) & 7;
  else return (row >> 2) & 3;
}

// MF is the MFMA block: 32 (v_mfma_f32_32x32x16, 16 of K per instruction,
// 16 accumulators per lane) or 16 (v_mfma_f32_16x16x32, 32 of K, 4
// accumulators per lane).  Both do the same work per cycle; under the power
// limit a stream of 16x16x32 MFMAs holds a higher clock (measured on MI355X:
// 1.86 vs 1.61 GHz, one wave per SIMD, random bf16 operands).
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int SWZ, int MF = 32>
struct TileCfg {
  static_assert(MF == 32 || MF == 16, "32x32x16 or 16x16x32 MFMA blocks");
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kBM = BM;
  static constexpr int kBN = BN;
  static constexpr int kMf = MF;          // rows (and columns) of one MFMA block
  static constexpr int kMfK = 512 / MF;   // K of one MFMA
  static constexpr int kWaveM = BM / WAVES_M;
  static constexpr int kWaveN = BN / WAVES_N;
  static constexpr int kFragM = kWaveM / MF;
  static constexpr int kFragN = kWaveN / MF;
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kCpr = BK / 8;      // 16-byte chunks per LDS row
  static constexpr int kSub = BK / kMfK;   // MFMA substeps per K-step
  using Acc = std::conditional_t<MF == 32, f32x16, f32x4>;  // one block's accumulators
  static constexpr int kABytes = BM * kRowBytes;
  static constexpr int kBBytes = BN * kRowBytes;
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kLdsBytes = STAGES * kStageBytes;
  static constexpr int kLoadsA = kABytes / (kThreads * 16);
  static constexpr int kLoadsB = kBBytes / (kThreads * 16);
  static constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
  static_assert(BK == 32 || BK == 64, "LDS rows of 64 or 128 bytes");
  static_assert(kWaveM % MF == 0 && kWaveN % MF == 0, "wave tile in MFMA blocks");
  static_assert(kABytes % (kThreads * 16) == 0, "A tile splits into loads");
  static_assert(kBBytes % (kThreads * 16) == 0, "B tile splits into loads");
  static_assert(kLdsBytes <= 160 * 1024, "LDS is 160 KB per CU");
  static_assert(STAGES >= 2, "ring needs two slots");
};

// ------------------------------------------------------------------- loads

// Issue the LDS-DMA loads of one operand tile (rows x BK) into LDS at byte
// address `dst`.  voff[i] holds row*ld*2 + chunk*16 (or kOOB for absent
// rows); the K offset goes in soffset, so this is only for K-steps that lie
// wholly inside K.
template <int NLOADS, int THREADS, bool NT = false>
__device__ __forceinline__ void issue_tile_loads(const u32x4& rsrc, uint32_t dst,
                                                 const uint32_t (&voff)[NLOADS], int k0,
                                                 int wave) {
#pragma unroll
  for (int i = 0; i < NLOADS; ++i)
    dma16<NT>(rsrc, dst + (i * THREADS + wave * 64) * 16, voff[i], (uint32_t)(k0 * 2));
}

// The K-step that reaches past K: chunks starting at or beyond K are sent
// out of range (read as zero); the K offset moves into the range-checked
// voffset.
template <int NLOADS, int THREADS, bool NT = false>
__device__ __forceinline__ void issue_tail_loads(const u32x4& rsrc, uint32_t dst,
                                                 const uint32_t (&voff)[NLOADS],
                                                 const int (&chunk)[NLOADS], int k0, int K,
                                                 int wave) {
#pragma unroll
  for (int i = 0; i < NLOADS; ++i) {
    const uint32_t v = (k0 + chunk[i] * 8) < K ? voff[i] + (uint32_t)(k0 * 2) : kOOB;
    dma16<NT>(rsrc, dst + (i * THREADS + wave * 64) * 16, v, 0u);
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

// --------------------------------------------------------------- fragments

// Read the MFMA fragments of one K substep (kMfK wide) from a ring slot.
// Lane l supplies 8 consecutive k of row (l % MF) at 16-byte chunk
// (kMfK / 8) * kk + l / MF of that row: for 32x32x16 blocks the two lane
// halves take the two 8-wide halves of the substep, for 16x16x32 blocks the
// four lane quarters its four 8-wide quarters.
template <typename Cfg, int SWZ>
__device__ __forceinline__ void read_frags(const lds_u8* sa, const lds_u8* sb, int kk, int wm,
                                           int wn, int lane, bf16x8 (&fa)[Cfg::kFragM],
                                           bf16x8 (&fb)[Cfg::kFragN]) {
  typedef const __attribute__((address_space(3))) bf16x8 lds_frag;
  constexpr int R = Cfg::kRowBytes, CPR = Cfg::kCpr, MF = Cfg::kMf;
  const int lrow = lane % MF, chunk = (Cfg::kMfK / 8) * kk + lane / MF;
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm) {
    const int row = wm * Cfg::kWaveM + fm * MF + lrow;
    fa[fm] = *(lds_frag*)(sa + row * R + ((chunk ^ swz<SWZ, CPR>(row)) << 4));
  }
#pragma unroll
  for (int fn = 0; fn < Cfg::kFragN; ++fn) {
    const int row = wn * Cfg::kWaveN + fn * MF + lrow;
    fb[fn] = *(lds_frag*)(sb + row * R + ((chunk ^ swz<SWZ, CPR>(row)) << 4));
  }
}

// One MFMA, D[n][m] += sum_k B[n][k] * A[m][k] (first operand from B, second
// from A): 32 x 32 x 16 on a 16-float accumulator block, 16 x 16 x 32 on a
// 4-float one.  The fragments hold raw 16-bit patterns; HALF reads them as
// fp16, otherwise as bf16.
template <bool HALF>
__device__ __forceinline__ f32x16 mfma_op(const bf16x8& b, const bf16x8& a, const f32x16& c) {
  if constexpr (HALF)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, b),
                                                  __builtin_bit_cast(f16x8, a), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
}
// The 16 x 16 x 32 form is written as asm with the accumulator tied in
// AGPRs: with the builtin, the compiler gave some of a 128 x 128 wave tile's
// 64 MFMAs a destination other than their accumulator input, and with all
// 256 AGPRs holding accumulators it then shuffled blocks through VGPRs
// every K-step.  The compiler cannot see the MFMA's latency through asm,
// so callers separate the accumulators' VALU writes before the first and
// reads after the last of these MFMAs by mfma16_settle().
template <bool HALF>
__device__ __forceinline__ f32x4 mfma_op(const bf16x8& b, const bf16x8& a, const f32x4& c) {
  f32x4 d = c;
  if constexpr (HALF)
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(d) : "v"(b), "v"(a));
  else
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(b), "v"(a));
  return d;
}

// Wait states between VALU accesses of accumulators and the asm MFMAs
// above (a 4-pass MFMA's result is readable 18 wait states after issue;
// 32 here), fenced so the scheduler moves nothing across.
__device__ __forceinline__ void mfma16_settle() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The order in which the MFMAs of a substep (fm-major, fn inner) first use
// their fragments: entry r is the r-th fragment needed, numbered as in
// read_frag_one (A fragments 0..kFragM-1, then B fragments).
template <typename Cfg>
constexpr int frag_need_order(int r) {
  bool seen[Cfg::kFragM + Cfg::kFragN] = {};
  int n = 0;
  for (int j = 0; j < Cfg::kFragM * Cfg::kFragN; ++j) {
    const int a = j / Cfg::kFragN, b = Cfg::kFragM + j % Cfg::kFragN;
    if (!seen[b]) {
      if (n++ == r) return b;
      seen[b] = true;
    }
    if (!seen[a]) {
      if (n++ == r) return a;
      seen[a] = true;
    }
  }
  return -1;
}

// Fragment IDX of read_frags alone (A fragments first, then B), so that the
// reads of a substep can be spread between MFMAs.
template <typename Cfg, int SWZ, int IDX>
__device__ __forceinline__ void read_frag_one(const lds_u8* sa, const lds_u8* sb, int kk, int wm,
                                              int wn, int lane, bf16x8 (&fa)[Cfg::kFragM],
                                              bf16x8 (&fb)[Cfg::kFragN]) {
  typedef const __attribute__((address_space(3))) bf16x8 lds_frag;
  constexpr int R = Cfg::kRowBytes, CPR = Cfg::kCpr, MF = Cfg::kMf;
  const int lrow = lane % MF, chunk = (Cfg::kMfK / 8) * kk + lane / MF;
  if constexpr (IDX < Cfg::kFragM) {
    const int row = wm * Cfg::kWaveM + IDX * MF + lrow;
    fa[IDX] = *(lds_frag*)(sa + row * R + ((chunk ^ swz<SWZ, CPR>(row)) << 4));
  } else {
    const int row = wn * Cfg::kWaveN + (IDX - Cfg::kFragM) * MF + lrow;
    fb[IDX - Cfg::kFragM] = *(lds_frag*)(sb + row * R + ((chunk ^ swz<SWZ, CPR>(row)) << 4));
  }
}

template <typename Cfg, bool HALF>
__device__ __forceinline__ void mfma_block(typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                           const bf16x8 (&fa)[Cfg::kFragM],
                                           const bf16x8 (&fb)[Cfg::kFragN]) {
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Cfg::kFragN; ++fn)
      acc[fm][fn] = mfma_op<HALF>(fb[fn], fa[fm], acc[fm][fn]);
}

// Call f(std::integral_constant<int, i>) for i = 0 .. N-1 in order.
template <int I, int N>
struct ConstexprFor {
  template <typename Fn>
  __device__ __forceinline__ static void run(Fn&& f) {
    if constexpr (I < N) {
      f(std::integral_constant<int, I>{});
      ConstexprFor<I + 1, N>::run(f);
    }
  }
};
template <int N, typename Fn>
__device__ __forceinline__ void constexpr_for(Fn&& f) {
  ConstexprFor<0, N>::run(f);
}

// Call f(lo, hi) with compile-time integral constants lo = w*L/F and
// hi = (w+1)*L/F (empty range for w >= F), for a run-time w in [1, 4].
template <int F, int L, typename Fn>
__device__ __forceinline__ void constexpr_for_window(int w, Fn&& f) {
  auto call = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr int lo = W < F ? W * L / F : L;
    constexpr int hi = W < F ? (W + 1) * L / F : L;
    f(std::integral_constant<int, lo>{}, std::integral_constant<int, hi>{});
  };
  switch (w) {
    case 1: call(std::integral_constant<int, 1>{}); break;
    case 2: call(std::integral_constant<int, 2>{}); break;
    case 3: call(std::integral_constant<int, 3>{}); break;
    default: call(std::integral_constant<int, 4>{}); break;
  }
}

// The MFMAs of one substep with G loads spaced evenly between them: load q
// goes after MFMA ceil((q+1)*n/G) - 1, and a scheduling barrier keeps each
// load at its place in the MFMA stream.
template <typename Cfg, bool HALF, int G, typename Dma>
__device__ __forceinline__ void mfma_block_dma(typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                               const bf16x8 (&fa)[Cfg::kFragM],
                                               const bf16x8 (&fb)[Cfg::kFragN], Dma&& dma) {
  constexpr int n = Cfg::kFragM * Cfg::kFragN;
#pragma unroll
  for (int j = 0; j < n; ++j) {
    const int fm = j / Cfg::kFragN, fn = j % Cfg::kFragN;
    acc[fm][fn] = mfma_op<HALF>(fb[fn], fa[fm], acc[fm][fn]);
#pragma unroll
    for (int q = (j * G) / n; q < ((j + 1) * G) / n; ++q) {
      dma(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// MFMAs J0 .. J1-1 of one substep (fm-major, fn inner) with G operations
// spaced evenly between them (op q right after the j-th of them for q in
// [j*G/n, (j+1)*G/n), n = J1 - J0, so several per MFMA when G > n), each
// pinned in place by a scheduling barrier.
template <typename Cfg, bool HALF, int J0, int J1, int G, int J = J0, typename Op>
__device__ __forceinline__ void mfma_range(typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                           const bf16x8 (&fa)[Cfg::kFragM],
                                           const bf16x8 (&fb)[Cfg::kFragN], Op&& op) {
  constexpr int n = J1 - J0;
  if constexpr (J < J1) {
    constexpr int fm = J / Cfg::kFragN, fn = J % Cfg::kFragN;
    acc[fm][fn] = mfma_op<HALF>(fb[fn], fa[fm], acc[fm][fn]);
    constexpr int qlo = ((J - J0) * G) / n, qhi = ((J - J0 + 1) * G) / n;
    constexpr_for<qhi - qlo>([&](auto qc) __attribute__((always_inline)) {
      op(std::integral_constant<int, qlo + decltype(qc)::value>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    mfma_range<Cfg, HALF, J0, J1, G, J + 1>(acc, fa, fb, op);
  }
}

// MFMAs J0 .. J1-1 of one substep (fm-major, fn inner), calling
// after(std::integral_constant<int, j>) after MFMA j.
template <typename Cfg, bool HALF, int J0, int J1, int J = J0, typename After>
__device__ __forceinline__ void mfma_each(typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                          const bf16x8 (&fa)[Cfg::kFragM],
                                          const bf16x8 (&fb)[Cfg::kFragN], After&& after) {
  if constexpr (J < J1) {
    constexpr int fm = J / Cfg::kFragN, fn = J % Cfg::kFragN;
    acc[fm][fn] = mfma_op<HALF>(fb[fn], fa[fm], acc[fm][fn]);
    after(std::integral_constant<int, J>{});
    mfma_each<Cfg, HALF, J0, J1, J + 1>(acc, fa, fb, after);
  }
}

// All MFMAs of one substep with G operations spaced evenly between them.
template <typename Cfg, bool HALF, int G, typename Op>
__device__ __forceinline__ void mfma_interleave(typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                                const bf16x8 (&fa)[Cfg::kFragM],
                                                const bf16x8 (&fb)[Cfg::kFragN], Op&& op) {
  mfma_range<Cfg, HALF, 0, Cfg::kFragM * Cfg::kFragN, G>(acc, fa, fb, op);
}

// True if swz(i*RPI + r) == swz((i & 1)*RPI + r) for all i < n, r < RPI.
template <int SWZ, int CPR, int RPI, int n>
constexpr bool swz_period_two() {
  for (int i = 0; i < n; ++i)
    for (int r = 0; r < RPI; ++r)
      if (swz<SWZ, CPR>(i * RPI + r) != swz<SWZ, CPR>((i & 1) * RPI + r)) return false;
  return true;
}

// ---------------------------------------------------------------- epilogue

// Four fp32 sums as four 16-bit values of OUT (kStoreBf16 / kStoreF16),
// rounded to nearest even, packed little-endian into two dwords.
template <int OUT>
__device__ __forceinline__ u32x2 pack_quad(const f32x4& v) {
  using T = std::conditional_t<OUT == kStoreF16, _Float16, __bf16>;
  typedef T t2 __attribute__((ext_vector_type(2)));
  const t2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, t2);
  const t2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, t2);
  return (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Store 4 consecutive fp32 sums v at row m, columns n .. n+3 of C, converted
// to OUT (kStoreBf16 / kStoreF16 / kStoreF32; the 16-bit conversions round to
// nearest even).  Columns >= N are skipped; the caller checks m < M.
template <int OUT>
__device__ __forceinline__ void store_quad(void* Cbase, int64_t ld, const f32x4& v, int m, int n,
                                           int N) {
  if constexpr (OUT == kStoreF32) {
    float* c = (float*)Cbase + (int64_t)m * ld + n;
    if (n + 3 < N) {
      *(f32x4*)c = v;
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < N) c[j] = v[j];
    }
  } else {
    const u32x2 q = pack_quad<OUT>(v);
    uint16_t* c = (uint16_t*)Cbase + (int64_t)m * ld + n;
    if (n + 3 < N) {
      *(u32x2*)c = q;
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < N) c[j] = (uint16_t)(q[j >> 1] >> (16 * (j & 1)));
    }
  }
}

// Accumulator layout of one MF x MF block (first MFMA operand from B,
// second from A): lane l holds row l % MF of the block, and its quad g
// (elements 4g .. 4g+3) holds the four consecutive columns starting at
// quad_col(g, l).  32 x 32 blocks: four quads, columns 8g + 4 (l / 32);
// 16 x 16 blocks: one quad, columns 4 (l / 16).
template <int MF>
__device__ __forceinline__ int quad_col(int g, int lane) {
  return 4 * (g * (64 / MF) + lane / MF);
}

// Store one accumulator block whose rows start at m0 and columns at n0.
// Rows >= M and columns >= N are skipped.
template <typename Cfg, int OUT>
__device__ __forceinline__ void store_block(void* Cbase, int64_t ld, const typename Cfg::Acc& blk,
                                            int m0, int n0, int lane, int M, int N) {
  constexpr int MF = Cfg::kMf;
  const int m = m0 + lane % MF;
  if (m >= M) return;
#pragma unroll
  for (int g = 0; g < MF * MF / 256; ++g)
    store_quad<OUT>(Cbase, ld, (f32x4){blk[4 * g], blk[4 * g + 1], blk[4 * g + 2], blk[4 * g + 3]},
                    m, n0 + quad_col<MF>(g, lane), N);
}

// The wave's accumulator blocks into C (bf16 or fp16, or fp32 for the debug
// output).
template <typename Cfg, int OUT>
__device__ __forceinline__ void store_tile(const KernelArgs& a, void* Cbase, int64_t ld,
                                           const typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                           int m_base, int n_base, int lane) {
#pragma unroll
  for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Cfg::kFragN; ++fn)
      store_block<Cfg, OUT>(Cbase, ld, acc[fm][fn], m_base + fm * Cfg::kMf,
                            n_base + fn * Cfg::kMf, lane, a.M, a.N);
}

// ------------------------------------------------- epilogue through LDS
//
// Stored straight from the accumulators, one store instruction writes 8 or
// 16 bytes into each of 32 rows (a lane holds 4 consecutive columns of one
// row), and the L2 takes one partial-line write per row and instruction: on
// MI355X that made the 256 x 256 tile's bf16 epilogue take 8-10 us.  Once
// the LDS ring is idle (after the main loop), the waves instead write their
// accumulator blocks into LDS and read them back by rows, so that 16
// consecutive lanes store 256 contiguous bytes of one row (whole 128-byte
// lines).
//
// Staging layout, per wave: row r of the wave block (kRB bytes) holds
// 16-byte chunk c at r*kRB + 16 (c ^ sw(r)), sw(r) = r % 16, or (r / 2) % 8
// for 128-byte rows.  A write instruction covers MF rows (lanes l and l + MF
// take the same row), a 16-byte read 64 / (kRB / 16) whole rows; with that
// XOR both fall in distinct banks, except that with 32 x 32 blocks rows r
// and r + 16 of one 16-bit write would share them, so there the two 8-byte
// halves of every chunk are swapped in rows with r % 32 >= 16.  Blocks too
// large for the LDS the staging may use (LIMIT bytes: the whole ring, or one
// slot of it while the other slots receive the next tile's first K-steps)
// go in passes of 32 rows through two alternating buffers.
template <typename Cfg, int OUT, int LIMIT = Cfg::kLdsBytes>
struct LdsStage {
  static constexpr int kMf = Cfg::kMf;
  static constexpr int kE = OUT == kStoreF32 ? 4 : 2;  // bytes per element
  static constexpr int kRB = Cfg::kWaveN * kE;         // bytes per staged row
  static constexpr bool kShape =
      kE == 4 ? (kRB == 256 || kRB == 512) : (kRB == 128 || kRB == 256);
  static constexpr int kWaves = Cfg::kThreads / 64;
  static constexpr bool kWhole = kWaves * Cfg::kWaveM * kRB <= LIMIT;
  // MFMA block rows per pass: all, or 32 rows
  static constexpr int kFmp = kWhole || Cfg::kFragM * kMf < 32 ? Cfg::kFragM : 32 / kMf;
  static constexpr int kPassRows = kFmp * kMf;
  static constexpr int kBufs = kFmp == Cfg::kFragM ? 1 : 2;
  static constexpr int kWaveBytes = kBufs * kPassRows * kRB;
  static constexpr bool kSwapHalves = kE == 2 && kMf == 32;
  static constexpr bool kOk = kShape && kWaves * kWaveBytes <= LIMIT;
  static_assert(Cfg::kFragM % kFmp == 0, "whole passes");

  __device__ static __forceinline__ uint32_t off(int r, int c) {
    const int sw = kRB == 128 ? (r >> 1) & 7 : r & 15;
    return (uint32_t)(r * kRB + ((c ^ sw) << 4));
  }
};

// NT stores the rows non-temporally: for C, which this kernel never reads
// back (measured 0.7-2 % faster at 4096^3 and 8192^3, where C would
// otherwise evict A and B panels from L2).  Split-K partials are stored
// normally, since the reduction reads them right after (non-temporal, their
// calls were ~1 % slower).  EDGE (a tile that C's last row or column cuts):
// rows at or past M are skipped, a 16-byte piece wholly inside N is stored
// whole, the one that N cuts element by element, pieces past N not at all.
template <typename Cfg, int OUT, int LIMIT = Cfg::kLdsBytes, bool NT = false, bool EDGE = false>
__device__ __forceinline__ void store_tile_lds(lds_u8* region, void* Cbase, int64_t ld,
                                               const typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                               int m_base, int n_base, int M = 0, int N = 0) {
  using St = LdsStage<Cfg, OUT, LIMIT>;
  static_assert(St::kOk, "staging fits the ring");
  // the lane index from the hardware rather than kept live through the main
  // loop (kept, it spilled to scratch in the 256 x 256 kernel)
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  constexpr int kE = St::kE, kRB = St::kRB, MF = Cfg::kMf;
  constexpr int LPR = kRB / 16;  // lanes per row when reading back
  constexpr int RPI = 64 / LPR;  // rows per read instruction (divides 16)
  static_assert(16 % RPI == 0, "a read instruction's rows share r / 16");
  static_assert(St::kPassRows % RPI == 0, "whole read instructions per pass");
  const int wr = lane % MF;
  const int rr = lane / LPR, rc = lane % LPR;
  uint8_t* out = (uint8_t*)Cbase + ((int64_t)(m_base + rr) * ld + n_base) * kE + rc * 16;
#pragma unroll
  for (int pass = 0; pass < Cfg::kFragM / St::kFmp; ++pass) {
    lds_u8* buf = region + (pass % St::kBufs) * (St::kPassRows * kRB);
#pragma unroll
    for (int fi = 0; fi < St::kFmp; ++fi) {
      const int r = fi * MF + wr;
#pragma unroll
      for (int fn = 0; fn < Cfg::kFragN; ++fn)
#pragma unroll
        for (int g = 0; g < MF * MF / 256; ++g) {
          const typename Cfg::Acc& b = acc[pass * St::kFmp + fi][fn];
          const f32x4 v = (f32x4){b[4 * g], b[4 * g + 1], b[4 * g + 2], b[4 * g + 3]};
          const int q4 = (fn * MF + quad_col<MF>(g, lane)) / 4;  // column / 4 in the wave row
          if constexpr (kE == 4) {
            *(__attribute__((address_space(3))) f32x4*)(buf + St::off(r, q4)) = v;
          } else {
            const uint32_t h = (uint32_t)((q4 ^ (St::kSwapHalves ? wr >> 4 : 0)) & 1);
            *(__attribute__((address_space(3))) u32x2*)(buf + St::off(r, q4 >> 1) + (h << 3)) =
                pack_quad<OUT>(v);
          }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < St::kPassRows / RPI; ++j) {
      const int r = j * RPI + rr;
      u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(buf + St::off(r, rc));
      if constexpr (St::kSwapHalves)
        if (((j * RPI) & 16) != 0) v = (u32x4){v[2], v[3], v[0], v[1]};
      u32x4* const dst = (u32x4*)(out + (int64_t)((pass * St::kPassRows + j * RPI) * kE) * ld);
      if constexpr (EDGE) {
        constexpr int kPer = 16 / kE;  // elements in a 16-byte piece
        const int row = m_base + pass * St::kPassRows + j * RPI + rr;
        const int col = n_base + rc * kPer;
        if (row >= M || col >= N) continue;
        if (col + kPer > N) {
#pragma unroll
          for (int e = 0; e < kPer; ++e) {
            if (col + e >= N) break;
            if constexpr (kE == 4)
              ((uint32_t*)dst)[e] = v[e];
            else
              ((uint16_t*)dst)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
          }
          continue;
        }
      }
      if constexpr (NT)
        __builtin_nontemporal_store(v, dst);
      else
        *dst = v;
    }
  }
}

// The epilogue of every kernel: C (OUT), or with SPLIT the K-slice's
// unrounded fp32 sums into its partial buffer (the reduction kernel in
// gemm_reduce.hip adds the slices in a fixed order), through LDS when the
// staging fits the ring, also for the tiles that C's last row or column
// cuts (their row pieces predicated; stored element by element from the
// accumulators instead, such tiles cost 3-4.5 % of a 4096^3-class call),
// else straight from the accumulators.  Called by all waves of the
// workgroup after the main loop (the LDS path has a barrier); the ring must
// not be written again.
// (An in-kernel reduction by the last slice to finish a tile was measured
// 2-3x slower: making the partials visible to the other XCDs needs a
// release fence per workgroup, which writes back that XCD's L2.)
template <typename Cfg, int OUT, bool SPLIT, int LIMIT = Cfg::kLdsBytes, bool kBarrier = true>
__device__ __forceinline__ void finish_tile(const KernelArgs& a, lds_u8* smem, int wave, int m0,
                                            int n0, const typename Cfg::Acc (&acc)[Cfg::kFragM][Cfg::kFragN],
                                            int m_base, int n_base, int lane, int split) {
  constexpr int kOut = SPLIT ? kStoreF32 : OUT;
  using St = LdsStage<Cfg, kOut, LIMIT>;
  void* const base = SPLIT ? (void*)(a.part + (int64_t)split * a.part_stride) : a.C;
  const int64_t ld = SPLIT ? a.ldp : a.ldc;
  if constexpr (St::kOk) {
    // every wave is done with the ring: loads landed, fragments read
    // (kBarrier false: the caller has made sure of it)
    if constexpr (kBarrier) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (m0 + Cfg::kBM <= a.M && n0 + Cfg::kBN <= a.N)
      store_tile_lds<Cfg, kOut, LIMIT, !SPLIT>(smem + wave * St::kWaveBytes, base, ld, acc,
                                               m_base, n_base);
    else
      store_tile_lds<Cfg, kOut, LIMIT, !SPLIT, true>(smem + wave * St::kWaveBytes, base, ld,
                                                     acc, m_base, n_base, a.M, a.N);
    return;
  }
  store_tile<Cfg, kOut>(a, base, ld, acc, m_base, n_base, lane);
}

// ------------------------------------------------------------------ kernel

// One workgroup per CU (the ring takes most of the 160 KB LDS): 4 waves run
// one per SIMD, 8 waves two per SIMD.
//
// PIPE selects how the LDS-DMA loads of a K-step are issued:
//   0 (burst):  all at once, right after the barrier that frees the slot;
//   1, 3, 4 (spread): one by one between MFMAs, over the first F substeps
//      of the window from that barrier to the next one (F = kSub, kSub-1,
//      kSub-2 for PIPE 1, 3, 4).
// A wave issues LDS-DMA loads at most about one per ~100 cycles (1 KB
// each), and while it waits to issue one, its in-order instruction stream
// cannot issue MFMAs either; a burst of loads therefore idles that SIMD's
// MFMA pipe.  Spread issue with at least three MFMAs between loads keeps
// the pipe busy.  With two ring slots, the loads of a step must land by the
// barrier that ends its window, so they are packed into the first F
// substeps and the rest of the window is latency slack.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int SWZ, int PIPE,
          int FLAGS>
__global__ __attribute__((amdgpu_flat_work_group_size(WAVES_M * WAVES_N * 64,
                                                      WAVES_M * WAVES_N * 64),
                          amdgpu_waves_per_eu(WAVES_M * WAVES_N / 4,
                                              WAVES_M * WAVES_N / 4))) void
gemm_bf16_kernel(KernelArgs a) {
  using Cfg = TileCfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, SWZ>;
  constexpr int T = Cfg::kThreads;
  constexpr int CPR = Cfg::kCpr;
  constexpr int LPS = Cfg::kLoadsPerStage;
  constexpr int LA = Cfg::kLoadsA;
  static_assert(PIPE != 2, "PIPE 2 is the ping-pong kernel");
  constexpr int kStore = store_kind<FLAGS>();
  constexpr bool kHalf = (FLAGS & kF16) != 0;
  constexpr bool kSplit = (FLAGS & kSplitK) != 0;
  constexpr bool kRagged = (FLAGS & kRaggedK) != 0;
  constexpr bool kStream = (FLAGS & kStreamB) != 0;  // B loads non-temporal
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
  const KOrder korder = make_korder(a, t, kt_begin, n_iter);
  const int full_tiles = a.K / BK;  // K-steps that need no K check

  // ---- buffer resources: tile-origin based, range = valid rows ----------
  const int rows_a = min(BM, a.M - m0);
  const int rows_b = min(BN, a.N - n0);
  const u32x4 rsrc_a = make_rsrc(a.A + (int64_t)m0 * a.lda, (uint32_t)(rows_a * a.lda * 2));
  const u32x4 rsrc_b = make_rsrc(a.B + (int64_t)n0 * a.ldb, (uint32_t)(rows_b * a.ldb * 2));

  // Per-lane load offsets.  Load i of this lane fills LDS slot
  // s = i*T + tid (16 B each): row s/CPR, position s%CPR, which holds
  // logical chunk (position ^ swz(row)) of that row.
  uint32_t voff_a[Cfg::kLoadsA], voff_b[Cfg::kLoadsB];
  int chunk_a[Cfg::kLoadsA], chunk_b[Cfg::kLoadsB];
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

  auto issue_stage = [&](int it) {
    const int kt = korder.kt(it);
    const uint32_t base = smem_addr + (it % STAGES) * Cfg::kStageBytes;
    if (kt < full_tiles) {
      issue_tile_loads<Cfg::kLoadsA, T>(rsrc_a, base, voff_a, kt * BK, wave);
      issue_tile_loads<Cfg::kLoadsB, T, kStream>(rsrc_b, base + Cfg::kABytes, voff_b, kt * BK,
                                                 wave);
    } else {
      issue_tail_loads<Cfg::kLoadsA, T>(rsrc_a, base, voff_a, chunk_a, kt * BK, a.K, wave);
      issue_tail_loads<Cfg::kLoadsB, T, kStream>(rsrc_b, base + Cfg::kABytes, voff_b, chunk_b,
                                                 kt * BK, a.K, wave);
    }
  };

  // Wait until step `it` has landed in every wave and publish it.  Steps
  // issued so far: 0 .. it+STAGES-2 (it >= 1; the refill of slot it-1
  // happens after this wait), or 0 .. STAGES-1 for it == 0 (the prologue),
  // so STAGES-2 (or STAGES-1) later steps' loads may stay in flight, fewer
  // near the end of the range.  A ragged K's last step is patched first.
  auto wait_step = [&](int it) {
    if constexpr (kRagged) {
      if (korder.kt(it) == a.k_tiles - 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_u8* st = smem + (it % STAGES) * Cfg::kStageBytes;
        fix_tail_chunks<Cfg::kLoadsA, T>(st, chunk_a, korder.kt(it) * BK, a.K, tid);
        fix_tail_chunks<Cfg::kLoadsB, T>(st + Cfg::kABytes, chunk_b, korder.kt(it) * BK, a.K,
                                         tid);
      }
    }
    const int later = min(it == 0 ? STAGES - 1 : STAGES - 2, n_iter - 1 - it);
    ring_wait_barrier_n<LPS, STAGES - 1>(later);
  };

  f32x16 acc[Cfg::kFragM][Cfg::kFragN];
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  constexpr int kReads = Cfg::kFragM + Cfg::kFragN;
  constexpr int kMfmas = Cfg::kFragM * Cfg::kFragN;
  bf16x8 fa[2][Cfg::kFragM], fb[2][Cfg::kFragN];

  if constexpr (PIPE == 0) {
    if (n_iter > 0) {
      // ---- prologue: every slot gets a K-step in flight -------------------
#pragma unroll
      for (int p = 0; p < STAGES; ++p)
        if (p < n_iter) issue_stage(p);
      wait_step(0);
      read_frags<Cfg, SWZ>(smem, smem + Cfg::kABytes, 0, wm, wn, lane, fa[0], fb[0]);

      // ---- main loop --------------------------------------------------------
      // Substep j of step `it` uses fragment buffer (it*kSub + j) & 1.
      for (int it = 0; it < n_iter; ++it) {
        const lds_u8* sa = smem + (it % STAGES) * Cfg::kStageBytes;
        const lds_u8* sb = sa + Cfg::kABytes;
        const int b0 = (it * Cfg::kSub) & 1;
#pragma unroll
        for (int kk = 0; kk + 1 < Cfg::kSub; ++kk) {
          const int cur = (b0 + kk) & 1, nxt = cur ^ 1;
          read_frags<Cfg, SWZ>(sa, sb, kk + 1, wm, wn, lane, fa[nxt], fb[nxt]);
          __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // DS reads
          mfma_block<Cfg, kHalf>(acc, fa[cur], fb[cur]);
          __builtin_amdgcn_sched_group_barrier(0x008, kMfmas, 0);  // MFMAs
        }
        const int cur = (b0 + Cfg::kSub - 1) & 1, nxt = cur ^ 1;
        if (it + 1 < n_iter) {
          // Every wave now holds step it's last fragments (lgkmcnt(0) inside
          // the wait), so slot it % STAGES is free: refill it with step
          // it+STAGES and start reading step it+1 under the last MFMAs.
          wait_step(it + 1);
          if (it + STAGES < n_iter) issue_stage(it + STAGES);
          const lds_u8* na = smem + ((it + 1) % STAGES) * Cfg::kStageBytes;
          read_frags<Cfg, SWZ>(na, na + Cfg::kABytes, 0, wm, wn, lane, fa[nxt], fb[nxt]);
          __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
        }
        mfma_block<Cfg, kHalf>(acc, fa[cur], fb[cur]);
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas, 0);
      }
    }
  } else {
    // ---- spread issue -------------------------------------------------------
    // The loads of step X form kSub groups of G.  Group 0 is issued right
    // after the barrier that frees slot X % STAGES (in the middle of step
    // X-STAGES), groups 1..kSub-1 during the first kSub-1 substeps of step
    // X-STAGES+1, each load between two MFMAs.  Steps past the end of the
    // range are not issued, and the wait counts shrink to match.
    // Window substep w (0 = the last substep of the step in which the
    // barrier freed the slot, 1..kSub-1 = the next step's first substeps)
    // issues loads [lo(w), lo(w+1)) of the step being loaded.
    constexpr int F = PIPE == 1 ? Cfg::kSub : PIPE == 3 ? Cfg::kSub - 1 : Cfg::kSub - 2;
    static_assert(F >= 1 && F <= Cfg::kSub, "issue window");
    static_assert(LPS <= F * kMfmas, "at most one load per MFMA");
    constexpr int G0 = LPS / F;  // loads in window substep 0

    // Load i (0..LPS-1; A loads first) of step `it`, if that step exists.
    auto dma_one = [&](int it, int i) {
      if (it >= n_iter) return;
      const int kt = korder.kt(it);
      const int k0 = kt * BK;
      const bool fast = kt < full_tiles;
      const int klim = a.K;
      const uint32_t base = smem_addr + (it % STAGES) * Cfg::kStageBytes;
      uint32_t dst, vbase;
      int chunk;
      if (i < LA) {
        dst = base + (i * T + wave * 64) * 16;
        vbase = voff_a[i];
        chunk = chunk_a[i];
      } else {
        dst = base + Cfg::kABytes + ((i - LA) * T + wave * 64) * 16;
        vbase = voff_b[i - LA];
        chunk = chunk_b[i - LA];
      }
      const uint32_t tailv = (k0 + chunk * 8 < klim) ? vbase + (uint32_t)(k0 * 2) : kOOB;
      const uint32_t vo = fast ? vbase : tailv;
      const uint32_t so = fast ? (uint32_t)(k0 * 2) : 0u;
      if (i < LA)
        dma16(rsrc_a, dst, vo, so);
      else
        dma16<kStream>(rsrc_b, dst, vo, so);
    };


    // "Step j has landed", in the middle of step j-1: every load of the
    // steps j+1 .. min(j+STAGES-2, n_iter-1) is issued and may still be in
    // flight; none of step j+STAGES-1.
    auto wait_mid = [&](int j) {
      if constexpr (kRagged) {
        if (korder.kt(j) == a.k_tiles - 1) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          lds_u8* st = smem + (j % STAGES) * Cfg::kStageBytes;
          fix_tail_chunks<Cfg::kLoadsA, T>(st, chunk_a, korder.kt(j) * BK, a.K, tid);
          fix_tail_chunks<Cfg::kLoadsB, T>(st + Cfg::kABytes, chunk_b, korder.kt(j) * BK, a.K,
                                           tid);
        }
      }
      ring_wait_barrier_n<LPS, STAGES - 2>(min(STAGES - 2, n_iter - 1 - j));
    };

    if (n_iter > 0) {
      // prologue: steps 0..STAGES-2 whole, group 0 of step STAGES-1
#pragma unroll
      for (int p = 0; p + 1 < STAGES; ++p)
#pragma unroll
        for (int i = 0; i < LPS; ++i) dma_one(p, i);
#pragma unroll
      for (int q = 0; q < G0; ++q) dma_one(STAGES - 1, q);
      if constexpr (kRagged) {
        if (korder.kt(0) == a.k_tiles - 1) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          fix_tail_chunks<Cfg::kLoadsA, T>(smem, chunk_a, korder.kt(0) * BK, a.K, tid);
          fix_tail_chunks<Cfg::kLoadsB, T>(smem + Cfg::kABytes, chunk_b, korder.kt(0) * BK, a.K, tid);
        }
      }
      // in flight: steps 1 .. min(STAGES-2, n_iter-1) whole, group 0 of
      // step STAGES-1 if it exists
      ring_wait_barrier_ng<LPS, STAGES - 2, G0>(min(STAGES - 2, n_iter - 1), STAGES - 1 < n_iter);
      read_frags<Cfg, SWZ>(smem, smem + Cfg::kABytes, 0, wm, wn, lane, fa[0], fb[0]);

      for (int it = 0; it < n_iter; ++it) {
        const lds_u8* sa = smem + (it % STAGES) * Cfg::kStageBytes;
        const lds_u8* sb = sa + Cfg::kABytes;
        const int b0 = (it * Cfg::kSub) & 1;
#pragma unroll
        for (int kk = 0; kk + 1 < Cfg::kSub; ++kk) {
          const int cur = (b0 + kk) & 1, nxt = cur ^ 1;
          read_frags<Cfg, SWZ>(sa, sb, kk + 1, wm, wn, lane, fa[nxt], fb[nxt]);
          // window substep kk+1 of step it+STAGES-1
          constexpr_for_window<F, LPS>(kk + 1, [&](auto lo, auto hi) {
            constexpr int kLo = decltype(lo)::value, kHi = decltype(hi)::value;
            mfma_block_dma<Cfg, kHalf, kHi - kLo>(acc, fa[cur], fb[cur],
                                           [&](int q) { dma_one(it + STAGES - 1, kLo + q); });
          });
        }
        const int cur = (b0 + Cfg::kSub - 1) & 1, nxt = cur ^ 1;
        if (it + 1 < n_iter) {
          wait_mid(it + 1);
          const lds_u8* na = smem + ((it + 1) % STAGES) * Cfg::kStageBytes;
          read_frags<Cfg, SWZ>(na, na + Cfg::kABytes, 0, wm, wn, lane, fa[nxt], fb[nxt]);
        }
        // (no load of step it+STAGES exists in the last step, so nothing is
        // written into the slot that other waves may still be reading)
        mfma_block_dma<Cfg, kHalf, G0>(acc, fa[cur], fb[cur], [&](int q) { dma_one(it + STAGES, q); });
      }
    }
  }

  finish_tile<Cfg, kStore, kSplit>(a, smem, wave, m0, n0, acc, m0 + wm * Cfg::kWaveM,
                                   n0 + wn * Cfg::kWaveN, lane, split);
}

}  // namespace gemm
