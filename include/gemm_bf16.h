/*
 * gemm_bf16 -- dense bf16 GEMM for AMD Instinct MI355X (gfx950), C ABI.
 *
 *   C[M,N] = A[M,K] * B[N,K]^T      bf16 inputs, fp32 accumulation,
 *                                   bf16 output (or fp32 for the debug call)
 *
 * (plus the same operation over fp16 operands: gemm_f16*, at the end)
 *
 * The operation is the one defined on the page "Matrix Multiplication on
 * NVIDIA's Blackwell: A Four-Part Deep Dive" (section on the definition of
 * matrix multiplication: C is M x N inner products over K; naive-kernel
 * section: the second operand is read as b[col, k], bf16 in and out with the
 * sum carried in fp32), and the linear-layer matmul of transformer prefill
 * and decode from the page "Hand-writing a Blackwell GEMM: from 164 to 1400
 * TFLOP/s" (section "two workloads, not one").  There is no alpha/beta: C is
 * overwritten with the product, as in that page's K-loop step, where a C tile
 * is the sum of A_k B_k^T starting from zero.
 *
 * Layouts.  All strides are in elements; all pointers are device pointers
 * on the current HIP device (hipGetDevice at the time of the call).
 *   A(m,k) = A[m*lda + k], lda >= K   (row-major, K contiguous)
 *   B(n,k) = B[n*ldb + k], ldb >= K   ("K-major": N rows of K)
 *   C(m,n) = C[m*ldc + n], ldc >= N   (row-major)
 * bf16 values are raw 16-bit patterns (uint16_t or __hip_bfloat16 storage).
 *
 * Shapes.  Any M, N, K >= 0.  M == 0 or N == 0: nothing is launched, the
 * call returns GEMM_OK.  K == 0: C is set to zeros (the empty sum).
 *
 * Alignment (required): A, B and C 16-byte aligned; lda, ldb and ldc
 * multiples of 8 elements.  Otherwise GEMM_ERR_MISALIGNED.  (Recommended:
 * A, B and C 128-byte aligned with lda, ldb and ldc multiples of 64
 * elements, so that every 128-byte piece of a row lies in one cache line;
 * with rows that start off a line, e.g. lda = ldb = K = 8168 or 7000, a
 * compute-bound call ran 10-12 % slower than with the rows padded to 8192
 * or 7040, and 4096 x 4088 x 4096 2 % slower with ldc = 4088 than with
 * ldc = 4096.)
 *
 * Numerics.  Products of bf16 values are exact in fp32; sums are fp32 in an
 * order fixed by the chosen configuration (so results are bitwise
 * reproducible run to run, split-K included).  The bf16 output is the fp32
 * sum rounded to nearest, ties to even.
 *
 * Ownership.  The caller owns A, B and C; the library neither frees nor
 * retains them.  C must not overlap A or B.  When a shape's configuration
 * splits K, the fp32 partial sums of the S slices (S * M * roundup8(N) * 4
 * bytes, or S * M * roundup8(N - N1) * 4 for a hybrid plan that splits only
 * the columns from N1 on; see gemm_bf16_config_name) go to a workspace the
 * library owns per (device, stream): allocated
 * on first need and grown when a larger one is needed.  Growth allocates a
 * new buffer and keeps the old one alive (work already queued, or a graph
 * captured earlier, may still use it); all of them are freed by
 * gemm_bf16_release_workspace, which therefore invalidates graphs captured
 * with calls that split K.  Allocation cannot be captured: pre-size the
 * workspace with gemm_bf16_reserve_workspace before stream capture; a call
 * under capture that would need to grow it returns GEMM_ERR_CAPTURE without
 * enqueueing anything.  gemm_bf16_ex_noalloc uses a static scratch array
 * instead and never allocates.
 *
 * Streams and errors.  Calls are asynchronous: work is enqueued on `stream`
 * (a hipStream_t passed as void*, NULL = the null stream) and the call never
 * synchronises it.  Argument errors are
 * returned synchronously before anything is enqueued.  A device fault shows
 * up at the caller's next synchronisation.  Calls on different streams may
 * run concurrently.  Nothing aborts and nothing prints.
 */
#ifndef GEMM_BF16_H
#define GEMM_BF16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point that returns int. */
#define GEMM_OK 0
#define GEMM_ERR_INVALID_ARG 1 /* negative size, ld too small, NULL with work */
#define GEMM_ERR_MISALIGNED 2  /* pointer not 16 B aligned or ld % 8 != 0 */
#define GEMM_ERR_UNSUPPORTED 3 /* operand too large for 32-bit tile offsets,
                                  unknown config name, or a config not
                                  built for fp16 passed to gemm_f16_ex */
#define GEMM_ERR_HIP 4         /* a HIP runtime call failed; see
                                  gemm_bf16_last_hip_error */
#define GEMM_ERR_CAPTURE 5     /* the stream is being captured and the call
                                  would have to allocate a larger split-K
                                  workspace (reserve it before capture) */
#define GEMM_ERR_SCRATCH 6     /* gemm_bf16_ex_noalloc: the plan's split-K
                                  partials exceed its static scratch */

/* C = A * B^T with bf16 output.  Arguments as described above.  Returns a
 * status code. */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const void* A, int64_t lda,
              const void* B, int64_t ldb,
              void* C, int64_t ldc,
              void* stream);

/* Debug variant: the same product with the fp32 sums stored unrounded.
 * C is float*, 16 B aligned, ldc in floats (a multiple of 8).  Same
 * configuration choice and summation order as
 * gemm_bf16 for the same shape, so rounding this output to bf16 gives
 * gemm_bf16's result. */
int gemm_bf16_f32out(int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda,
                     const void* B, int64_t ldb,
                     float* C, int64_t ldc,
                     void* stream);

/* As gemm_bf16 / gemm_bf16_f32out, but with the kernel configuration named
 * explicitly (one of the names gemm_bf16_config_at enumerates), for
 * ablations, tuning sweeps and tests that compare configurations.
 * config == NULL or "" selects automatically.  out_f32 != 0 writes fp32 to C
 * (then C is float*).  Unknown name: GEMM_ERR_UNSUPPORTED. */
int gemm_bf16_ex(const char* config,
                 int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 void* C, int64_t ldc,
                 int out_f32, void* stream);

/* Name of the configuration gemm_bf16 (and gemm_f16: the plan choice is the
 * same for both operand types) would choose for this shape, e.g.
 * "t256x256x64_w2x2_s2_x3_p10_k1_g4": tile BM x BN x BK, waves, ring stages,
 * LDS swizzle, load schedule, then K splits and GROUP_M (and "_r<n>", the
 * K-step rotation, when on, "_n1" when B is loaded non-temporally,
 * "_h<S>" for a hybrid plan and "_m1" / "_m2" for a mixed one).
 * Per-thread static storage, valid until the thread's next call; never NULL.
 *
 * "_h<S>" (a hybrid plan; with "_k1" only, and not with "_P"): where the
 * tiles fill their last pass over the GPU's 256 compute units only in part,
 * the tile columns that make up the whole passes (N1 = the largest number
 * of whole tile columns within them, times the tile width) are computed
 * unsplit, and columns N1 .. N-1 as a second launch with K split S ways and
 * the fixed-order reduction.  Each element's sum is that of the part that
 * covers it, so results are reproducible run to run; the columns from N1 on
 * may differ from the unsplit plan's in the last bits, as any split does.
 * The automatic choice weighs it against the plain plans: for M > 256 with
 * a model of launch time fitted on MI355X, for smaller M when the left-over
 * tiles times S fit in one pass.  Named on a shape where it does not apply (whole passes, one pass or
 * less, or too few K-steps to split), it is dropped and the plain plan runs.
 *
 * "_m1" / "_m2" (a mixed plan; on the 256 x 256 tile
 * t256x256x64_w2x2_s2_x3_p10 only, with "_k1", and not with "_P" or "_h"):
 * the same whole passes as a hybrid, columns 0 .. N1-1 on 256 x 256 tiles,
 * and columns N1 .. N-1 as a second launch on 256 x 128 ("_m1") or
 * 128 x 128 ("_m2") tiles, unsplit, so the narrower tiles fill the compute
 * units that the wide tiles' last pass would leave idle.  No
 * workspace.  Both tiles add the same K-steps in the same order, so the
 * result is the plain plan's, bit for bit (with "_r<n>" the rotation
 * follows each launch's own tiles).  The automatic choice weighs it against
 * the other plans for M > 256.  Named on a shape with no whole pass, or
 * one pass or less, it is dropped and the plain plan runs.
 *
 * "_n1" (accepted by gemm_bf16_ex / gemm_f16_ex on the tiles built for it:
 * the 256 x 128 direct-to-LDS tile and the M <= 64 tiles) marks B's loads
 * non-temporal, so the L2 does not keep B for reuse.  It is meant for one
 * row of tiles (M no larger than the tile's BM), where no other workgroup
 * reads the same B; it changes only the cache policy, so results are the
 * same bits as without it.  Calls with fp32 output, or a K that is not a
 * whole number of the tile's K-steps, run the ordinary kernel.  "_n0" is
 * accepted and means the default (no suffix).
 *
 * gemm_bf16_ex also accepts a "_P<n>" suffix on the tile built for it
 * (t256x256x64_w2x2_s2_x3_p10): a persistent grid of n workgroups (rounded
 * down to a multiple of 8, at most the tile count) that walk the tiles in
 * the same order, each draining one tile's C through one LDS ring slot
 * while the next tile's first K-steps load into the others.  Same tiles and
 * per-tile summation order, so the same bits as the plan without it.  bf16
 * operands only, never with a split ("_k1"); its fp32 output runs the
 * ordinary kernel (same sums).  This is the persistent scheduling of "Matrix
 * Multiplication on NVIDIA's Blackwell" (Kernels 7 and 8: double-buffered
 * output, persistent kernel), re-designed for one LDS ring per CU. */
const char* gemm_bf16_config_name(int64_t M, int64_t N, int64_t K);

/* Enumerate the built configurations: the i-th name, or NULL past the end. */
const char* gemm_bf16_config_at(int i);

/* ------------------------------------------------------------------ fp16
 * The same product over fp16 operands (IEEE binary16 bit patterns): fp16
 * inputs, fp32 accumulation, fp16 output rounded to nearest even, with
 * overflow past 65504 giving +-infinity.  This is the input type the page
 * "Hand-writing a Blackwell GEMM: from 164 to 1400 TFLOP/s" measures with
 * (section "how I measured": its checks run on fp16 tensors).  Layouts,
 * shapes, alignment, ownership, workspaces, streams and status codes are
 * exactly as for the bf16 calls above; the kernels are the same with the
 * fp16 matrix-core instruction. */

/* C = A * B^T with fp16 operands and fp16 output.  Returns a status code. */
int gemm_f16(int64_t M, int64_t N, int64_t K,
             const void* A, int64_t lda,
             const void* B, int64_t ldb,
             void* C, int64_t ldc,
             void* stream);

/* Debug variant: fp16 operands, the fp32 sums stored unrounded (C is
 * float*, ldc in floats, a multiple of 8).  Rounding it to fp16 gives
 * gemm_f16's result. */
int gemm_f16_f32out(int64_t M, int64_t N, int64_t K,
                    const void* A, int64_t lda,
                    const void* B, int64_t ldb,
                    float* C, int64_t ldc,
                    void* stream);

/* gemm_f16 / gemm_f16_f32out with the configuration named explicitly.  Only
 * the configurations gemm_f16_config_at enumerates are built for fp16; any
 * other name returns GEMM_ERR_UNSUPPORTED.  config == NULL or "" selects
 * automatically. */
int gemm_f16_ex(const char* config,
                int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda,
                const void* B, int64_t ldb,
                void* C, int64_t ldc,
                int out_f32, void* stream);

/* Enumerate the configurations built for fp16 operands: the i-th name, or
 * NULL past the end. */
const char* gemm_f16_config_at(int i);

/* ------------------------------------------------------- no allocation
 * For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as gemm_bf16_ex (config NULL or "" = automatic, out_f32 as there,
 * the same plans and summation order, so the same bits), but the split-K
 * partials go to a static array of GEMM_NOALLOC_SCRATCH_BYTES that every
 * device holds from the library's first use on it until the process ends,
 * instead of the per-stream workspace.  It calls no hipMalloc or hipFree
 * and never synchronises.  A plan whose partials (S * M * roundup8(N) * 4
 * bytes) exceed the array is refused with GEMM_ERR_SCRATCH before anything
 * is enqueued; the automatic plans of every shape stay below it.  Every
 * call on one device shares that device's array, so calls that may overlap
 * on one device (different streams, or concurrent graph replays) race and
 * must be ordered by the caller; nothing in the array needs clearing
 * between calls.  Returns a status code. */
#define GEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gemm_bf16_ex_noalloc(const char* config,
                         int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda,
                         const void* B, int64_t ldb,
                         void* C, int64_t ldc,
                         int out_f32, void* stream);

/* Human-readable text for a status code.  Static storage; never NULL. */
const char* gemm_bf16_status_string(int status);

/* The hipError_t value of the most recent failed HIP call made by this
 * library on the calling thread (0 if none). */
int gemm_bf16_last_hip_error(void);

/* Make sure the workspace of (current device, stream) holds at least
 * `bytes` bytes, allocating now rather than inside a later gemm call.
 * Returns a status code. */
int gemm_bf16_reserve_workspace(size_t bytes, void* stream);

/* Bytes of workspace the automatic choice needs for this shape (0 when it
 * does not split K). */
size_t gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K);

/* Free every workspace this library holds, on every device.  Synchronises
 * the streams they belong to first, so every stream that has made a split-K
 * call (or reserved a workspace) must still exist when this is called:
 * destroying a stream does not free its workspace, and a destroyed stream
 * cannot be synchronised.  Returns a status code. */
int gemm_bf16_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_BF16_H */
