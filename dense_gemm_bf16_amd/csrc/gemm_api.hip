// C-ABI front end of the bf16 (and fp16) GEMM library: argument checks, the
// choice of kernel configuration, split-K workspaces, launch.  The contract of every
// entry point is stated in include/gemm_bf16.h.
#include "../../include/gemm_bf16.h"

#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "gemm_internal.h"

namespace gemm {
namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return GEMM_ERR_HIP;
}

// ---------------------------------------------------------------- workspaces
// One split-K workspace per (device, stream), holding the fp32 partial
// products of the K-slices.  Work on one stream runs in order, so one buffer
// per stream is never used by two calls at once.
//
// Growth allocates a larger buffer and retires the old one without freeing
// it: work already queued on the stream, or a graph captured earlier with
// the old pointer, may still write it.  Retired buffers are freed only by
// gemm_bf16_release_workspace.  No allocation happens while the stream is
// being captured (it could not be captured, and the synchronisation that a
// safe free would need invalidates the capture): the call fails with
// GEMM_ERR_CAPTURE instead, before anything is enqueued.
struct Workspace {
  int device;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};

std::mutex g_ws_mu;
std::vector<Workspace> g_ws;
std::vector<Workspace> g_retired;

// GEMM_OK if the stream is not being captured, else GEMM_ERR_CAPTURE (or
// GEMM_ERR_HIP if the query fails).
int check_not_capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return hip_fail(e);
  return st == hipStreamCaptureStatusNone ? GEMM_OK : GEMM_ERR_CAPTURE;
}

int get_workspace(int device, hipStream_t stream, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* have = nullptr;
  for (Workspace& w : g_ws)
    if (w.device == device && w.stream == stream) have = &w;
  if (have && have->bytes >= bytes) {
    *out = have->ptr;
    return GEMM_OK;
  }
  int rc = check_not_capturing(stream);
  if (rc != GEMM_OK) return rc;
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) return hip_fail(e);
  if (have) {
    g_retired.push_back(*have);
    have->ptr = p;
    have->bytes = bytes;
  } else {
    g_ws.push_back(Workspace{device, stream, p, bytes});
  }
  *out = p;
  return GEMM_OK;
}

int64_t partial_ld(int64_t N) { return (N + 7) / 8 * 8; }


size_t workspace_bytes(const Plan& p, int64_t M, int64_t N) {
  if (p.split_n > 0) {  // hybrid: only the columns past split_n are split
    if (p.tail_splits <= 1) return 0;  // mixed: nothing is split
    return (size_t)p.tail_splits * (size_t)M * (size_t)partial_ld(N - p.split_n) * 4;
  }
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * (size_t)M * (size_t)partial_ld(N) * 4;
}

// ------------------------------------------------------------ config choice
// Shape -> configuration, from sweeps on MI355X (HIP events, cold B for the
// memory-bound shapes).  The tuned table first (exact shapes); for M > 256
// the cost model below (model_plan), which picks among the direct-to-LDS
// tiles, split counts and hybrids; otherwise these rules (for M > 256 they
// were the choice before the model, which keeps their plans for 4096^3 and
// the M = 8192 prefill shapes):
//  * M <= 64 (small decode batches): the small-M kernel, one workgroup per
//    BM x 32 block over all of K (BM = 32 up to M = 32, else 64), so
//    N = 8192 gives 256 workgroups with no split-K pass; K-step rotation on
//    (the operands' power-of-two row strides otherwise send concurrent
//    workgroups to the same memory channels).  12-17 % faster than the
//    earlier 32 x 128 tiles split four ways at M = 1 and 17, 6 % at M = 48.
//    When the strips need more than one pass over the CUs (N = 10240: 320,
//    N = 28672: 896), or M > 48 (a 64 x 32 strip reads twice as much A as
//    B), the 32 x 128 / 64 x 128 tiles instead, K split to about 256
//    workgroups: 33-34 vs 38-42 us at N = 10240 and M = 1, 32; 37 vs 57 us
//    at 64 x 10240 x 8192, 80 vs 90 us at 32 x 28672 x 8192, 28 vs 33 us at
//    64 x 4096 x 14336;
//  * enough 256 x 256 tiles to fill the chip (4096^3, M = 8192 prefill):
//    the direct-to-LDS 256 x 256 x 64 kernel, no split (at steady clock 6 %
//    faster than the register-staged kernel at 4096^3 and on both M = 8192
//    prefill shapes);
//  * otherwise direct-to-LDS 256 x 128 tiles with a three-slot ring (0.5-6 %
//    faster than the register-staged 256 x 128 tiles at M = 256; with two
//    slots 6-8 % slower, a step's loads then have one step to land),
//    rotation on for a single row of tiles, K split to about 256
//    workgroups -- unless they would need
//    a split while 128 x 128 tiles fill the chip without one (M = 512, N =
//    8192: 44 vs 52 us; 1024 x 4096 x 4096: 35 vs 43 us), or the split
//    leaves fewer than 24 K-steps per slice, where first loads and partial
//    stores weigh more than the smaller tile costs (512 x 4096 x 4096: 128 x
//    128 split 2, 26.5 vs 28.6 us).  Then direct-to-LDS 128 x 128 tiles with
//    a four-slot ring, split to about 256 workgroups.
//  * and where the tiles chosen above (unsplit) fill their last pass over
//    the CUs only in part, a hybrid plan ("_h<S>"): the whole passes, taken
//    as whole tile columns, run unsplit, and the tile columns left over run
//    as a second call with K split S ways, when those tiles times S fit in
//    one pass.  The left-over pass then takes 1/S of a tile's time plus the
//    split's partial round trip.  Measured (as the two calls, against the
//    plain plan): 2048 x 10240 x 8192 329.5 -> 272.1 us, 1024 x 10240 x 8192
//    195.3 -> 156.6, 512 x 10240 x 8192 111.7 -> 91.0, 1024 / 2048 / 4096 x
//    5376 x 5376 -11 to -12 %, 4096 x 10240 x 8192 -2.3 %, 2048 x 28672 x
//    8192 -3.2 %.
// All three direct-to-LDS tiles run with 16 x 16 x 32 MFMAs: at the same
// cycles per FLOP the chip holds a higher clock under its power limit with
// them, and measured against the 32 x 32 x 16 form of the same tiles they
// are 9 % faster at 4096^3, 4-6 % on the M = 8192 prefill shapes (10 % with
// fp16 operands), 2-7 % at 512 x 8192 x 5376 and level (+-2 %) on the
// M = 256 decode shapes.
constexpr int kCUs = 256;
constexpr const char* kBig = "t256x256x64_w2x2_s2_x3_p10";
constexpr const char* kMid = "t256x128x64_w2x2_s3_x3_p10";
constexpr const char* kMid128 = "t128x128x64_w2x2_s4_x3_p10";
constexpr const char* kSmallM32 = "t32x32x64_w1x1_s8_x2_p9";
constexpr const char* kSmallM64 = "t64x32x64_w1x1_s6_x2_p9";
constexpr const char* kSkinny32 = "t32x128x64_w1x4_s6_x2_p0";
constexpr const char* kSkinny64 = "t64x128x64_w1x4_s6_x2_p0";

// Shapes measured by the offline tuning sweep (dense_gemm_bf16_amd/tune.py):
// exact (M, N, K) -> plan name, consulted before the cost model and the
// rules below.
struct TunedPlan {
  int64_t M, N, K;
  const char* plan;
};
constexpr TunedPlan kTuned[] = {
#include "gemm_tuned.inc"
    {0, 0, 0, nullptr}};

int64_t tiles_of(const TileConfig* t, int64_t M, int64_t N) {
  return ((M + t->bm - 1) / t->bm) * ((N + t->bn - 1) / t->bn);
}

// Splits so that tiles * splits is about `target` workgroups, keeping at
// least 8 K-steps per slice.
int choose_splits(int64_t tiles, int64_t k_tiles, int64_t target = kCUs) {
  if (tiles <= 0 || tiles >= target) return 1;  // tiles == 0: empty M or N
  int s = (int)((target + tiles / 2) / tiles);
  while (s > 1 && k_tiles / s < 8) --s;
  return s < 1 ? 1 : s;
}

void finish_plan(Plan* p, int64_t M, int64_t N, int64_t K) {
  const int64_t bk = p->tile->bk;
  const int64_t k_tiles = (K + bk - 1) / bk;
  if (p->persist > 0) {
    // a persistent grid walks whole tiles (no split); it is a multiple of 8
    // workgroups, so each keeps its XCD's tiles, and no larger than the
    // tile count
    p->splits = 1;
    const int64_t tiles = ((M + p->tile->bm - 1) / p->tile->bm) * ((N + p->tile->bn - 1) / p->tile->bn);
    int64_t g = p->persist / 8 * 8;
    if (g < 8) g = 8;
    if (g > tiles) g = tiles;
    p->persist = (int)(g > 0 ? g : 8);
  }
  if (p->splits > k_tiles) p->splits = (int)(k_tiles > 0 ? k_tiles : 1);
  if (p->splits < 1) p->splits = 1;
  if (p->splits > 1) {
    // equal slices of ceil(k_tiles / S) steps; drop slices left empty
    const int64_t per = (k_tiles + p->splits - 1) / p->splits;
    p->splits = (int)((k_tiles + per - 1) / per);
  }
  // Hybrid: the first whole passes over the CUs, as whole tile columns, run
  // unsplit; the columns after them form a second call with K split.  Only
  // where both parts are non-empty and the tail still splits after the
  // same clamping as above; otherwise the plain plan.
  p->split_n = 0;
  if (p->tail_splits > 1 && p->splits == 1 && p->persist == 0) {
    const int64_t tiles_m = (M + p->tile->bm - 1) / p->tile->bm;
    const int64_t tiles_n = (N + p->tile->bn - 1) / p->tile->bn;
    const int64_t head_cols = tiles_m > 0 ? (tiles_m * tiles_n / kCUs) * kCUs / tiles_m : 0;
    int64_t s = p->tail_splits < k_tiles ? p->tail_splits : k_tiles;
    if (s > 1) {
      const int64_t per = (k_tiles + s - 1) / s;
      s = (k_tiles + per - 1) / per;
    }
    if (head_cols > 0 && head_cols < tiles_n && s > 1) {
      p->tail_splits = (int)s;
      p->split_n = head_cols * p->tile->bn;
    }
  }
  if (p->split_n == 0) p->tail_splits = 0;
  // Mixed: the same head as the hybrid, the columns after it unsplit on
  // tail_tile (only 256 x 256 over 256 x 128 or 128 x 128, unsplit, no
  // persistent grid, no non-temporal B); otherwise the plain plan.
  int mixed = 0;
  if (p->tail_tile) {
    const int64_t tiles_m = (M + p->tile->bm - 1) / p->tile->bm;
    const int64_t tiles_n = (N + p->tile->bn - 1) / p->tile->bn;
    const int64_t head_cols = tiles_m > 0 ? (tiles_m * tiles_n / kCUs) * kCUs / tiles_m : 0;
    mixed = p->tail_tile == find_tile_config(kMid) ? 1 : p->tail_tile == find_tile_config(kMid128) ? 2 : 0;
    const bool ok = p->split_n == 0 && p->splits == 1 && p->persist == 0 && p->stream_b == 0 &&
                    p->tile == find_tile_config(kBig) && mixed > 0;
    if (ok && head_cols > 0 && head_cols < tiles_n)
      p->split_n = head_cols * p->tile->bn;
    else
      p->tail_tile = nullptr;
  }
  int n = snprintf(p->name, sizeof p->name, "%s_k%d_g%d", p->tile->name, p->splits, p->group_m);
  if (p->k_rot > 0 && n > 0 && n < (int)sizeof p->name)
    n += snprintf(p->name + n, sizeof p->name - n, "_r%d", p->k_rot);
  if (p->persist > 0 && n > 0 && n < (int)sizeof p->name)
    n += snprintf(p->name + n, sizeof p->name - n, "_P%d", p->persist);
  if (p->stream_b > 0 && n > 0 && n < (int)sizeof p->name)
    n += snprintf(p->name + n, sizeof p->name - n, "_n1");
  if (p->split_n > 0 && !p->tail_tile && n > 0 && n < (int)sizeof p->name)
    snprintf(p->name + n, sizeof p->name - n, "_h%d", p->tail_splits);
  if (p->tail_tile && n > 0 && n < (int)sizeof p->name)
    snprintf(p->name + n, sizeof p->name - n, "_m%d", mixed);
}

bool plan_from_name(const char* name, int64_t M, int64_t N, int64_t K, Plan* out);

// ------------------------------------------------------- plan cost model
// For M > 256 the plan is the cheapest under a model of a launch's time on
// MI355X, fitted (least squares on log time) to 1,000 timings of 77 shapes:
// M from 320 to 6144, N x K among 4096 x 4096, 14336 x 4096, 4096 x 14336,
// 8192 x 8192, 10240 x 8192, 5376 x 5376 and 28672 x 8192, each direct-to-LDS
// tile unsplit, split 2-8 and hybrid.  RMS error 4.5 %; on 42 other shapes
// (M 288-5120, N x K with N or K of 3072-16384) its choice ran within 0.1 %
// of the fastest plan timed (geometric mean; 3.5 % at worst), against 7.2 %
// (and up to 50 %) for the earlier rules; on 30 shapes of up to 8.75 passes
// of tiles, swept afterwards, within 0.2 % (1.6 % at worst, with the hybrid
// margin below).  dense_gemm_bf16_amd/plan_model.py holds the same model,
// the sweep and the fit, with the measurements.
//
// A launch of `tiles` tiles split S ways runs units = tiles * S workgroups,
// one per CU at a time: each pass over the 256 CUs costs a unit's time,
// steps * step_us + tile_us (steps: K-steps per slice; tile_us: first loads
// and epilogue), and a last pass with a fraction f of the CUs busy costs
// kPartialPass + (1 - kPartialPass) * f of a full one (fewer workgroups
// share L2, HBM and the power budget).  A split adds the partial slices'
// round trip (written by the GEMM, read by the reduction) and the
// reduction's launch.
struct TileCost {
  const char* name;
  double step_us, tile_us;
};
constexpr TileCost kTileCosts[] = {  // in this order (the mixed plans take [1] and [2])
    {kBig, 1.4295, 2.6456}, {kMid, 0.8187, 1.9745}, {kMid128, 0.4817, 1.8138}};
constexpr double kPartialPass = 0.6767;
constexpr double kLaunchUs = 1.1184;
constexpr double kSplitUs = 1.4115;
constexpr double kSplitUsPerMB = 0.3239;  // per MB of partial slices
// A hybrid whose unsplit part makes two or more whole passes is taken only
// if its estimate is 3 % below the others': after whole passes a partial
// last pass runs faster than the partial-pass term says, and without the
// margin the model preferred hybrids up to 4.7 % slower on a sweep of 30
// such shapes (with it: 1.6 % at worst).
constexpr double kHybridMargin = 0.03;
constexpr int64_t kModelMinM = 257;

// K splits as finish_plan equalises them: ceil(k_tiles / S) steps a slice.
int64_t even_splits(int64_t S, int64_t k_tiles) {
  if (S > k_tiles) S = k_tiles;
  if (S <= 1) return 1;
  const int64_t per = (k_tiles + S - 1) / S;
  return (k_tiles + per - 1) / per;
}

// Bytes of fp32 partial slices, in floating point: the product can exceed
// 64 bits for shapes that are only named, never run.
double partial_bytes(int64_t S, int64_t M, int64_t N) {
  return (double)S * (double)M * (double)partial_ld(N) * 4.0;
}

double launch_cost(const TileCost& c, int64_t tiles, int64_t S, int64_t k_tiles, int64_t M,
                   int64_t N) {
  const int64_t units = tiles * S;
  const int64_t steps = (k_tiles + S - 1) / S;
  double passes = (double)(units / kCUs);
  if (units % kCUs) passes += kPartialPass + (1 - kPartialPass) * (double)(units % kCUs) / kCUs;
  double t = (steps * c.step_us + c.tile_us) * passes + kLaunchUs;
  if (S > 1) t += kSplitUs + kSplitUsPerMB * partial_bytes(S, M, N) * 1e-6;
  return t;
}

// The cheapest plan under the model: each direct-to-LDS tile unsplit, with
// K split 2, 3, 4, 6 or 8 ways (at least 8 K-steps a slice, at most 4
// workgroups per CU, partials within the no-allocation scratch), and the
// hybrids of an unsplit plan whose last pass is partial, its left-over
// columns split 2, 3, 4, 6 or 8 ways, and for the 256 x 256 tile the mixed
// plans, its left-over columns unsplit on 256 x 128 or 128 x 128 tiles.
Plan model_plan(int64_t M, int64_t N, int64_t K, bool half) {
  Plan best{};
  double best_t = 0;
  auto consider = [&](const TileConfig* t, int64_t S, int64_t h, double cost,
                      const TileConfig* tail = nullptr) {
    if (best.tile && cost >= best_t) return;
    best = Plan{};
    best.tile = t;
    best.splits = (int)S;
    best.tail_splits = (int)h;
    best.tail_tile = tail;
    best.group_m = 4;
    best_t = cost;
  };
  const TileConfig* big = find_tile_config(kBig);
  const TileConfig* mid = find_tile_config(kMid);
  const TileConfig* m128 = find_tile_config(kMid128);
  for (const TileCost& c : kTileCosts) {
    const TileConfig* t = find_tile_config(c.name);
    if (!t || (half && !t->f16)) continue;
    const int64_t kt = (K + t->bk - 1) / t->bk;
    const int64_t tm = (M + t->bm - 1) / t->bm, tn = (N + t->bn - 1) / t->bn;
    const int64_t tiles = tm * tn;
    for (int64_t S : {1, 2, 3, 4, 6, 8}) {
      if (S > 1 && (kt / S < 8 || tiles * S > 4 * kCUs)) continue;
      const int64_t s = even_splits(S, kt);
      if (S > 1 && s <= 1) continue;
      if (s > 1 && partial_bytes(s, M, N) > (double)GEMM_NOALLOC_SCRATCH_BYTES) continue;
      consider(t, s, 0, launch_cost(c, tiles, s, kt, M, N));
    }
    if (tiles > kCUs && tiles % kCUs) {
      const int64_t head_cols = (tiles / kCUs) * kCUs / tm;
      if (head_cols <= 0 || head_cols >= tn) continue;
      const int64_t n1 = head_cols * t->bn;
      for (int64_t h : {2, 3, 4, 6, 8}) {
        const int64_t hs = even_splits(h, kt);
        if (hs <= 1) continue;
        if (partial_bytes(hs, M, N - n1) > (double)GEMM_NOALLOC_SCRATCH_BYTES) continue;
        const double est = launch_cost(c, tm * head_cols, 1, kt, M, n1) +
                           launch_cost(c, tm * (tn - head_cols), hs, kt, M, N - n1);
        consider(t, 1, hs, tm * head_cols / kCUs >= 2 ? est * (1 + kHybridMargin) : est);
      }
      // mixed: the same head, the columns after it unsplit on 256 x 128
      // or 128 x 128 tiles (the same margin as a hybrid after two or more
      // whole passes)
      for (int i = 1; i <= 2 && t == big; ++i) {
        const TileConfig* tt = i == 1 ? mid : m128;
        if (!tt || (half && !tt->f16)) continue;
        const TileCost& mc = kTileCosts[i];
        const int64_t mkt = (K + tt->bk - 1) / tt->bk;
        const int64_t mtiles = ((M + tt->bm - 1) / tt->bm) * ((N - n1 + tt->bn - 1) / tt->bn);
        const double est = launch_cost(c, tm * head_cols, 1, kt, M, n1) +
                           launch_cost(mc, mtiles, 1, mkt, M, N - n1);
        consider(t, 1, 0, tm * head_cols / kCUs >= 2 ? est * (1 + kHybridMargin) : est, tt);
      }
    }
  }
  return best;
}

// The plan for a shape: the tuned table's entry if there is one (and its
// tile is built for the operand type), else for M > 256 the cost model's
// choice, else the rules.
Plan choose_plan(int64_t M, int64_t N, int64_t K, bool half = false) {
  for (const TunedPlan* e = kTuned; e->plan; ++e) {
    if (e->M != M || e->N != N || e->K != K) continue;
    Plan p{};
    if (plan_from_name(e->plan, M, N, K, &p) && (!half || p.tile->f16)) return p;
    break;
  }
  Plan p{};
  p.group_m = 4;
  const TileConfig* big = find_tile_config(kBig);
  constexpr int64_t kMaxDim = int64_t(1) << 31;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) {
    // Beyond the kernels' 32-bit shape fields (such calls are refused): a
    // name only, computed without the tile and byte counts below, which
    // could overflow for such sizes.
    p.tile = big;
    p.splits = 1;
    snprintf(p.name, sizeof p.name, "%s_k1_g4", big->name);
    return p;
  }
  const int64_t big_tiles = tiles_of(big, M, N);
  if (M >= kModelMinM) {
    Plan m = model_plan(M, N, K, half);
    if (m.tile) {
      finish_plan(&m, M, N, K);
      return m;
    }
  }
  if (M <= 64) {
    // One BM x 32 strip per workgroup while the strips fit in one pass over
    // the CUs (and BM x 32 strips re-read little A: M <= 48); otherwise
    // 128-wide tiles, a quarter as many workgroups, split along K to fill.
    const TileConfig* strip = find_tile_config(M <= 32 ? kSmallM32 : kSmallM64);
    p.tile = (M <= 48 && tiles_of(strip, M, N) <= kCUs)
                 ? strip
                 : find_tile_config(M <= 32 ? kSkinny32 : kSkinny64);
    p.splits = choose_splits(tiles_of(p.tile, M, N), (K + p.tile->bk - 1) / p.tile->bk);
    p.k_rot = 1;
    // one row of tiles: no other workgroup reads a workgroup's B, so its
    // loads are non-temporal (M = 1 and 17 at 8192 x 8192: 25.7 -> 21.9 and
    // 24.7 -> 21.7 us)
    p.stream_b = (M + p.tile->bm - 1) / p.tile->bm == 1 && p.tile->stream ? 1 : 0;
  } else if (M <= 128) {
    // One row of 128 x 128 tiles, K split to about 256 workgroups, rotation
    // on: the 256-row tiles would pad M to 256, loading and multiplying
    // twice the A rows.  Swept with B cold at M = 96 and 128 over seven N x K
    // (4096-28672 x 4096-28672): 4-27 % faster than the 256 x 128 tiles on
    // 12 of the 14 shapes and within 1 % of the fastest plan on them.
    const TileConfig* m128 = find_tile_config(kMid128);
    p.tile = m128;
    p.splits = choose_splits(tiles_of(m128, M, N), (K + m128->bk - 1) / m128->bk);
    p.k_rot = 1;
  } else if (big_tiles >= kCUs - kCUs / 8) {
    p.tile = big;
    p.splits = 1;
    p.k_rot = 0;
  } else {
    const TileConfig* mid = find_tile_config(kMid);
    const TileConfig* m128 = find_tile_config(kMid128);
    const int64_t k_tiles = (K + mid->bk - 1) / mid->bk;
    const int mid_splits = choose_splits(tiles_of(mid, M, N), k_tiles);
    if (mid_splits == 1 || (tiles_of(m128, M, N) < kCUs - kCUs / 8 && k_tiles / mid_splits >= 24)) {
      p.tile = mid;
      p.splits = mid_splits;
      // rotation only for a single row of tiles: with several, the tiles
      // that share a B panel read it together from L2 when unrotated
      // (1024 x 8192 x 8192: 117 vs 128 us)
      p.k_rot = (M + mid->bm - 1) / mid->bm == 1 ? 1 : 0;
    } else {
      p.tile = m128;
      p.splits = choose_splits(tiles_of(m128, M, N), k_tiles);
      // Two rows of tiles: rotation when each workgroup runs 32 K-steps or
      // more.  Interleaved, B cold, M = 160-256: 2.0-4.4 % faster on the 12
      // such shapes (N or K 11008-14336), 0.5-5 % slower on the 12 with
      // 16-27 steps (4096 x 4096, 5120 x 5120, 6144 x 4096).
      p.k_rot = (M + m128->bm - 1) / m128->bm <= 2 && k_tiles / p.splits >= 32 ? 1 : 0;
    }
  }
  if (M > 64 && p.splits == 1) {
    // A last pass over the CUs that the tiles fill only in part: run the
    // whole passes (as whole tile columns) unsplit and the columns left
    // over with K split, when that fits the left-over tiles into one pass.
    const int64_t tiles_m = (M + p.tile->bm - 1) / p.tile->bm;
    const int64_t tiles = tiles_of(p.tile, M, N);
    const int64_t head_tiles = tiles_m > 0 ? (tiles / kCUs) * kCUs / tiles_m * tiles_m : 0;
    const int64_t tail_tiles = tiles - head_tiles;
    if (head_tiles > 0 && tail_tiles > 0) {
      const int s = choose_splits(tail_tiles, (K + p.tile->bk - 1) / p.tile->bk);
      if (s > 1 && tail_tiles * s <= kCUs) p.tail_splits = s;
    }
  }
  finish_plan(&p, M, N, K);
  return p;
}

// Parse "tile[_k<splits>][_g<group>][_r<rotation>][_P<grid>][_n<0|1>][_h<splits>][_m<0|1|2>]"
// where tile is a table name (_P: a persistent grid of that many workgroups
// walking the tiles; only for tiles built with it, bf16 operands, and never
// split.  _n1: non-temporal B loads, only for tiles built with them.  _h:
// the hybrid of finish_plan, only with _k1 and no _P.  _m1 / _m2: the mixed
// plan of finish_plan with its tail on 256 x 128 / 128 x 128 tiles, only on
// the 256 x 256 tile with _k1 and none of _P, _n1 and _h).
bool plan_from_name(const char* name, int64_t M, int64_t N, int64_t K, Plan* out) {
  char buf[64];
  if (strlen(name) >= sizeof buf) return false;
  strcpy(buf, name);
  int splits = 1, group = 4, rot = 0, persist = 0, stream = 0, tail = 0, mixed = 0;
  for (;;) {
    char* u = strrchr(buf, '_');
    if (!u) break;
    int v = 0;
    if (u[1] == 'k' && sscanf(u + 2, "%d", &v) == 1 && v >= 1) {
      splits = v;
      *u = 0;
    } else if (u[1] == 'g' && sscanf(u + 2, "%d", &v) == 1 && v >= 1) {
      group = v;
      *u = 0;
    } else if (u[1] == 'r' && sscanf(u + 2, "%d", &v) == 1 && v >= 0) {
      rot = v;
      *u = 0;
    } else if (u[1] == 'P' && sscanf(u + 2, "%d", &v) == 1 && v >= 1) {
      persist = v;
      *u = 0;
    } else if (u[1] == 'n' && sscanf(u + 2, "%d", &v) == 1 && (v == 0 || v == 1)) {
      stream = v;
      *u = 0;
    } else if (u[1] == 'h' && sscanf(u + 2, "%d", &v) == 1 && v >= 0) {
      tail = v;
      *u = 0;
    } else if (u[1] == 'm' && sscanf(u + 2, "%d", &v) == 1 && v >= 0 && v <= 2) {
      mixed = v;
      *u = 0;
    } else {
      break;
    }
  }
  const TileConfig* t = find_tile_config(buf);
  if (!t) return false;
  if (persist > 0 && (!t->persist || splits > 1)) return false;
  if (stream && !t->stream) return false;
  if (tail > 1 && (splits > 1 || persist > 0)) return false;
  if (mixed && (t != find_tile_config(kBig) || splits > 1 || persist > 0 || stream || tail > 1))
    return false;
  out->tile = t;
  out->splits = splits;
  out->group_m = group;
  out->k_rot = rot;
  out->persist = persist;
  out->stream_b = stream;
  out->tail_splits = tail;
  out->tail_tile = mixed == 1 ? find_tile_config(kMid) : mixed == 2 ? find_tile_config(kMid128) : nullptr;
  finish_plan(out, M, N, K);
  return true;
}

// ----------------------------------------------------------------- checks
int check_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
               int64_t ldb, const void* C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
  if (lda < K || ldb < K || ldc < N) return GEMM_ERR_INVALID_ARG;
  if (M > 0 && N > 0) {
    if (!C) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && (!A || !B)) return GEMM_ERR_INVALID_ARG;
  }
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15) return GEMM_ERR_MISALIGNED;
  if ((lda | ldb | ldc) & 7) return GEMM_ERR_MISALIGNED;
  return GEMM_OK;
}

// One launch plan (not hybrid) on the whole of C.  `fixed_ws`: the device
// address of a caller-side partial buffer of `fixed_bytes` bytes to use
// instead of the per-stream workspace (the no-allocation entry point), or
// NULL.
int run_one(const Plan& p, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
            const void* B, int64_t ldb, void* C, int64_t ldc, bool out_f32, bool half,
            hipStream_t stream, void* fixed_ws, size_t fixed_bytes) {
  const TileConfig& t = *p.tile;
  if (half && !t.f16) return GEMM_ERR_UNSUPPORTED;
  if (p.persist > 0 && (half || !t.persist || p.splits > 1)) return GEMM_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return GEMM_OK;
  // 32-bit limits: tile-relative byte offsets of the operands, grid size,
  // and the int32 shape fields of the kernel.
  // (a tile's operand range plus the 4 KB a load may move its resource base
  // back by must stay below 2^31, the voffset that marks an absent chunk)
  constexpr int64_t kRangeLimit = (int64_t(1) << 31) - 4096;
  if ((int64_t)t.bm * lda * 2 >= kRangeLimit || (int64_t)t.bn * ldb * 2 >= kRangeLimit)
    return GEMM_ERR_UNSUPPORTED;
  if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 31))
    return GEMM_ERR_UNSUPPORTED;
  const int64_t tiles_m = (M + t.bm - 1) / t.bm, tiles_n = (N + t.bn - 1) / t.bn;
  const int64_t k_tiles = (K + t.bk - 1) / t.bk;
  const int64_t units = tiles_m * tiles_n * p.splits;
  if (units >= (int64_t(1) << 31)) return GEMM_ERR_UNSUPPORTED;
  const int64_t grid = p.persist > 0 && !out_f32 && p.persist < units ? p.persist : units;

  KernelArgs a{};
  a.A = (const uint16_t*)A;
  a.B = (const uint16_t*)B;
  a.C = C;
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.tiles_m = (int32_t)tiles_m;
  a.tiles_n = (int32_t)tiles_n;
  a.k_tiles = (int32_t)k_tiles;
  a.splits = p.splits;
  a.k_tiles_per_split = (int32_t)((k_tiles + p.splits - 1) / p.splits);
  a.group_m = p.group_m;
  a.k_rot = p.k_rot;
  int flags = out_f32 ? kOutF32 : 0;
  if ((K & 7) != 0) flags |= kRaggedK;
  if (half) flags |= kF16;
  if (K % t.bk != 0) flags |= kPartialK;
  // (fp32 output: the ordinary kernel, whose per-tile K order is the same)
  if (p.persist > 0 && !out_f32) flags |= kPersistent;
  // (where no kernel with non-temporal B loads is built for the other
  // flags, the launcher runs the ordinary one: same sums, same results)
  if (p.stream_b > 0) flags |= kStreamB;
  void* ws = nullptr;
  if (p.splits > 1) {
    const size_t need = workspace_bytes(p, M, N);
    if (fixed_ws) {
      if (need > fixed_bytes) return GEMM_ERR_SCRATCH;
      ws = fixed_ws;
    } else {
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return hip_fail(e);
      int rc = get_workspace(dev, stream, need, &ws);
      if (rc != GEMM_OK) return rc;
    }
    a.part = (float*)ws;
    a.ldp = partial_ld(N);
    a.part_stride = M * a.ldp;
    flags |= kSplitK;
  }
  hipError_t e = t.launch(a, (int)grid, stream, flags);
  if (e != hipSuccess) return hip_fail(e);
  if (p.splits > 1) {
    const int out_kind = out_f32 ? kStoreF32 : half ? kStoreF16 : kStoreBf16;
    e = launch_splitk_reduce(a.part, a.ldp, a.part_stride, p.splits, C, ldc, (int)M, (int)N,
                             out_kind, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return GEMM_OK;
}

// A plan on C: a hybrid plan as two calls on column ranges, each a plain
// plan of the same tile -- columns [split_n, N) with K split tail_splits
// ways first (it is the part that may need a workspace, so an error there
// leaves nothing enqueued), then columns [0, split_n) unsplit.  A mixed plan
// the same way, with the columns [split_n, N) unsplit on tail_tile.  The two
// ranges share no element of C, so each element's sum is that of the plan
// that covers it (for a mixed plan without rotation the same as the plain
// plan's: both tiles add the same K-steps in the same order).
int run(const Plan& p, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
        const void* B, int64_t ldb, void* C, int64_t ldc, bool out_f32, bool half,
        hipStream_t stream, void* fixed_ws = nullptr, size_t fixed_bytes = 0) {
  if (p.split_n <= 0 || p.split_n >= N)
    return run_one(p, M, N, K, A, lda, B, ldb, C, ldc, out_f32, half, stream, fixed_ws,
                   fixed_bytes);
  const int64_t n1 = p.split_n;
  Plan part = p;
  part.split_n = 0;
  part.tail_splits = 0;
  part.tail_tile = nullptr;
  part.splits = p.tail_splits;
  if (p.tail_tile) {
    part.tile = p.tail_tile;
    part.splits = 1;
  }
  const uint16_t* B1 = (const uint16_t*)B + n1 * ldb;
  uint8_t* C1 = (uint8_t*)C + n1 * (out_f32 ? 4 : 2);
  int rc = run_one(part, M, N - n1, K, A, lda, B1, ldb, C1, ldc, out_f32, half, stream,
                   fixed_ws, fixed_bytes);
  if (rc != GEMM_OK) return rc;
  part.tile = p.tile;
  part.splits = 1;
  return run_one(part, M, n1, K, A, lda, B, ldb, C, ldc, out_f32, half, stream, fixed_ws,
                 fixed_bytes);
}

// The plan of a call: the named configuration, or the automatic choice.
int make_plan(const char* config, int64_t M, int64_t N, int64_t K, bool half, Plan* p) {
  if (config && config[0]) {
    if (!plan_from_name(config, M, N, K, p)) return GEMM_ERR_UNSUPPORTED;
  } else {
    *p = choose_plan(M, N, K, half);
  }
  return GEMM_OK;
}

int gemm_entry(const char* config, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
               const void* B, int64_t ldb, void* C, int64_t ldc, bool out_f32, bool half,
               void* stream) {
  int rc = check_args(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != GEMM_OK) return rc;
  Plan p{};
  rc = make_plan(config, M, N, K, half, &p);
  if (rc != GEMM_OK) return rc;
  return run(p, M, N, K, A, lda, B, ldb, C, ldc, out_f32, half, (hipStream_t)stream);
}

// ------------------------------------------------- static scratch (no-alloc)
// The no-allocation entry point keeps its split-K partials in this array.
// Each device that loads the library holds its own copy, at its own
// address, until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up
// once per device (hipGetSymbolAddress with that device current) and only
// that address is ever passed to a kernel.
constexpr size_t kScratchBytes = GEMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return GEMM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GEMM_OK;
}

// The i-th table entry with f16 set (or with no condition), or NULL.
const char* config_at(int i, bool f16_only) {
  if (i < 0) return nullptr;
  for (const TileConfig* t = tile_configs(); t->name; ++t) {
    if (f16_only && !t->f16) continue;
    if (i-- == 0) return t->name;
  }
  return nullptr;
}

thread_local char g_name_buf[64];

}  // namespace
}  // namespace gemm

extern "C" {

int gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, void* stream) {
  return gemm::gemm_entry(nullptr, M, N, K, A, lda, B, ldb, C, ldc, false, false, stream);
}

int gemm_bf16_f32out(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, float* C, int64_t ldc, void* stream) {
  return gemm::gemm_entry(nullptr, M, N, K, A, lda, B, ldb, C, ldc, true, false, stream);
}

int gemm_bf16_ex(const char* config, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                 const void* B, int64_t ldb, void* C, int64_t ldc, int out_f32, void* stream) {
  return gemm::gemm_entry(config, M, N, K, A, lda, B, ldb, C, ldc, out_f32 != 0, false, stream);
}

int gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
             int64_t ldb, void* C, int64_t ldc, void* stream) {
  return gemm::gemm_entry(nullptr, M, N, K, A, lda, B, ldb, C, ldc, false, true, stream);
}

int gemm_f16_f32out(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                    int64_t ldb, float* C, int64_t ldc, void* stream) {
  return gemm::gemm_entry(nullptr, M, N, K, A, lda, B, ldb, C, ldc, true, true, stream);
}

int gemm_f16_ex(const char* config, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                const void* B, int64_t ldb, void* C, int64_t ldc, int out_f32, void* stream) {
  return gemm::gemm_entry(config, M, N, K, A, lda, B, ldb, C, ldc, out_f32 != 0, true, stream);
}

const char* gemm_f16_config_at(int i) { return gemm::config_at(i, true); }

int gemm_bf16_ex_noalloc(const char* config, int64_t M, int64_t N, int64_t K, const void* A,
                         int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                         int out_f32, void* stream) {
  int rc = gemm::check_args(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != GEMM_OK) return rc;
  gemm::Plan p{};
  rc = gemm::make_plan(config, M, N, K, false, &p);
  if (rc != GEMM_OK) return rc;
  if (gemm::workspace_bytes(p, M, N) > gemm::kScratchBytes) return GEMM_ERR_SCRATCH;
  if (M == 0 || N == 0) return GEMM_OK;
  void* ws = nullptr;
  rc = gemm::scratch_of_current_device(&ws);
  if (rc != GEMM_OK) return rc;
  return gemm::run(p, M, N, K, A, lda, B, ldb, C, ldc, out_f32 != 0, false,
                   (hipStream_t)stream, ws, gemm::kScratchBytes);
}

const char* gemm_bf16_config_name(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return "invalid";
  gemm::Plan p = gemm::choose_plan(M, N, K);
  memcpy(gemm::g_name_buf, p.name, sizeof p.name);
  return gemm::g_name_buf;
}

const char* gemm_bf16_config_at(int i) { return gemm::config_at(i, false); }

const char* gemm_bf16_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_ARG: return "invalid argument (negative size, ld too small, or NULL)";
    case GEMM_ERR_MISALIGNED: return "misaligned (pointers need 16 B, leading dims a multiple of 8)";
    case GEMM_ERR_UNSUPPORTED:
      return "unsupported (size beyond 32-bit offsets, unknown config, or a config not built "
             "for fp16)";
    case GEMM_ERR_HIP: return "HIP runtime error (see gemm_bf16_last_hip_error)";
    case GEMM_ERR_CAPTURE:
      return "the stream is being captured and this shape needs a larger split-K workspace than "
             "the one reserved for it (reserve it before capture)";
    case GEMM_ERR_SCRATCH:
      return "this plan's split-K partials exceed the static scratch of the no-allocation "
             "entry point";
    default: return "unknown status";
  }
}

int gemm_bf16_last_hip_error(void) { return gemm::g_last_hip_error; }

int gemm_bf16_reserve_workspace(size_t bytes, void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gemm::hip_fail(e);
  void* ws = nullptr;
  return gemm::get_workspace(dev, (hipStream_t)stream, bytes < 256 ? 256 : bytes, &ws);
}

size_t gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 0) return 0;
  gemm::Plan p = gemm::choose_plan(M, N, K);
  return gemm::workspace_bytes(p, M, N);
}

int gemm_bf16_release_workspace(void) {
  std::lock_guard<std::mutex> lk(gemm::g_ws_mu);
  int rc = GEMM_OK;
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  auto release = [&](std::vector<gemm::Workspace>& list) {
    for (gemm::Workspace& w : list) {
      hipError_t e = hipSetDevice(w.device);
      if (e == hipSuccess) e = hipStreamSynchronize(w.stream);
      if (e == hipSuccess) e = hipFree(w.ptr);
      if (e != hipSuccess) rc = gemm::hip_fail(e);
    }
    list.clear();
  };
  release(gemm::g_ws);
  release(gemm::g_retired);
  // restore the caller's device; a failure here is reported like the rest
  if (have_cur) {
    hipError_t e = hipSetDevice(cur);
    if (e != hipSuccess) rc = gemm::hip_fail(e);
  }
  return rc;
}

}  // extern "C"
