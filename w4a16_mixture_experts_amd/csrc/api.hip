// api.hip -- host side of the C ABI: argument checks, the variant plan,
// workspace carving and kernel enqueueing.  Nothing here allocates device
// memory, synchronizes or reads device values back.
//
// Sources: [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE
// backend" (Modification: small-batch split-K, route-count-based tile
// selection; BC-breaking: explicit selections are strict errors);
// [P3] TensorRT-LLM PR #18313, "Add W4A16 per-channel weight-only support for
// Cutlass fused MoE" (Description: diagnostics that name the offending tensor
// instead of a bare assertion).
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

#include "../../include/w4a16_moe.h"
#include "device.h"
#include "internal.h"
#include "router.h"

static_assert(W4A16_ROUTE_CHUNKS_MAX == w4moe::kRouteChunksMax,
              "the header states the route scratch size");

namespace {

thread_local std::string g_last_error;

w4a16_status_t fail(w4a16_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Plan {
  int path = 2, bm = 64, kslice = 128, nkb = 1;
  int n_tiles_up = 0, n_tiles_down = 0, mode_up = 0;
  bool down_resident = false;  // grouped path: down GEMM with the tile's rows resident in LDS
  int col_steps = 0;
  int splitk_S = 0, splitk_cb = 0;  // split-K gate/up chunks and blocks per chunk (0: off)
  int splitk_nc = 0, splitk_passes = 0;  // column chunks, column passes per chunk
  int small_slots = 1;    // small batch: gate/up grid rows (distinct experts expected)
  int64_t R = 0, P = 0, MT = 0, items = 0;
  int N1 = 0;
  bool x16 = false;       // streaming tile launches take the exact fp16 route
  bool x16_down = false;  // so does the resident down GEMM
  int64_t n_redo_up = 0, n_redo_down = 0;  // rerun flags of those launches
  bool fused_fin = false;  // the combine runs inside the down launch
  // split-K gate/up with the resident down kernel: the down kernel forms the
  // activations from the partials while staging (no activation launch)
  bool act_in_down = false;
  bool tile_sort = false;  // tile launches take tiles biggest first (tile order)
  size_t off_counts = 0, off_offsets = 0, off_slot = 0, off_sorted = 0, off_tile = 0,
         off_order = 0,
         off_act = 0, off_y = 0, off_part = 0, off_chunks = 0, off_redo = 0, off_fin = 0,
         total = 0;
};

w4a16_status_t check_desc(const w4a16_moe_desc_t* d) {
  if (d == nullptr) return fail(W4A16_ERR_INVALID_ARG, "desc: null pointer");
  if (d->num_tokens < 0) return fail(W4A16_ERR_INVALID_ARG, "desc.num_tokens: %d < 0", d->num_tokens);
  if (d->hidden <= 0) return fail(W4A16_ERR_INVALID_ARG, "desc.hidden: %d <= 0", d->hidden);
  if (d->intermediate <= 0)
    return fail(W4A16_ERR_INVALID_ARG, "desc.intermediate: %d <= 0", d->intermediate);
  if (d->num_local_experts <= 0)
    return fail(W4A16_ERR_INVALID_ARG, "desc.num_local_experts: %d <= 0", d->num_local_experts);
  if (d->top_k <= 0) return fail(W4A16_ERR_INVALID_ARG, "desc.top_k: %d <= 0", d->top_k);
  if (d->dtype != W4A16_DT_BF16 && d->dtype != W4A16_DT_FP16)
    return fail(W4A16_ERR_INVALID_ARG, "desc.dtype: unknown value %d", d->dtype);
  if (d->act != W4A16_ACT_SILU_GATED && d->act != W4A16_ACT_RELU2)
    return fail(W4A16_ERR_INVALID_ARG, "desc.act: unknown value %d", d->act);
  if (d->qlayout != W4A16_Q_GROUP_K && d->qlayout != W4A16_Q_PER_CHANNEL &&
      d->qlayout != W4A16_Q_FP4_GROUP_K)
    return fail(W4A16_ERR_INVALID_ARG, "desc.qlayout: unknown value %d", d->qlayout);
  if (d->num_local_experts > 1024)
    return fail(W4A16_ERR_UNSUPPORTED, "desc.num_local_experts: %d > 1024", d->num_local_experts);
  if (d->top_k > 32) return fail(W4A16_ERR_UNSUPPORTED, "desc.top_k: %d > 32", d->top_k);
  if (d->qlayout != W4A16_Q_PER_CHANNEL && d->group_size != 32)
    return fail(W4A16_ERR_UNSUPPORTED, "desc.group_size: %d (only 32 is supported)", d->group_size);
  if (d->hidden % 64 != 0)
    return fail(W4A16_ERR_UNSUPPORTED,
                "w13_packed/w2_packed: hidden=%d is not a multiple of 64", d->hidden);
  if (d->intermediate % 64 != 0)
    return fail(W4A16_ERR_UNSUPPORTED,
                "w13_packed/w2_packed: intermediate=%d is not a multiple of 64", d->intermediate);
  const int64_t R = static_cast<int64_t>(d->num_tokens) * d->top_k;
  if (R > (int64_t(1) << 26))
    return fail(W4A16_ERR_UNSUPPORTED, "topk_ids: %lld routes exceed 2^26", (long long)R);
  if (d->force_block_m != 0 && d->force_block_m != 64)
    return fail(W4A16_ERR_INVALID_ARG, "desc.force_block_m: %d (0 or 64)", d->force_block_m);
  if (d->force_path < 0 || d->force_path > 2)
    return fail(W4A16_ERR_INVALID_ARG, "desc.force_path: %d (0, 1 or 2)", d->force_path);
  if (d->force_tile_order < 0 || d->force_tile_order > 2)
    return fail(W4A16_ERR_INVALID_ARG, "desc.force_tile_order: %d (0, 1 or 2)",
                d->force_tile_order);
  if (d->force_splitk < 0 || d->force_splitk > 2)
    return fail(W4A16_ERR_INVALID_ARG, "desc.force_splitk: %d (0, 1 or 2)", d->force_splitk);
  if (d->fp16_route != 0 && d->fp16_route != 1)
    return fail(W4A16_ERR_INVALID_ARG, "desc.fp16_route: %d (0 or 1)", d->fp16_route);
  if (d->fused_finalize < 0 || d->fused_finalize > 1)
    return fail(W4A16_ERR_INVALID_ARG, "desc.fused_finalize: %d (0 or 1)", d->fused_finalize);
  if (d->num_global_experts != 0 && d->num_global_experts < d->num_local_experts)
    return fail(W4A16_ERR_INVALID_ARG, "desc.num_global_experts: %d < num_local_experts %d",
                d->num_global_experts, d->num_local_experts);
  return W4A16_OK;
}

// Variant selection from the route count R = T*K ([P1] Modification:
// route-count-based tile selection and small-batch split-K).
//   path 2 (small batch): R <= 128.  No route preparation; the gate/up kernel
//     finds each touched expert's rows in the ids and splits the reduction
//     over 8 waves; the down kernel combines per token.
//   path 1 (grouped): route preparation into 64-row expert tiles (empty
//     16-row subtiles are skipped at run time), the gate/up GEMM per tile
//     (streaming or split-K), the down GEMM and the FP32 combine.
// Expected routes per touched expert under uniform routing: R routes over E
// experts touch E (1 - (1 - 1/E)^R) of them in expectation.  With a local
// share (E of num_global_experts), routes are counted valid in proportion.
double routes_per_touched_expert(const w4a16_moe_desc_t* d, int64_t routes, bool local_share) {
  const double E = static_cast<double>(d->num_local_experts);
  const double share = local_share && d->num_global_experts > d->num_local_experts
                           ? E / d->num_global_experts
                           : 1.0;
  const double R = static_cast<double>(routes) * share;
  const double D = std::max(1.0, E * (1.0 - std::pow(1.0 - 1.0 / E, R)));
  return R / D;
}

Plan make_plan(const w4a16_moe_desc_t* d) {
  Plan pl;
  const int E = d->num_local_experts, H = d->hidden, I = d->intermediate, K = d->top_k;
  const bool gated = d->act == W4A16_ACT_SILU_GATED;
  pl.R = static_cast<int64_t>(d->num_tokens) * K;
  pl.N1 = gated ? 2 * I : I;
  pl.mode_up = gated ? w4moe::MODE_UP_GATED : w4moe::MODE_UP_RELU2;
  const int down_blocks = (I + 127) / 128;
  pl.items = static_cast<int64_t>(K) *
             ((down_blocks + w4moe::kDecDownSliceBlocks - 1) / w4moe::kDecDownSliceBlocks);

  // share of the routes expected to be local (uniform routing over the
  // global experts)
  const double share = d->num_global_experts > E
                           ? static_cast<double>(E) / d->num_global_experts : 1.0;
  if (d->force_path) pl.path = d->force_path;
  // the small-batch down kernel stages the pre-activations of every valid
  // route of its token per 32-column workgroup, so the choice counts the
  // routes expected to be local (in proportion to the local share of the
  // global experts).  Measured faster than the grouped path for 1-8 tokens
  // when that count times I is small: the I=256 top-8 shard, the I=1408
  // top-4 per-channel model, the I=2048 top-8 share of 32 of 256 experts
  // (one local route per token: 57 -> 16 us at 1 token, 96 -> 82 us at 8);
  // several times slower for an I=2048 top-8 model whose routes are all local.
  // Past 64 routes (the second ballot) only when every route is expected to
  // be local: the gate/up grid has a workgroup per (16 columns, route slot),
  // and one whose slot owns no local expert still pays the ids round trip
  // before it exits.  Measured: the 384-expert shard at 12 and 16 tokens
  // 125 -> 78 and 124 -> 94 us, the per-channel model at 16 and 32 tokens
  // 111 -> 79 and 132 -> 123 us; the 32-of-256 share at 16 tokens 107 ->
  // 170 us (about 29,000 of its 32,768 workgroups exit)
  // Refined by forced runs of both paths (cold us, small batch / grouped):
  // - the work of the gate/up grid, (N1 / 16) x the local experts expected,
  //   decides past a few tokens: the per-channel model 78 / 89 at 16 tokens
  //   (about 6,970 working workgroups) but 107 / 91 at 24 (8,450) and 133 /
  //   92 at 32; the skewed ReLU^2 model 72 / 95 at 8 tokens (4,640) but 121 /
  //   114 at 16 (7,790); the 384-expert shard 86 / 92 at 16 (3,490);
  // - K x local share x I up to 12,288: the skewed ReLU^2 model (top-6, I =
  //   1856: 11,136) 24 / 50 us at 1 token and 72 / 95 at 8;
  // - the 32-of-256 share up to 96 routes: 67 / 82 at 12 tokens, 123 / 106
  //   at 16.
  else {
    const int64_t max_routes = share < 1.0 ? 96 : w4moe::kSmallMaxRoutes;
    const double Ed = static_cast<double>(E);
    const double local = static_cast<double>(pl.R) * share;
    const double dexp = Ed * (1.0 - std::pow(1.0 - 1.0 / Ed, local));
    const double working = (pl.N1 / 16) * dexp;
    pl.path = (pl.R <= max_routes && pl.items <= w4moe::kDecMaxItems &&
               H <= 8 * w4moe::kSmallMaxSlice && K * share * I <= 12288.0 &&
               working <= 7400.0 &&
               static_cast<int64_t>(K) * I <= w4moe::kDecActLoads * w4moe::kDecThreadsAll * 8)
                  ? 2 : 1;
  }

  // small batch: one gate/up workgroup row per route slot, or, when far
  // fewer distinct local experts than routes are expected, a row per
  // distinct expert expected with a margin (a row takes a second expert when
  // there are more).  The compact grid spares the rows whose slot owns no
  // local expert their ids round trip, but every row then finds the owners
  // with a chain of ballots, one per distinct expert: measured on the
  // 32-of-256 share at 8 tokens 82 -> 74 us; with rows about as many as
  // experts (the 60-expert model at 32 tokens) it was 123 -> 188 us
  pl.small_slots = static_cast<int>(std::max<int64_t>(pl.R, 1));
  if (pl.R > 0) {
    const double Ed = static_cast<double>(E);
    const double dexp = Ed * (1.0 - std::pow(1.0 - 1.0 / Ed, static_cast<double>(pl.R) * share));
    const int64_t rows = static_cast<int64_t>(std::ceil(1.5 * dexp)) + 2;
    if (2 * rows < pl.R) pl.small_slots = static_cast<int>(rows);
  }
  // per-wave reduction slice of the small-batch gate/up kernel (8 waves)
  const int up_blocks = (H + 127) / 128;
  const int per_wave = (up_blocks + w4moe::kSmallWaves - 1) / w4moe::kSmallWaves;
  pl.kslice = per_wave * 128;
  pl.nkb = per_wave;

  const int64_t touched = std::min<int64_t>(E, pl.R);
  pl.P = pl.R + touched * (pl.bm - 1);
  pl.MT = pl.P / pl.bm;
  pl.n_tiles_up = gated ? (I + w4moe::kTileColsGated - 1) / w4moe::kTileColsGated
                        : (I + w4moe::kTileColsPlain - 1) / w4moe::kTileColsPlain;
  pl.n_tiles_down = (H + w4moe::kTileColsPlain - 1) / w4moe::kTileColsPlain;
  // split-K gate/up when tiles are expected to hold few routes (every route
  // counted) and the streaming launch would leave much of its last round of
  // workgroups (one per CU) empty, and only before the resident down kernel,
  // which then forms the activations from the partials (no activation launch;
  // N1 small, so are the partials).  Measured, forced split-K against the
  // streaming kernel (cold us): Kimi shard 153 / 161 at 32 tokens (fill 0.73),
  // 237 / 244 at 64 (0.74), even at 80 (0.83), 181 streaming against 197 at
  // 48 (0.95) and 255-269 against 276-296 at 96-128 (0.86-0.93); with a
  // larger intermediate (the DeepSeek share, the per-channel model, the
  // skewed ReLU^2 model: 8-16 column tiles per expert tile) the streaming
  // kernel won at every token count from 16 to 128, by 9-54 us.
  if (pl.R > 0) {
    const double rpe_all = routes_per_touched_expert(d, pl.R, false);
    const double Ed = static_cast<double>(E);
    const double touched =
        std::max(1.0, Ed * (1.0 - std::pow(1.0 - 1.0 / Ed, static_cast<double>(pl.R))));
    const double wgs = touched * pl.n_tiles_up;
    const double fill = wgs / (w4moe::kComputeUnits * std::ceil(wgs / w4moe::kComputeUnits));
    bool use = rpe_all <= 3.0 && I <= w4moe::kResidentK && fill < 0.8;
    if (d->force_splitk == 1) use = true;
    if (d->force_splitk == 2) use = false;
    if (use) {
      const int nblk = (H + 127) / 128;
      // chunks of an even number of blocks (scales load per block pair)
      const int cb_max = ((w4moe::kSplitkMaxLds / (16 * 2) - 8) / 128) & ~1;
      const int64_t mt = std::max<int64_t>(pl.MT, 1);
      int S = static_cast<int>(std::max<int64_t>((1024 + mt - 1) / mt, (nblk + cb_max - 1) / cb_max));
      S = std::max(1, std::min(S, (nblk + 1) / 2));
      pl.splitk_cb = std::min(cb_max, (((nblk + S - 1) / S) + 1) & ~1);
      pl.splitk_S = (nblk + pl.splitk_cb - 1) / pl.splitk_cb;
      // column chunks so that even a single touched expert spreads over the
      // GPU (the tile capacity overcounts tiles when few routes are local)
      const int passes = (pl.N1 + w4moe::kSplitkPassRows - 1) / w4moe::kSplitkPassRows;
      const int64_t wgs = mt * pl.splitk_S;
      const int nc = static_cast<int>(
          std::min<int64_t>(passes, std::max<int64_t>(1, (1024 + wgs - 1) / wgs)));
      pl.splitk_passes = (passes + nc - 1) / nc;
      pl.splitk_nc = (passes + pl.splitk_passes - 1) / pl.splitk_passes;
    }
  }
  // short reductions: one workgroup per (tile, column chunk) keeps the tile's
  // activation rows in LDS and walks col_steps column tiles; chunks are sized
  // so that the tile capacity times the chunks fills the GPU about 8 times
  // Exact fp16 route of the streaming tile kernels (bf16 activations, bf16
  // group scales): it drops the per-group scaling of the output, which pays
  // when tiles hold several 16-row subtiles; each such launch is followed by
  // a small launch that reruns tiles with activations outside fp16's range.
  // Measured on the Kimi shard: 549 -> 532 us at about 43 routes per expert
  // (2048 tokens), 373 -> 369 us at about 21 (1024 tokens); tiles of one
  // subtile (5 routes per expert at 256 tokens) keep the per-group form.
  // Routes are counted as valid in proportion to the local share of the
  // global experts (uniform routing).
  if (pl.R > 0 && d->dtype == W4A16_DT_BF16 && d->qlayout == W4A16_Q_GROUP_K &&
      d->fp16_route == 1) {
    pl.x16 = routes_per_touched_expert(d, pl.R, true) >= 16.0;
  }
  pl.down_resident = I <= w4moe::kResidentK;
  // Tile order: with many routes per expert the tiles differ in size (two to
  // four non-empty subtiles around 43 routes per expert, a full tile and a
  // tail around 64), and workgroups taken in route order leave the last ones
  // on each CU at random sizes (the SQ busy counters of the Kimi shard's
  // gate/up at 2048 tokens: shader engines idle 17 % of the launch); the
  // biggest tiles first end the launch sooner.  It costs each workgroup one
  // more round trip before its loads.  Measured, forward: the Kimi shard 510
  // -> 495 us at 2048 tokens, 361 -> 358 at 1024, 281 -> 283 at 256; the
  // 32-of-256 share 461 -> 423 at 2048, 231 -> 227 at 512; the skewed ReLU^2
  // model (mostly full tiles) 1035 -> 1055 at 4096 tokens, 355 -> 357 at 1024.
  // Refined by forced runs (route order / biggest first, cold us): the Kimi
  // shard 313 / 307 at 512 tokens (10.7 routes per expert); the DeepSeek
  // share 236 / 224, 276 / 266, 463 / 447 at 512-2048 (16-64); the
  // per-channel model 109 / 106 and 235 / 228 at 256 and 1024 (17, 68); the
  // skewed ReLU^2 model 363 / 354 at 1024 (48) but 626 / 652 at 2048 (96);
  // the tiny model 26 / 27 at 256, whose 24 workgroups are one round: the
  // order only shortens the tail of a launch of several rounds.
  if (pl.path == 1 && pl.R > 0) {
    const double rpe = routes_per_touched_expert(d, pl.R, true);
    const double Ed = static_cast<double>(E);
    const double local = static_cast<double>(pl.R) * share;
    const double touched = Ed * (1.0 - std::pow(1.0 - 1.0 / Ed, local));
    const double wgs = touched * std::ceil(rpe / pl.bm) * pl.n_tiles_up;
    pl.tile_sort = rpe >= w4moe::kTileSortMinRoutes && rpe <= w4moe::kTileSortMaxRoutes &&
                   wgs > w4moe::kComputeUnits;
    if (d->force_tile_order == 1) pl.tile_sort = false;
    if (d->force_tile_order == 2) pl.tile_sort = true;
  }
  // The down GEMM takes the fp16 route under the same condition (measured on
  // the Kimi shard's resident kernel: 167 -> 148 us at 2048 tokens; tiles of
  // one subtile were slower on it).
  pl.x16_down = pl.x16;
  // Measured on the Kimi shard (one workgroup-pass of loads per tile: the
  // padding rows load nothing): the activation launch and its dependent
  // start are saved at 32-128 tokens.
  pl.act_in_down = pl.path == 1 && pl.splitk_S > 0 && pl.down_resident && !pl.x16_down;
  if (pl.down_resident) {
    const int64_t steps = pl.n_tiles_down;
    const int64_t mt = std::max<int64_t>(pl.MT, 1);
    // workgroups aimed at (over the tile capacity): fewer, longer ones when
    // tiles hold few routes, more when tiles are full and compute-heavy.
    // Measured on the Kimi shard against a flat 2048: 1024 at 32 tokens
    // (down GEMM 55.4 -> 50.8 us; 512 was no better than 2048), 4096 at 2048
    // tokens (147.8 -> 141.2 us; 8192 was no better); 256 and 1024 tokens flat
    const double rpe = routes_per_touched_expert(d, pl.R, true);
    const int64_t target = rpe < 4.0 ? 1024 : (rpe >= 32.0 ? 4096 : 2048);
    const int64_t chunks = std::min<int64_t>(steps, std::max<int64_t>(1, (target + mt - 1) / mt));
    pl.col_steps = static_cast<int>((steps + chunks - 1) / chunks);
    pl.n_tiles_down = static_cast<int>((steps + pl.col_steps - 1) / pl.col_steps);
  }

  // fused finalize on request ([P2]'s fused mode: the combine inside the down
  // launch, arrival counters per token and column chunk), except on the
  // opted-in fp16 down route, whose rerun launch would count routes twice.
  // Not the default: measured on MI355X it is about twice as slow as the
  // combine launch of its own (Kimi shard down + combine at 256 tokens: 212
  // against 110 us), since each workgroup's agent-scope release is an L2
  // write-back
  pl.fused_fin = pl.path == 1 && pl.R > 0 && !pl.x16_down && d->fused_finalize == 1;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  if (pl.path == 2) {
    pl.off_act = take(sizeof(float) * std::max<int64_t>(pl.R, 1) * pl.N1);  // FP32 pre-activations
  } else {
    pl.off_counts = take(sizeof(int32_t) * E);
    pl.off_chunks = take(sizeof(int32_t) * w4moe::kRouteChunksMax * E);
    pl.off_offsets = take(sizeof(int32_t) * (E + 1));
    pl.off_slot = take(sizeof(int32_t) * std::max<int64_t>(pl.R, 1));
    pl.off_sorted = take(sizeof(int32_t) * std::max<int64_t>(pl.P, 1));
    pl.off_tile = take(sizeof(int32_t) * std::max<int64_t>(pl.MT, 1));
    if (pl.tile_sort) pl.off_order = take(sizeof(int32_t) * std::max<int64_t>(pl.MT, 1));
    pl.off_act = take(sizeof(uint16_t) * pl.P * I);
    pl.off_y = take(sizeof(uint16_t) * std::max<int64_t>(pl.R, 1) * H);  // Y rows by route
    if (pl.splitk_S > 0)
      pl.off_part = take(sizeof(float) * static_cast<size_t>(pl.splitk_S) * pl.R * pl.N1);
    if (pl.fused_fin)
      pl.off_fin = take(sizeof(int32_t) * static_cast<size_t>(d->num_tokens) * pl.n_tiles_down);
    // rerun flags of the fp16-route launches: the gate/up launch's, then the
    // down launch's
    const int64_t mt = std::max<int64_t>(pl.MT, 1);
    pl.n_redo_up = (pl.x16 && pl.splitk_S == 0) ? w4moe::tile_launch_workgroups(pl.n_tiles_up, mt) : 0;
    pl.n_redo_down = pl.x16_down ? w4moe::tile_launch_workgroups(pl.n_tiles_down, mt) : 0;
    if (pl.n_redo_up + pl.n_redo_down > 0)
      pl.off_redo = take(sizeof(int32_t) * (pl.n_redo_up + pl.n_redo_down));
  }
  pl.total = off;
  return pl;
}

// Grid limits of the launches a plan makes.
w4a16_status_t check_plan(const w4a16_moe_desc_t* d, const Plan& pl) {
  if (pl.MT > 65535)
    return fail(W4A16_ERR_UNSUPPORTED, "topk_ids: %lld expert tiles exceed 65535 (too many routes)",
                (long long)pl.MT);
  if (d->num_tokens > 65535)
    return fail(W4A16_ERR_UNSUPPORTED, "x: num_tokens=%d exceeds 65535", d->num_tokens);
  // 32-bit buffer offsets: x and one expert's packed weights or scales
  if (static_cast<int64_t>(d->num_tokens) * d->hidden * 2 >= (int64_t(1) << 31))
    return fail(W4A16_ERR_UNSUPPORTED, "x: %lld bytes (2^31 or more)",
                (long long)d->num_tokens * d->hidden * 2);
  if (static_cast<int64_t>(pl.N1) * d->hidden >= (int64_t(1) << 31))
    return fail(W4A16_ERR_UNSUPPORTED, "w13_packed: one expert's weights reach 2^30 bytes");
  if (pl.path == 2 && pl.R > w4moe::kSmallMaxRoutes)
    return fail(W4A16_ERR_UNSUPPORTED, "topk_ids: %lld routes exceed the small-batch path's %d",
                (long long)pl.R, w4moe::kSmallMaxRoutes);
  if (pl.path == 2 && d->hidden > 8 * w4moe::kSmallMaxSlice)
    return fail(W4A16_ERR_UNSUPPORTED, "x: hidden=%d exceeds the small-batch path's %d",
                d->hidden, 8 * w4moe::kSmallMaxSlice);
  if (pl.path == 2 &&
      static_cast<int64_t>(d->top_k) * d->intermediate > w4moe::kDecActLoads * w4moe::kDecThreadsAll * 8)
    return fail(W4A16_ERR_UNSUPPORTED,
                "topk_ids/w2_packed: top_k * intermediate = %lld exceeds the small-batch path's %d",
                (long long)d->top_k * d->intermediate, w4moe::kDecActLoads * w4moe::kDecThreadsAll * 8);
  if (pl.path == 2 && pl.items > w4moe::kDecMaxItems)
    return fail(W4A16_ERR_UNSUPPORTED,
                "w2_packed: top_k * slices = %lld exceeds the small-batch path's %d",
                (long long)pl.items, w4moe::kDecMaxItems);
  return W4A16_OK;
}

bool misaligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

w4a16_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return W4A16_OK;
  return fail(W4A16_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* w4a16_status_string(w4a16_status_t s) {
  switch (s) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_ARG: return "invalid argument";
    case W4A16_ERR_UNSUPPORTED: return "unsupported configuration";
    case W4A16_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case W4A16_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* w4a16_last_error_message(void) { return g_last_error.c_str(); }

w4a16_status_t w4a16_moe_workspace_size(const w4a16_moe_desc_t* desc, size_t* bytes) {
  const w4a16_status_t st = check_desc(desc);
  if (st != W4A16_OK) return st;
  if (bytes == nullptr) return fail(W4A16_ERR_INVALID_ARG, "bytes: null pointer");
  const Plan pl = make_plan(desc);
  const w4a16_status_t st2 = check_plan(desc, pl);
  if (st2 != W4A16_OK) return st2;
  *bytes = pl.total;
  return W4A16_OK;
}

w4a16_status_t w4a16_moe_get_plan(const w4a16_moe_desc_t* desc, w4a16_moe_plan_t* plan) {
  const w4a16_status_t st = check_desc(desc);
  if (st != W4A16_OK) return st;
  if (plan == nullptr) return fail(W4A16_ERR_INVALID_ARG, "plan: null pointer");
  const Plan pl = make_plan(desc);
  const w4a16_status_t st2 = check_plan(desc, pl);
  if (st2 != W4A16_OK) return st2;
  plan->path = pl.path;
  plan->block_m = pl.bm;
  plan->k_slice = pl.kslice;
  plan->splitk_chunks = pl.splitk_S;
  plan->max_positions = pl.P;
  plan->max_tiles = pl.MT;
  plan->workspace_bytes = pl.total;
  const bool up16 = pl.path == 1 && pl.n_redo_up > 0;
  const bool dn16 = pl.path == 1 && pl.n_redo_down > 0;
  plan->fp16_route = (up16 ? 1 : 0) | (dn16 ? 2 : 0);
  plan->rerun_flags_up = up16 ? static_cast<int32_t>(pl.n_redo_up) : 0;
  plan->rerun_flags_down = dn16 ? static_cast<int32_t>(pl.n_redo_down) : 0;
  plan->rerun_flags_offset = (up16 || dn16) ? pl.off_redo : 0;
  plan->fused_combine = pl.fused_fin ? 1 : 0;
  plan->tile_order = pl.tile_sort ? 1 : 0;
  plan->act_in_down = pl.act_in_down ? 1 : 0;
  return W4A16_OK;
}

}  // extern "C"

namespace {

struct StageEvents {
  hipEvent_t* ev;
  int n;
  hipStream_t s;
  hipError_t mark(int i) const {
    return (ev != nullptr && i < n && ev[i] != nullptr) ? hipEventRecord(ev[i], s) : hipSuccess;
  }
};

// Checks of the router arguments of a routed call (logits [T][Eg] fp32).
w4a16_status_t check_route(const w4a16_moe_desc_t* d, const float* logits, int renormalize,
                           int* eg) {
  const int Eg = d->num_global_experts > 0 ? d->num_global_experts : d->num_local_experts;
  if (Eg > w4moe::kRouterMaxExperts)
    return fail(W4A16_ERR_UNSUPPORTED, "router_logits: num_global_experts=%d exceeds %d", Eg,
                w4moe::kRouterMaxExperts);
  if (d->top_k > Eg)
    return fail(W4A16_ERR_UNSUPPORTED, "topk_ids: top_k=%d exceeds num_global_experts=%d",
                d->top_k, Eg);
  if (renormalize != 0 && renormalize != 1)
    return fail(W4A16_ERR_INVALID_ARG, "renormalize: %d (0 or 1)", renormalize);
  if (d->num_tokens > 0 && logits == nullptr)
    return fail(W4A16_ERR_INVALID_ARG, "router_logits: null pointer");
  if (misaligned(logits, 4))
    return fail(W4A16_ERR_INVALID_ARG, "router_logits: address not 4-byte aligned");
  *eg = Eg;
  return W4A16_OK;
}

// route != nullptr: the tokens are routed from route->logits inside the
// forward's first launch, which writes topk_ids and topk_weights (the
// caller's buffers, then read by the later kernels).
w4a16_status_t forward_impl(const void* x, const uint8_t* w13_packed, const void* w13_scales,
                            const uint8_t* w2_packed, const void* w2_scales,
                            const int32_t* topk_ids, const float* topk_weights, void* out,
                            const w4a16_moe_desc_t* desc, void* workspace, size_t workspace_bytes,
                            w4a16_stream_t stream_, hipEvent_t* events, int n_events,
                            const w4moe::RouteArgs* route = nullptr) {
  w4a16_status_t st = check_desc(desc);
  if (st != W4A16_OK) return st;
  const Plan pl = make_plan(desc);
  st = check_plan(desc, pl);
  if (st != W4A16_OK) return st;
  if (n_events < 0) return fail(W4A16_ERR_INVALID_ARG, "n_events: %d < 0", n_events);
  if (desc->num_tokens == 0) return W4A16_OK;

  struct {
    const void* p;
    const char* name;
    size_t align;
  } ptrs[] = {{x, "x", 16},           {w13_packed, "w13_packed", 16}, {w13_scales, "w13_scales", 4},
              {w2_packed, "w2_packed", 16}, {w2_scales, "w2_scales", 4}, {topk_ids, "topk_ids", 4},
              {topk_weights, "topk_weights", 4}, {out, "out", 16}, {workspace, "workspace", 16}};
  for (const auto& q : ptrs) {
    if (q.p == nullptr) return fail(W4A16_ERR_INVALID_ARG, "%s: null pointer", q.name);
    if (misaligned(q.p, q.align))
      return fail(W4A16_ERR_INVALID_ARG, "%s: address not %zu-byte aligned", q.name, q.align);
  }
  if (workspace_bytes < pl.total)
    return fail(W4A16_ERR_WORKSPACE_TOO_SMALL, "workspace: %zu bytes given, %zu needed",
                workspace_bytes, pl.total);

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const StageEvents evs{events, n_events, stream};
  const int E = desc->num_local_experts, H = desc->hidden, I = desc->intermediate;
  const int K = desc->top_k;
  const bool group = desc->qlayout != W4A16_Q_PER_CHANNEL;  // INT4 or FP4 groups along K
  char* ws = static_cast<char*>(workspace);
  auto* counts = reinterpret_cast<int32_t*>(ws + pl.off_counts);
  auto* offsets = reinterpret_cast<int32_t*>(ws + pl.off_offsets);
  auto* slot = reinterpret_cast<int32_t*>(ws + pl.off_slot);
  auto* sorted = reinterpret_cast<int32_t*>(ws + pl.off_sorted);
  auto* tile = reinterpret_cast<int32_t*>(ws + pl.off_tile);
  auto* order = pl.tile_sort ? reinterpret_cast<int32_t*>(ws + pl.off_order) : nullptr;
  auto* act = reinterpret_cast<uint16_t*>(ws + pl.off_act);
  auto* ybuf = reinterpret_cast<uint16_t*>(ws + pl.off_y);

  const int64_t w13_bytes = static_cast<int64_t>(pl.N1) * H / 2;
  const int64_t w13_sc = group ? static_cast<int64_t>(pl.N1) * (H / 32) : pl.N1;
  const int64_t w2_bytes = static_cast<int64_t>(H) * I / 2;
  const int64_t w2_sc = group ? static_cast<int64_t>(H) * (I / 32) : H;
  const bool gated = desc->act == W4A16_ACT_SILU_GATED;

  if (pl.path == 2) {
    // small batch: FP32 pre-activations per touched expert (rows found in the
    // ids), then the activation, the down GEMM and the combine per token
    w4moe::SmallHParams sh{};
    sh.x = static_cast<const uint16_t*>(x);
    sh.lda = H;
    sh.T = static_cast<int>(desc->num_tokens);
    sh.ids = topk_ids;
    sh.R = static_cast<int>(pl.R);
    sh.slots = pl.small_slots;
    sh.top_k = K;
    sh.E = E;
    sh.off = desc->expert_offset;
    sh.wq = w13_packed;
    sh.ws = static_cast<const uint16_t*>(w13_scales);
    sh.wq_expert_bytes = w13_bytes;
    sh.ws_expert_elems = w13_sc;
    sh.K = H;
    sh.kslice = pl.kslice;
    sh.h = reinterpret_cast<float*>(ws + pl.off_act);
    sh.ldh = pl.N1;
    if (route != nullptr) {
      if (route->Eg <= 64 * w4moe::kSmallRouteNpl && pl.R <= w4moe::kSmallRouteMaxRoutes &&
          static_cast<int64_t>(pl.N1 / 16) * pl.small_slots <= w4moe::kSmallRouteMaxWorkgroups) {
        sh.ra = *route;  // routed inside the gate/up launch
      } else {
        // every gate/up workgroup routes all tokens itself, so beyond a few
        // routes or workgroups (or with more global experts than that launch
        // routes) the router kernel runs first
        st = hip_status(w4moe::launch_router_topk(route->logits, route->T, route->Eg, K,
                                                  route->renorm, route->ids, route->wts, stream),
                        "router launch");
        if (st != W4A16_OK) return st;
      }
    }
    st = hip_status(evs.mark(2), "stage event");
    if (st != W4A16_OK) return st;
    st = hip_status(w4moe::launch_small_h(sh, desc->dtype, desc->qlayout, pl.nkb, pl.N1, stream),
                    "gate/up GEMM launch");
    if (st == W4A16_OK) st = hip_status(evs.mark(3), "stage event");
    if (st != W4A16_OK) return st;
    w4moe::DecodeDownParams dd{};
    dd.h = sh.h;
    dd.ldh = pl.N1;
    dd.wq = w2_packed;
    dd.ws = static_cast<const uint16_t*>(w2_scales);
    dd.wq_expert_bytes = w2_bytes;
    dd.ws_expert_elems = w2_sc;
    dd.ids = topk_ids;
    dd.wts = topk_weights;
    dd.top_k = K;
    dd.E = E;
    dd.off = desc->expert_offset;
    dd.I = I;
    dd.H = H;
    dd.out = static_cast<uint16_t*>(out);
    // the prefetching variant when a token's valid routes are expected to
    // give each wave more than one item (the local share of the routes
    // counted; its two register sets halve the workgroups per CU).  The
    // 32-of-256 share, about one valid route of 8 slices per token, which the
    // top-k count alone sent to it: 59.1 -> 57.4 us at 8 tokens.
    {
      const int nsl = ((I + 127) / 128 + w4moe::kDecDownSliceBlocks - 1) / w4moe::kDecDownSliceBlocks;
      const double share = desc->num_global_experts > E
                               ? static_cast<double>(E) / desc->num_global_experts : 1.0;
      dd.prefetch = K * share * nsl > w4moe::kDecWavesAll ? 1 : 0;
    }
    st = hip_status(evs.mark(4), "stage event");
    if (st != W4A16_OK) return st;
    st = hip_status(w4moe::launch_decode_down(dd, desc->dtype, desc->qlayout, gated,
                                              desc->num_tokens, stream),
                    "down GEMM launch");
    if (st == W4A16_OK) st = hip_status(evs.mark(5), "stage event");
    return st;
  }

  // a1: route preparation into block_m-row expert tiles
  st = hip_status(evs.mark(0), "stage event");
  if (st != W4A16_OK) return st;
  auto* fin_cnt = pl.fused_fin ? reinterpret_cast<int32_t*>(ws + pl.off_fin) : nullptr;
  st = hip_status(w4moe::launch_route_prep(topk_ids, static_cast<int>(pl.R), E,
                                           desc->expert_offset, pl.bm, counts, offsets, sorted,
                                           slot, tile,
                                           reinterpret_cast<int32_t*>(ws + pl.off_chunks), stream,
                                           K, route, fin_cnt,
                                           static_cast<int64_t>(desc->num_tokens) * pl.n_tiles_down,
                                           order),
                  route != nullptr ? "routing and route preparation launch"
                                   : "route preparation launch");
  if (st == W4A16_OK) st = hip_status(evs.mark(1), "stage event");
  if (st != W4A16_OK) return st;

  // a2-a4: gathered gate/up (or w1) GEMM with the activation epilogue
  st = hip_status(evs.mark(2), "stage event");
  if (st != W4A16_OK) return st;
  {
    w4moe::GemmParams up{};
    up.a = static_cast<const uint16_t*>(x);
    up.lda = H;
    up.a_bytes = static_cast<uint32_t>(sizeof(uint16_t) * desc->num_tokens * H);
    up.sorted = sorted;
    up.top_k = K;
    up.wq = w13_packed;
    up.ws = static_cast<const uint16_t*>(w13_scales);
    up.wq_expert_bytes = w13_bytes;
    up.ws_expert_elems = w13_sc;
    up.K = H;
    up.n_cols = I;
    up.up_rows = I;
    up.tile_expert = tile;
    up.tile_order = pl.splitk_S > 0 ? nullptr : order;  // split-K: tiles of similar size
    up.tiles = static_cast<int>(pl.MT);
    up.offsets = offsets;
    up.E = E;
    up.bm = pl.bm;
    up.out = act;
    up.ldo = I;
    up.n_tiles = pl.n_tiles_up;
    up.redo = pl.n_redo_up > 0 ? reinterpret_cast<int32_t*>(ws + pl.off_redo) : nullptr;
    if (pl.splitk_S > 0) {
      up.redo = nullptr;
      up.part = reinterpret_cast<float*>(ws + pl.off_part);
      up.S = pl.splitk_S;
      up.cb = pl.splitk_cb;
      up.R = static_cast<int>(pl.R);
      up.n_cols = pl.N1;
      up.slot = slot;
      up.n_tiles = pl.splitk_nc;
      up.col_steps = pl.splitk_passes;
      st = hip_status(w4moe::launch_up_splitk(up, desc->dtype, desc->qlayout,
                                              static_cast<int>(pl.MT), stream),
                      "gate/up GEMM launch");
      if (st == W4A16_OK && !pl.act_in_down)
        st = hip_status(w4moe::launch_splitk_act(up, desc->dtype, gated, stream),
                        "activation launch");
    } else {
      st = hip_status(w4moe::launch_tile_gemm(up, desc->dtype, desc->qlayout, pl.mode_up,
                                              static_cast<int>(pl.MT), stream),
                      "gate/up GEMM launch");
    }
  }
  if (st == W4A16_OK) st = hip_status(evs.mark(3), "stage event");
  if (st != W4A16_OK) return st;

  // a5: grouped down GEMM -> 16-bit expert outputs
  w4moe::GemmParams dn{};
  dn.a = act;
  dn.lda = I;
  dn.sorted = sorted;
  dn.top_k = K;
  dn.wq = w2_packed;
  dn.ws = static_cast<const uint16_t*>(w2_scales);
  dn.wq_expert_bytes = w2_bytes;
  dn.ws_expert_elems = w2_sc;
  dn.K = I;
  dn.n_cols = H;
  dn.up_rows = 0;
  dn.tile_expert = tile;
  dn.tile_order = order;
  dn.tiles = static_cast<int>(pl.MT);
  dn.offsets = offsets;
  dn.E = E;
  dn.bm = pl.bm;
  dn.out = ybuf;
  dn.ldo = H;
  dn.n_tiles = pl.n_tiles_down;
  dn.redo = pl.n_redo_down > 0
                ? reinterpret_cast<int32_t*>(ws + pl.off_redo) + pl.n_redo_up
                : nullptr;
  if (pl.fused_fin) {
    dn.fin_cnt = fin_cnt;
    dn.wts = topk_weights;
    dn.fin_out = static_cast<uint16_t*>(out);
    dn.fin_chunks = pl.n_tiles_down;
    dn.T = desc->num_tokens;
    dn.slot = slot;
    dn.n_main = static_cast<int>(
        w4moe::tile_launch_workgroups(pl.n_tiles_down, std::max<int64_t>(pl.MT, 1)));
  }
  st = hip_status(evs.mark(4), "stage event");
  if (st != W4A16_OK) return st;
  dn.col_steps = pl.col_steps;
  if (pl.act_in_down) {
    dn.part = reinterpret_cast<float*>(ws + pl.off_part);
    dn.S = pl.splitk_S;
    dn.R = static_cast<int>(pl.R);
    dn.part_ld = pl.N1;
    dn.up_rows = gated ? I : 0;
  }
  st = hip_status(pl.down_resident
                      ? w4moe::launch_down_resident(dn, desc->dtype, desc->qlayout,
                                                    static_cast<int>(pl.MT), stream)
                  : w4moe::launch_tile_gemm(dn, desc->dtype, desc->qlayout, w4moe::MODE_DOWN,
                                            static_cast<int>(pl.MT), stream),
                  "down GEMM launch");
  if (st == W4A16_OK) st = hip_status(evs.mark(5), "stage event");
  if (st != W4A16_OK) return st;

  // a6: FP32 combine in fixed top-k order, one 16-bit cast (inside the down
  // launch when fused)
  if (pl.fused_fin) {  // the combine stage is empty: events back to back
    st = hip_status(evs.mark(6), "stage event");
    if (st == W4A16_OK) st = hip_status(evs.mark(7), "stage event");
    return st;
  }
  w4moe::CombineParams cb{};
  cb.y = ybuf;
  cb.slot = slot;
  cb.wts = topk_weights;
  cb.top_k = K;
  cb.H = H;
  cb.out = static_cast<uint16_t*>(out);
  st = hip_status(evs.mark(6), "stage event");
  if (st != W4A16_OK) return st;
  st = hip_status(w4moe::launch_combine(cb, desc->dtype, desc->num_tokens, stream),
                  "combine launch");
  if (st == W4A16_OK) st = hip_status(evs.mark(7), "stage event");
  return st;
}

}  // namespace

extern "C" {

w4a16_status_t w4a16_moe_forward(const void* x, const uint8_t* w13_packed, const void* w13_scales,
                                 const uint8_t* w2_packed, const void* w2_scales,
                                 const int32_t* topk_ids, const float* topk_weights, void* out,
                                 const w4a16_moe_desc_t* desc, void* workspace,
                                 size_t workspace_bytes, w4a16_stream_t stream) {
  return forward_impl(x, w13_packed, w13_scales, w2_packed, w2_scales, topk_ids, topk_weights,
                      out, desc, workspace, workspace_bytes, stream, nullptr, 0);
}

w4a16_status_t w4a16_moe_forward_timed(const void* x, const uint8_t* w13_packed,
                                       const void* w13_scales, const uint8_t* w2_packed,
                                       const void* w2_scales, const int32_t* topk_ids,
                                       const float* topk_weights, void* out,
                                       const w4a16_moe_desc_t* desc, void* workspace,
                                       size_t workspace_bytes, w4a16_stream_t stream,
                                       void* const* stage_events, int32_t n_events) {
  return forward_impl(x, w13_packed, w13_scales, w2_packed, w2_scales, topk_ids, topk_weights,
                      out, desc, workspace, workspace_bytes, stream,
                      reinterpret_cast<hipEvent_t*>(const_cast<void**>(stage_events)), n_events);
}

w4a16_status_t w4a16_moe_forward_routed(
    const void* x, const uint8_t* w13_packed, const void* w13_scales, const uint8_t* w2_packed,
    const void* w2_scales, const float* router_logits, int32_t renormalize, int32_t* topk_ids,
    float* topk_weights, void* out, const w4a16_moe_desc_t* desc, void* workspace,
    size_t workspace_bytes, w4a16_stream_t stream, void* const* stage_events, int32_t n_events) {
  w4a16_status_t st = check_desc(desc);
  if (st != W4A16_OK) return st;
  int Eg = 0;
  st = check_route(desc, router_logits, renormalize, &Eg);
  if (st != W4A16_OK) return st;
  w4moe::RouteArgs ra{};
  ra.logits = router_logits;
  ra.T = desc->num_tokens;
  ra.Eg = Eg;
  ra.renorm = renormalize;
  ra.ids = topk_ids;
  ra.wts = topk_weights;
  return forward_impl(x, w13_packed, w13_scales, w2_packed, w2_scales, topk_ids, topk_weights,
                      out, desc, workspace, workspace_bytes, stream,
                      reinterpret_cast<hipEvent_t*>(const_cast<void**>(stage_events)), n_events,
                      &ra);
}

w4a16_status_t w4a16_moe_route_and_prepare(const w4a16_moe_desc_t* desc,
                                           const float* router_logits, int32_t renormalize,
                                           int32_t block_m, int32_t* topk_ids,
                                           float* topk_weights, int32_t* counts,
                                           int32_t* offsets, int32_t* sorted_routes,
                                           int64_t sorted_capacity, int32_t* route_slot,
                                           int32_t* chunk_scratch, w4a16_stream_t stream_) {
  if (desc == nullptr) return fail(W4A16_ERR_INVALID_ARG, "desc: null pointer");
  if (desc->num_tokens < 0)
    return fail(W4A16_ERR_INVALID_ARG, "desc.num_tokens: %d < 0", desc->num_tokens);
  if (desc->top_k <= 0 || desc->top_k > w4moe::kRouterMaxTopK)
    return fail(W4A16_ERR_INVALID_ARG, "desc.top_k: %d (1..%d)", desc->top_k,
                w4moe::kRouterMaxTopK);
  if (desc->num_local_experts <= 0 || desc->num_local_experts > 1024)
    return fail(W4A16_ERR_INVALID_ARG, "desc.num_local_experts: %d (1..1024)",
                desc->num_local_experts);
  if (block_m < 1 || block_m > 256)
    return fail(W4A16_ERR_INVALID_ARG, "block_m: %d (1..256)", block_m);
  int Eg = 0;
  w4a16_status_t st = check_route(desc, router_logits, renormalize, &Eg);
  if (st != W4A16_OK) return st;
  const int64_t R = static_cast<int64_t>(desc->num_tokens) * desc->top_k;
  if (R > (int64_t(1) << 26))
    return fail(W4A16_ERR_UNSUPPORTED, "topk_ids: %lld routes exceed 2^26", (long long)R);
  const int64_t need = R + std::min<int64_t>(desc->num_local_experts, R) * (block_m - 1);
  if (sorted_capacity < need)
    return fail(W4A16_ERR_INVALID_ARG, "sorted_routes: capacity %lld < %lld",
                (long long)sorted_capacity, (long long)need);
  struct {
    const void* p;
    const char* name;
  } ptrs[] = {{counts, "counts"}, {offsets, "offsets"}, {sorted_routes, "sorted_routes"},
              {route_slot, "route_slot"}, {topk_ids, "topk_ids"}, {topk_weights, "topk_weights"}};
  for (const auto& q : ptrs) {
    if (q.p == nullptr && !(R == 0 && q.p != counts && q.p != offsets))
      return fail(W4A16_ERR_INVALID_ARG, "%s: null pointer", q.name);
  }
  w4moe::RouteArgs ra{};
  ra.logits = router_logits;
  ra.T = desc->num_tokens;
  ra.Eg = Eg;
  ra.renorm = renormalize;
  ra.ids = topk_ids;
  ra.wts = topk_weights;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_route_prep(topk_ids, static_cast<int>(R),
                                             desc->num_local_experts, desc->expert_offset,
                                             block_m, counts, offsets, sorted_routes, route_slot,
                                             nullptr, chunk_scratch, stream, desc->top_k, &ra),
                    "routing and route preparation launch");
}

w4a16_status_t w4a16_moe_prepare_routes(const w4a16_moe_desc_t* desc, const int32_t* topk_ids,
                                        int32_t block_m, int32_t* counts, int32_t* offsets,
                                        int32_t* sorted_routes, int64_t sorted_capacity,
                                        int32_t* route_slot, int32_t* chunk_scratch,
                                        w4a16_stream_t stream_) {
  if (desc == nullptr) return fail(W4A16_ERR_INVALID_ARG, "desc: null pointer");
  if (desc->num_tokens < 0)
    return fail(W4A16_ERR_INVALID_ARG, "desc.num_tokens: %d < 0", desc->num_tokens);
  if (desc->top_k <= 0 || desc->top_k > 32)
    return fail(W4A16_ERR_INVALID_ARG, "desc.top_k: %d (1..32)", desc->top_k);
  if (desc->num_local_experts <= 0 || desc->num_local_experts > 1024)
    return fail(W4A16_ERR_INVALID_ARG, "desc.num_local_experts: %d (1..1024)",
                desc->num_local_experts);
  if (block_m < 1 || block_m > 256)
    return fail(W4A16_ERR_INVALID_ARG, "block_m: %d (1..256)", block_m);
  const int64_t R = static_cast<int64_t>(desc->num_tokens) * desc->top_k;
  if (R > (int64_t(1) << 26))
    return fail(W4A16_ERR_UNSUPPORTED, "topk_ids: %lld routes exceed 2^26", (long long)R);
  const int64_t need = R + std::min<int64_t>(desc->num_local_experts, R) * (block_m - 1);
  if (sorted_capacity < need)
    return fail(W4A16_ERR_INVALID_ARG, "sorted_routes: capacity %lld < %lld",
                (long long)sorted_capacity, (long long)need);
  struct {
    const void* p;
    const char* name;
  } ptrs[] = {{counts, "counts"}, {offsets, "offsets"}, {sorted_routes, "sorted_routes"},
              {route_slot, "route_slot"}, {topk_ids, "topk_ids"}};
  for (const auto& q : ptrs) {
    if (q.p == nullptr && !(R == 0 && (q.p == route_slot || q.p == topk_ids || q.p == sorted_routes)))
      return fail(W4A16_ERR_INVALID_ARG, "%s: null pointer", q.name);
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_route_prep(topk_ids, static_cast<int>(R),
                                             desc->num_local_experts, desc->expert_offset,
                                             block_m, counts, offsets, sorted_routes, route_slot,
                                             nullptr, chunk_scratch, stream),
                    "route preparation launch");
}

w4a16_status_t w4a16_unpack_int4(const uint8_t* packed, int64_t n_bytes, int8_t* out,
                                 w4a16_stream_t stream_) {
  if (n_bytes < 0) return fail(W4A16_ERR_INVALID_ARG, "n_bytes: %lld < 0", (long long)n_bytes);
  if (n_bytes == 0) return W4A16_OK;
  if (packed == nullptr) return fail(W4A16_ERR_INVALID_ARG, "packed: null pointer");
  if (out == nullptr) return fail(W4A16_ERR_INVALID_ARG, "out: null pointer");
  if (n_bytes > (int64_t(1) << 33))
    return fail(W4A16_ERR_UNSUPPORTED, "n_bytes: %lld too large", (long long)n_bytes);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_unpack(packed, n_bytes, out, stream), "unpack launch");
}

w4a16_status_t w4a16_decode_fp4(const uint8_t* packed, int64_t n_bytes, int32_t dtype, float* out,
                                w4a16_stream_t stream_) {
  if (n_bytes < 0) return fail(W4A16_ERR_INVALID_ARG, "n_bytes: %lld < 0", (long long)n_bytes);
  if (dtype != W4A16_DT_BF16 && dtype != W4A16_DT_FP16)
    return fail(W4A16_ERR_INVALID_ARG, "dtype: %d (bf16 or fp16)", dtype);
  if (n_bytes == 0) return W4A16_OK;
  if (packed == nullptr) return fail(W4A16_ERR_INVALID_ARG, "packed: null pointer");
  if (out == nullptr) return fail(W4A16_ERR_INVALID_ARG, "out: null pointer");
  if (n_bytes > (int64_t(1) << 33))
    return fail(W4A16_ERR_UNSUPPORTED, "n_bytes: %lld too large", (long long)n_bytes);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_decode_fp4(packed, n_bytes, dtype == W4A16_DT_BF16 ? w4moe::DT_BF16
                                                                                  : w4moe::DT_FP16,
                                             out, stream),
                    "FP4 decode launch");
}

w4a16_status_t w4a16_stream_probe(const uint8_t* buf, int64_t bytes, int32_t row_bytes,
                                  uint32_t* sink, w4a16_stream_t stream_) {
  if (row_bytes <= 0 || row_bytes % 64 != 0 || row_bytes > w4moe::kProbeMaxRowBytes)
    return fail(W4A16_ERR_INVALID_ARG, "row_bytes: %d (a multiple of 64, at most %d)", row_bytes,
                w4moe::kProbeMaxRowBytes);
  if (bytes < row_bytes)
    return fail(W4A16_ERR_INVALID_ARG, "bytes: %lld below one row", (long long)bytes);
  if (bytes / row_bytes > (int64_t(1) << 34))
    return fail(W4A16_ERR_UNSUPPORTED, "bytes: %lld too large", (long long)bytes);
  if (buf == nullptr) return fail(W4A16_ERR_INVALID_ARG, "buf: null pointer");
  if (sink == nullptr) return fail(W4A16_ERR_INVALID_ARG, "sink: null pointer");
  if (misaligned(buf, 16)) return fail(W4A16_ERR_INVALID_ARG, "buf: address not 16-byte aligned");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_stream_probe(buf, bytes, row_bytes, sink, stream),
                    "probe launch");
}

w4a16_status_t w4a16_e8m0_to_scales(const uint8_t* e8m0, int64_t n, int32_t dtype, void* out,
                                    w4a16_stream_t stream_) {
  if (n < 0) return fail(W4A16_ERR_INVALID_ARG, "n: %lld < 0", (long long)n);
  if (dtype != W4A16_DT_BF16 && dtype != W4A16_DT_FP16)
    return fail(W4A16_ERR_INVALID_ARG, "dtype: unknown value %d", dtype);
  if (n == 0) return W4A16_OK;
  if (e8m0 == nullptr) return fail(W4A16_ERR_INVALID_ARG, "e8m0: null pointer");
  if (out == nullptr) return fail(W4A16_ERR_INVALID_ARG, "out: null pointer");
  if (misaligned(out, 2)) return fail(W4A16_ERR_INVALID_ARG, "out: address not 2-byte aligned");
  if (n > (int64_t(1) << 36)) return fail(W4A16_ERR_UNSUPPORTED, "n: %lld too large", (long long)n);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_e8m0_to_h16(e8m0, n, dtype, static_cast<uint16_t*>(out), stream),
                    "scale conversion launch");
}

w4a16_status_t w4a16_repack_per_channel(const uint8_t* packed, const void* scales,
                                        int64_t n_experts, int32_t n_out, int32_t k_in,
                                        uint8_t* out_packed, void* out_scales,
                                        w4a16_stream_t stream_) {
  if (n_experts < 0) return fail(W4A16_ERR_INVALID_ARG, "n_experts: %lld < 0", (long long)n_experts);
  if (n_out <= 0 || n_out % 2 != 0)
    return fail(W4A16_ERR_INVALID_ARG, "packed: n_out=%d (a positive even count)", n_out);
  if (k_in <= 0 || k_in % 64 != 0)
    return fail(W4A16_ERR_UNSUPPORTED, "packed: k_in=%d is not a multiple of 64", k_in);
  if (n_experts > 65535)
    return fail(W4A16_ERR_UNSUPPORTED, "n_experts: %lld exceeds 65535", (long long)n_experts);
  if (n_experts == 0) return W4A16_OK;
  const struct {
    const void* p;
    const char* name;
  } ptrs[] = {{packed, "packed"}, {scales, "scales"}, {out_packed, "out_packed"},
              {out_scales, "out_scales"}};
  for (const auto& q : ptrs)
    if (q.p == nullptr) return fail(W4A16_ERR_INVALID_ARG, "%s: null pointer", q.name);
  if (misaligned(out_packed, 4))
    return fail(W4A16_ERR_INVALID_ARG, "out_packed: address not 4-byte aligned");
  if (misaligned(scales, 2) || misaligned(out_scales, 2))
    return fail(W4A16_ERR_INVALID_ARG, "scales/out_scales: address not 2-byte aligned");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_repack_per_channel(
                        packed, static_cast<const uint16_t*>(scales), n_experts, n_out, k_in,
                        out_packed, static_cast<uint16_t*>(out_scales), stream),
                    "repack launch");
}

w4a16_status_t w4a16_moe_route_topk(const float* logits, int64_t num_tokens,
                                    int32_t num_global_experts, int32_t top_k,
                                    int32_t renormalize, int32_t* topk_ids, float* topk_weights,
                                    w4a16_stream_t stream_) {
  if (num_tokens < 0) return fail(W4A16_ERR_INVALID_ARG, "logits: num_tokens=%lld < 0", (long long)num_tokens);
  if (num_tokens > INT32_MAX)
    return fail(W4A16_ERR_UNSUPPORTED, "logits: num_tokens=%lld exceeds %d", (long long)num_tokens,
                INT32_MAX);
  if (num_global_experts < 1 || num_global_experts > w4moe::kRouterMaxExperts)
    return fail(W4A16_ERR_UNSUPPORTED, "logits: num_global_experts=%d (1..%d)", num_global_experts,
                w4moe::kRouterMaxExperts);
  if (top_k < 1 || top_k > w4moe::kRouterMaxTopK || top_k > num_global_experts)
    return fail(W4A16_ERR_UNSUPPORTED, "topk_ids: top_k=%d (1..min(%d, num_global_experts))", top_k,
                w4moe::kRouterMaxTopK);
  if (renormalize != 0 && renormalize != 1)
    return fail(W4A16_ERR_INVALID_ARG, "renormalize: %d (0 or 1)", renormalize);
  if (num_tokens == 0) return W4A16_OK;
  const struct {
    const void* p;
    const char* name;
  } ptrs[] = {{logits, "logits"}, {topk_ids, "topk_ids"}, {topk_weights, "topk_weights"}};
  for (const auto& q : ptrs) {
    if (q.p == nullptr) return fail(W4A16_ERR_INVALID_ARG, "%s: null pointer", q.name);
    if (misaligned(q.p, 4)) return fail(W4A16_ERR_INVALID_ARG, "%s: address not 4-byte aligned", q.name);
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  return hip_status(w4moe::launch_router_topk(logits, static_cast<int>(num_tokens), num_global_experts,
                                              top_k, renormalize, topk_ids, topk_weights, stream),
                    "router launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Forward without a caller workspace (for callers that cannot allocate: code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The scratch is a file-scope device array, one copy per GPU;
// its device address is looked up once per device (with that device
// current) and only that address is handed to kernels or copies.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[W4A16_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on the first call).
w4a16_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W4A16_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(W4A16_ERR_UNSUPPORTED, "device %d: no-alloc scratch supports devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(W4A16_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return W4A16_OK;
}

}  // namespace

extern "C" w4a16_status_t w4a16_moe_forward_noalloc(
    const void* x, const uint8_t* w13_packed, const void* w13_scales, const uint8_t* w2_packed,
    const void* w2_scales, const int32_t* topk_ids, const float* topk_weights, void* out,
    const w4a16_moe_desc_t* desc, w4a16_stream_t stream) {
  w4a16_status_t st = check_desc(desc);
  if (st != W4A16_OK) return st;
  const Plan pl = make_plan(desc);
  st = check_plan(desc, pl);
  if (st != W4A16_OK) return st;
  if (pl.total > static_cast<size_t>(W4A16_NOALLOC_SCRATCH_BYTES))
    return fail(W4A16_ERR_UNSUPPORTED,
                "workspace: %zu bytes needed exceed the no-alloc scratch of %zu bytes "
                "(use w4a16_moe_forward with a caller workspace)",
                pl.total, static_cast<size_t>(W4A16_NOALLOC_SCRATCH_BYTES));
  if (desc->num_tokens == 0) return W4A16_OK;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != W4A16_OK) return st;
  // nothing in the workspace has to start at zero: every kernel writes what
  // a later one reads (flags included) within the same forward
  return forward_impl(x, w13_packed, w13_scales, w2_packed, w2_scales, topk_ids, topk_weights,
                      out, desc, ws, static_cast<size_t>(W4A16_NOALLOC_SCRATCH_BYTES), stream,
                      nullptr, 0);
}
