// internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4moe {

enum : int { MODE_UP_GATED = 0, MODE_UP_RELU2 = 1, MODE_DOWN = 2 };

constexpr int kComputeUnits = 256;   // MI355X
constexpr int kCombineCols = 2048;
constexpr int kTileRows = 64;        // route positions of one LDS-staged expert tile
constexpr int kTileWaves = 8;
constexpr int kTileColsGated = 128;  // activation columns per tile workgroup (gated)
constexpr int kTileColsPlain = 256;  // output columns per tile workgroup otherwise

struct GemmParams {
  const uint16_t* a;          // UP: x [T][lda]; DOWN: act [P][lda] (A operand order)
  int lda;
  uint32_t a_bytes;           // UP: bytes of x (below 2^31)
  const int32_t* sorted;      // [P] route index or -1 (padding)
  int top_k;
  const uint8_t* wq;          // packed weights, expert 0
  const uint16_t* ws;         // scales, expert 0
  int64_t wq_expert_bytes;
  int64_t ws_expert_elems;
  int K;                      // reduction length
  int n_cols;                 // logical output columns (I for gated UP)
  int up_rows;                // gated: row offset of the up weights (= I)
  const int32_t* tile_expert; // [max tiles]
  // null, or the used tiles by descending count of non-empty 16-row
  // subtiles: workgroups take tile_order[position] instead of the position
  const int32_t* tile_order;
  const int32_t* offsets;     // [E+1]; offsets[E] = padded total
  int E;
  int bm;
  uint16_t* out;              // UP: act [P][ldo]; DOWN: Y [T*K][ldo] by route
  int ldo;
  int n_tiles;                // column tiles (resident down / split-K: column chunks)
  int col_steps;              // resident down / split-K: column passes per chunk
  // split-K gate/up (tiles of few rows)
  float* part;                // [S][R][n_cols] FP32 partial pre-activations
  int S;                      // reduction chunks
  int cb;                     // 128-blocks per chunk
  int R;                      // routes (T*K)
  // resident down kernel: non-null part selects activations formed from the
  // split-K partials [S][R][part_ld] while staging (the up values of a
  // partial row at column offset up_rows; 0: ReLU^2) instead of reading `a`
  int part_ld;
  const int32_t* slot;        // [R] route -> position, -1 for invalid routes
  int tiles;                  // entries of tile_expert (positions / bm)
  // streaming tile kernel, bf16 group layout: non-null selects the exact
  // fp16 route; one flag per workgroup (set when its tile is to be rerun)
  int32_t* redo;
  // DOWN with the combine fused in: non-null selects it.  fin_cnt holds one
  // arrival counter per (token, column chunk), zeroed by route preparation;
  // the workgroup whose arrival completes a token's valid routes for a chunk
  // combines them (slot: route -> position, -1 invalid; wts [T][K]) into
  // fin_out; workgroups from n_main on write zeros for tokens without a
  // valid route.
  int32_t* fin_cnt;
  const float* wts;
  uint16_t* fin_out;
  int fin_chunks;
  int T;
  int n_main;
};

// Workgroups that zero the output rows of tokens without a valid route
// (fused combine): one wave per token.
constexpr int kFinZeroTokens = kTileWaves;
inline int fin_zero_workgroups(int T) { return (T + kFinZeroTokens - 1) / kFinZeroTokens; }

// small-batch path
constexpr int kDecMaxItems = 256;         // (route, slice) items per token
constexpr int kDecDownSliceBlocks = 2;    // 128-blocks of the reduction per item
// small-batch gate/up kernel (pre-activations h in FP32)
constexpr int kSmallMaxRoutes = 128;      // T*K: the row search is two ballots of one wave
constexpr int kSmallWaves = 8;            // reduction slices
constexpr int kSmallThreads = kSmallWaves * 64;
constexpr int kSmallRows = 4;             // token rows per pass (MFMA rows 0, 4, 8, 12)
constexpr int kSmallMaxSlice = 1024;      // reduction per slice: hidden <= 8 * 1024
constexpr int kSmallRouteNpl = 8;         // routed: logits per lane (E_global <= 512)
constexpr int kSmallRouteMaxRoutes = 16;  // routed inside the launch up to this T*K
// ... and at most this many gate/up workgroups: each of them routes the
// tokens itself (the same bits in every one), which beyond about two
// workgroups per CU costs more than the router launch it saves (the 32-of-256
// share at 1 token, 2048 workgroups: 23 -> 41 us)
constexpr int kSmallRouteMaxWorkgroups = 512;
inline size_t small_h_lds_bytes(int kslice) {
  return sizeof(uint16_t) * static_cast<size_t>(kSmallWaves) * (kSmallRows * (kslice + 8) + 16 * 32);
}

// Router arguments (router.h) of a forward that routes the tokens itself:
// logits [T][Eg] fp32 in, ids/wts [T][K] out; logits == nullptr: ids given.
struct RouteArgs {
  const float* logits;
  int T, Eg, renorm;
  int32_t* ids;
  float* wts;
};

struct SmallHParams {
  const uint16_t* x;          // [T][lda]
  int lda;
  int T;                      // tokens (rows of x)
  const int32_t* ids;         // [R] global ids (unless routed: ra.logits set)
  RouteArgs ra;               // routed: ids and weights come from the logits
  int R, top_k, E, off;
  int slots;                  // grid rows: workgroup row y takes distinct local
                              // experts y, y + slots, ... (1 <= slots <= R)
  const uint8_t* wq;          // w13 packed, expert 0
  const uint16_t* ws;         // w13 scales, expert 0
  int64_t wq_expert_bytes;
  int64_t ws_expert_elems;
  int K;                      // reduction length (H)
  int kslice;                 // per-wave slice of K, multiple of 128
  float* h;                   // [R][ldh] pre-activations (route-indexed)
  int ldh;                    // N1
};

struct DecodeDownParams {
  const float* h;             // [R][ldh] FP32 pre-activations, route-indexed
  int ldh;                    // N1
  const uint8_t* wq;
  const uint16_t* ws;
  int64_t wq_expert_bytes;
  int64_t ws_expert_elems;
  const int32_t* ids;         // [T][K]
  const float* wts;           // [T][K]
  int top_k, E, off;
  int I, H;
  uint16_t* out;              // [T][H]
  int prefetch;               // 1: the variant that loads a wave's next item while
                              // it computes one (more items than waves expected)
};

constexpr int kDecThreadsAll = 512;       // threads of the small-batch down kernel
constexpr int kDecWavesAll = kDecThreadsAll / 64;
constexpr int kDecActLoads = 8;           // activation chunks per thread: top_k * I <= 8 * 512 * 8
inline size_t decode_down_lds_bytes(int top_k, int I) {
  // the activations [top_k][I + 8] 16-bit, then FP32 partials [items][32]
  const int nsl = ((I + 127) / 128 + kDecDownSliceBlocks - 1) / kDecDownSliceBlocks;
  return sizeof(uint16_t) * static_cast<size_t>(top_k) * (I + 8) +
         sizeof(float) * 32 * static_cast<size_t>(top_k) * nsl;
}

struct CombineParams {
  const uint16_t* y;          // [T*K][H] expert outputs by route
  const int32_t* slot;        // [T*K]
  const float* wts;           // [T][K]
  int top_k, H;
  uint16_t* out;              // [T][H]
};

// Route preparation (one launch up to 2048 routes, else two).  chunk_hist:
// kRouteChunksMax * E ints of scratch, or null for a single-chunk (slower for
// many routes) preparation.
// With `route` (router logits instead of ids; see router.h) route->ids and
// route->wts are written first: up to 16 tokens inside the one-workgroup
// preparation launch (one token per wave), else by the router kernel before
// the preparation.  top_k: routes per token.
constexpr int kRouteChunksMax = 32;
int route_prep_chunk(int R);
// zero: n_zero int32 that the preparation sets to 0 (the fused combine's
// arrival counters), or null.
hipError_t launch_route_prep(const int32_t* ids, int R, int E, int off, int bm, int32_t* counts,
                             int32_t* offsets, int32_t* sorted, int32_t* slot,
                             int32_t* tile_expert, int32_t* chunk_hist, hipStream_t stream,
                             int top_k = 1, const RouteArgs* route = nullptr,
                             int32_t* zero = nullptr, int64_t n_zero = 0,
                             int32_t* tile_order = nullptr);

// 64-row expert tiles (route positions), LDS-staged activations
constexpr int kResidentK = 256;      // reduction the resident down kernel holds in LDS
// tile launches take tiles biggest first between these expected valid routes
// per touched expert (tiles of mixed sizes; far above, most tiles are full)
constexpr double kTileSortMinRoutes = 9.0;
constexpr double kTileSortMaxRoutes = 80.0;
constexpr int kSplitkNsub = 2;       // 16-row weight subtiles per wave in the split-K kernel
constexpr int kSplitkPassRows = kTileWaves * 16 * kSplitkNsub;  // weight rows per column pass
constexpr int kSplitkMaxLds = 78 * 1024;   // two workgroups per CU
hipError_t launch_up_splitk(const GemmParams& p, int dtype, int layout, int max_tiles,
                            hipStream_t stream);
// act rows from split-K partials (GemmParams: part, S, R, n_cols = N1, ldo = I,
// slot, out = act)
hipError_t launch_splitk_act(const GemmParams& p, int dtype, bool gated, hipStream_t stream);
hipError_t launch_down_resident(const GemmParams& p, int dtype, int layout, int max_tiles,
                                hipStream_t stream);
hipError_t launch_tile_gemm(const GemmParams& p, int dtype, int layout, int mode, int max_tiles,
                            hipStream_t stream);
// workgroups of the kernel that reruns flagged tiles of a fp16-route launch
// (one per XCD)
constexpr int kTileRedoWorkgroups = 8;
// workgroups of a streaming tile launch (the size of its flag array)
inline int64_t tile_launch_workgroups(int n_tiles, int64_t max_tiles) {
  return 8 * static_cast<int64_t>(n_tiles) * ((max_tiles + 7) / 8);
}

hipError_t launch_small_h(const SmallHParams& p, int dtype, int layout, int nkb, int n1,
                          hipStream_t stream);

hipError_t launch_decode_down(const DecodeDownParams& p, int dtype, int layout, bool gated, int T,
                              hipStream_t stream);

hipError_t launch_combine(const CombineParams& p, int dtype, int T, hipStream_t stream);

hipError_t launch_unpack(const uint8_t* packed, int64_t n_bytes, int8_t* out, hipStream_t stream);
hipError_t launch_decode_fp4(const uint8_t* packed, int64_t n_bytes, int dtype, float* out,
                             hipStream_t stream);
hipError_t launch_e8m0_to_h16(const uint8_t* e8m0, int64_t n, int dtype, uint16_t* out,
                              hipStream_t stream);
hipError_t launch_repack_per_channel(const uint8_t* in, const uint16_t* sc_in, int64_t n_experts,
                                     int n_out, int k_in, uint8_t* out, uint16_t* sc_out,
                                     hipStream_t stream);

// Streaming-read probe over [bytes / row_bytes][row_bytes] (row_bytes a
// multiple of 64, at most 8 * 16 * 64).
constexpr int kProbeMaxRowBytes = 8 * 16 * 64;
hipError_t launch_stream_probe(const uint8_t* buf, int64_t bytes, int row_bytes, uint32_t* sink,
                               hipStream_t stream);

// Router scoring and top-k (softmax over E_global logits, K largest).
constexpr int kRouterMaxExperts = 1024;
constexpr int kRouterMaxTopK = 32;
hipError_t launch_router_topk(const float* logits, int T, int Eg, int K, int renorm, int32_t* ids,
                              float* wts, hipStream_t stream);

}  // namespace w4moe
