// route_prep.hip -- route preparation for the local W4A16 MoE forward.
//
// Sources: [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE
// backend" (Benchmark: route preparation is part of the timed MoE;
// Modification: local experts, invalid routes, masked expert counts);
// [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
// overhead" (Description: route guards, padded fallback).
//
// From topk_ids [R = T*K] it builds
//   counts[e]       valid routes of local expert e
//   offsets[e]      exclusive prefix of counts rounded up to block_m
//   sorted[p]       route index r = t*K + k at padded position p, ascending
//                   within an expert; -1 in padding
//   slot[r]         p of route r, or -1 for an invalid route
//   tile_expert[i]  expert of tile i (positions [i*block_m, (i+1)*block_m));
//                   skipped when the pointer is null
//   tile_order[k]   optional: the used tiles by descending count of non-empty
//                   block_m/4-row subtiles, ties in tile order
//
// A stable counting sort without atomics.  Up to kRpOneRoutes routes: one
// workgroup (rp_one_kernel), which sorts the routes in LDS and writes the
// padded list in order.  Otherwise two launches:
//   1. rp_rank_kernel: workgroup c takes the contiguous chunk c of routes;
//      each of its waves walks a slab of the chunk 64 routes at a time.
//      Lanes holding the same expert are found with one ballot per expert-id
//      bit; a lane's rank is the number of matching lanes below it.  A
//      wave's LDS histogram gives ranks across its chunks; a prefix over the
//      waves gives each route's rank within the chunk (written to slot[r])
//      and the chunk's per-expert counts (chunk_hist[c][e]).
//   2. rp_scatter_kernel: each workgroup redoes the per-expert scan (chunk
//      bases, totals, padded sizes, offsets), scatters its chunk,
//      p = offsets[e] + base[c][e] + rank, and writes the padding and the
//      tile -> expert map of its share of the experts; workgroup 0 writes
//      counts and offsets.
// Ascending order within an expert follows from chunks, slabs, 64-route
// pieces and lanes all being in route order.
#include <algorithm>
#include <cstdint>

#include "device.h"
#include "internal.h"
#include "router.h"

namespace w4moe {

namespace {

constexpr int kRpThreads = 256;            // ranking workgroup (4 waves)
constexpr int kRpWaves = kRpThreads / 64;
constexpr int kRpScanThreads = 1024;       // one thread per expert (E <= 1024)
constexpr int kRpMaxExperts = 1024;

__device__ __forceinline__ int local_expert(int32_t g, int E, int off) {
  const int64_t e = static_cast<int64_t>(g) - off;
  return (e >= 0 && e < E) ? static_cast<int>(e) : -1;
}

// The wave's index in the workgroup, as a value the compiler knows is the
// same in every lane (wave-strided loops then run on scalar counters).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Inclusive prefix sum over the 64 lanes of a wave.  Shift-and-add steps of
// 1, 2, 4 and 8 lanes inside each 16-lane row through DPP row shifts (a lane
// shifted in from outside its row reads 0); then the totals of rows 0 and 2
// are added to rows 1 and 3 (broadcast of lanes 15 and 47), and the total of
// rows 0-1 to rows 2-3 (broadcast of lane 31).  No LDS round trip, unlike a
// shuffle.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Padding positions (-1) and the tile -> expert map of experts [eb, ee).
// Wave w takes experts eb + [w * per, (w + 1) * per) (per <= 64: E <= 64 *
// waves); lane j reads the
// bounds of the wave's j-th expert, then the wave walks its experts with
// those values broadcast from lane j, each store instruction writing
// consecutive positions of one expert (a thread per expert would scatter
// every store over 64 experts' ranges).
__device__ __forceinline__ void fill_padding_and_tiles(int eb, int ee, int bm,
                                                       const int32_t* s_off, const int32_t* s_cnt,
                                                       int32_t* sorted, int32_t* tile_expert,
                                                       int waves) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int per = (ee - eb + waves - 1) / waves;
  const int e0 = eb + w * per;
  const int me = e0 + lane;
  int pad_v = 0, end_v = 0, t0_v = 0, t1_v = 0;
  if (lane < per && me < ee) {
    const int beg = s_off[me];
    end_v = s_off[me + 1];
    pad_v = beg + s_cnt[me];
    t0_v = beg / bm;
    t1_v = end_v / bm;
  }
  const int n = min(per, ee - e0);
  for (int j = 0; j < n; ++j) {
    const int pad = __builtin_amdgcn_readlane(pad_v, j), end = __builtin_amdgcn_readlane(end_v, j);
    for (int p = pad + lane; p < end; p += 64) sorted[p] = -1;
    if (tile_expert != nullptr) {
      const int t1 = __builtin_amdgcn_readlane(t1_v, j);
      for (int i = __builtin_amdgcn_readlane(t0_v, j) + lane; i < t1; i += 64) tile_expert[i] = e0 + j;
    }
  }
}

// tile_order (optional): the used 64-row tiles by descending count of
// non-empty 16-row subtiles (4, 3, 2, 1), ties in tile order: a stable
// counting sort over four buckets.  An expert of n routes has n / 64 full
// tiles and, if n % 64 > 0, a last tile of ceil((n % 64) / 16) subtiles; the
// four per-expert bucket counts are scanned over the experts (thread e:
// expert e, E <= 1024), and each workgroup writes the entries of the tiles of
// experts [eb, ee).  All threads of the workgroup call it (it has barriers).
// The tile kernels take tiles in this order, so the last workgroups to start
// on a CU are the shortest.
__device__ __forceinline__ void write_tile_order(int E, int bm, const int32_t* s_off,
                                                 const int32_t* s_cnt, int eb, int ee,
                                                 int32_t* tile_order, int32_t (*s_tot)[16]) {
  constexpr int kW = kRpScanThreads / 64;
  static_assert(kW <= 16, "wave totals");
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int sub = bm / 4;  // rows per subtile (16 for 64-row tiles)
  int n[4] = {0, 0, 0, 0};
  int full = 0, part_b = -1;
  if (tid < E) {
    const int cnt = s_cnt[tid];
    full = cnt / bm;
    const int rem = cnt - full * bm;
    n[0] = full;
    if (rem > 0) {
      part_b = 4 - (rem + sub - 1) / sub;
      n[part_b] += 1;
    }
  }
  int incl[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    incl[b] = wave_incl_scan(n[b]);
    if (lane == 63) s_tot[b][w] = incl[b];  // per-wave totals
  }
  __syncthreads();
  if (tid >= eb && tid < ee) {
    int start[4], ex[4];  // first entry of each bucket; its tiles before expert tid
    int run = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      start[b] = run;
      ex[b] = incl[b] - n[b];
#pragma unroll
      for (int v = 0; v < kW; ++v) {
        const int t = s_tot[b][v];
        run += t;
        if (v < w) ex[b] += t;
      }
    }
    const int t0 = s_off[tid] / bm;
    for (int j = 0; j < full; ++j) tile_order[start[0] + ex[0] + j] = t0 + j;
    if (part_b >= 0) {
      const int pb = part_b == 0 ? full : 0;  // after the expert's full tiles in bucket 0
      int sb = 0, eb2 = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b == part_b) sb = start[b], eb2 = ex[b];
      tile_order[sb + eb2 + pb] = t0 + full;
    }
  }
}

}  // namespace

// Up to kRpOneRoutes routes: the whole preparation in one workgroup.  Wave w
// takes the contiguous slab of np 64-route pieces starting at piece w * np
// (NP >= np, a compile-time bound) and ranks its pieces in order, its LDS
// histogram carrying the counts of its earlier pieces; the scan over the
// waves' histograms gives each wave's base within an expert.  The routes are
// then gathered into an LDS list by expert and rank, each tile records its
// first list entry and valid rows, and the padded list is written tile by
// tile in one pass: consecutive lanes, every position once, no per-expert
// loop (which a wave walks serially, instruction by instruction).
// (Measured: up to 2048 routes, one workgroup beats the two launches by 0-2
// us; at 4 pieces per wave, 3072 and 4096 routes on the 384-expert shard, it
// is 1-4 us slower.)
constexpr int kRpOneMaxPieces = 2;
constexpr int kRpOneRoutes = kRpOneMaxPieces * kRpScanThreads;

// NPL > 0: the ids come from routing the tokens' logits first (router.h, NPL
// logits per lane); wave w routes token w (at most 16 tokens), keeps the ids
// in LDS and writes ids and weights out.
template <int NP, int NPL>
__global__ void __launch_bounds__(kRpScanThreads)
rp_one_kernel(const int32_t* __restrict__ ids, int R, int E, int off, int bm, int cap,
              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
              int32_t* __restrict__ sorted, int32_t* __restrict__ slot,
              int32_t* __restrict__ tile_expert, int top_k, RouteArgs ra,
              int32_t* __restrict__ zero, int64_t n_zero, int32_t* __restrict__ tile_order) {
  constexpr int kW = kRpScanThreads / 64;
  static_assert(kW <= 16, "wave totals");
  for (int64_t i = threadIdx.x; i < n_zero; i += kRpScanThreads) zero[i] = 0;
  __shared__ int32_t hist[kW][kRpMaxExperts];
  __shared__ int32_t wave_tot[2][kW];
  __shared__ int32_t s_off[kRpMaxExperts + 1];
  __shared__ int32_t s_cnt[kRpMaxExperts];
  __shared__ int32_t s_pre[kRpMaxExperts];
  __shared__ int32_t s_ids[NPL > 0 ? NP * kRpScanThreads : 1];
  // route list: the route of rank k of expert e at s_pre[e] + k (one spare
  // entry: a tile's rows past its valid ones read at most one past the end)
  __shared__ int32_t s_route[NP * kRpScanThreads + 1];
  // per tile: first list entry, valid rows (an expert of n > 0 routes has
  // ceil(n / block_m) <= n tiles)
  constexpr int kTiles = NP * kRpScanThreads;
  __shared__ int2 s_tile[kTiles];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  if constexpr (NPL > 0) {
    route_tokens<NPL>(ra, top_k, w, ra.T, kW, lane, [&](int t, int id, float pw) {
      if (lane < top_k) {
        const int r = t * top_k + lane;
        s_ids[r] = id;
        ra.ids[r] = id;
        ra.wts[r] = pw;
      }
    });
    __syncthreads();
  }
  const int np = ((R + 63) / 64 + kW - 1) / kW;  // pieces per wave
  const int r0 = 64 * np * w + lane;              // route of piece 0 of this lane
  int ev[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int r = r0 + 64 * q;
    ev[q] = (q < np && r < R) ? local_expert(NPL > 0 ? s_ids[r] : ids[r], E, off) : -1;
  }
  for (int x = lane; x < E; x += 64) hist[w][x] = 0;  // read back by this wave only
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // rank within the wave's slab: lanes of a piece holding the same expert are
  // found with one ballot per expert-id bit
  int rk[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    rk[q] = 0;
    if (q < np) {
      const int e = ev[q];
      uint64_t match = __ballot(e >= 0);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        match &= bit ? m : ~m;
      }
      if (e >= 0) {
        const int rank = __popcll(match & below);
        const int before = hist[w][e];
        if (rank == 0) hist[w][e] = before + __popcll(match);
        rk[q] = before + rank;
      }
    }
  }
  __syncthreads();
  // per expert: wave bases (in place, all loads in flight first), totals,
  // padded sizes
  int padded = 0, total = 0;
  if (tid < E) {
    int n[kW];
#pragma unroll
    for (int v = 0; v < kW; ++v) n[v] = hist[v][tid];
#pragma unroll
    for (int v = 0; v < kW; ++v) {
      hist[v][tid] = total;
      total += n[v];
    }
    counts[tid] = total;
    padded = (total + bm - 1) / bm * bm;
  }
  // prefixes over the experts of the padded sizes (first positions) and of
  // the totals (first entries of the route list below)
  const int incl_p = wave_incl_scan(padded);
  const int incl_c = wave_incl_scan(total);
  if (lane == 63) {
    wave_tot[0][w] = incl_p;
    wave_tot[1][w] = incl_c;
  }
  __syncthreads();
  int P = 0, excl = incl_p - padded, pre = incl_c - total;
#pragma unroll
  for (int v = 0; v < kW; ++v) {
    const int tp = wave_tot[0][v], tc = wave_tot[1][v];
    P += tp;
    if (v < w) excl += tp, pre += tc;
  }
  const int n_tiles = min(P / bm, min(cap / bm, kTiles));
  if (tid < E) {
    offsets[tid] = excl;
    s_off[tid] = excl;
    s_cnt[tid] = total;
    s_pre[tid] = pre;
    // each tile of the expert: its first route-list entry and valid rows
    const int t0 = excl / bm;
    for (int j = 0, k = 0; k < total && t0 + j < n_tiles; ++j, k += bm) {
      s_tile[t0 + j] = make_int2(pre + k, min(bm, total - k));
      if (tile_expert != nullptr) tile_expert[t0 + j] = tid;
    }
  }
  if (tid == 0) {
    offsets[E] = P;
    s_off[E] = P;
  }
  __syncthreads();
  // the route list: routes by expert, then rank (route order)
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int r = r0 + 64 * q;
    if (q < np && r < R) {
      const int e = ev[q];
      if (e >= 0) {
        const int k = hist[w][e] + rk[q];
        slot[r] = s_off[e] + k;
        s_route[s_pre[e] + k] = r;
      } else {
        slot[r] = -1;
      }
    }
  }
  __syncthreads();
  // the padded list, tile by tile (a wave per tile, lane j: row j): the
  // route-list entry of a valid row, -1 in padding; every position written
  // once, by consecutive lanes.  With 64-row tiles, four tiles per pass keep
  // their LDS reads in flight together.
  if (bm == 64) {
    constexpr int U = 4;
    for (int i0 = w; i0 < n_tiles; i0 += U * kW) {
      int2 inf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) inf[u] = s_tile[min(i0 + u * kW, n_tiles - 1)];
      int rv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) rv[u] = s_route[inf[u].x + min(lane, inf[u].y)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kW;
        if (i < n_tiles) sorted[i * 64 + lane] = lane < inf[u].y ? rv[u] : -1;
      }
    }
  } else {
    for (int i = w; i < n_tiles; i += kW) {
      const int2 inf = s_tile[i];
      for (int j = lane; j < bm; j += 64) {
        const int rv = s_route[inf.x + min(j, inf.y)];
        sorted[i * bm + j] = j < inf.y ? rv : -1;
      }
    }
  }
  if (tile_order != nullptr) {
    __shared__ int32_t s_tot[4][16];
    write_tile_order(E, bm, s_off, s_cnt, 0, E, tile_order, s_tot);
  }
}

__global__ void __launch_bounds__(kRpThreads)
rp_rank_kernel(const int32_t* __restrict__ ids, int R, int E, int off, int chunk,
               int32_t* __restrict__ slot, int32_t* __restrict__ chunk_hist,
               int32_t* __restrict__ zero, int64_t n_zero) {
  constexpr int NW = kRpWaves;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kRpThreads + threadIdx.x; i < n_zero;
       i += static_cast<int64_t>(gridDim.x) * kRpThreads)
    zero[i] = 0;
  __shared__ int32_t hist[NW][kRpMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int c = blockIdx.x;
  for (int e = lane; e < E; e += 64) hist[w][e] = 0;  // read back by this wave only

  const int c_beg = c * chunk;
  const int c_end = min(R, c_beg + chunk);
  const int slab = ((chunk + NW - 1) / NW + 63) & ~63;
  const int r_beg = c_beg + w * slab;
  const int r_end = min(c_end, r_beg + slab);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;

  // rank of each route within this wave's slab (ids of kRound pieces in
  // flight).  A slab of one round keeps ids and ranks in registers for the
  // pass after the scan; a longer one parks the ranks in slot[].
  constexpr int kRound = 4;
  const bool one_round = slab <= 64 * kRound;
  int ek[kRound], rk[kRound];
#pragma unroll
  for (int q = 0; q < kRound; ++q) ek[q] = -1, rk[q] = 0;
  for (int rb = r_beg; rb < r_end; rb += 64 * kRound) {
    int ev[kRound];
#pragma unroll
    for (int q = 0; q < kRound; ++q) {
      const int r = rb + 64 * q + lane;
      ev[q] = (r < r_end) ? local_expert(ids[r], E, off) : -1;
    }
#pragma unroll
    for (int q = 0; q < kRound; ++q) {
      ek[q] = ev[q];
      rk[q] = 0;
      if (rb + 64 * q >= r_end) continue;
      const int r = rb + 64 * q + lane;
      const int e = ev[q];
      uint64_t match = __ballot(e >= 0);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        match &= bit ? m : ~m;
      }
      if (e >= 0) {
        const int rank = __popcll(match & below);
        const int before = hist[w][e];
        if (rank == 0) hist[w][e] = before + __popcll(match);
        rk[q] = before + rank;
        if (!one_round) slot[r] = before + rank;  // rank within the wave's slab
      } else if (!one_round && r < r_end) {
        slot[r] = -1;
      }
    }
  }
  __syncthreads();
  // per expert: wave bases within the chunk (in place) and the chunk total
  for (int e = tid; e < E; e += (NW * 64)) {
    int run = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int n = hist[v][e];
      hist[v][e] = run;
      run += n;
    }
    chunk_hist[static_cast<int64_t>(c) * E + e] = run;
  }
  __syncthreads();
  // rank within the chunk
  if (one_round) {
#pragma unroll
    for (int q = 0; q < kRound; ++q) {
      const int r = r_beg + 64 * q + lane;
      if (r < r_end) slot[r] = ek[q] >= 0 ? rk[q] + hist[w][ek[q]] : -1;
    }
  } else {
    for (int rb = r_beg; rb < r_end; rb += 64) {
      const int r = rb + lane;
      if (r < r_end) {
        const int e = local_expert(ids[r], E, off);
        if (e >= 0) slot[r] += hist[w][e];
      }
    }
  }
}

// Every workgroup redoes the (small) per-expert scan, so that no separate
// launch is needed: chunk counts of each expert (all loads in flight), the
// totals, their padded sizes, the scan over experts; then workgroup c
// scatters chunk c and writes the padding and tile map of its share of the
// experts, and workgroup 0 writes counts and offsets.  chunk_hist may alias
// counts (one chunk: the only workgroup reads a count before writing it, in
// the same thread).
__global__ void __launch_bounds__(kRpScanThreads)
rp_scatter_kernel(const int32_t* __restrict__ ids, int R, int E, int off, int bm, int chunk,
                  int n_chunks, const int32_t* chunk_hist, int32_t* counts,
                  int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                  int32_t* __restrict__ slot, int32_t* __restrict__ tile_expert,
                  int32_t* __restrict__ tile_order) {
  constexpr int kW = kRpScanThreads / 64;
  __shared__ int32_t wave_tot[kW];
  __shared__ int32_t s_off[kRpMaxExperts + 1];
  __shared__ int32_t s_cnt[kRpMaxExperts];
  __shared__ int32_t s_base[kRpMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int c = blockIdx.x;
  const int c_end = min(R, (c + 1) * chunk);
  // a chunk of at most one route per thread: the route's expert and rank
  // are requested with the chunk counts
  const bool one_pass = chunk <= kRpScanThreads;
  const int r1 = c * chunk + tid;
  int e1 = -1, k1 = 0;
  if (one_pass && r1 < c_end) {
    e1 = local_expert(ids[r1], E, off);
    k1 = slot[r1];
  }
  int padded = 0, total = 0, base = 0;
  if (tid < E) {
    int n[kRouteChunksMax];
#pragma unroll
    for (int q = 0; q < kRouteChunksMax; ++q)
      n[q] = q < n_chunks ? chunk_hist[static_cast<int64_t>(q) * E + tid] : 0;
#pragma unroll
    for (int q = 0; q < kRouteChunksMax; ++q) {
      if (q == c) base = total;
      total += n[q];
    }
    padded = (total + bm - 1) / bm * bm;
  }
  const int incl = wave_incl_scan(padded);
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  int P = 0, excl = incl - padded;
#pragma unroll
  for (int v = 0; v < kW; ++v) {
    const int t = wave_tot[v];
    P += t;
    if (v < w) excl += t;
  }
  if (tid < E) {
    s_off[tid] = excl;
    s_cnt[tid] = total;
    s_base[tid] = base;
  }
  if (tid == 0) s_off[E] = P;
  __syncthreads();
  if (one_pass) {
    if (e1 >= 0) {  // slot[r1] is already -1 for an invalid route
      const int pos = s_off[e1] + s_base[e1] + k1;
      sorted[pos] = r1;
      slot[r1] = pos;
    }
  } else {
    for (int r = c * chunk + tid; r < c_end; r += kRpScanThreads) {
      const int e = local_expert(ids[r], E, off);
      if (e < 0) continue;
      const int pos = s_off[e] + s_base[e] + slot[r];
      sorted[pos] = r;
      slot[r] = pos;
    }
  }
  if (c == 0) {
    if (tid < E) {
      counts[tid] = s_cnt[tid];
      offsets[tid] = s_off[tid];
    }
    if (tid == 0) offsets[E] = s_off[E];
  }
  const int per_wg = (E + n_chunks - 1) / n_chunks;
  const int eb = min(E, c * per_wg);
  fill_padding_and_tiles(eb, min(E, eb + per_wg), bm, s_off, s_cnt, sorted, tile_expert, kW);
  if (tile_order != nullptr) {
    __shared__ int32_t s_tot[4][16];
    write_tile_order(E, bm, s_off, s_cnt, eb, min(E, eb + per_wg), tile_order, s_tot);
  }
}

int route_prep_chunk(int R) {
  // at most kRouteChunksMax chunks, at least 256 routes per chunk
  const int per = (R + kRouteChunksMax - 1) / kRouteChunksMax;
  return std::max(256, (per + 63) & ~63);
}

// Up to this many tokens the one-workgroup preparation routes its tokens
// itself (one token per wave); a wave routes a token in about 1300 dependent
// VALU instructions, so more tokens per wave cost more than the router
// launch they save, and the router kernel (one wave per token over the
// whole GPU) runs first instead.
constexpr int kRpRouteMaxTokens = kRpScanThreads / 64;

hipError_t launch_route_prep(const int32_t* ids, int R, int E, int off, int bm, int32_t* counts,
                             int32_t* offsets, int32_t* sorted, int32_t* slot,
                             int32_t* tile_expert, int32_t* chunk_hist, hipStream_t stream,
                             int top_k, const RouteArgs* route, int32_t* zero, int64_t n_zero,
                             int32_t* tile_order) {
  if (E < 1 || E > kRpMaxExperts || R < 0 || bm < 1) return hipErrorInvalidValue;
  if (tile_order != nullptr && bm % 4 != 0) return hipErrorInvalidValue;
  // positions the padded list may take (its callers' capacity)
  const int64_t cap64 = R + std::min<int64_t>(E, R) * (bm - 1);
  if (cap64 > INT32_MAX) return hipErrorInvalidValue;
  const int cap = static_cast<int>(cap64);
  if (zero == nullptr) n_zero = 0;
  // without scratch: one chunk, whose counts live in `counts` itself (the
  // scan overwrites them with the totals) and whose base is 0
  const bool one = chunk_hist == nullptr;
  const int chunk = one ? std::max(R, 1) : route_prep_chunk(R);
  const int n_chunks = R > 0 ? (R + chunk - 1) / chunk : 0;
  int32_t* hist = one ? counts : chunk_hist;
  if (route != nullptr && R > 0) {
    const RouteArgs& ra = *route;
    if (ra.Eg < 1 || ra.Eg > kRouterMaxExperts || top_k < 1 || top_k > kRouterMaxTopK ||
        top_k > ra.Eg || static_cast<int64_t>(ra.T) * top_k != R)
      return hipErrorInvalidValue;
    if (R <= kRpScanThreads && ra.T <= kRpRouteMaxTokens) {
      auto k = rp_one_kernel<1, 16>;
      switch (router_npl(ra.Eg)) {
        case 1: k = rp_one_kernel<1, 1>; break;
        case 2: k = rp_one_kernel<1, 2>; break;
        case 4: k = rp_one_kernel<1, 4>; break;
        case 8: k = rp_one_kernel<1, 8>; break;
        default: break;
      }
      hipLaunchKernelGGL(k, dim3(1), dim3(kRpScanThreads), 0, stream, ids, R, E, off, bm, cap,
                         counts, offsets, sorted, slot, tile_expert, top_k, ra, zero, n_zero,
                         tile_order);
      return hipGetLastError();
    }
    const hipError_t err = launch_router_topk(ra.logits, ra.T, ra.Eg, top_k, ra.renorm, ra.ids,
                                              ra.wts, stream);
    if (err != hipSuccess) return err;
    ids = ra.ids;  // the preparation reads the ids the router wrote
  }
  if (R <= kRpOneRoutes) {
    static_assert(kRpOneMaxPieces == 1 || kRpOneMaxPieces == 2 || kRpOneMaxPieces == 4,
                  "pieces per wave");
    auto k = rp_one_kernel<1, 0>;
    if (R > 2 * kRpScanThreads) k = rp_one_kernel<(kRpOneMaxPieces > 2 ? 4 : 1), 0>;
    else if (R > kRpScanThreads) k = rp_one_kernel<(kRpOneMaxPieces > 1 ? 2 : 1), 0>;
    hipLaunchKernelGGL(k, dim3(1), dim3(kRpScanThreads), 0, stream, ids, R, E, off, bm, cap,
                       counts, offsets, sorted, slot, tile_expert, top_k, RouteArgs{}, zero,
                       n_zero, tile_order);
    return hipGetLastError();
  }
  // R > kRpOneRoutes here, so there is at least one chunk
  hipLaunchKernelGGL(rp_rank_kernel, dim3(n_chunks), dim3(kRpThreads), 0, stream, ids, R, E, off,
                     chunk, slot, hist, zero, n_zero);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(rp_scatter_kernel, dim3(n_chunks), dim3(kRpScanThreads), 0, stream, ids, R,
                     E, off, bm, chunk, n_chunks, hist, counts, offsets, sorted, slot,
                     tile_expert, tile_order);
  return hipGetLastError();
}

}  // namespace w4moe
