// route_prep.hip -- route preparation for the local W4A16 MoE forward.
//
// Sources: [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE
// backend" (Benchmark: route preparation is part of the timed MoE;
// Modification: local experts, invalid routes, masked expert counts);
// [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
// overhead" (Description: route guards, padded fallback).
//
// One workgroup of 1024 threads (16 waves) builds, from topk_ids [R = T*K]:
//   counts[e]       valid routes of local expert e
//   offsets[e]      exclusive prefix of counts rounded up to block_m
//   sorted[p]       route index r = t*K + k at padded position p, ascending
//                   within an expert; -1 in padding
//   slot[r]         p of route r, or -1 for an invalid route
//   tile_expert[i]  expert of tile i (positions [i*block_m, (i+1)*block_m));
//                   skipped when the pointer is null
// and zeroes the split-K arrival counters of the gate/up kernel.
//
// Stable counting sort without atomics: wave w owns the contiguous slab
// [w*S, (w+1)*S) of routes and walks it 64 routes at a time.  Lanes holding
// the same expert are found with one ballot per expert-id bit; a lane's rank
// is the number of matching lanes below it, and the lowest matching lane
// bumps the wave's LDS histogram.  A block-wide pass turns the 16 histograms
// into per-wave bases and padded offsets, and a second walk over the slabs
// scatters every route to offsets[e] + base[w][e] + rank.  Ascending order
// within an expert follows from slabs, chunks and lanes all being in order.
#include "device.h"
#include "internal.h"

namespace w4moe {

constexpr int kRpThreads = 1024;
constexpr int kRpWaves = kRpThreads / 64;
constexpr int kRpMaxExperts = 1024;
constexpr int kRpRound = 16;  // 64-route chunks whose id loads are in flight together

__device__ __forceinline__ int local_expert(int32_t g, int E, int off) {
  const int64_t e = static_cast<int64_t>(g) - off;
  return (e >= 0 && e < E) ? static_cast<int>(e) : -1;
}

__global__ void __launch_bounds__(kRpThreads)
route_prep_kernel(const int32_t* __restrict__ ids, int R, int E, int off, int bm,
                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                  int32_t* __restrict__ sorted, int32_t* __restrict__ slot,
                  int32_t* __restrict__ tile_expert, int32_t* __restrict__ zero_buf,
                  int zero_n) {
  __shared__ int32_t hist[kRpWaves][kRpMaxExperts];
  __shared__ int32_t wave_tot[kRpWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int i = tid; i < zero_n; i += kRpThreads) zero_buf[i] = 0;
  for (int e = lane; e < E; e += 64) hist[w][e] = 0;
  __syncthreads();

  const int slab = ((R + kRpWaves - 1) / kRpWaves + 63) & ~63;
  const int r_beg = w * slab;
  const int r_end = min(R, r_beg + slab);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;

  // pass 1: per-wave histogram and rank of each route within its wave's slab.
  // The slab is walked in rounds of kRpRound chunks of 64 routes; every id
  // load of a round is issued before the first is used.
  for (int rb = r_beg; rb < r_end; rb += 64 * kRpRound) {
    int ev[kRpRound];
#pragma unroll
    for (int q = 0; q < kRpRound; ++q) {
      const int r = rb + 64 * q + lane;
      ev[q] = (r < r_end) ? local_expert(ids[r], E, off) : -1;
    }
#pragma unroll
    for (int q = 0; q < kRpRound; ++q) {
      if (rb + 64 * q >= r_end) break;
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
        slot[r] = before + rank;  // temporary: rank within the slab
      } else if (r < r_end) {
        slot[r] = -1;
      }
    }
  }
  __syncthreads();

  // per expert: exclusive prefix over waves, counts, padded sizes
  // (one thread per expert; E <= 1024)
  int padded = 0, my_count = 0;
  if (tid < E) {
    int run = 0;
    for (int v = 0; v < kRpWaves; ++v) {
      const int c = hist[v][tid];
      hist[v][tid] = run;
      run += c;
    }
    counts[tid] = run;
    my_count = run;
    padded = (run + bm - 1) / bm * bm;
  }
  // block-wide exclusive scan of padded sizes over experts
  int incl = padded;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  if (w == 0) {
    int t = (lane < kRpWaves) ? wave_tot[lane] : 0;
    for (int d = 1; d < kRpWaves; d <<= 1) {
      const int v = __shfl_up(t, d, 64);
      if (lane >= d) t += v;
    }
    if (lane < kRpWaves) wave_tot[lane] = t;  // inclusive totals per wave
  }
  __syncthreads();
  const int excl = incl - padded + (w > 0 ? wave_tot[w - 1] : 0);
  __shared__ int32_t s_off[kRpMaxExperts + 1];
  if (tid < E) {
    offsets[tid] = excl;
    s_off[tid] = excl;
  }
  if (tid == 0) {
    offsets[E] = wave_tot[kRpWaves - 1];
    s_off[E] = wave_tot[kRpWaves - 1];
  }
  __syncthreads();

  // pass 2: scatter (each thread revisits exactly the routes it ranked)
  for (int rb = r_beg; rb < r_end; rb += 64 * kRpRound) {
    int ev[kRpRound], rk[kRpRound];
#pragma unroll
    for (int q = 0; q < kRpRound; ++q) {
      const int r = rb + 64 * q + lane;
      ev[q] = (r < r_end) ? local_expert(ids[r], E, off) : -1;
      rk[q] = (ev[q] >= 0) ? slot[r] : 0;
    }
#pragma unroll
    for (int q = 0; q < kRpRound; ++q) {
      const int r = rb + 64 * q + lane;
      if (ev[q] >= 0) {
        const int pos = s_off[ev[q]] + hist[w][ev[q]] + rk[q];
        sorted[pos] = r;
        slot[r] = pos;
      }
    }
  }
  // padding positions and the tile -> expert map (thread e owns expert e)
  if (tid < E) {
    const int beg = s_off[tid], end = s_off[tid + 1];
    for (int p = beg + my_count; p < end; ++p) sorted[p] = -1;
    if (tile_expert != nullptr)
      for (int i = beg / bm; i < end / bm; ++i) tile_expert[i] = tid;
  }
}

hipError_t launch_route_prep(const int32_t* ids, int R, int E, int off, int bm, int32_t* counts,
                             int32_t* offsets, int32_t* sorted, int32_t* slot,
                             int32_t* tile_expert, int32_t* zero_buf, int zero_n,
                             hipStream_t stream) {
  hipLaunchKernelGGL(route_prep_kernel, dim3(1), dim3(kRpThreads), 0, stream, ids, R, E, off, bm,
                     counts, offsets, sorted, slot, tile_expert, zero_buf, zero_n);
  return hipGetLastError();
}

}  // namespace w4moe
