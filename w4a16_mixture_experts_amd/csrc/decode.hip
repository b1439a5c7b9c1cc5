// decode.hip -- the small-batch path of the local W4A16 MoE forward: two
// kernels, no route preparation pass.
//
// Sources (web pages, cited by tag and section):
//   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
//        Modification: small-batch split-K, register-side INT4 dequantization,
//        FP32 accumulation; invalid routes and masked expert counts.
//   [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
//        overhead"  Description, "Contract": FP32 combine in fixed top-k
//        order before one 16-bit cast, no atomics.
//
// small_h_kernel  grid (16-column weight subtiles) x (route slots), 8 waves:
//   the workgroup of the first route of each touched expert (two ballots
//   over the <= 128 ids) computes that expert's FP32 pre-activations for every route of
//   the expert, the reduction split over the 8 waves and summed in LDS in
//   slice order.
// decode_down_kernel  grid (32 output columns) x (tokens), 8 waves.  Work
//   items are (valid route k, 256-wide slice of the reduction); each wave computes
//   its items' 32 partial outputs in FP32 (one MFMA row: a route is a single
//   activation row) into LDS; then 32 lanes add, for k = 0..K-1 in order,
//   w[t,k] * (sum of k's slices in slice order) and cast once to 16 bits.
#include "device.h"
#include "internal.h"
#include "router.h"

namespace w4moe {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;

template <int LAYOUT>
struct BBlk {
  uint32_t d[is_group(LAYOUT) ? 4 : 8];
  uint32_t s[2];
};

template <int LAYOUT>
__device__ __forceinline__ void tr_b(BBlk<LAYOUT>& b) {
  if constexpr (is_group(LAYOUT)) {
    transpose_rows4(b.d[0], b.d[1], b.d[2], b.d[3]);
  } else {
    transpose_rows4(b.d[0], b.d[2], b.d[4], b.d[6]);
    transpose_rows4(b.d[1], b.d[3], b.d[5], b.d[7]);
  }
}

template <int DT, int LAYOUT>
__device__ __forceinline__ u32x4 b_op(const BBlk<LAYOUT>& b, int j, int par) {
  if constexpr (is_group(LAYOUT)) {
    return group_to_h16<DT, LAYOUT>(b.d[j]);
  } else {
    const int sh = 4 * par;
    return bytes_to_h16<DT>(b.d[2 * j] >> sh, b.d[2 * j + 1] >> sh);
  }
}

template <int DT>
__device__ __forceinline__ float sc_of(uint32_t pair, int j) {
  return H16<DT>::to_f32((j & 1) ? (pair >> 16) : (pair & 0xffffu));
}

__device__ __forceinline__ int local_id(int32_t g, int E, int off) {
  const int64_t e = static_cast<int64_t>(g) - off;
  return (e >= 0 && e < E) ? static_cast<int>(e) : -1;
}

}  // namespace

// ---------------------------------------------------------------------------
// small batch gate/up (T*K <= 128): pre-activations h = x W13^T in FP32 for one
// 16-row weight subtile of one touched expert; 8 waves split the reduction.
// ---------------------------------------------------------------------------
// The rows of the expert come from one ballot over the ids; the workgroup of
// the first route of an expert does the work, so each touched expert's
// weights are streamed once.  Gate and up subtiles are separate workgroups
// (the activation is applied by the down kernel), which gives 2*I/16
// workgroups per touched expert.
// Up to 4 rows per pass sit at MFMA rows 0, 4, 8, 12: result row 4q is
// element 0 of lane row q, so one FMA per MFMA applies the group scale.
// Memory order: one load of the ids; then, in flight together, every weight,
// group scale and x value of the wave's slice (raw buffer loads: masked
// lanes read zeros, so nothing waits on a load before its use).  Each wave
// stages only its own slice of x (no barrier), and one barrier precedes the
// fixed-order sum over slices.  Two dependent memory round trips in all.
// ROUTE: the ids come from routing the tokens' logits first (router.h): wave
// w routes tokens w, w + 8, ... into LDS (every workgroup the same way, so
// each sees the same ids), and workgroup (0, 0) writes the ids and weights
// out for the down kernel and the caller.  One barrier more; the logits load
// takes the place of the ids load.
template <int DT, int LAYOUT, int NKB, bool ROUTE>
__global__ void __launch_bounds__(kSmallThreads)
small_h_kernel(const SmallHParams p) {
  using T = H16<DT>;
  constexpr bool GROUP = is_group(LAYOUT);
  constexpr int CH = NKB * 16;  // 8-value chunks per staged x row of a slice
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4, par = c & 1;
  // column tiles are the fast grid dimension: consecutive workgroups stream
  // consecutive 16-row slabs of one expert
  const int nt = blockIdx.x;
  const int r0 = blockIdx.y;

  extern __shared__ uint16_t s_dyn[];  // per wave [kSmallRows][kslice + 8] x (A order), then
                                       // per wave [16][32] group scales
  __shared__ float s_red[kSmallWaves][64];
  __shared__ int32_t s_rid[ROUTE ? kSmallMaxRoutes : 1];

  // lane l holds the ids of routes l and l + 64 (R <= 128)
  int32_t my_id, my_id1 = -1;
  if constexpr (ROUTE) {
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
    route_tokens<kSmallRouteNpl>(p.ra, p.top_k, w, p.T, kSmallWaves, lane,
                                 [&](int t, int id, float pw) {
      if (lane < p.top_k) {
        const int r = t * p.top_k + lane;
        s_rid[r] = id;
        if (writer) {
          p.ra.ids[r] = id;
          p.ra.wts[r] = pw;
        }
      }
    });
    __syncthreads();
    my_id = lane < p.R ? s_rid[lane] : 0;
  } else {
    // rows: the routes whose id equals route r0's id (R <= 128: one load of
    // two ids per lane, two ballots)
    const auto rids = make_rsrc(p.ids, 4u * static_cast<uint32_t>(p.R));
    my_id = static_cast<int32_t>(bload4(rids, 4u * lane, lane < p.R));
    my_id1 = static_cast<int32_t>(bload4(rids, 4u * (lane + 64), lane + 64 < p.R));
  }
  // Grid rows.  One row per route slot (gridDim.y == R): row r works iff
  // route r is the first route of a local expert.  Fewer rows (most routes
  // expected not local): the owner slots, the first route of each distinct
  // local expert, are found with one ballot per distinct local id, and row y
  // takes the distinct experts y, y + rows, ...  (a serial chain of ballots:
  // with one row per slot it would only delay the weight loads).
  const bool direct = static_cast<int>(gridDim.y) == p.R;
  uint64_t own0 = 0, own1 = 0;
  int n_own = r0 + 1;  // direct: the loop below runs once, for slot r0
  if (!direct) {
    uint64_t rem0 = __ballot(lane < p.R && local_id(my_id, p.E, p.off) >= 0);
    uint64_t rem1 = __ballot(lane + 64 < p.R && local_id(my_id1, p.E, p.off) >= 0);
    while (rem0 != 0) {
      const int j = __builtin_ctzll(rem0);
      const int32_t v = __builtin_amdgcn_readlane(my_id, j);
      own0 |= 1ull << j;
      rem0 &= ~__ballot(my_id == v);
      rem1 &= ~__ballot(my_id1 == v);
    }
    while (rem1 != 0) {
      const int j = __builtin_ctzll(rem1);
      const int32_t v = __builtin_amdgcn_readlane(my_id1, j);
      own1 |= 1ull << j;
      rem1 &= ~__ballot(my_id1 == v);
    }
    n_own = __popcll(own0) + __popcll(own1);
  }
  const int my_tok = lane / p.top_k;          // token of route `lane`
  const int my_tok1 = (lane + 64) / p.top_k;  // token of route `lane + 64`

  for (int kx = r0; kx < n_own; kx += static_cast<int>(gridDim.y)) {
    int slot = r0;  // the route slot that owns this row's expert
    if (!direct) {  // the owner slot of distinct expert kx
      uint64_t m0 = own0, m1 = own1;
      const int c0 = __popcll(m0);
      if (kx < c0) {
        for (int i = 0; i < kx; ++i) m0 &= m0 - 1;
        slot = __builtin_ctzll(m0);
      } else {
        for (int i = 0; i < kx - c0; ++i) m1 &= m1 - 1;
        slot = 64 + __builtin_ctzll(m1);
      }
    }
    const int32_t gid = slot < 64 ? __builtin_amdgcn_readlane(my_id, slot)
                                  : __builtin_amdgcn_readlane(my_id1, slot - 64);
    const int e = local_id(gid, p.E, p.off);
    if (e < 0) return;  // direct: invalid route, nothing to do (uniform)
    const uint64_t match0 = __ballot(lane < p.R && my_id == gid);
    const uint64_t match1 = __ballot(lane + 64 < p.R && my_id1 == gid);
    // direct: an earlier slot owns this expert (uniform)
    if (slot != (match0 != 0 ? __builtin_ctzll(match0) : 64 + __builtin_ctzll(match1))) return;
    const int M = __popcll(match0) + __popcll(match1);

    const int wrow = nt * 16 + c;  // weight row (output column of h)
    const auto rw = make_rsrc(p.wq + static_cast<int64_t>(e) * p.wq_expert_bytes,
                              static_cast<uint32_t>(p.wq_expert_bytes));
    const auto rs = make_rsrc(p.ws + static_cast<int64_t>(e) * p.ws_expert_elems,
                              static_cast<uint32_t>(2 * p.ws_expert_elems));
    const auto rx = make_rsrc(p.x, 2u * static_cast<uint32_t>(p.T) * static_cast<uint32_t>(p.lda));
    const uint32_t boff = GROUP ? static_cast<uint32_t>(wrow) * (p.K >> 1)
                                : static_cast<uint32_t>(wrow >> 1) * p.K;
    const uint32_t soff = GROUP ? 2u * static_cast<uint32_t>(wrow) * (p.K >> 5) : 2u * wrow;
    const int xs = p.kslice + 8;  // staged x row stride (16 B padding)
    uint16_t* my_x = s_dyn + w * kSmallRows * xs;
    uint16_t* my_sc = s_dyn + kSmallWaves * kSmallRows * xs + w * 16 * 32;  // [16 rows][32 scales]
    const int kb = w * p.kslice;
    const int ke = min(p.K, kb + p.kslice);
    const int q_row = c >> 2;
    const u32x4 bconst = {T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2};
    const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};

    // one pass per 4 rows (more than 4 only if one expert takes more than 4 of
    // the routes; then the weights are streamed once per pass)
    uint64_t rest0 = match0, rest1 = match1;  // the expert's routes not yet taken
    for (int m0 = 0; m0 < M; m0 += kSmallRows) {
      const int nr = min(kSmallRows, M - m0);
      int rrow[kSmallRows], tok[kSmallRows];
  #pragma unroll
      for (int q = 0; q < kSmallRows; ++q) {
        rrow[q] = slot;
        tok[q] = 0;
        if (q < nr) {  // uniform
          if (rest0 != 0) {
            const int b = __builtin_ctzll(rest0);
            rest0 &= rest0 - 1;
            rrow[q] = b;
            tok[q] = __builtin_amdgcn_readlane(my_tok, b);
          } else {
            const int b = __builtin_ctzll(rest1);
            rest1 &= rest1 - 1;
            rrow[q] = 64 + b;
            tok[q] = __builtin_amdgcn_readlane(my_tok1, b);
          }
        }
      }
      // (1) this wave's slice of the staged rows (issued first: they are staged
      //     while the weights are still in flight): chunk idx -> row idx / CH
      u32x4 xv[NKB];
  #pragma unroll
      for (int i = 0; i < NKB; ++i) {
        const int idx = lane + 64 * i;
        const int q = idx / CH, ck = idx - q * CH;
        const int tq = q == 0 ? tok[0] : q == 1 ? tok[1] : q == 2 ? tok[2] : tok[3];
        const bool ok = q < nr && kb + 8 * ck < ke;
        xv[i] = bload16(rx, 2u * (static_cast<uint32_t>(tq) * p.lda + kb + 8 * ck), ok);
      }
      // (2) group scales of the slice (at most 64 bytes per row): one 16-byte
      //     load per lane covers the wave's 16 rows (lane l: row l / 4, part
      //     l % 4), staged in the wave's own LDS region
      u32x4 scv;
      uint32_t scol_bits = 0;
      if constexpr (GROUP) {
        const uint32_t so = 2u * (static_cast<uint32_t>(nt * 16 + (lane >> 2)) * (p.K >> 5) +
                                  (kb >> 5)) + 16u * (lane & 3);
        scv = bload16(rs, so, kb < p.K);
      } else {
        scol_bits = bload4(rs, soff & ~3u, true) >> (16 * (wrow & 1));
      }
      // (3) every weight of this wave's slice (kslice <= NKB * 128)
      u32x4 bw[NKB];
      u32x4 bw2[GROUP ? 1 : NKB];
  #pragma unroll
      for (int i = 0; i < NKB; ++i) {
        const int k0 = kb + 128 * i;
        const int ng = k0 < ke ? min(4, (ke - k0) >> 5) : 0;
        if constexpr (GROUP) {
          bw[i] = bload16(rw, boff + (k0 >> 1) + 16 * g, g < ng);
        } else {
          bw[i] = bload16(rw, boff + k0 + 32 * g, g < ng);
          bw2[i] = bload16(rw, boff + k0 + 32 * g + 16, g < ng);
        }
      }
      // every load above is issued before anything below is scheduled (the
      // scheduler would otherwise sink weight loads next to their use)
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int i = 0; i < NKB; ++i) {
        const int idx = lane + 64 * i;
        const int q = idx / CH, ck = idx - q * CH;
        *reinterpret_cast<u32x4*>(my_x + q * xs + 8 * ck) = permute_a(xv[i]);
      }
      if constexpr (GROUP) *reinterpret_cast<u32x4*>(my_sc + 8 * lane) = scv;
      // the wave reads back only what its own lanes wrote: LDS order suffices.
      // Every lane feeds staged row c / 4: rows 4q of the MFMA carry route q;
      // the other rows only reach outputs t[1..3], which are never used, and
      // rows q >= nr are staged zeros whose outputs are never stored.
      const uint16_t* arow = my_x + q_row * xs;
      const float scol = T::to_f32(scol_bits & 0xffffu);

      // A fragments of a block, read one block ahead of their use
      u32x4 af[2][4];
  #pragma unroll
      for (int j = 0; j < 4; ++j) af[0][j] = *reinterpret_cast<const u32x4*>(arow + 32 * j + 8 * g);
      float acc = 0.0f;
  #pragma unroll
      for (int i = 0; i < NKB; ++i) {
        if (i + 1 < NKB) {
  #pragma unroll
          for (int j = 0; j < 4; ++j)
            af[(i + 1) & 1][j] =
                *reinterpret_cast<const u32x4*>(arow + 128 * (i + 1) + 32 * j + 8 * g);
        }
        uint32_t d[4], d2[4];
        d[0] = bw[i][0]; d[1] = bw[i][1]; d[2] = bw[i][2]; d[3] = bw[i][3];
        if constexpr (GROUP) {
          transpose_rows4(d[0], d[1], d[2], d[3]);
        } else {
          d2[0] = bw2[i][0]; d2[1] = bw2[i][1]; d2[2] = bw2[i][2]; d2[3] = bw2[i][3];
          // 8 dwords per lane: evens and odds transposed separately
          transpose_rows4(d[0], d[2], d2[0], d2[2]);
          transpose_rows4(d[1], d[3], d2[1], d2[3]);
        }
        u32x2 sc2 = {0u, 0u};
        if constexpr (GROUP) sc2 = *reinterpret_cast<const u32x2*>(my_sc + 32 * c + 4 * i);
        // groups past the end of the reduction have zero x and zero weights,
        // so t = 0 there and the (finite) scale read beside them is harmless
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 a = af[i & 1][j];
          float sc;
          u32x4 bop;
          if constexpr (GROUP) {
            const uint32_t pair = sc2[j >> 1];
            sc = T::to_f32((j & 1) ? (pair >> 16) : (pair & 0xffffu));
            bop = group_to_h16<DT, LAYOUT>(d[j]);
          } else {
            sc = scol;
            // sub-chunk j = dwords (2j, 2j+1) of the lane's 8
            const uint32_t lo = (j < 2) ? d[2 * j] : d2[2 * j - 4];
            const uint32_t hi = (j < 2) ? d[2 * j + 1] : d2[2 * j - 3];
            bop = bytes_to_h16<DT>(lo >> (4 * par), hi >> (4 * par));
          }
          // INT4: the -1.5 * sum(a) term of the (24 + q) / 16 encoding; FP4 needs none
          const f32x4 corr = LAYOUT == Q_FP4_GROUP_K ? fzero : T::mfma(a, bconst, fzero);
          const f32x4 t = T::mfma(a, bop, corr);
          acc = fmaf(sc, t[0], acc);
        }
      }
      s_red[w][lane] = acc;
      __syncthreads();
      // wave 0: slices in order; lane row g holds staged row g (element 0)
      if (w == 0 && g < nr) {
        float v = s_red[0][lane];
        for (int q = 1; q < kSmallWaves; ++q) v += s_red[q][lane];
        p.h[static_cast<int64_t>(rrow[g]) * p.ldh + wrow] = 16.0f * v;
      }
      __syncthreads();
    }
  }  // distinct experts kx
}

// ---------------------------------------------------------------------------
// small batch down GEMM of each route of one token + FP32 combine in top-k
// order; the activation of the token's routes is formed in the prologue
// ---------------------------------------------------------------------------
// Memory order: one load of the token's ids and weights (lane k holds route
// k); then, in flight together, the FP32 pre-activations of the token's
// routes and the weights of each wave's first work item (raw buffer loads:
// masked lanes read zeros, nothing waits on a load before its use).
// SiLU(gate)*up or ReLU^2 is computed once per value, rounded to 16 bits and
// staged in LDS in A operand order.  Work items are (valid route k, 256-wide
// slice of the reduction): invalid routes take none; each wave computes its
// items' 32 partial outputs (one MFMA row: a route is a single activation row)
// into LDS, and with PF (more items than waves possible) the loads of its next
// item are in flight while it computes one; then 32 lanes add, for k =
// 0..K-1 in order, w[t,k] * (sum of k's slices in slice order) over the valid
// routes and cast once.
template <int DT, int LAYOUT, bool GATED, int AL, bool PF>
__global__ void __launch_bounds__(kDecThreads)
decode_down_kernel(const DecodeDownParams p) {
  using T = H16<DT>;
  constexpr int NSUB = 2;
  constexpr int SL = kDecDownSliceBlocks;  // blocks of 128 per item
  // the wave index as a wave-uniform value: items, routes and expert ids
  // derived from it stay scalar (buffer descriptors included)
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c = lane & 15, g = lane >> 4, par = c & 1;
  const int n0 = blockIdx.x * 32;
  const int t = blockIdx.y;
  const int nblk = (p.I + 127) / 128;
  const int nsl = (nblk + SL - 1) / SL;
  const int as = p.I + 8;                  // staged activation row stride

  extern __shared__ uint16_t s_dyn[];      // [top_k][I + 8] activations (A operand
                                           // order), then [top_k * nsl][32] partials
  uint16_t* const s_act = s_dyn;
  float (*const s_y)[32] = reinterpret_cast<float (*)[32]>(
      s_dyn + static_cast<size_t>(p.top_k) * as);

  // (1) the token's routes: lane k < top_k holds id, local expert and weight
  const uint32_t r_base = static_cast<uint32_t>(t) * p.top_k;
  const auto rids = make_rsrc(p.ids + r_base, 4u * p.top_k);
  const auto rwts = make_rsrc(p.wts + r_base, 4u * p.top_k);
  const int e_lane = local_id(static_cast<int32_t>(bload4(rids, 4u * lane, lane < p.top_k)), p.E, p.off);
  const float wt_lane = __uint_as_float(bload4(rwts, 4u * lane, lane < p.top_k));
  // work items are (valid route, slice): item it is slice it % nsl of the
  // (it / nsl)-th valid route in top-k order (invalid routes take no item)
  const uint32_t vmask = static_cast<uint32_t>(__ballot(lane < p.top_k && e_lane >= 0));
  const int items = __popc(vmask) * nsl;

  bool on[NSUB];
  int wrow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    on[s] = n0 + 16 * s < p.H;
    wrow[s] = n0 + 16 * s + c;
  }

  // (2) pre-activations of the token's routes (8 values per chunk)
  const int ich = p.I >> 3;
  const int nch = p.top_k * ich;
  const auto rh = make_rsrc(p.h + static_cast<int64_t>(r_base) * p.ldh, 4u * p.top_k * p.ldh);
  f32x4 hg[AL][2], hu[AL][2];  // AL: activation chunks per thread (>= top_k * I / 8 / 512)
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int idx = tid + kDecThreads * i;
    const int k = idx < nch ? idx / ich : 0, cc = idx < nch ? idx - k * ich : 0;
    const bool ok = idx < nch && ((vmask >> k) & 1u) != 0;
    const uint32_t off = 4u * (static_cast<uint32_t>(k) * p.ldh + 8 * cc);
    hg[i][0] = __builtin_bit_cast(f32x4, bload16(rh, off, ok));
    hg[i][1] = __builtin_bit_cast(f32x4, bload16(rh, off + 16, ok));
    if constexpr (GATED) {
      hu[i][0] = __builtin_bit_cast(f32x4, bload16(rh, off + 4u * p.I, ok));
      hu[i][1] = __builtin_bit_cast(f32x4, bload16(rh, off + 4u * p.I + 16, ok));
    }
  }

  // (3) weights of a work item (route k, reduction slice sl); an item past
  // the last loads nothing (e = -1)
  const uint32_t boff[NSUB] = {
      is_group(LAYOUT) ? static_cast<uint32_t>(wrow[0]) * (p.I >> 1)
                          : static_cast<uint32_t>(wrow[0] >> 1) * p.I,
      is_group(LAYOUT) ? static_cast<uint32_t>(wrow[1]) * (p.I >> 1)
                          : static_cast<uint32_t>(wrow[1] >> 1) * p.I};
  auto item_route = [&](int it) {  // top-k index of item it's route
    uint32_t m = vmask;
    for (int i = it / nsl; i > 0; --i) m &= m - 1;
    return __builtin_ctz(m);
  };
  auto load_item = [&](int it, BBlk<LAYOUT> (&b)[SL][NSUB], float (&scol)[NSUB], int& e) {
    const bool have = it < items;
    const int k = have ? item_route(it) : 0;
    e = have ? __builtin_amdgcn_readlane(e_lane, k) : -1;
    const int ee = e >= 0 ? e : 0;
    const auto rw = make_rsrc(p.wq + static_cast<int64_t>(ee) * p.wq_expert_bytes,
                              static_cast<uint32_t>(p.wq_expert_bytes));
    const auto rs = make_rsrc(p.ws + static_cast<int64_t>(ee) * p.ws_expert_elems,
                              static_cast<uint32_t>(2 * p.ws_expert_elems));
    const int sl = it % nsl;
    const int kb = sl * SL * 128;
    const int ke = min(p.I, kb + SL * 128);
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int k0 = kb + 128 * i;
      const int ng = k0 < ke ? min(4, (ke - k0) >> 5) : 0;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const bool ok = e >= 0 && on[s] && ng > 0;
        if constexpr (is_group(LAYOUT)) {
          const u32x4 v = bload16(rw, boff[s] + (k0 >> 1) + 16 * g, ok && g < ng);
          b[i][s].d[0] = v[0]; b[i][s].d[1] = v[1]; b[i][s].d[2] = v[2]; b[i][s].d[3] = v[3];
          const uint32_t so = 2u * (static_cast<uint32_t>(wrow[s]) * (p.I >> 5) + (k0 >> 5));
          const u32x2 sv = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, ok ? so : kOob, 0, 0));
          b[i][s].s[0] = sv[0];
          b[i][s].s[1] = sv[1];
        } else {
          const u32x4 v0 = bload16(rw, boff[s] + k0 + 32 * g, ok && g < ng);
          const u32x4 v1 = bload16(rw, boff[s] + k0 + 32 * g + 16, ok && g < ng);
          b[i][s].d[0] = v0[0]; b[i][s].d[1] = v0[1]; b[i][s].d[2] = v0[2]; b[i][s].d[3] = v0[3];
          b[i][s].d[4] = v1[0]; b[i][s].d[5] = v1[1]; b[i][s].d[6] = v1[2]; b[i][s].d[7] = v1[3];
          b[i][s].s[0] = b[i][s].s[1] = 0u;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
      scol[s] = (is_group(LAYOUT))
                    ? 0.0f
                    : T::to_f32(bload4(rs, (2u * wrow[s]) & ~3u, e >= 0 && on[s]) >> (16 * (wrow[s] & 1)));
  };

  BBlk<LAYOUT> b[PF ? 2 : 1][SL][NSUB];
  float scol[PF ? 2 : 1][NSUB];
  int e_cur[PF ? 2 : 1];
  load_item(w, b[0], scol[0], e_cur[0]);

  // (4) activation of the valid routes: computed once per value, 16-bit, A
  // operand order (the rows of invalid routes are never read)
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int idx = tid + kDecThreads * i;
    const int k = idx < nch ? idx / ich : 0, cc = idx - k * ich;
    if (idx < nch && ((vmask >> k) & 1u) != 0) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float hv = hg[i][q >> 2][q & 3];
        if constexpr (GATED) {
          v[q] = silu(hv) * hu[i][q >> 2][q & 3];
        } else {
          const float hp = fmaxf(hv, 0.0f);
          v[q] = hp * hp;
        }
      }
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = static_cast<uint32_t>(T::from_f32(v[2 * q])) |
               (static_cast<uint32_t>(T::from_f32(v[2 * q + 1])) << 16);
      *reinterpret_cast<u32x4*>(s_act + k * as + 8 * cc) = permute_a(o);
    }
  }
  __syncthreads();

  const u32x4 bconst = {T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2};
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  // one item's 32 partial outputs into s_y[it]
  auto compute_item = [&](int it, BBlk<LAYOUT> (&bb)[SL][NSUB], const float (&sc_col)[NSUB],
                          int e) {
    const int k = item_route(it), sl = it % nsl;
    float y[NSUB] = {0.0f, 0.0f};
    if (e >= 0) {
      const uint16_t* arow = s_act + k * as;
      const int kb = sl * SL * 128;
      const int ke = min(p.I, kb + SL * 128);
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int k0 = kb + 128 * i;
        const int ng = k0 < ke ? min(4, (ke - k0) >> 5) : 0;
#pragma unroll
        for (int s = 0; s < NSUB; ++s) tr_b<LAYOUT>(bb[i][s]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool gv = j < ng;
          const bool fa = c == 0 && gv;
          const u32x4 av = *reinterpret_cast<const u32x4*>(arow + (fa ? k0 + 32 * j + 8 * g : 0));
          u32x4 a;
          a[0] = fa ? av[0] : 0u;
          a[1] = fa ? av[1] : 0u;
          a[2] = fa ? av[2] : 0u;
          a[3] = fa ? av[3] : 0u;
          const f32x4 corr = LAYOUT == Q_FP4_GROUP_K ? fzero : T::mfma(a, bconst, fzero);
#pragma unroll
          for (int s = 0; s < NSUB; ++s) {
            float sc = (is_group(LAYOUT)) ? sc_of<DT>(bb[i][s].s[j >> 1], j) : sc_col[s];
            sc = (gv && on[s]) ? sc : 0.0f;
            const f32x4 tt = T::mfma(a, b_op<DT, LAYOUT>(bb[i][s], j, par), corr);
            y[s] = fmaf(sc, tt[0], y[s]);
          }
        }
      }
    }
    if (lane < 16) {
      s_y[it][c] = y[0];
      s_y[it][16 + c] = y[1];
    }
  };
  if constexpr (PF) {
    // two register sets used alternately: the next item's loads (masked
    // past the last) are in flight while an item is computed
    for (int it = w; it < items; it += 2 * kDecWaves) {
      load_item(it + kDecWaves, b[1], scol[1], e_cur[1]);
      compute_item(it, b[0], scol[0], e_cur[0]);
      if (it + kDecWaves >= items) break;
      load_item(it + 2 * kDecWaves, b[0], scol[0], e_cur[0]);
      compute_item(it + kDecWaves, b[1], scol[1], e_cur[1]);
    }
  } else {
    for (int it = w; it < items; it += kDecWaves) {
      if (it != w) load_item(it, b[0], scol[0], e_cur[0]);
      compute_item(it, b[0], scol[0], e_cur[0]);
    }
  }
  __syncthreads();
  if (tid < 32) {
    float acc = 0.0f;
    int kv = 0;  // items of the valid routes before route k
    for (int k = 0; k < p.top_k; ++k) {
      if (((vmask >> k) & 1u) == 0) continue;  // invalid route: nothing
      float y = s_y[kv * nsl][tid];
      for (int sl = 1; sl < nsl; ++sl) y += s_y[kv * nsl + sl][tid];
      const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wt_lane), k));
      acc += wk * (16.0f * y);
      ++kv;
    }
    if (n0 + tid < p.H) p.out[static_cast<int64_t>(t) * p.H + n0 + tid] = T::from_f32(acc);
  }
}

// ---------------------------------------------------------------------------
// launchers

template <typename F>
static hipError_t allow_lds(F* kernel, size_t lds) {
  // dynamic LDS beyond 64 KiB must be opted into per kernel (gfx950 has 160 KiB)
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}


template <int DT, int LAYOUT, int NKB>
static hipError_t launch_small_h_k(const SmallHParams& p, dim3 grid, size_t lds, hipStream_t st) {
  if (p.ra.logits != nullptr) {
    const hipError_t err = allow_lds(small_h_kernel<DT, LAYOUT, NKB, true>, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((small_h_kernel<DT, LAYOUT, NKB, true>), grid, dim3(kSmallThreads), lds,
                       st, p);
    return hipGetLastError();
  }
  const hipError_t err = allow_lds(small_h_kernel<DT, LAYOUT, NKB, false>, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((small_h_kernel<DT, LAYOUT, NKB, false>), grid, dim3(kSmallThreads), lds, st,
                     p);
  return hipGetLastError();
}

template <int DT, int LAYOUT>
static hipError_t launch_small_h_nkb(const SmallHParams& p, int nkb, dim3 grid, size_t lds,
                                     hipStream_t st) {
  // one instantiation per blocks-per-slice count: no wasted loads or registers
  switch (nkb) {
    case 1: return launch_small_h_k<DT, LAYOUT, 1>(p, grid, lds, st);
    case 2: return launch_small_h_k<DT, LAYOUT, 2>(p, grid, lds, st);
    case 3: return launch_small_h_k<DT, LAYOUT, 3>(p, grid, lds, st);
    case 4: return launch_small_h_k<DT, LAYOUT, 4>(p, grid, lds, st);
    case 5: return launch_small_h_k<DT, LAYOUT, 5>(p, grid, lds, st);
    case 6: return launch_small_h_k<DT, LAYOUT, 6>(p, grid, lds, st);
    case 7: return launch_small_h_k<DT, LAYOUT, 7>(p, grid, lds, st);
    case 8: return launch_small_h_k<DT, LAYOUT, 8>(p, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_small_h(const SmallHParams& p, int dtype, int layout, int nkb, int n1,
                          hipStream_t stream) {
  if (p.R < 1 || p.R > kSmallMaxRoutes || p.slots < 1 || p.slots > p.R) return hipErrorInvalidValue;
  const dim3 grid(n1 / 16, p.slots);
  const size_t lds = small_h_lds_bytes(p.kslice);
  if (dtype == DT_BF16)
    return layout == Q_GROUP_K ? launch_small_h_nkb<DT_BF16, Q_GROUP_K>(p, nkb, grid, lds, stream)
         : layout == Q_FP4_GROUP_K ? launch_small_h_nkb<DT_BF16, Q_FP4_GROUP_K>(p, nkb, grid, lds, stream)
                               : launch_small_h_nkb<DT_BF16, Q_PER_CHANNEL>(p, nkb, grid, lds, stream);
  return layout == Q_GROUP_K ? launch_small_h_nkb<DT_FP16, Q_GROUP_K>(p, nkb, grid, lds, stream)
       : layout == Q_FP4_GROUP_K ? launch_small_h_nkb<DT_FP16, Q_FP4_GROUP_K>(p, nkb, grid, lds, stream)
                             : launch_small_h_nkb<DT_FP16, Q_PER_CHANNEL>(p, nkb, grid, lds, stream);
}

template <int DT, int LAYOUT, bool GATED, int AL>
static hipError_t launch_dd_k(const DecodeDownParams& p, dim3 grid, size_t lds, hipStream_t st) {
  // items (valid routes x slices) expected to outnumber the waves: the
  // prefetching variant (two register sets; fewer workgroups per CU)
  if (p.prefetch) {
    const hipError_t err = allow_lds(decode_down_kernel<DT, LAYOUT, GATED, AL, true>, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((decode_down_kernel<DT, LAYOUT, GATED, AL, true>), grid, dim3(kDecThreads),
                       lds, st, p);
    return hipGetLastError();
  }
  const hipError_t err = allow_lds(decode_down_kernel<DT, LAYOUT, GATED, AL, false>, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_down_kernel<DT, LAYOUT, GATED, AL, false>), grid, dim3(kDecThreads),
                     lds, st, p);
  return hipGetLastError();
}

template <int DT, int LAYOUT, bool GATED>
static hipError_t launch_dd_al(const DecodeDownParams& p, dim3 grid, size_t lds, hipStream_t st) {
  const int need = (p.top_k * (p.I / 8) + kDecThreads - 1) / kDecThreads;
  if (need <= 1) return launch_dd_k<DT, LAYOUT, GATED, 1>(p, grid, lds, st);
  if (need <= 2) return launch_dd_k<DT, LAYOUT, GATED, 2>(p, grid, lds, st);
  if (need <= 4) return launch_dd_k<DT, LAYOUT, GATED, 4>(p, grid, lds, st);
  if (need <= kDecActLoads) return launch_dd_k<DT, LAYOUT, GATED, kDecActLoads>(p, grid, lds, st);
  return hipErrorInvalidValue;
}

template <int DT, int LAYOUT>
static hipError_t launch_dd(const DecodeDownParams& p, bool gated, dim3 grid, size_t lds,
                            hipStream_t st) {
  return gated ? launch_dd_al<DT, LAYOUT, true>(p, grid, lds, st)
               : launch_dd_al<DT, LAYOUT, false>(p, grid, lds, st);
}

hipError_t launch_decode_down(const DecodeDownParams& p, int dtype, int layout, bool gated, int T,
                              hipStream_t stream) {
  const dim3 grid((p.H + 31) / 32, T);
  const size_t lds = decode_down_lds_bytes(p.top_k, p.I);
  if (dtype == DT_BF16)
    return layout == Q_GROUP_K ? launch_dd<DT_BF16, Q_GROUP_K>(p, gated, grid, lds, stream)
         : layout == Q_FP4_GROUP_K ? launch_dd<DT_BF16, Q_FP4_GROUP_K>(p, gated, grid, lds, stream)
                               : launch_dd<DT_BF16, Q_PER_CHANNEL>(p, gated, grid, lds, stream);
  return layout == Q_GROUP_K ? launch_dd<DT_FP16, Q_GROUP_K>(p, gated, grid, lds, stream)
       : layout == Q_FP4_GROUP_K ? launch_dd<DT_FP16, Q_FP4_GROUP_K>(p, gated, grid, lds, stream)
                             : launch_dd<DT_FP16, Q_PER_CHANNEL>(p, gated, grid, lds, stream);
}

}  // namespace w4moe
