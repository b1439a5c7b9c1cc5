// router.h -- one token's router scoring and top-k by one wave, shared by the
// standalone router kernel and the kernels that fuse routing with the first
// step of the forward (route preparation, or the small-batch gate/up GEMM).
//
// Sources (web pages, cited by tag and section):
//   [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
//        overhead"  Final performance: routing is part of the timed MoE.
//   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
//        Benchmark: FP32 routing weights, INT32 expert ids, no
//        renormalization of the selected weights.
//
// The softmax of the token's logits over all global experts, then the K
// experts of largest probability in descending order, ties to the lower id,
// with their probabilities as weights (optionally divided by their sum in
// top-k order).  The selection compares logits: the softmax is strictly
// increasing in the logit, so the order is the same and no tie is decided
// between probabilities that only rounding made equal.
//
// Lane l holds logits l, l + 64, ... (one coalesced pass over the row); the
// maximum and the sum of exp(l - max) are butterfly reductions over the wave
// done in VALU (DPP and permlane swaps, a fixed order: bitwise repeatable, and
// the same bits in every kernel that calls this); the K winners come from K
// rounds of a wave argmax over the untaken logits, each lane keeping a bit
// mask of its taken slots.  Lane k ends up holding winner k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "internal.h"  // RouteArgs

namespace w4moe {

// (value, id) order of the selection: larger value first, then lower id
// (bitwise operators: evaluated as selects, not branches)
__device__ __forceinline__ bool rt_before(float a, int ia, float b, int ib) {
  return (a > b) | ((a == b) & (ia < ib));
}

// Butterfly partner of this lane at step S (0..5) of a 64-lane all-reduce,
// all in VALU (no LDS permutes): quad_perm [1,0,3,2] and [2,3,0,1], the
// half-row and row mirrors (lane i with 7 - i, then 15 - i), then the other
// 16-lane row and the other 32-lane half through the gfx950 permlane swaps.
// After step S every lane holds the combination over its group of 2^(S+1)
// lanes; combining with a commutative operation gives every lane the same
// bits, since each pair of partners adds or compares the same two values.
template <int S>
__device__ __forceinline__ uint32_t bfly_partner(uint32_t v, int lane) {
  if constexpr (S == 0) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  else if constexpr (S == 1) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  else if constexpr (S == 2) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
  else if constexpr (S == 3) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
  else if constexpr (S == 4) {
    // rows 0/1 and 2/3 swapped: an even row finds its partner in the second result
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((lane >> 4) & 1) ? p[0] : p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return lane >= 32 ? p[0] : p[1];
  }
}

template <int S>
__device__ __forceinline__ float bfly_partner_f(float v, int lane) {
  return __uint_as_float(bfly_partner<S>(__float_as_uint(v), lane));
}

__device__ __forceinline__ float wave_max(float m, int lane) {
  m = fmaxf(m, bfly_partner_f<0>(m, lane));
  m = fmaxf(m, bfly_partner_f<1>(m, lane));
  m = fmaxf(m, bfly_partner_f<2>(m, lane));
  m = fmaxf(m, bfly_partner_f<3>(m, lane));
  m = fmaxf(m, bfly_partner_f<4>(m, lane));
  return fmaxf(m, bfly_partner_f<5>(m, lane));
}

__device__ __forceinline__ float wave_sum(float z, int lane) {
  z += bfly_partner_f<0>(z, lane);
  z += bfly_partner_f<1>(z, lane);
  z += bfly_partner_f<2>(z, lane);
  z += bfly_partner_f<3>(z, lane);
  z += bfly_partner_f<4>(z, lane);
  return z + bfly_partner_f<5>(z, lane);
}

template <int S>
__device__ __forceinline__ void argmax_step(float& bv, int& bi, int lane) {
  const float ov = bfly_partner_f<S>(bv, lane);
  const int oi = static_cast<int>(bfly_partner<S>(static_cast<uint32_t>(bi), lane));
  const bool take = rt_before(ov, oi, bv, bi);
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

// Logits per lane of a router instantiation: E_global <= 64 * NPL.
__host__ __device__ constexpr int router_npl(int Eg) {
  return Eg <= 64 ? 1 : Eg <= 128 ? 2 : Eg <= 256 ? 4 : Eg <= 512 ? 8 : 16;
}

// A token's logits, lane l holding logits l, l + 64, ... (slots past E_global
// hold -inf with ids >= E_global: they lose every tie against a real expert,
// and K <= E_global keeps them out of the result).
template <int NPL>
struct RouteRow {
  float v[NPL];
};

template <int NPL>
__device__ __forceinline__ RouteRow<NPL> route_load(const float* row, int Eg, int lane) {
  // the row is the wave's (uniform): said so, the buffer resource lives in
  // scalar registers (else every load becomes a loop over lane values)
  const uint64_t a = reinterpret_cast<uint64_t>(row);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  row = reinterpret_cast<const float*>((static_cast<uint64_t>(hi) << 32) | lo);
  Eg = __builtin_amdgcn_readfirstlane(Eg);
  const auto rl = make_rsrc(row, 4u * static_cast<uint32_t>(Eg));
  RouteRow<NPL> r;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    const float x = __uint_as_float(bload4(rl, 4u * static_cast<uint32_t>(e), e < Eg));
    r.v[j] = e < Eg ? x : -INFINITY;
  }
  return r;
}

// Selection by the calling wave (all 64 lanes, wave-uniform arguments): on
// return lane k < K holds the k-th expert id and its weight.
template <int NPL>
__device__ __forceinline__ void route_select(const RouteRow<NPL>& row, int K, int renorm,
                                             int lane, int& my_id, float& p_out) {
  const float* v = row.v;
  float m = v[0];
#pragma unroll
  for (int j = 1; j < NPL; ++j) m = fmaxf(m, v[j]);
  m = wave_max(m, lane);
  const bool none = m == -INFINITY;  // every logit of the token is -inf
  float z = 0.0f;
  if (!none) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) z += expf(v[j] - m);
  }
  z = wave_sum(z, lane);

  uint32_t taken = 0;
  my_id = 0;
  float my_v = -INFINITY;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      const bool take = (((taken >> j) & 1u) == 0u) & rt_before(v[j], e, bv, bi);
      bv = take ? v[j] : bv;
      bi = take ? e : bi;
    }
    argmax_step<0>(bv, bi, lane);
    argmax_step<1>(bv, bi, lane);
    argmax_step<2>(bv, bi, lane);
    argmax_step<3>(bv, bi, lane);
    argmax_step<4>(bv, bi, lane);
    argmax_step<5>(bv, bi, lane);
    taken |= (lane == (bi & 63)) ? (1u << (bi >> 6)) : 0u;
    my_id = lane == k ? bi : my_id;
    my_v = lane == k ? bv : my_v;
  }
  // weights of the K winners (lane k holds winner k), all at once
  float my_p = (none || my_v == -INFINITY) ? 0.0f : expf(my_v - m) / z;
  if (renorm) {
    float sum = 0.0f;
    for (int k = 0; k < K; ++k)  // top-k order
      sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_p), k));
    my_p = sum > 0.0f ? my_p / sum : 0.0f;
  }
  p_out = my_p;
}

// Routes tokens t0, t0 + step, ... < t1 with the calling wave, the next
// token's logits requested before the current one is selected; f(t, id, p)
// is called by every lane after each token (lane k < K holding winner k).
template <int NPL, typename F>
__device__ __forceinline__ void route_tokens(const RouteArgs& ra, int K, int t0, int t1, int step,
                                             int lane, F&& f) {
  if (t0 >= t1) return;
  RouteRow<NPL> next = route_load<NPL>(ra.logits + static_cast<int64_t>(t0) * ra.Eg, ra.Eg, lane);
  for (int t = t0; t < t1; t += step) {
    const RouteRow<NPL> cur = next;
    if (t + step < t1)
      next = route_load<NPL>(ra.logits + static_cast<int64_t>(t + step) * ra.Eg, ra.Eg, lane);
    int id;
    float p;
    route_select<NPL>(cur, K, ra.renorm, lane, id, p);
    f(t, id, p);
  }
}

}  // namespace w4moe
