// router.hip -- router scoring and top-k, the step before route preparation.
//
// Sources (web pages, cited by tag and section):
//   [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
//        overhead"  Final performance: routing is part of the timed MoE.
//   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
//        Benchmark: FP32 routing weights, INT32 expert ids, no
//        renormalization of the selected weights.
//
// For each token: the softmax of its router logits over all global experts,
// then the K experts of largest probability in descending order, ties to the
// lower id, with their probabilities as weights (optionally divided by their
// sum).  The selection compares logits: the softmax is strictly increasing in
// the logit, so the order is the same and no tie is decided between
// probabilities that only rounding made equal.
//
// One wave per token.  Lane l holds logits l, l + 64, ... in registers (one
// coalesced pass over the row); the maximum and the sum of exp(l - max) are
// butterfly reductions over the wave (a fixed order, so results are bitwise
// repeatable); the K winners come from K rounds of a wave argmax over the
// untaken logits, each lane keeping a bit mask of its taken slots.  Lane k
// ends up holding winner k and writes it.
#include <stdint.h>

#include "device.h"
#include "internal.h"

namespace w4moe {

namespace {

constexpr int kRtWaves = 4;  // tokens per workgroup

// (value, id) order of the selection: larger value first, then lower id
__device__ __forceinline__ bool rt_before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

}  // namespace

template <int NPL>  // logits per lane: E_global <= 64 * NPL
__global__ void __launch_bounds__(64 * kRtWaves)
router_topk_kernel(const float* __restrict__ logits, int T, int Eg, int K, int renorm,
                   int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRtWaves + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const auto rl = make_rsrc(logits + static_cast<int64_t>(t) * Eg, 4u * static_cast<uint32_t>(Eg));
  // slots past E_global hold -inf with ids >= E_global: they lose every tie
  // against a real expert, and K <= E_global keeps them out of the result
  float v[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    const float x = __uint_as_float(bload4(rl, 4u * static_cast<uint32_t>(e), e < Eg));
    v[j] = e < Eg ? x : -INFINITY;
  }
  float m = v[0];
#pragma unroll
  for (int j = 1; j < NPL; ++j) m = fmaxf(m, v[j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const bool none = m == -INFINITY;  // every logit of the token is -inf
  float z = 0.0f;
  if (!none) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) z += expf(v[j] - m);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);

  uint32_t taken = 0;
  int my_id = 0;
  float my_p = 0.0f;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      if (!((taken >> j) & 1u) && rt_before(v[j], e, bv, bi)) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (rt_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
    if (lane == k) {
      my_id = bi;
      my_p = (none || bv == -INFINITY) ? 0.0f : expf(bv - m) / z;
    }
  }
  if (renorm) {
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum += __shfl(my_p, k, 64);  // top-k order
    my_p = sum > 0.0f ? my_p / sum : 0.0f;
  }
  if (lane < K) {
    ids[static_cast<int64_t>(t) * K + lane] = my_id;
    wts[static_cast<int64_t>(t) * K + lane] = my_p;
  }
}

hipError_t launch_router_topk(const float* logits, int T, int Eg, int K, int renorm, int32_t* ids,
                              float* wts, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (Eg < 1 || Eg > kRouterMaxExperts || K < 1 || K > kRouterMaxTopK || K > Eg)
    return hipErrorInvalidValue;
  const dim3 grid((T + kRtWaves - 1) / kRtWaves), block(64 * kRtWaves);
  const int npl = (Eg + 63) / 64;
  if (npl <= 1) hipLaunchKernelGGL(router_topk_kernel<1>, grid, block, 0, stream, logits, T, Eg, K, renorm, ids, wts);
  else if (npl <= 2) hipLaunchKernelGGL(router_topk_kernel<2>, grid, block, 0, stream, logits, T, Eg, K, renorm, ids, wts);
  else if (npl <= 4) hipLaunchKernelGGL(router_topk_kernel<4>, grid, block, 0, stream, logits, T, Eg, K, renorm, ids, wts);
  else if (npl <= 8) hipLaunchKernelGGL(router_topk_kernel<8>, grid, block, 0, stream, logits, T, Eg, K, renorm, ids, wts);
  else hipLaunchKernelGGL(router_topk_kernel<16>, grid, block, 0, stream, logits, T, Eg, K, renorm, ids, wts);
  return hipGetLastError();
}

}  // namespace w4moe
