// router.hip -- router scoring and top-k, the step before route preparation.
//
// Sources (web pages, cited by tag and section):
//   [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
//        overhead"  Final performance: routing is part of the timed MoE.
//   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
//        Benchmark: FP32 routing weights, INT32 expert ids, no
//        renormalization of the selected weights.
//
// One wave per token (route_load and route_select in router.h).
#include <stdint.h>

#include "device.h"
#include "internal.h"
#include "router.h"

namespace w4moe {

namespace {

constexpr int kRtWaves = 4;  // tokens per workgroup

}  // namespace

template <int NPL>  // logits per lane: E_global <= 64 * NPL
__global__ void __launch_bounds__(64 * kRtWaves)
router_topk_kernel(const float* __restrict__ logits, int T, int Eg, int K, int renorm,
                   int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRtWaves + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  int my_id;
  float my_p;
  route_select<NPL>(route_load<NPL>(logits + static_cast<int64_t>(t) * Eg, Eg, lane), K, renorm,
                    lane, my_id, my_p);
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
