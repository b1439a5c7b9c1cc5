// gemm.hip -- the FP32 combine of the grouped path of the local W4A16 MoE
// forward on gfx950, and the nibble-unpacking test export.
//
// Sources (web pages, cited by tag and section):
//   [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
//        overhead"  Description, "Contract": 16-bit expert outputs combined in
//        FP32 in fixed top-k order before one 16-bit cast, no atomics.
//   [P3] TensorRT-LLM PR #18313, "Add W4A16 per-channel weight-only support
//        for Cutlass fused MoE"  Checkpoint format (nibble packing).
//
// Kernels
//   combine_kernel  out[t] = cast16(sum_k w[t,k] * Y[t*K+k]) in FP32 over the
//                   valid routes (slot[t*K+k] >= 0).
//   unpack_kernel   nibbles through the GEMMs' bit conversion, back to int8.
//   decode_fp4_kernel  E2M1 codes through the GEMMs' conversion, back to FP32.
//   e8m0_kernel     MXFP4 block scales to 16-bit scales (setup).
//   repack_pc_kernel  per-channel INT4 into the group layout (setup).
#include "device.h"
#include "internal.h"

namespace w4moe {

template <int DT>
__global__ void __launch_bounds__(256)
combine_kernel(const CombineParams p) {
  using T = H16<DT>;
  constexpr int kBatch = 8;  // routes whose Y loads are in flight together
  const int t = blockIdx.y;
  const int col = (blockIdx.x * 256 + threadIdx.x) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < p.top_k; kb += kBatch) {
    // the token's slots and weights (wave-uniform), then every Y load of the
    // batch: one buffer resource per route, empty for an invalid route (its
    // loads return zeros), and columns past H read out of range as well
    int pos[kBatch];
    float wk[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int r = t * p.top_k + kb + k;
      pos[k] = kb + k < p.top_k ? p.slot[r] : -1;
      wk[k] = kb + k < p.top_k ? p.wts[r] : 0.0f;
    }
    u32x4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const bool ok = pos[k] >= 0;
      const int64_t r = static_cast<int64_t>(t) * p.top_k + kb + k;  // Y row of the route
      const auto ry = make_rsrc(p.y + (ok ? r : 0) * p.H, ok ? static_cast<uint32_t>(2 * p.H) : 0u);
      v[k] = bload16(ry, 2u * static_cast<uint32_t>(col), true);
    }
    // fixed order: ascending k, invalid routes contribute nothing
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (pos[k] < 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wk[k] * T::to_f32(v[k][i] & 0xffffu);
        acc[2 * i + 1] += wk[k] * T::to_f32(v[k][i] >> 16);
      }
    }
  }
  if (col >= p.H) return;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(T::from_f32(acc[2 * i])) |
           (static_cast<uint32_t>(T::from_f32(acc[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(p.out + static_cast<int64_t>(t) * p.H + col) = o;
}

// Test export: nibbles through the same bit conversion the GEMMs use, then
// back to integers: q = 16 * value - 24 (exact).
__global__ void __launch_bounds__(256)
unpack_kernel(const uint8_t* __restrict__ in, int64_t n, int8_t* __restrict__ out) {
  using T = H16<DT_BF16>;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (b0 >= n) return;
  const int nb = static_cast<int>(min<int64_t>(4, n - b0));
  uint32_t d = 0;
  for (int q = 0; q < nb; ++q) d |= static_cast<uint32_t>(in[b0 + q]) << (8 * q);
  const u32x4 h = nibbles_to_h16<DT_BF16>(d);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lo = static_cast<int>(T::to_f32(h[j] & 0xffffu) * 16.0f) - 24;
    const int hi = static_cast<int>(T::to_f32(h[j] >> 16) * 16.0f) - 24;
    if (j < 2 * nb) out[2 * b0 + j] = static_cast<int8_t>(lo);
    if (j + 4 < 2 * nb) out[2 * b0 + j + 4] = static_cast<int8_t>(hi);
  }
}

// Test export: FP4 (E2M1) codes through the conversion the GEMMs use (each
// value / 16 as a 16-bit float), back to FP32 values (times 16: exact).
// Four bytes (eight codes) per thread, in the GEMMs' pair order.
template <int DT>
__global__ void __launch_bounds__(256)
decode_fp4_kernel(const uint8_t* __restrict__ in, int64_t n, float* __restrict__ out) {
  using T = H16<DT>;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (b0 >= n) return;
  const int nb = static_cast<int>(min<int64_t>(4, n - b0));
  uint32_t d = 0;
  for (int q = 0; q < nb; ++q) d |= static_cast<uint32_t>(in[b0 + q]) << (8 * q);
  const u32x4 h = e2m1_to_h16<DT>(d);  // (n_j, n_j+4) in dword j
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < 2 * nb) out[2 * b0 + j] = 16.0f * T::to_f32(h[j] & 0xffffu);
    if (j + 4 < 2 * nb) out[2 * b0 + j + 4] = 16.0f * T::to_f32(h[j] >> 16);
  }
}

// MXFP4 block scales: E8M0 code e -> 2^(e - 127) as a 16-bit float (the
// FP32 value is exact; its 16-bit rounding is exact wherever the dtype holds
// the power of two).
template <int DT>
__global__ void __launch_bounds__(256)
e8m0_kernel(const uint8_t* __restrict__ in, int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t e = in[i];
  // 2^(e - 127): e >= 1 is a normal FP32 exponent field, e = 0 the subnormal 2^-127
  const float v = e == 255u ? __uint_as_float(0x7FC00000u)
                            : (e == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23));
  out[i] = H16<DT>::from_f32(v);
}

// Setup-only re-layout of per-channel INT4 (packed along N, [E][N/2][K],
// scales [E][N]) into the group layout (packed along K, [E][N][K/2], the
// channel scale repeated per 32 values, [E][N][K/32]).  Thread i writes
// output bytes 4i..4i+3 of one expert; the scales are written by the threads
// of each row's first K/32 bytes.
__global__ void __launch_bounds__(256)
repack_pc_kernel(const uint8_t* __restrict__ in, const uint16_t* __restrict__ sc_in, int n_out,
                 int k_in, uint8_t* __restrict__ out, uint16_t* __restrict__ sc_out) {
  const int64_t e = blockIdx.y;
  const int64_t per_e = static_cast<int64_t>(n_out) * (k_in / 2);   // output bytes per expert
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (b0 >= per_e) return;
  const uint8_t* src = in + e * per_e;   // the input has as many bytes per expert
  const int n = static_cast<int>(b0 / (k_in / 2));
  const int kb = static_cast<int>(b0 % (k_in / 2));   // first output byte within the row
  const int sh = 4 * (n & 1);                          // odd channels: high nibbles
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = 2 * (kb + j);
    const uint32_t lo = (src[static_cast<int64_t>(n >> 1) * k_in + k] >> sh) & 0xFu;
    const uint32_t hi = (src[static_cast<int64_t>(n >> 1) * k_in + k + 1] >> sh) & 0xFu;
    word |= (lo | (hi << 4)) << (8 * j);
  }
  *reinterpret_cast<uint32_t*>(out + e * per_e + b0) = word;
  // scales: the row's K/32 group scales, 4 per thread (K/2 bytes per row is a
  // multiple of 4, so a thread's bytes stay in one row)
  const int groups = k_in / 32;
  const uint16_t s = sc_in[e * n_out + n];
  for (int gi = kb; gi < min(groups, kb + 4); ++gi)
    sc_out[(e * n_out + n) * groups + gi] = s;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_combine(const CombineParams& p, int dtype, int T, hipStream_t stream) {
  const dim3 grid((p.H + kCombineCols - 1) / kCombineCols, T);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL((combine_kernel<DT_BF16>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((combine_kernel<DT_FP16>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_fp4(const uint8_t* packed, int64_t n_bytes, int dtype, float* out,
                             hipStream_t stream) {
  const int64_t threads = (n_bytes + 3) / 4;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(decode_fp4_kernel<DT_BF16>, grid, dim3(256), 0, stream, packed, n_bytes, out);
  else
    hipLaunchKernelGGL(decode_fp4_kernel<DT_FP16>, grid, dim3(256), 0, stream, packed, n_bytes, out);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t n_bytes, int8_t* out, hipStream_t stream) {
  const int64_t threads = (n_bytes + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(unpack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     packed, n_bytes, out);
  return hipGetLastError();
}

}  // namespace w4moe

namespace w4moe {

hipError_t launch_e8m0_to_h16(const uint8_t* e8m0, int64_t n, int dtype, uint16_t* out,
                              hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(e8m0_kernel<DT_BF16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, e8m0, n, out);
  else
    hipLaunchKernelGGL(e8m0_kernel<DT_FP16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, e8m0, n, out);
  return hipGetLastError();
}

}  // namespace w4moe

namespace w4moe {

hipError_t launch_repack_per_channel(const uint8_t* in, const uint16_t* sc_in, int64_t n_experts,
                                     int n_out, int k_in, uint8_t* out, uint16_t* sc_out,
                                     hipStream_t stream) {
  const int64_t per_e = static_cast<int64_t>(n_out) * (k_in / 2);
  const dim3 grid(static_cast<unsigned>((per_e / 4 + 255) / 256), static_cast<unsigned>(n_experts));
  hipLaunchKernelGGL(repack_pc_kernel, grid, dim3(256), 0, stream, in, sc_in, n_out, k_in, out,
                     sc_out);
  return hipGetLastError();
}

}  // namespace w4moe
