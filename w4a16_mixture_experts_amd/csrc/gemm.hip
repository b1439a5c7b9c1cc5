// gemm.hip -- expert GEMMs, activation epilogues and the FP32 combine of the
// local W4A16 MoE forward on gfx950.
//
// Sources (web pages, cited by tag and section):
//   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
//        Modification: register-side INT4 dequantization, FP32 accumulation,
//        small-batch split-K, route-count-based tile selection.
//        Validation: empty split-K partitions must produce zeros.
//   [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
//        overhead"  Description, "Contract": 16-bit expert outputs combined in
//        FP32 in fixed top-k order before one 16-bit cast, no atomics.
//   [P3] TensorRT-LLM PR #18313, "Add W4A16 per-channel weight-only support
//        for Cutlass fused MoE"  Checkpoint format (packing, per-channel
//        scales) and Validation (gated and non-gated ReLU^2 experts).
//
// Kernels
//   grouped_gemm_kernel  one workgroup = one expert tile of block_m padded
//       route positions x 64 (gated) or 128 output columns over the whole
//       reduction.  UP mode gathers token rows of x and writes the 16-bit
//       activation (SiLU(gate)*up or ReLU^2) in A operand order; DOWN mode
//       reads those rows and writes 16-bit expert outputs Y.
//   combine_kernel       out[t] = cast16(sum_k w[t,k] * Y[slot[t,k]]) in FP32.
//
// Weight streaming: lane (c, g) of a wave reads 16 bytes = one 32-value group
// of weight row c (group layout) at reduction offset 32*g; a 4x4 dword
// transpose across the wave's four 16-lane rows (two permlane swaps each way)
// regroups them so that MFMA j sees group j, lane row g holding its values
// 8g..8g+7.  Each MFMA therefore spans exactly one quantization group.
#include "device.h"
#include "internal.h"

namespace w4moe {

namespace {

__device__ __forceinline__ int a_store_col(int col) { return (col & ~7) | a_pos(col & 7); }

template <int DT>
__device__ __forceinline__ float scale_of(uint32_t pair, int j) {
  return H16<DT>::to_f32((j & 1) ? (pair >> 16) : (pair & 0xffffu));
}

// Raw weights of one subtile for one k-block of 128 (before the transpose).
template <int LAYOUT>
struct BRaw {
  uint32_t d[LAYOUT == Q_GROUP_K ? 4 : 8];
  uint32_t s[2];  // group layout: scales of groups 0..3 of the block, two per dword
};

template <int LAYOUT>
__device__ __forceinline__ void load_b(BRaw<LAYOUT>& b, const uint8_t* brow, const uint16_t* srow,
                                     int k0, int ng, int g, bool on, const void* safe) {
  if constexpr (LAYOUT == Q_GROUP_K) {
    const u32x4 v = load16_if(on && g < ng, brow + (k0 >> 1) + 16 * g, safe);
    b.d[0] = v[0]; b.d[1] = v[1]; b.d[2] = v[2]; b.d[3] = v[3];
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(srow + (k0 >> 5));
    b.s[0] = load4_if(on, sp, safe);
    b.s[1] = load4_if(on && ng > 2, sp + 1, safe);
  } else {
    const bool ok = on && g < ng;
    const u32x4 v0 = load16_if(ok, brow + k0 + 32 * g, safe);
    const u32x4 v1 = load16_if(ok, brow + k0 + 32 * g + 16, safe);
    b.d[0] = v0[0]; b.d[1] = v0[1]; b.d[2] = v0[2]; b.d[3] = v0[3];
    b.d[4] = v1[0]; b.d[5] = v1[1]; b.d[6] = v1[2]; b.d[7] = v1[3];
    b.s[0] = b.s[1] = 0u;
    (void)srow;
  }
}

template <int LAYOUT>
__device__ __forceinline__ void transpose_b(BRaw<LAYOUT>& b) {
  if constexpr (LAYOUT == Q_GROUP_K) {
    transpose_rows4(b.d[0], b.d[1], b.d[2], b.d[3]);
  } else {
    transpose_rows4(b.d[0], b.d[2], b.d[4], b.d[6]);
    transpose_rows4(b.d[1], b.d[3], b.d[5], b.d[7]);
  }
}

// B operand of MFMA j (after transpose_b); par = output column parity for
// the per-channel layout (odd columns live in the high nibbles).
template <int DT, int LAYOUT>
__device__ __forceinline__ u32x4 b_operand(const BRaw<LAYOUT>& b, int j, int par) {
  if constexpr (LAYOUT == Q_GROUP_K) {
    return nibbles_to_h16<DT>(b.d[j]);
  } else {
    const int sh = 4 * par;
    return bytes_to_h16<DT>(b.d[2 * j] >> sh, b.d[2 * j + 1] >> sh);
  }
}

__device__ __forceinline__ u32x4 zero4() {
  u32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

}  // namespace

template <int DT, int LAYOUT, int MS, int MODE>
__global__ void __launch_bounds__(256)
grouped_gemm_kernel(const GemmParams p) {
  using T = H16<DT>;
  constexpr int NSUB = 2;
  constexpr bool UP = MODE != MODE_DOWN;

  const int mt = blockIdx.y;
  const int total = p.offsets[p.E];
  if (mt * p.bm >= total) return;  // whole workgroup: tiles past the padded total
  const int e = p.tile_expert[mt];
  const int nt = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;

  // this wave's two weight-row subtiles and the output column of this lane
  int col[NSUB], wrow[NSUB];
  bool on[NSUB];
  if constexpr (MODE == MODE_UP_GATED) {
    const int i0 = nt * kWgColsGated + w * 16;
    on[0] = on[1] = i0 < p.n_cols;
    col[0] = col[1] = i0 + c;
    wrow[0] = i0 + c;
    wrow[1] = p.up_rows + i0 + c;
  } else {
    const int n0 = nt * kWgColsPlain + w * 32;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      on[s] = n0 + 16 * s < p.n_cols;
      col[s] = n0 + 16 * s + c;
      wrow[s] = col[s];
    }
  }
  const int par = c & 1;

  const uint8_t* wq_e = p.wq + static_cast<int64_t>(e) * p.wq_expert_bytes;
  const uint16_t* ws_e = p.ws + static_cast<int64_t>(e) * p.ws_expert_elems;
  const uint8_t* brow[NSUB];
  const uint16_t* srow[NSUB];
  float scol[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    if constexpr (LAYOUT == Q_GROUP_K) {
      brow[s] = wq_e + static_cast<int64_t>(wrow[s]) * (p.K >> 1);
      srow[s] = ws_e + static_cast<int64_t>(wrow[s]) * (p.K >> 5);
      scol[s] = 0.0f;
    } else {
      brow[s] = wq_e + static_cast<int64_t>(wrow[s] >> 1) * p.K;
      srow[s] = nullptr;
      scol[s] = on[s] ? T::to_f32(ws_e[wrow[s]]) : 0.0f;
    }
  }

  // A rows: position p_row of the tile -> token row of x (UP) or act row (DOWN)
  const int row_base = mt * p.bm;
  const uint16_t* arow[MS];
  bool ms_on[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int prow = row_base + 16 * ms + c;
    const int r = p.sorted[prow];
    if (r >= 0) {
      arow[ms] = UP ? p.a + static_cast<int64_t>(r / p.top_k) * p.lda
                    : p.a + static_cast<int64_t>(prow) * p.lda;
    } else {
      arow[ms] = nullptr;
    }
    ms_on[ms] = __ballot(r >= 0) != 0ull;
  }

  f32x4 acc[MS][NSUB];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[ms][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 bconst;
  bconst[0] = bconst[1] = bconst[2] = bconst[3] = T::kNegOneHalf2;
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};

  const int kb = 0;
  const int ke = p.K;

  BRaw<LAYOUT> bnext[NSUB];
  if (kb < ke) {
    const int ng0 = min(4, (ke - kb) >> 5);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) load_b<LAYOUT>(bnext[s], brow[s], srow[s], kb, ng0, g, on[s], p.wq);
  }

  for (int k0 = kb; k0 < ke; k0 += 128) {
    const int ng = min(4, (ke - k0) >> 5);
    BRaw<LAYOUT> bcur[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) bcur[s] = bnext[s];
    // prefetch the next block's weights while this one is computed
    const int k1 = k0 + 128;
    if (k1 < ke) {
      const int ng1 = min(4, (ke - k1) >> 5);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) load_b<LAYOUT>(bnext[s], brow[s], srow[s], k1, ng1, g, on[s], p.wq);
    }
    // activation fragments of this block
    u32x4 av[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = load16_if(arow[ms] != nullptr && j < ng, arow[ms] + k0 + 32 * j + 8 * g, p.a);
        av[ms][j] = UP ? permute_a(v) : v;
      }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) transpose_b<LAYOUT>(bcur[s]);

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= ng) break;
      u32x4 bh[NSUB];
      float sc[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        bh[s] = b_operand<DT, LAYOUT>(bcur[s], j, par);
        if constexpr (LAYOUT == Q_GROUP_K) sc[s] = scale_of<DT>(bcur[s].s[j >> 1], j);
        else sc[s] = scol[s];
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        if (!ms_on[ms]) continue;
        const f32x4 corr = T::mfma(av[ms][j], bconst, fzero);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          if (!on[s]) continue;
          const f32x4 t = T::mfma(av[ms][j], bh[s], corr);
          acc[ms][s][0] = fmaf(sc[s], t[0], acc[ms][s][0]);
          acc[ms][s][1] = fmaf(sc[s], t[1], acc[ms][s][1]);
          acc[ms][s][2] = fmaf(sc[s], t[2], acc[ms][s][2]);
          acc[ms][s][3] = fmaf(sc[s], t[3], acc[ms][s][3]);
        }
      }
    }
  }

  // values of this lane: rows row_base + 16ms + 4g + i, columns col[s]
  float val[MS][NSUB][4];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) val[ms][s][i] = 16.0f * acc[ms][s][i];

  bool valid[MS][4];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) valid[ms][i] = p.sorted[row_base + 16 * ms + 4 * g + i] >= 0;

  // epilogue
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t prow = row_base + 16 * ms + 4 * g + i;
      uint16_t* orow = p.out + prow * p.ldo;
      if constexpr (MODE == MODE_UP_GATED) {
        if (on[0]) {
          const float a = valid[ms][i] ? silu(val[ms][0][i]) * val[ms][1][i] : 0.0f;
          orow[a_store_col(col[0])] = T::from_f32(a);
        }
      } else if constexpr (MODE == MODE_UP_RELU2) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          if (!on[s]) continue;
          const float h = fmaxf(val[ms][s][i], 0.0f);
          orow[a_store_col(col[s])] = T::from_f32(valid[ms][i] ? h * h : 0.0f);
        }
      } else {
        if (valid[ms][i]) {
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            if (on[s]) orow[col[s]] = T::from_f32(val[ms][s][i]);
        }
      }
    }
}

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
      const auto ry = make_rsrc(p.y + static_cast<int64_t>(ok ? pos[k] : 0) * p.H,
                                ok ? static_cast<uint32_t>(2 * p.H) : 0u);
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int DT, int LAYOUT, int MODE>
static hipError_t launch_gg_ms(const GemmParams& p, int ms, dim3 grid, hipStream_t st) {
  switch (ms) {
    case 1: hipLaunchKernelGGL((grouped_gemm_kernel<DT, LAYOUT, 1, MODE>), grid, dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((grouped_gemm_kernel<DT, LAYOUT, 2, MODE>), grid, dim3(256), 0, st, p); break;
    case 4: hipLaunchKernelGGL((grouped_gemm_kernel<DT, LAYOUT, 4, MODE>), grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT, int LAYOUT>
static hipError_t launch_gg_mode(const GemmParams& p, int ms, int mode, dim3 grid, hipStream_t st) {
  switch (mode) {
    case MODE_UP_GATED: return launch_gg_ms<DT, LAYOUT, MODE_UP_GATED>(p, ms, grid, st);
    case MODE_UP_RELU2: return launch_gg_ms<DT, LAYOUT, MODE_UP_RELU2>(p, ms, grid, st);
    case MODE_DOWN: return launch_gg_ms<DT, LAYOUT, MODE_DOWN>(p, ms, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_grouped_gemm(const GemmParams& p, int dtype, int layout, int ms, int mode,
                               int max_tiles, hipStream_t stream) {
  const dim3 grid(p.n_tiles, max_tiles);
  if (dtype == DT_BF16) {
    return layout == Q_GROUP_K ? launch_gg_mode<DT_BF16, Q_GROUP_K>(p, ms, mode, grid, stream)
                               : launch_gg_mode<DT_BF16, Q_PER_CHANNEL>(p, ms, mode, grid, stream);
  }
  return layout == Q_GROUP_K ? launch_gg_mode<DT_FP16, Q_GROUP_K>(p, ms, mode, grid, stream)
                             : launch_gg_mode<DT_FP16, Q_PER_CHANNEL>(p, ms, mode, grid, stream);
}

hipError_t launch_combine(const CombineParams& p, int dtype, int T, hipStream_t stream) {
  const dim3 grid((p.H + kCombineCols - 1) / kCombineCols, T);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL((combine_kernel<DT_BF16>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((combine_kernel<DT_FP16>), grid, dim3(256), 0, stream, p);
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
