// tile.hip -- grouped expert GEMMs for larger batches (route-prepared tiles).
//
// Sources (web pages, cited by tag and section):
//   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
//        Modification: register-side INT4 dequantization with 16-bit
//        activations in shared memory and FP32 accumulation; multi-stage
//        buffering of the operand loads.
//   [P3] TensorRT-LLM PR #18313, "Add W4A16 per-channel weight-only support
//        for Cutlass fused MoE"  Checkpoint format and Validation (gated and
//        non-gated ReLU^2 experts).
//
// tile_gemm_kernel: one workgroup = one expert tile of up to 64 route
// positions (four 16-row subtiles; empty subtiles are skipped) x 64 (gated:
// 64 gate + 64 up weight rows) or 128 output columns, over the whole
// reduction, in 128-wide blocks:
//   - the tile's activation rows for block b+1 are loaded while block b is
//     computed (one 32-value group per thread) and staged in a double-buffered
//     LDS tile, already in A operand order; UP mode gathers token rows of x,
//     DOWN mode reads the activation rows of the tile's positions;
//   - each wave streams its two 16-row weight subtiles with the lane layout
//     described in device.h (16 bytes per lane = one quantization group,
//     a 4x4 dword transpose across lane rows), prefetched one block ahead;
//   - MFMA j of a block spans one quantization group: exact dequantization,
//     the group scale applied to the FP32 result;
//   - one barrier per block.
// Epilogue: UP writes the 16-bit activation (SiLU(gate)*up or ReLU^2) in A
// operand order; DOWN writes the 16-bit expert outputs Y.
#include "device.h"
#include "internal.h"

namespace w4moe {

namespace {

constexpr int kTileMs = kTileRows / 16;      // 16-row subtiles
constexpr int kTileThreads = 256;            // 4 waves
constexpr int kAStride = 128 + 8;            // staged row stride (16 B padding)

template <int DT>
__device__ __forceinline__ float scale_lo(uint32_t pair) { return H16<DT>::to_f32(pair & 0xffffu); }
template <int DT>
__device__ __forceinline__ float scale_hi(uint32_t pair) { return H16<DT>::to_f32(pair >> 16); }

template <int LAYOUT>
struct WBlk {
  u32x4 d;                       // group layout: 16 bytes; per-channel: first 16 bytes
  u32x4 d2;                      // per-channel: second 16 bytes
  uint32_t s0, s1;               // group layout: scales of groups 0..3 (two per dword)
};

}  // namespace

// One expert tile with NMS active 16-row subtiles (valid routes come first in
// a tile, so the active subtiles are a prefix).
template <int DT, int LAYOUT, int MODE, int NMS>
__device__ __forceinline__ void tile_run(const GemmParams& p, const int row_base, const int e,
                                         const int nt, uint16_t (*s_a)[kTileRows][kAStride],
                                         float (*s_corr)[4][kTileRows]) {
  using T = H16<DT>;
  constexpr int NSUB = 2;
  constexpr bool UP = MODE != MODE_DOWN;
  constexpr bool GROUP = LAYOUT == Q_GROUP_K;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4, par = c & 1;

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
  const auto rw = make_rsrc(p.wq + static_cast<int64_t>(e) * p.wq_expert_bytes,
                            static_cast<uint32_t>(p.wq_expert_bytes));
  const auto rs = make_rsrc(p.ws + static_cast<int64_t>(e) * p.ws_expert_elems,
                            static_cast<uint32_t>(2 * p.ws_expert_elems));
  uint32_t boff[NSUB], soff[NSUB];
  float scol[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    boff[s] = GROUP ? static_cast<uint32_t>(wrow[s]) * (p.K >> 1)
                    : static_cast<uint32_t>(wrow[s] >> 1) * p.K;
    soff[s] = GROUP ? 2u * static_cast<uint32_t>(wrow[s]) * (p.K >> 5) : 0u;
    scol[s] = GROUP ? 0.0f : T::to_f32(bload4(rs, 2u * (wrow[s] & ~1), on[s]) >> (16 * (wrow[s] & 1)));
  }

  // staging role of this thread: row st_row, 32-value group st_q of each block
  const int st_row = tid >> 2, st_q = tid & 3;
  const int st_r = p.sorted[row_base + st_row];
  const bool st_ok = st_r >= 0;
  const auto ra = UP ? make_rsrc(p.a, p.a_bytes)
                     : make_rsrc(p.a + static_cast<int64_t>(row_base) * p.lda,
                                 static_cast<uint32_t>(2 * kTileRows * p.lda));
  const uint32_t st_off = 2u * static_cast<uint32_t>(UP ? (st_ok ? st_r / p.top_k : 0) : st_row) *
                          static_cast<uint32_t>(p.lda);

  auto load_a = [&](int k0, u32x4 (&v)[4]) {
    const bool ok = st_ok && k0 + 32 * st_q < p.K;
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = bload16(ra, st_off + 2u * (k0 + 32 * st_q + 8 * h), ok);
  };
  // staged activations in A operand order, plus the group's correction
  // -1.5 * sum(a) that turns (24 + q) / 16 back into q / 16
  auto store_a = [&](int buf, const u32x4 (&v)[4]) {
    uint16_t* dst = &s_a[buf][st_row][32 * st_q];
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      *reinterpret_cast<u32x4*>(dst + 8 * h) = UP ? permute_a(v[h]) : v[h];
#pragma unroll
      for (int q = 0; q < 4; ++q) sum = T::dot2_ones(v[h][q], sum);
    }
    s_corr[buf][st_q][st_row] = -1.5f * sum;
  };
  auto load_w = [&](int k0, WBlk<LAYOUT> (&b)[NSUB]) {
    const int ng = k0 < p.K ? min(4, (p.K - k0) >> 5) : 0;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const bool ok = on[s] && g < ng;
      if constexpr (GROUP) {
        b[s].d = bload16(rw, boff[s] + (k0 >> 1) + 16 * g, ok);
        const uint32_t so = soff[s] + 2u * (k0 >> 5);
        b[s].s0 = bload4(rs, so, on[s] && ng > 0);
        b[s].s1 = bload4(rs, so + 4, on[s] && ng > 2);
      } else {
        b[s].d = bload16(rw, boff[s] + k0 + 32 * g, ok);
        b[s].d2 = bload16(rw, boff[s] + k0 + 32 * g + 16, ok);
        b[s].s0 = b[s].s1 = 0u;
      }
    }
  };

  f32x4 acc[NMS][NSUB];
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[ms][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: block 0 of A staged, block 0 of the weights in registers
  {
    u32x4 av[4];
    load_a(0, av);
    store_a(0, av);
  }
  WBlk<LAYOUT> wcur[NSUB];
  load_w(0, wcur);
  __syncthreads();

  const int nblk = (p.K + 127) >> 7;
  for (int blk = 0; blk < nblk; ++blk) {
    const int k0 = blk * 128;
    const int buf = blk & 1;
    // next block (reads nothing past the reduction: those loads are masked)
    u32x4 anext[4];
    WBlk<LAYOUT> wnext[NSUB];
    load_a(k0 + 128, anext);
    load_w(k0 + 128, wnext);
    const int ng = min(4, (p.K - k0) >> 5);
    // weights of this block: transpose so that MFMA j sees group j
    uint32_t d[NSUB][8];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      d[s][0] = wcur[s].d[0]; d[s][1] = wcur[s].d[1]; d[s][2] = wcur[s].d[2]; d[s][3] = wcur[s].d[3];
      if constexpr (GROUP) {
        transpose_rows4(d[s][0], d[s][1], d[s][2], d[s][3]);
      } else {
        d[s][4] = wcur[s].d2[0]; d[s][5] = wcur[s].d2[1]; d[s][6] = wcur[s].d2[2]; d[s][7] = wcur[s].d2[3];
        transpose_rows4(d[s][0], d[s][2], d[s][4], d[s][6]);
        transpose_rows4(d[s][1], d[s][3], d[s][5], d[s][7]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 bop[NSUB];
      float sc[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if constexpr (GROUP) {
          bop[s] = nibbles_to_h16<DT>(d[s][j]);
          const uint32_t pr = (j < 2) ? wcur[s].s0 : wcur[s].s1;
          sc[s] = (j & 1) ? scale_hi<DT>(pr) : scale_lo<DT>(pr);
        } else {
          bop[s] = bytes_to_h16<DT>(d[s][2 * j] >> (4 * par), d[s][2 * j + 1] >> (4 * par));
          sc[s] = scol[s];
        }
        sc[s] = (j < ng && on[s]) ? sc[s] : 0.0f;
      }
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&s_a[buf][16 * ms + c][32 * j + 8 * g]);
        const f32x4 corr = *reinterpret_cast<const f32x4*>(&s_corr[buf][j][16 * ms + 4 * g]);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          const f32x4 t = T::mfma(a, bop[s], corr);
          acc[ms][s][0] = fmaf(sc[s], t[0], acc[ms][s][0]);
          acc[ms][s][1] = fmaf(sc[s], t[1], acc[ms][s][1]);
          acc[ms][s][2] = fmaf(sc[s], t[2], acc[ms][s][2]);
          acc[ms][s][3] = fmaf(sc[s], t[3], acc[ms][s][3]);
        }
      }
    }
    store_a(buf ^ 1, anext);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) wcur[s] = wnext[s];
    __syncthreads();
  }

  // epilogue: lane (c, g) holds rows row_base + 16ms + 4g + i, column col[s]
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t prow = row_base + 16 * ms + 4 * g + i;
      const bool valid = p.sorted[prow] >= 0;
      uint16_t* orow = p.out + prow * p.ldo;
      if constexpr (MODE == MODE_UP_GATED) {
        if (on[0]) {
          const float a = valid ? silu(16.0f * acc[ms][0][i]) * (16.0f * acc[ms][1][i]) : 0.0f;
          orow[(col[0] & ~7) | a_pos(col[0] & 7)] = T::from_f32(a);
        }
      } else if constexpr (MODE == MODE_UP_RELU2) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          if (!on[s]) continue;
          const float h = fmaxf(16.0f * acc[ms][s][i], 0.0f);
          orow[(col[s] & ~7) | a_pos(col[s] & 7)] = T::from_f32(valid ? h * h : 0.0f);
        }
      } else {
        if (valid) {
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            if (on[s]) orow[col[s]] = T::from_f32(16.0f * acc[ms][s][i]);
        }
      }
    }
  }
}

template <int DT, int LAYOUT, int MODE>
__global__ void __launch_bounds__(kTileThreads, 2)
tile_gemm_kernel(const GemmParams p) {
  __shared__ uint16_t s_a[2][kTileRows][kAStride];
  __shared__ float s_corr[2][4][kTileRows];

  const int mt = blockIdx.y;
  const int row_base = mt * kTileRows;
  if (row_base >= p.offsets[p.E]) return;  // whole workgroup: tile past the padded total
  int nms = 0;
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) nms += p.sorted[row_base + 16 * ms] >= 0 ? 1 : 0;
  const int e = p.tile_expert[mt];
  const int nt = blockIdx.x;
  switch (nms) {
    case 1: tile_run<DT, LAYOUT, MODE, 1>(p, row_base, e, nt, s_a, s_corr); break;
    case 2: tile_run<DT, LAYOUT, MODE, 2>(p, row_base, e, nt, s_a, s_corr); break;
    case 3: tile_run<DT, LAYOUT, MODE, 3>(p, row_base, e, nt, s_a, s_corr); break;
    default: tile_run<DT, LAYOUT, MODE, 4>(p, row_base, e, nt, s_a, s_corr); break;
  }
}

template <int DT, int LAYOUT, int MODE>
static hipError_t launch_tile_k(const GemmParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((tile_gemm_kernel<DT, LAYOUT, MODE>), grid, dim3(kTileThreads), 0, st, p);
  return hipGetLastError();
}

template <int DT, int LAYOUT>
static hipError_t launch_tile_mode(const GemmParams& p, int mode, dim3 grid, hipStream_t st) {
  switch (mode) {
    case MODE_UP_GATED: return launch_tile_k<DT, LAYOUT, MODE_UP_GATED>(p, grid, st);
    case MODE_UP_RELU2: return launch_tile_k<DT, LAYOUT, MODE_UP_RELU2>(p, grid, st);
    case MODE_DOWN: return launch_tile_k<DT, LAYOUT, MODE_DOWN>(p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tile_gemm(const GemmParams& p, int dtype, int layout, int mode, int max_tiles,
                            hipStream_t stream) {
  const dim3 grid(p.n_tiles, max_tiles);
  if (dtype == DT_BF16)
    return layout == Q_GROUP_K ? launch_tile_mode<DT_BF16, Q_GROUP_K>(p, mode, grid, stream)
                               : launch_tile_mode<DT_BF16, Q_PER_CHANNEL>(p, mode, grid, stream);
  return layout == Q_GROUP_K ? launch_tile_mode<DT_FP16, Q_GROUP_K>(p, mode, grid, stream)
                             : launch_tile_mode<DT_FP16, Q_PER_CHANNEL>(p, mode, grid, stream);
}

}  // namespace w4moe
