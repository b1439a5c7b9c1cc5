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
// tile_gemm_kernel: one workgroup (8 waves) = one expert tile of up to 64
// route positions (four 16-row subtiles; empty subtiles are skipped) x 256
// weight rows (gated: 128 gate + 128 up rows = 128 activation columns;
// otherwise 256 output columns), over the whole reduction in 128-wide blocks:
//   - the tile's activation rows are staged in LDS in A operand order, two
//     128-blocks per stage and two stages: while blocks 2s and 2s+1 are
//     computed, blocks 2s+2 and 2s+3 (loaded one step earlier, 16 values
//     per thread and block) are written to the other stage; UP mode gathers
//     token rows of x, DOWN mode reads the activation rows of the tile's
//     positions;
//   - each wave streams its two 16-row weight subtiles with the lane layout
//     described in device.h (16 bytes per lane = one quantization group,
//     a 4x4 dword transpose across lane rows), prefetched half a step ahead;
//   - group scales: for a tile of one active subtile, the 256 rows' scales
//     staged in LDS (the whole reduction, or phases of 112 groups);
//     otherwise fetched with the weights, 16 bytes per row and block pair;
//   - MFMA j of a block spans one quantization group: exact dequantization,
//     the group scale applied to the FP32 result;
//   - one barrier per two blocks.
// The activation tile is as large as the weight block it meets, and the
// workgroups of one tile are launched onto one XCD one after another (the
// dispatcher deals consecutive workgroups to the 8 XCDs in turn), so the
// re-reads of a tile's activations by its column workgroups hit that XCD's L2.
// Epilogue: UP writes the 16-bit activation (SiLU(gate)*up or ReLU^2) in A
// operand order; DOWN writes the 16-bit expert outputs Y.
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace w4moe {

namespace {

constexpr int kTileMs = kTileRows / 16;      // 16-row subtiles
constexpr int kTileThreads = 64 * kTileWaves;
constexpr int kAStride = 128 + 8;            // staged row stride (16 B padding)
constexpr int kXcds = 8;
constexpr int kNsub = 2;                     // 16-row weight subtiles per wave
constexpr int kSplitkRing = 4;               // split-K: weight blocks in registers
constexpr int kSplitkXLoads = 10;            // split-K: staged x chunks per thread (cb <= 19)
constexpr int kSplitkScLoads = 10;           // split-K: 8-byte scale loads per lane (32 rows x cb <= 640)
// Streaming tile kernel LDS: activations in two stages of two 128-blocks,
// then (group layout) the group scales of the workgroup's 256 weight rows:
// the whole reduction when it fits beside the stages (K / 32 <=
// kScWholeGroups), else phases of kScPhaseGroups groups (K / 32 a multiple of
// 8 then, so that a row's share of a phase is whole 16-byte chunks).
constexpr int kStageElems = kTileRows * kAStride;  // one staged 128-block
constexpr int kScWholeGroups = 176;                // 4 blocks + 2 * 256 * 176 B + 16 <= 160 KiB
constexpr int kScWholeLoads = 256 * kScWholeGroups * 2 / 16 / kTileThreads;  // 16-byte chunks per thread
constexpr int kScPhaseGroups = 112;                // 28 blocks
constexpr int kScPhaseLoads = 256 * kScPhaseGroups * 2 / 16 / kTileThreads;
static_assert(kScWholeLoads * 16 * kTileThreads == 256 * kScWholeGroups * 2, "whole chunks");
static_assert(kScPhaseLoads * 16 * kTileThreads == 256 * kScPhaseGroups * 2, "phase chunks");
static_assert(kScPhaseGroups % 8 == 0, "a phase is whole 128-block pairs");
inline bool tile_scales_in_lds(int layout, int K) {
  return is_group(layout) && (K / 32 <= kScWholeGroups || (K / 32) % 8 == 0);
}
inline size_t tile_lds_bytes(bool scl, int K) {
  size_t b = sizeof(uint16_t) * 4 * kStageElems;
  if (scl) b += sizeof(uint16_t) * 256 * (K / 32 <= kScWholeGroups ? K / 32 : kScPhaseGroups) + 16;
  return b;
}

template <int DT>
__device__ __forceinline__ float scale_lo(uint32_t pair) { return H16<DT>::to_f32(pair & 0xffffu); }
template <int DT>
__device__ __forceinline__ float scale_hi(uint32_t pair) { return H16<DT>::to_f32(pair >> 16); }

// acc += s * t for every output of a group (s: this lane's column scale);
// NI = 1: only element 0 of each lane (rows 0, 4, 8 and 12 of a subtile
// whose routes sit there), the other rows' products are never used
template <int NMS, int NSUB, int NI = 4>
__device__ __forceinline__ void scale_accumulate(f32x4 (&acc)[NMS][NSUB],
                                                 const f32x4 (&t)[NMS][NSUB],
                                                 const float (&sc)[NSUB]) {
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[ms][s][i] = fmaf(sc[s], t[ms][s][i], acc[ms][s][i]);
}

// One 128-wide reduction block of one 16-row weight subtile, as one lane holds
// it: group layout: 16 bytes (one quantization group of the lane's row) and
// the 4 group scales of the row; per-channel: 32 bytes and the dword holding
// the row's scale.
template <int LAYOUT>
struct WBlk {
  u32x4 d;
  u32x4 d2;                      // per-channel only
  uint32_t s0, s1;               // scales of this block (group layout: 4 groups)
  uint32_t s2, s3;               // group layout, first block of a pair: the next block's
};

// How a block's group scales arrive.  Each row's scales of a 128-block are 8
// bytes; fetched per block, every scale load of a wave touches 16 cache lines
// for 128 useful bytes, and that dominated the weight stream.  So blocks come
// in pairs: the first block of a pair loads 16 bytes (both blocks' scales) and
// hands the second half to its partner (pass_scales).  SC_NONE loads no
// scales: the streaming tile kernel reads them from LDS.
enum : int { SC_SINGLE = 0, SC_PAIR_FIRST = 1, SC_PAIR_SECOND = 2, SC_NONE = 3 };

// One expert's packed weights and scales (wave-uniform), and where a wave's
// NSUB subtiles sit in them (per lane).
struct WExpert {
  __amdgpu_buffer_rsrc_t rw, rs;
};
template <int NSUB = kNsub>
struct WSrc {
  uint32_t boff[NSUB], soff[NSUB];
  bool on[NSUB];
};

__device__ __forceinline__ WExpert make_wexpert(const GemmParams& p, int e) {
  WExpert x;
  x.rw = make_rsrc(p.wq + static_cast<int64_t>(e) * p.wq_expert_bytes,
                   static_cast<uint32_t>(p.wq_expert_bytes));
  x.rs = make_rsrc(p.ws + static_cast<int64_t>(e) * p.ws_expert_elems,
                   static_cast<uint32_t>(2 * p.ws_expert_elems));
  return x;
}

template <int LAYOUT, int NSUB = kNsub>
__device__ __forceinline__ WSrc<NSUB> make_wsrc(int K, const int (&wrow)[NSUB],
                                                const bool (&on)[NSUB]) {
  constexpr bool GROUP = is_group(LAYOUT);
  WSrc<NSUB> w;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    w.on[s] = on[s];
    w.boff[s] = GROUP ? static_cast<uint32_t>(wrow[s]) * (K >> 1)
                      : static_cast<uint32_t>(wrow[s] >> 1) * K;
    w.soff[s] = GROUP ? 2u * static_cast<uint32_t>(wrow[s]) * (K >> 5)
                      : 2u * static_cast<uint32_t>(wrow[s] & ~1);
  }
  return w;
}

// Loads of block k0 (reads nothing past the reduction or the output rows:
// those lanes get zeros, scales included).
template <int LAYOUT, int NSUB = kNsub, int SC = SC_SINGLE>
__device__ __forceinline__ void load_wblk(const WExpert& x, const WSrc<NSUB>& w, int k0, int K,
                                          int g, WBlk<LAYOUT> (&b)[NSUB]) {
  const int ng = k0 < K ? min(4, (K - k0) >> 5) : 0;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const bool ok = w.on[s] && g < ng;
    if constexpr (is_group(LAYOUT)) {
      b[s].d = bload16(x.rw, w.boff[s] + (k0 >> 1) + 16 * g, ok);
      const uint32_t so = w.soff[s] + 2u * (k0 >> 5);
      if constexpr (SC == SC_PAIR_FIRST) {
        // groups past the reduction in the window only ever meet A zeros
        const u32x4 v = bload16(x.rs, so, w.on[s] && ng > 0);
        b[s].s0 = v[0]; b[s].s1 = v[1]; b[s].s2 = v[2]; b[s].s3 = v[3];
      } else if constexpr (SC == SC_SINGLE) {
        b[s].s0 = bload4(x.rs, so, w.on[s] && ng > 0);
        b[s].s1 = bload4(x.rs, so + 4, w.on[s] && ng > 2);
      }
    } else {
      b[s].d = bload16(x.rw, w.boff[s] + k0 + 32 * g, ok);
      b[s].d2 = bload16(x.rw, w.boff[s] + k0 + 32 * g + 16, ok);
      b[s].s0 = bload4(x.rs, w.soff[s], w.on[s] && ng > 0);
      b[s].s1 = 0u;
    }
  }
}

template <int LAYOUT, int NSUB>
__device__ __forceinline__ void pass_scales(const WBlk<LAYOUT> (&first)[NSUB],
                                            WBlk<LAYOUT> (&second)[NSUB]) {
  if constexpr (is_group(LAYOUT)) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      second[s].s0 = first[s].s2;
      second[s].s1 = first[s].s3;
    }
  }
}

// acc += A[rows 0..16*NMS) x deq(W block)^T for one 128-block.  `sa` points
// at LDS element (row 0, first column of the block), rows `stride` apart.
// All A fragments are read first (LDS latency paid once per block); the
// correction -1.5 * sum(a) of each group comes from one MFMA against a
// constant operand.
template <int DT, int LAYOUT, int NMS, bool UPFRONT = true, int NSUB = kNsub, int NI = 4>
__device__ __forceinline__ void mma_block(const uint16_t* sa, int stride,
                                          const WBlk<LAYOUT> (&wb)[NSUB],
                                          f32x4 (&acc)[NMS][NSUB], int c, int g, int par) {
  using T = H16<DT>;
  constexpr bool GROUP = is_group(LAYOUT);
  // scheduling fences keep the compiler from hoisting the LDS reads of later
  // blocks (or, without UPFRONT, of later groups) into this one, which would
  // hold every fragment live at once
  __builtin_amdgcn_sched_barrier(0);
  const u32x4 bconst = {T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2};
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  auto frag = [&](int ms, int j) {
    return *reinterpret_cast<const u32x4*>(sa + (16 * ms + c) * stride + 32 * j + 8 * g);
  };
  u32x4 af[NMS][4];
  if constexpr (UPFRONT) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms) af[ms][j] = frag(ms, j);
  }
  // transpose so that MFMA j sees group j
  uint32_t d[NSUB][8];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    d[s][0] = wb[s].d[0]; d[s][1] = wb[s].d[1]; d[s][2] = wb[s].d[2]; d[s][3] = wb[s].d[3];
    if constexpr (GROUP) {
      transpose_rows4(d[s][0], d[s][1], d[s][2], d[s][3]);
    } else {
      d[s][4] = wb[s].d2[0]; d[s][5] = wb[s].d2[1]; d[s][6] = wb[s].d2[2]; d[s][7] = wb[s].d2[3];
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
        bop[s] = group_to_h16<DT, LAYOUT>(d[s][j]);
        const uint32_t pr = (j < 2) ? wb[s].s0 : wb[s].s1;
        sc[s] = (j & 1) ? scale_hi<DT>(pr) : scale_lo<DT>(pr);
      } else {
        bop[s] = bytes_to_h16<DT>(d[s][2 * j] >> (4 * par), d[s][2 * j + 1] >> (4 * par));
        sc[s] = par ? scale_hi<DT>(wb[s].s0) : scale_lo<DT>(wb[s].s0);
      }
      // no mask needed: a group past the reduction or a column past the
      // output reads scale 0 (out-of-range load) and A rows of zeros
    }
    f32x4 t[NMS][NSUB];
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms) {
      const u32x4 a = UPFRONT ? af[ms][j] : frag(ms, j);
      // INT4: the -1.5 * sum(a) term of the (24 + q) / 16 encoding; FP4 needs none
      const f32x4 corr = LAYOUT == Q_FP4_GROUP_K ? fzero : T::mfma(a, bconst, fzero);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) t[ms][s] = T::mfma(a, bop[s], corr);
    }
    scale_accumulate<NMS, NSUB, NI>(acc, t, sc);
    if constexpr (!UPFRONT) __builtin_amdgcn_sched_barrier(0);
  }
}

// mma_block with the group scales taken from the first block of the pair
// (`second` selects its upper half); per-channel layouts use wb's own scale.
template <int DT, int LAYOUT, int NMS, int NSUB, int NI = 4>
__device__ __forceinline__ void mma_block2(const uint16_t* sa, int stride,
                                           const WBlk<LAYOUT> (&wb)[NSUB],
                                           const WBlk<LAYOUT> (&wsc)[NSUB], int second,
                                           f32x4 (&acc)[NMS][NSUB], int c, int g, int par) {
  using T = H16<DT>;
  constexpr bool GROUP = is_group(LAYOUT);
  __builtin_amdgcn_sched_barrier(0);
  const u32x4 bconst = {T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2, T::kNegOneHalf2};
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  u32x4 af[NMS][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
      af[ms][j] = *reinterpret_cast<const u32x4*>(sa + (16 * ms + c) * stride + 32 * j + 8 * g);
  uint32_t d[NSUB][8];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    d[s][0] = wb[s].d[0]; d[s][1] = wb[s].d[1]; d[s][2] = wb[s].d[2]; d[s][3] = wb[s].d[3];
    if constexpr (GROUP) {
      transpose_rows4(d[s][0], d[s][1], d[s][2], d[s][3]);
    } else {
      d[s][4] = wb[s].d2[0]; d[s][5] = wb[s].d2[1]; d[s][6] = wb[s].d2[2]; d[s][7] = wb[s].d2[3];
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
        bop[s] = group_to_h16<DT, LAYOUT>(d[s][j]);
        const uint32_t pr = second ? ((j < 2) ? wsc[s].s2 : wsc[s].s3)
                                   : ((j < 2) ? wsc[s].s0 : wsc[s].s1);
        sc[s] = (j & 1) ? scale_hi<DT>(pr) : scale_lo<DT>(pr);
      } else {
        bop[s] = bytes_to_h16<DT>(d[s][2 * j] >> (4 * par), d[s][2 * j + 1] >> (4 * par));
        sc[s] = par ? scale_hi<DT>(wb[s].s0) : scale_lo<DT>(wb[s].s0);
      }
    }
    f32x4 t[NMS][NSUB];
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms) {
      const f32x4 corr = LAYOUT == Q_FP4_GROUP_K ? fzero : T::mfma(af[ms][j], bconst, fzero);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) t[ms][s] = T::mfma(af[ms][j], bop[s], corr);
    }
    scale_accumulate<NMS, NSUB, NI>(acc, t, sc);
  }
}

// Exact dequantization to fp16 for bf16 activations and bf16 group scales.
//   A bf16 activation converts to fp16 exactly when its magnitude is below
//   2^16 (fp16 carries more significand bits; values below 2^-17 lose low
//   bits, an error under 2^-24); the conversion rounds to nearest, so a
//   magnitude of 2^16 or more (no bf16 value lies between fp16's largest
//   65504 and 65520) becomes an infinity, which makes the tile's accumulators
//   non-finite (an infinity times a zero weight is NaN).  Such a tile is
//   rerun with the per-group form (tile_redo_kernel), which also gives
//   infinite or NaN activations their plain meaning.  q * s, with q in [-8, 7] and a bf16
//   scale s, has at most 3 + 8 significant bits, so it is exact in fp16 as
//   well when 2^-17 <= |s| <= 2720 (or s = 0): its lowest bit is then at
//   least 2^-24, and 16s and 24s are exact fp16 values.  It is formed per
//   value pair as one fused multiply-add (24 + q)/16 * 16s - 24s whose exact
//   result is representable.  A scale outside that range (or an infinity or
//   NaN) marks the tile for the same rerun.  The MFMA then accumulates
//   x * (q s) over every group in FP32: no per-group scaling and no
//   correction term.
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  // round to nearest (one packed conversion)
  const f16x2 r = {static_cast<_Float16>(__uint_as_float(v << 16)),
                   static_cast<_Float16>(__uint_as_float(v & 0xffff0000u))};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
  r[0] = bf16x2_to_f16x2(v[0]);
  r[1] = bf16x2_to_f16x2(v[1]);
  r[2] = bf16x2_to_f16x2(v[2]);
  r[3] = bf16x2_to_f16x2(v[3]);
  return r;
}
// (24 + q)/16 * 16s - 24s for one pair.  The operand comes in by value: a
// bit cast applied directly to a vector element was compiled as a cast of
// element 0 for every element.
__device__ __forceinline__ uint32_t dequant_pair_f16(uint32_t q2, f16x2 s16, f16x2 m24) {
  const f16x2 qv = __builtin_bit_cast(f16x2, q2);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qv, s16, m24));
}

// bf16 magnitudes (sign cleared) of the group scales the fp16 route takes:
// 0, and 2^-17 (0x3700) to 2720 (0x452A); q * 0 is exact, so all-zero
// groups (zero-padded or pruned weights) stay on the route
constexpr uint32_t kX16ScaleLo = 0x3700u;
constexpr uint32_t kX16ScaleEnd = 0x452Bu;

// acc += A[rows 0..16*NMS) x deq(W block)^T for one 128-block with the exact
// fp16 dequantization above (A staged as fp16; group layout, bf16 scales in
// wb[s].s0 / s1 as for mma_block).  acc holds the plain sum (no factor 16).
// sbad is set if a group scale of the block lies outside the exact range
// (lane g checks group g of its row, so the 64 lanes cover every scale).
template <int NMS, bool UPFRONT = true, int NSUB = kNsub>
__device__ __forceinline__ void mma_block_x(const uint16_t* sa, int stride,
                                            const WBlk<Q_GROUP_K> (&wb)[NSUB],
                                            f32x4 (&acc)[NMS][NSUB], int c, int g, bool& sbad) {
  __builtin_amdgcn_sched_barrier(0);
  auto frag = [&](int ms, int j) {
    return *reinterpret_cast<const u32x4*>(sa + (16 * ms + c) * stride + 32 * j + 8 * g);
  };
  u32x4 af[NMS][4];
  if constexpr (UPFRONT) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms) af[ms][j] = frag(ms, j);
  }
  uint32_t d[NSUB][4];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    d[s][0] = wb[s].d[0]; d[s][1] = wb[s].d[1]; d[s][2] = wb[s].d[2]; d[s][3] = wb[s].d[3];
    transpose_rows4(d[s][0], d[s][1], d[s][2], d[s][3]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 bop[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const uint32_t pr = (j < 2) ? wb[s].s0 : wb[s].s1;
      const float sf = (j & 1) ? __uint_as_float(pr & 0xffff0000u) : __uint_as_float(pr << 16);
      const f16x2 s16 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(16.0f * sf, 16.0f * sf));
      const f16x2 m24 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(-24.0f * sf, -24.0f * sf));
      const u32x4 q = nibbles_to_h16<DT_FP16>(d[s][j]);
      bop[s][0] = dequant_pair_f16(q[0], s16, m24);
      bop[s][1] = dequant_pair_f16(q[1], s16, m24);
      bop[s][2] = dequant_pair_f16(q[2], s16, m24);
      bop[s][3] = dequant_pair_f16(q[3], s16, m24);
    }
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms) {
      const u32x4 a = UPFRONT ? af[ms][j] : frag(ms, j);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[ms][s] = H16<DT_FP16>::mfma(a, bop[s], acc[ms][s]);
    }
    if constexpr (!UPFRONT) __builtin_amdgcn_sched_barrier(0);
  }
  // range of the block's group scales, checked after its products are
  // issued (the scales have arrived by then)
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const uint32_t dw = (g & 2) ? wb[s].s1 : wb[s].s0;
    const uint32_t mag = __builtin_amdgcn_ubfe(dw, 16 * (g & 1), 15);
    sbad |= (mag - kX16ScaleLo >= kX16ScaleEnd - kX16ScaleLo) & (mag != 0u);
  }
}

// ---------------------------------------------------------------------------
// Fused finalize: the combine inside the down GEMM launch ([P2] Description:
// fused and non-fused finalize modes; "Contract": the 16-bit expert outputs
// are combined in FP32 in fixed top-k order before one 16-bit cast, with no
// atomic or reduction into the output).  Each down
// workgroup, once its Y rows for output columns [c0, c1) are stored, releases
// them device-wide and counts its routes as arrived, one counter per (token,
// column chunk).  The workgroup whose arrival completes a token's valid
// routes for the chunk acquires and combines that token: acc = sum over k
// ascending of w[t,k] * Y[t*K+k] (valid routes only), cast once.  Which
// workgroup does it changes nothing in the result.  The counters (integer
// atomics) only decide who combines; no value is accumulated atomically.
// ---------------------------------------------------------------------------
// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

template <int DT>
__device__ __forceinline__ void finalize_arrivals(const GemmParams& p, int row_base, int chunk,
                                                  int c0, int c1) {
  using T = H16<DT>;
  __shared__ int s_rows[kTileRows];
  __shared__ int s_nlast;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // release, once per workgroup: every wave waits for its Y stores to reach
  // the L2, then one agent-scope release (on this chip an L2 write-back, the
  // dominant cost of the fused form) makes them visible device-wide before
  // any of the workgroup's routes counts as arrived
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (w == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int route = p.sorted[row_base + lane];
    bool last = false;
    if (route >= 0) {
      const int t = route / p.top_k;
      int nvalid = 0;
      for (int k = 0; k < p.top_k; ++k) nvalid += p.slot[t * p.top_k + k] >= 0 ? 1 : 0;
      const int old = __hip_atomic_fetch_add(p.fin_cnt + static_cast<int64_t>(t) * p.fin_chunks + chunk,
                                             1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = old == nvalid - 1;
    }
    const uint64_t m = __ballot(last);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    if (last) s_rows[__popcll(m & below)] = route / p.top_k;
    if (lane == 0) s_nlast = __popcll(m);
  }
  __syncthreads();
  const int nlast = s_nlast;
  if (nlast == 0) return;
  // acquire: the other workgroups' Y rows of these tokens are visible
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int ng = (c1 - c0) / 8;  // 16-byte column groups of the chunk
  constexpr int kB = 8;          // routes whose Y loads are in flight together
  for (int i = tid; i < nlast * ng; i += kTileThreads) {
    const int t = s_rows[i / ng];
    const int col = c0 + 8 * (i % ng);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < p.top_k; kb += kB) {
      u32x4 v[kB];
      float wk[kB];
      bool ok[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int r = t * p.top_k + kb + k;
        ok[k] = kb + k < p.top_k && p.slot[r] >= 0;
        wk[k] = ok[k] ? p.wts[r] : 0.0f;
        v[k] = ok[k] ? *reinterpret_cast<const u32x4*>(p.out + static_cast<int64_t>(r) * p.ldo + col)
                     : u32x4{0u, 0u, 0u, 0u};
      }
      // fixed order: ascending k, invalid routes contribute nothing
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        if (!ok[k]) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += wk[k] * T::to_f32(v[k][j] & 0xffffu);
          acc[2 * j + 1] += wk[k] * T::to_f32(v[k][j] >> 16);
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = static_cast<uint32_t>(T::from_f32(acc[2 * j])) |
             (static_cast<uint32_t>(T::from_f32(acc[2 * j + 1])) << 16);
    *reinterpret_cast<u32x4*>(p.fin_out + static_cast<int64_t>(t) * p.ldo + col) = o;
  }
}

// Zeros of the output rows of tokens without a valid route (they never
// arrive anywhere): workgroup z takes tokens kFinZeroTokens * z + wave.
__device__ __forceinline__ void finalize_zero_rows(const GemmParams& p, int z) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = z * kFinZeroTokens + w;
  if (t >= p.T) return;  // whole wave
  const bool any = __ballot(lane < p.top_k && p.slot[t * p.top_k + lane] >= 0) != 0ull;
  if (any) return;
  uint16_t* row = p.fin_out + static_cast<int64_t>(t) * p.ldo;
  for (int col = 8 * lane; col < p.n_cols; col += 8 * 64)
    *reinterpret_cast<u32x4*>(row + col) = u32x4{0u, 0u, 0u, 0u};
}

// Valid rows of the lane's 16 * NMS output rows as a bit mask: bit 4ms + i
// stands for tile row 16ms + 4g + i.
template <int NMS>
__device__ __forceinline__ uint32_t valid_rows(const GemmParams& p, int row_base, int g) {
  uint32_t m = 0;
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m |= (p.sorted[row_base + 16 * ms + 4 * g + i] >= 0 ? 1u : 0u) << (4 * ms + i);
  return m;
}

// Epilogue: lane (c, g) holds rows row_base + 16ms + 4g + i of column col[s].
// UP writes the 16-bit activation in A operand order (padding rows get 0)
// through a buffer resource over the tile's 64 rows (masked lanes store
// nothing); DOWN writes the 16-bit expert outputs of valid rows into Y, whose
// rows are indexed by route (t * K + k).
template <int DT, int MODE, int NMS>
__device__ __forceinline__ void store_outputs(const GemmParams& p, int row_base,
                                              const f32x4 (&acc)[NMS][kNsub],
                                              const int (&col)[kNsub], const bool (&on)[kNsub],
                                              int g, uint32_t vmask) {
  using T = H16<DT>;
  const auto ro = make_rsrc(p.out + static_cast<int64_t>(row_base) * p.ldo,
                            static_cast<uint32_t>(2 * kTileRows * p.ldo));
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = (vmask >> (4 * ms + i)) & 1u;
      const uint32_t rowoff = static_cast<uint32_t>((16 * ms + 4 * g + i) * p.ldo);
      if constexpr (MODE == MODE_UP_GATED) {
        const float a = valid ? silu(16.0f * acc[ms][0][i]) * (16.0f * acc[ms][1][i]) : 0.0f;
        bstore2(ro, 2u * (rowoff + ((col[0] & ~7) | a_pos(col[0] & 7))), on[0], T::from_f32(a));
      } else if constexpr (MODE == MODE_UP_RELU2) {
#pragma unroll
        for (int s = 0; s < kNsub; ++s) {
          const float h = fmaxf(16.0f * acc[ms][s][i], 0.0f);
          bstore2(ro, 2u * (rowoff + ((col[s] & ~7) | a_pos(col[s] & 7))), on[s],
                  T::from_f32(valid ? h * h : 0.0f));
        }
      } else {
        // expert outputs are rows of Y by route index (16-bit, H columns)
        const int route = p.sorted[row_base + 16 * ms + 4 * g + i];
        uint16_t* yrow = p.out + static_cast<int64_t>(valid ? route : 0) * p.ldo;
#pragma unroll
        for (int s = 0; s < kNsub; ++s)
          if (on[s] && valid) yrow[col[s]] = T::from_f32(16.0f * acc[ms][s][i]);
      }
    }
  }
}

// Rows and columns of wave w's two subtiles in column tile nt.
template <int MODE>
__device__ __forceinline__ void wave_columns(const GemmParams& p, int nt, int w, int c,
                                             int (&col)[kNsub], int (&wrow)[kNsub],
                                             bool (&on)[kNsub]) {
  if constexpr (MODE == MODE_UP_GATED) {
    const int i0 = nt * kTileColsGated + w * 16;
    on[0] = on[1] = i0 < p.n_cols;
    col[0] = col[1] = i0 + c;
    wrow[0] = i0 + c;
    wrow[1] = p.up_rows + i0 + c;
  } else {
    const int n0 = nt * kTileColsPlain + w * 32;
#pragma unroll
    for (int s = 0; s < kNsub; ++s) {
      on[s] = n0 + 16 * s < p.n_cols;
      col[s] = n0 + 16 * s + c;
      wrow[s] = col[s];
    }
  }
}

// Workgroup L's place in the tile order and its column tile: workgroup L
// runs on XCD L % 8, XCD x takes positions x, x + 8, ... and walks the column
// tiles of each back to back (a tile's activation rows are then read through
// one L2).
__device__ __forceinline__ int tile_position(const GemmParams& p, int L, int& nt) {
  const int q = L / kXcds;
  nt = q % p.n_tiles;
  return kXcds * (q / p.n_tiles) + L % kXcds;
}

// The tile at position k: tile_order[k] with a tile order (the used tiles,
// biggest first), else k; -1 for a position past the used tiles (tile order
// only: one round trip for the padded total and the entry).  Without an
// order a position past the used tiles is found later, from its row base.
__device__ __forceinline__ int tile_at(const GemmParams& p, int k) {
  if (p.tile_order == nullptr) return k;
  const int total = p.offsets[p.E];
  const int o = p.tile_order[min(k, p.tiles - 1)];
  asm volatile("" : : "s"(total), "s"(o));  // both loads in flight together
  return k * kTileRows < total ? o : -1;
}

// Active 16-row subtiles of a tile: valid routes come first, so they are a
// prefix (uniform).
__device__ __forceinline__ int active_subtiles(const GemmParams& p, int row_base) {
  int nms = 0;
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) nms += p.sorted[row_base + 16 * ms] >= 0 ? 1 : 0;
  return nms;
}

}  // namespace

// ---------------------------------------------------------------------------
// Streaming tile kernel: the reduction in steps of two 128-blocks, the
// activations of a step staged into one of two LDS stages (one barrier per
// step).
// ---------------------------------------------------------------------------

// X16: the exact fp16 dequantization (bf16 activations and scales, group
// layout); returns false, with nothing stored, if an accumulator is not
// finite (an activation of magnitude 2^16 or more, an infinity or a NaN),
// true otherwise.
template <int DT, int LAYOUT, int MODE, int NMS, bool SCL, bool X16 = false>
__device__ __forceinline__ bool tile_run(const GemmParams& p, const int row_base, const int e,
                                         const int nt, uint16_t* s_lds, const int st_r) {
  constexpr bool UP = MODE != MODE_DOWN;
  static_assert(!X16 || (DT == DT_BF16 && LAYOUT == Q_GROUP_K && !SCL), "fp16 route");
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4, par = c & 1;

  int col[kNsub], wrow[kNsub];
  bool on[kNsub];
  wave_columns<MODE>(p, nt, w, c, col, wrow, on);
  const WExpert wx = make_wexpert(p, e);
  const WSrc<> ws = make_wsrc<LAYOUT>(p.K, wrow, on);

  // staging role of this thread: row st_row, kVals consecutive values of each
  // 128-block starting at kVals * st_c
  constexpr int kVals = kTileRows * 128 / kTileThreads;  // 32 (4 waves) or 16 (8 waves)
  constexpr int kChunks = kVals / 8;                     // 16-byte loads per thread
  constexpr int kPerRow = 128 / kVals;
  static_assert(kVals == 32 || kVals == 16, "16 or 32 staged values per thread");
  const int st_row = tid / kPerRow, st_c = tid % kPerRow;  // st_r = sorted[row_base + st_row]
  const bool st_ok = st_r >= 0;
  const auto ra = UP ? make_rsrc(p.a, p.a_bytes)
                     : make_rsrc(p.a + static_cast<int64_t>(row_base) * p.lda,
                                 static_cast<uint32_t>(2 * kTileRows * p.lda));
  const uint32_t st_off = 2u * static_cast<uint32_t>(UP ? (st_ok ? st_r / p.top_k : 0) : st_row) *
                          static_cast<uint32_t>(p.lda);
  auto load_a = [&](int k0, u32x4 (&v)[kChunks]) {
    const bool ok = st_ok && k0 + kVals * st_c < p.K;
#pragma unroll
    for (int h = 0; h < kChunks; ++h)
      v[h] = bload16(ra, st_off + 2u * (k0 + kVals * st_c + 8 * h), ok);
  };
  // one block's activations, in A operand order, into staged block `blk`
  auto store_a = [&](uint16_t* blk, const u32x4 (&v)[kChunks]) {
    uint16_t* dst = blk + st_row * kAStride + kVals * st_c;
#pragma unroll
    for (int h = 0; h < kChunks; ++h) {
      const u32x4 a = UP ? permute_a(v[h]) : v[h];
      if constexpr (X16) {
        *reinterpret_cast<u32x4*>(dst + 8 * h) = bf16x8_to_f16x8(a);
      } else {
        *reinterpret_cast<u32x4*>(dst + 8 * h) = a;
      }
    }
  };

  f32x4 acc[NMS][kNsub];
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int s = 0; s < kNsub; ++s) acc[ms][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Group scales in LDS.  A row's scales are contiguous and so are the rows
  // of a range (gated: the 128 gate rows, then the 128 up rows): the whole
  // reduction's scales are one linear copy per range, every load covering
  // whole cache lines (fetched per block from HBM, each scale load touched 16
  // lines for 128 useful bytes).  A phase copies each row's share of the
  // phase, whole 16-byte chunks.
  const int gpr = p.K >> 5;  // groups (scales) per row
  const uint32_t rbytes = 2u * gpr;
  const bool whole = gpr <= kScWholeGroups;
  const int pg = whole ? gpr : kScPhaseGroups;  // LDS scale row stride (groups)
  uint16_t* const s_sc = s_lds + 4 * kStageElems;
  // scale row (within the expert) of the workgroup's weight row r
  auto sc_row = [&](int r) {
    return MODE == MODE_UP_GATED ? (r < 128 ? 0 : p.up_rows - 128) + nt * kTileColsGated + r
                                 : nt * kTileColsPlain + r;
  };
  auto load_whole = [&](u32x4 (&v)[kScWholeLoads]) {
    const int nranges = MODE == MODE_UP_GATED ? 2 : 1;
    const int rrows = MODE == MODE_UP_GATED ? 128 : 256;                   // rows per range
    const uint32_t rchunks = static_cast<uint32_t>(rrows) * rbytes / 16;  // 16-byte chunks per range
#pragma unroll
    for (int i = 0; i < kScWholeLoads; ++i) {
      const uint32_t ch = static_cast<uint32_t>(tid + kTileThreads * i);
      const int rg = ch < rchunks ? 0 : 1;
      const uint32_t lc = ch - rg * rchunks;
      v[i] = bload16(wx.rs, static_cast<uint32_t>(sc_row(rrows * rg)) * rbytes + 16u * lc,
                     rg < nranges && lc < rchunks);
    }
  };
  auto store_whole = [&](const u32x4 (&v)[kScWholeLoads]) {
    const uint32_t nchunks = 256u * rbytes / 16;
#pragma unroll
    for (int i = 0; i < kScWholeLoads; ++i) {
      const uint32_t ch = static_cast<uint32_t>(tid + kTileThreads * i);
      if (ch < nchunks) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(s_sc) + 16u * ch) = v[i];
    }
  };
  // phase ph: groups [kScPhaseGroups * ph, +kScPhaseGroups) of every row
  auto load_phase = [&](int ph, u32x4 (&v)[kScPhaseLoads]) {
    const int g0 = kScPhaseGroups * ph;
    const int cpr = min(gpr - g0, kScPhaseGroups) >> 3;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < kScPhaseLoads; ++i) {
      const int ch = tid + kTileThreads * i;
      const int r = ch / cpr, part = ch - r * cpr;
      v[i] = bload16(wx.rs, static_cast<uint32_t>(sc_row(r)) * rbytes + 2u * g0 + 16u * part,
                     r < 256);
    }
  };
  auto store_phase = [&](int ph, const u32x4 (&v)[kScPhaseLoads]) {
    const int cpr = min(gpr - kScPhaseGroups * ph, kScPhaseGroups) >> 3;
#pragma unroll
    for (int i = 0; i < kScPhaseLoads; ++i) {
      const int ch = tid + kTileThreads * i;
      const int r = ch / cpr, part = ch - r * cpr;
      if (r < 256)
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(s_sc) + 2 * kScPhaseGroups * r +
                                  16 * part) = v[i];
    }
  };
  // LDS rows of this lane's two weight rows; scales of block bp of the phase
  int lrow[kNsub];
#pragma unroll
  for (int s2 = 0; s2 < kNsub; ++s2)
    lrow[s2] = MODE == MODE_UP_GATED ? 128 * s2 + 16 * w + c : 32 * w + 16 * s2 + c;
  auto set_scales = [&](int bp, WBlk<LAYOUT> (&b)[kNsub]) {
#pragma unroll
    for (int s2 = 0; s2 < kNsub; ++s2) {
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(s_sc + lrow[s2] * pg + 4 * bp);
      b[s2].s0 = sp[0];
      b[s2].s1 = sp[1];
    }
  };

  // Pipeline.  Step s computes blocks 2s and 2s + 1 from stage s & 1 while
  // the other stage receives blocks 2s + 2 and 2s + 3 (loaded one step
  // earlier) and blocks 2s + 4 and 2s + 5 are requested.  Weights: a ring
  // of two register sets, a block requested half a step before it is used
  // (without LDS scales the pair's first block fetches both blocks' scales).
  // Steps past the last block only issue masked loads.
  constexpr int SC_FIRST = SCL ? SC_NONE : SC_PAIR_FIRST;
  constexpr int SC_SECOND = SCL ? SC_NONE : SC_PAIR_SECOND;
  WBlk<LAYOUT> wr[2][kNsub];
  u32x4 an[2][kChunks];
  bool sbad = false;  // X16: a group scale outside the route's exact range
  const int nblk = (p.K + 127) >> 7;
  const int nsteps = (nblk + 1) >> 1;
  auto step = [&](int s, int pb0) {  // pb0: first block of the scale phase
    const int b = 2 * s;
    const uint16_t* sx = s_lds + 2 * kStageElems * (s & 1);
    uint16_t* sy = s_lds + 2 * kStageElems * ((s & 1) ^ 1);
    load_wblk<LAYOUT, kNsub, SC_SECOND>(wx, ws, 128 * (b + 1), p.K, g, wr[1]);
    if constexpr (SCL) set_scales(b - pb0, wr[0]);
    if constexpr (X16) mma_block_x<NMS>(sx, kAStride, wr[0], acc, c, g, sbad);
    else mma_block<DT, LAYOUT, NMS>(sx, kAStride, wr[0], acc, c, g, par);
    if constexpr (!SCL) pass_scales<LAYOUT, kNsub>(wr[0], wr[1]);
    store_a(sy, an[0]);
    store_a(sy + kStageElems, an[1]);
    load_a(128 * (b + 4), an[0]);
    load_a(128 * (b + 5), an[1]);
    load_wblk<LAYOUT, kNsub, SC_FIRST>(wx, ws, 128 * (b + 2), p.K, g, wr[0]);
    if (b + 1 < nblk) {
      if constexpr (SCL) set_scales(b + 1 - pb0, wr[1]);
      if constexpr (X16) mma_block_x<NMS>(sx + kStageElems, kAStride, wr[1], acc, c, g, sbad);
      else mma_block<DT, LAYOUT, NMS>(sx + kStageElems, kAStride, wr[1], acc, c, g, par);
    }
    __syncthreads();
  };

  // prologue: blocks 0 and 1 into stage 0 (with the first scales), blocks 2
  // and 3 requested
  load_a(0, an[0]);
  load_a(128, an[1]);
  load_wblk<LAYOUT, kNsub, SC_FIRST>(wx, ws, 0, p.K, g, wr[0]);
  if constexpr (SCL) {
    // the fences keep the compiler from pairing each load with its store
    if (whole) {
      u32x4 v[kScWholeLoads];
      load_whole(v);
      __builtin_amdgcn_sched_barrier(0);
      store_whole(v);
    } else {
      u32x4 v[kScPhaseLoads];
      load_phase(0, v);
      __builtin_amdgcn_sched_barrier(0);
      store_phase(0, v);
    }
  }
  store_a(s_lds, an[0]);
  store_a(s_lds + kStageElems, an[1]);
  load_a(256, an[0]);
  load_a(384, an[1]);
  __syncthreads();

  const int psteps = SCL && !whole ? kScPhaseGroups / 8 : nsteps;  // steps per scale phase
  for (int s0 = 0; s0 < nsteps; s0 += psteps) {
    const int s1 = min(nsteps, s0 + psteps);
    // the next phase's scales are stored after the closing barrier of the
    // phase's last step (no wave reads the old ones any more); the up
    // projections request them before that step, the down projection (whose
    // step holds more registers) after it
    const bool next = SCL && s1 < nsteps;
    for (int s = s0; s < (next ? s1 - 1 : s1); ++s) step(s, 2 * s0);
    if constexpr (SCL) {
      if (next) {
        const int ph = s1 / psteps;
        u32x4 v[kScPhaseLoads];
        if constexpr (UP) {
          load_phase(ph, v);
          __builtin_amdgcn_sched_barrier(0);
          step(s1 - 1, 2 * s0);
        } else {
          step(s1 - 1, 2 * s0);
          load_phase(ph, v);
          __builtin_amdgcn_sched_barrier(0);
        }
        store_phase(ph, v);
        __syncthreads();
      }
    }
  }
  if constexpr (X16) {
    bool bad = false;
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
      for (int s2 = 0; s2 < kNsub; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad |= !__builtin_isfinite(acc[ms][s2][i]);
    if (__syncthreads_or(bad || sbad)) return false;
    // the epilogue applies the per-group form's factor 16 (exact)
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
      for (int s2 = 0; s2 < kNsub; ++s2) acc[ms][s2] *= 0.0625f;
  }
  store_outputs<DT, MODE, NMS>(p, row_base, acc, col, on, g, valid_rows<NMS>(p, row_base, g));
  return true;
}

// The work of tile-kernel workgroup L.  X16: tiles of several subtiles take
// the exact fp16 route; returns false if such a tile must be rerun.
template <int DT, int LAYOUT, int MODE, bool SCL, bool X16>
__device__ __forceinline__ bool tile_work(const GemmParams& p, const int L, uint16_t* s_lds) {
  int nt;
  const int mt = tile_at(p, tile_position(p, L, nt));
  if (mt < 0) return true;  // whole workgroup: position past the used tiles
  const int row_base = mt * kTileRows;
  // every index the workgroup needs comes in one batch of loads before the
  // first decision (a tile past the padded total reads a clamped tile)
  const int rb = min(mt, p.tiles - 1) * kTileRows;
  const int total = p.offsets[p.E];
  const int e = p.tile_expert[rb / kTileRows];
  int first[kTileMs];
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) first[ms] = p.sorted[rb + 16 * ms];
  constexpr int kPerRow = 128 / (kTileRows * 128 / kTileThreads);  // staging threads per row
  const int st_r = p.sorted[rb + static_cast<int>(threadIdx.x) / kPerRow];
  // an empty statement that reads every index keeps the compiler from moving
  // the loads behind the exit below (one round trip instead of several)
  asm volatile("" : : "s"(total), "s"(e), "s"(first[0]), "s"(first[1]), "s"(first[2]), "s"(first[3]),
               "v"(st_r));
  if (row_base >= total) return true;  // whole workgroup: tile past the padded total
  int nms = 0;
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) nms += first[ms] >= 0 ? 1 : 0;
  // LDS scales serve tiles of one active subtile, which stream weights at
  // the memory's pace; with more subtiles the tile is bound by its MFMA and
  // VALU issue, and scales fetched with the weights (per block pair) keep
  // the register count lower and measured faster
  switch (nms) {
    case 1: return tile_run<DT, LAYOUT, MODE, 1, SCL>(p, row_base, e, nt, s_lds, st_r);
    case 2: return tile_run<DT, LAYOUT, MODE, 2, false, X16>(p, row_base, e, nt, s_lds, st_r);
    case 3: return tile_run<DT, LAYOUT, MODE, 3, false, X16>(p, row_base, e, nt, s_lds, st_r);
    default: return tile_run<DT, LAYOUT, MODE, 4, false, X16>(p, row_base, e, nt, s_lds, st_r);
  }
}

template <int DT, int LAYOUT, int MODE, bool SCL, bool X16>
__global__ void __launch_bounds__(kTileThreads)
tile_gemm_kernel(const GemmParams p) {
  // [2 stages][2 blocks][kTileRows][kAStride] activations, then (SCL) the
  // group scales: [256 rows][K / 32] or [256 rows][kScPhaseGroups]
  extern __shared__ __align__(16) uint16_t s_lds[];
  const int L = static_cast<int>(blockIdx.x);
  if constexpr (MODE == MODE_DOWN && !X16) {
    if (p.fin_cnt != nullptr && L >= p.n_main) {  // fused combine: empty tokens' rows
      finalize_zero_rows(p, L - p.n_main);
      return;
    }
  }
  // X16: every workgroup records whether its tile must be rerun (the flag
  // array needs no clearing)
  const bool done = tile_work<DT, LAYOUT, MODE, SCL, X16>(p, L, s_lds);
  if constexpr (X16) {
    if (threadIdx.x == 0) p.redo[blockIdx.x] = done ? 0 : 1;
  }
  if constexpr (MODE == MODE_DOWN && !X16) {
    if (p.fin_cnt != nullptr) {
      // the workgroup's tile and column tile (as tile_work derives them)
      int nt;
      const int mt = tile_at(p, tile_position(p, L, nt));
      const int row_base = mt * kTileRows;
      const int c0 = nt * kTileColsPlain, c1 = min(p.n_cols, c0 + kTileColsPlain);
      if (mt >= 0 && row_base < p.offsets[p.E] && c0 < c1)
        finalize_arrivals<DT>(p, row_base, nt, c0, c1);
    }
  }
}

// Reruns, with the per-group form, the tiles of a fp16-route launch of
// n_wg workgroups whose activations left fp16's range.  Workgroup b owns
// flags b, b + G, b + 2G, ... (G workgroups); each pass reads one flag per
// thread, and only a pass with a flag set walks its flags one by one
// (normally none is: every workgroup makes one pass of loads and exits).
template <int DT, int LAYOUT, int MODE>
__global__ void __launch_bounds__(kTileThreads)
tile_redo_kernel(const GemmParams p, const int n_wg) {
  extern __shared__ __align__(16) uint16_t s_lds[];
  const int G = static_cast<int>(gridDim.x);
  for (int base = static_cast<int>(blockIdx.x); base < n_wg; base += G * kTileThreads) {
    const int L = base + G * static_cast<int>(threadIdx.x);
    const bool f = L < n_wg && p.redo[L] != 0;
    if (!__syncthreads_or(f)) continue;
    for (int i = 0; i < kTileThreads; ++i) {
      const int Li = base + G * i;
      if (Li >= n_wg) break;
      if (p.redo[Li] == 0) continue;  // uniform
      tile_work<DT, LAYOUT, MODE, false, false>(p, Li, s_lds);
      __syncthreads();  // LDS reuse by the next tile
    }
  }
}

// ---------------------------------------------------------------------------
// Down GEMM for short reductions (K <= kResidentK): the tile's activation rows
// stay in LDS for the whole workgroup, which walks p.col_steps column steps of
// 8 x 32 output columns.  Waves never synchronize after the staging; each
// requests the next step's weights while it computes the current one.
// ---------------------------------------------------------------------------

// Expert outputs of one column step leave through the wave's own LDS region
// (rows of 32 columns, stride kOutStride): each lane then stores 16 bytes of
// one row, eight lanes' worth of rows per instruction, instead of a 16-bit
// value per lane per output.
constexpr int kOutStride = 40;  // 16-bit elements per staged row (80 B)

// Activation values i0 .. i0 + 7 of route r from the split-K partials
// [S][R][ld] FP32: the chunks summed in order 0 .. S-1 (four chunks' loads in
// flight at a time), then SiLU(gate) * up (gated: the up values at column
// offset `up` of a partial row) or ReLU^2 (up == 0), one 16-bit rounding
// each; packed in A operand order.  The activation kernel and the resident
// down kernel's staging both form activations here, so their bits agree.
template <int DT>
__device__ __forceinline__ u32x4 act_from_partials(const float* part, int S, int R, int ld,
                                                   int up, int r, int i0) {
  float h[8], u[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = u[j] = 0.0f;
  for (int kb = 0; kb < S; kb += 4) {
    f32x4 a[4][2], b[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j][0] = a[j][1] = b[j][0] = b[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (kb + j < S) {
        const float* row = part + (static_cast<int64_t>(kb + j) * R + r) * ld + i0;
        a[j][0] = *reinterpret_cast<const f32x4*>(row);
        a[j][1] = *reinterpret_cast<const f32x4*>(row + 4);
        if (up > 0) {
          b[j][0] = *reinterpret_cast<const f32x4*>(row + up);
          b[j][1] = *reinterpret_cast<const f32x4*>(row + up + 4);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kb + j < S) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[q] += a[j][0][q];
          h[4 + q] += a[j][1][q];
          u[q] += b[j][0][q];
          u[4 + q] += b[j][1][q];
        }
      }
    }
  }
  uint16_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v;
    if (up > 0) {
      v = silu(h[j]) * u[j];
    } else {
      const float z = fmaxf(h[j], 0.0f);
      v = z * z;
    }
    o[a_pos(j)] = H16<DT>::from_f32(v);
  }
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] = static_cast<uint32_t>(o[2 * q]) | (static_cast<uint32_t>(o[2 * q + 1]) << 16);
  return v;
}

template <int DT, int LAYOUT, int NMS, int NKB, bool PART = false>
__device__ __forceinline__ void down_resident_run(const GemmParams& p, const int row_base,
                                                  const int e, const int chunk, uint16_t* s_ar,
                                                  uint16_t* s_out) {
  constexpr int S = NKB * 128 + 8;   // row stride of the resident tile
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4, par = c & 1;

  // stage the tile's activation rows once (padding rows and columns past K
  // read zeros)
  if constexpr (PART) {
    // from the split-K partials of the gate/up launch.  Rows past the NMS
    // non-empty subtiles hold no route: their passes load nothing.
    constexpr int kPerRow = NKB * 16;                   // 8-value chunks per row
    constexpr int kRowsPer = kTileThreads / kPerRow;    // rows per pass
    constexpr int kIters = kTileRows / kRowsPer;
    static_assert(kTileRows % kRowsPer == 0, "staging passes");
    const int srt = p.sorted[row_base + lane];          // every wave: all 64 rows
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int idx = tid + i * kTileThreads;
      const int row = idx / kPerRow, ch = idx % kPerRow;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kRowsPer * i < 16 * NMS) {
        const int r = __shfl(srt, row, 64);
        if (r >= 0 && 8 * ch < p.K)
          v = act_from_partials<DT>(p.part, p.S, p.R, p.part_ld, p.up_rows, r, 8 * ch);
      }
      *reinterpret_cast<u32x4*>(s_ar + row * S + 8 * ch) = v;
    }
  } else {
    constexpr int kPerRow = NKB * 16;                       // 16-byte chunks per row
    constexpr int kIters = kTileRows * kPerRow / kTileThreads;
    static_assert(kTileRows * kPerRow % kTileThreads == 0, "staging covers the tile");
    const auto ra = make_rsrc(p.a + static_cast<int64_t>(row_base) * p.lda,
                              static_cast<uint32_t>(2 * kTileRows * p.lda));
    u32x4 v[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int idx = tid + i * kTileThreads;
      const int row = idx / kPerRow, ch = idx % kPerRow;
      const bool ok = p.sorted[row_base + row] >= 0 && 8 * ch < p.K;
      v[i] = bload16(ra, 2u * static_cast<uint32_t>(row * p.lda + 8 * ch), ok);
    }
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int idx = tid + i * kTileThreads;
      const int row = idx / kPerRow, ch = idx % kPerRow;
      *reinterpret_cast<u32x4*>(s_ar + row * S + 8 * ch) = v[i];
    }
  }
  __syncthreads();

  const int step_begin = chunk * p.col_steps;
  const int step_end = min(step_begin + p.col_steps, (p.n_cols + kTileColsPlain - 1) / kTileColsPlain);

  const WExpert wx = make_wexpert(p, e);
  const uint32_t vmask = valid_rows<NMS>(p, row_base, g);
  // wave w's columns in step st: st * 256 + 32 w + 16 k + c (k = subtile)
  auto step_src = [&](int st, int (&col)[kNsub], bool (&on)[kNsub]) {
    const int n0 = st * kTileColsPlain + w * 32;
#pragma unroll
    for (int k = 0; k < kNsub; ++k) {
      col[k] = n0 + 16 * k + c;
      on[k] = st < step_end && n0 + 16 * k < p.n_cols;
    }
    return make_wsrc<LAYOUT>(p.K, col, on);
  };
  // two register sets: the next block's weights are requested while the
  // current block is computed
  auto load_blk = [&](int st, int kb, WBlk<LAYOUT> (&wb)[kNsub]) {
    int col[kNsub];
    bool on[kNsub];
    const WSrc<> ws = step_src(st, col, on);
    if constexpr (NKB == 1) load_wblk<LAYOUT, kNsub, SC_SINGLE>(wx, ws, 128 * kb, p.K, g, wb);
    else if (kb == 0) load_wblk<LAYOUT, kNsub, SC_PAIR_FIRST>(wx, ws, 0, p.K, g, wb);
    else load_wblk<LAYOUT, kNsub, SC_PAIR_SECOND>(wx, ws, 128, p.K, g, wb);
  };
  f32x4 acc[NMS][kNsub];
  auto zero_acc = [&]() {
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
      for (int k = 0; k < kNsub; ++k) acc[ms][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // rows of the tile holding a route (bit r: tile row r)
  const uint64_t rows_valid = __ballot(p.sorted[row_base + lane] >= 0);
  const bool vec_out = (p.n_cols & 7) == 0;  // a 16-byte chunk is all in or all out
  // route index of the row each lane stores in the vectorized epilogue
  int route[NMS];
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) route[ms] = p.sorted[row_base + 16 * ms + (lane >> 2)];
  auto store_step = [&](int st) {
    int col[kNsub];
    bool on[kNsub];
    step_src(st, col, on);
    if (!vec_out) {
      store_outputs<DT, MODE_DOWN, NMS>(p, row_base, acc, col, on, g, vmask);
      return;
    }
    // lane (c, g) holds rows 16 ms + 4 g + i of columns 16 s + c
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
      for (int s = 0; s < kNsub; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_out[(16 * ms + 4 * g + i) * kOutStride + 16 * s + c] =
              H16<DT>::from_f32(16.0f * acc[ms][s][i]);
    // lane l: row 16 ms + l / 4, columns 8 (l % 4) .. + 8 of the wave's 32
    const int n0 = st * kTileColsPlain + w * 32 + 8 * (lane & 3);
    const bool col_ok = st < step_end && n0 < p.n_cols;
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms) {
      const int r = 16 * ms + (lane >> 2);
      const u32x4 v = *reinterpret_cast<const u32x4*>(s_out + r * kOutStride + 8 * (lane & 3));
      const bool ok = col_ok && ((rows_valid >> r) & 1u);
      // Y rows by route index
      if (ok) *reinterpret_cast<u32x4*>(p.out + static_cast<int64_t>(route[ms]) * p.ldo + n0) = v;
    }
  };

  static_assert(NKB == 1 || NKB == 2, "one or two 128-blocks per step");
  // tiles of one or two subtiles hold few accumulators: their weights stream
  // through a ring of four blocks, two column steps ahead (the register
  // count of the kernel is set by the larger tiles)
  constexpr bool kDeep = NKB == 2 && NMS <= 2;
  if constexpr (kDeep) {
    WBlk<LAYOUT> w[4][kNsub];
    load_blk(step_begin, 0, w[0]);
    load_blk(step_begin, 1, w[1]);
    load_blk(step_begin + 1, 0, w[2]);
    load_blk(step_begin + 1, 1, w[3]);
    for (int st = step_begin; st < step_end; st += 2) {
      zero_acc();
      pass_scales<LAYOUT, kNsub>(w[0], w[1]);
      mma_block<DT, LAYOUT, NMS, false>(s_ar, S, w[0], acc, c, g, par);
      mma_block<DT, LAYOUT, NMS, false>(s_ar + 128, S, w[1], acc, c, g, par);
      store_step(st);
      load_blk(st + 2, 0, w[0]);
      load_blk(st + 2, 1, w[1]);
      if (st + 1 < step_end) {
        zero_acc();
        pass_scales<LAYOUT, kNsub>(w[2], w[3]);
        mma_block<DT, LAYOUT, NMS, false>(s_ar, S, w[2], acc, c, g, par);
        mma_block<DT, LAYOUT, NMS, false>(s_ar + 128, S, w[3], acc, c, g, par);
        store_step(st + 1);
      }
      load_blk(st + 3, 0, w[2]);
      load_blk(st + 3, 1, w[3]);
    }
    return;
  }
  WBlk<LAYOUT> w0[kNsub], w1[kNsub];
  load_blk(step_begin, 0, w0);
  if constexpr (NKB == 2) {
    for (int st = step_begin; st < step_end; ++st) {
      load_blk(st, 1, w1);
      zero_acc();
      mma_block<DT, LAYOUT, NMS, false>(s_ar, S, w0, acc, c, g, par);
      pass_scales<LAYOUT, kNsub>(w0, w1);
      load_blk(st + 1, 0, w0);
      mma_block<DT, LAYOUT, NMS, false>(s_ar + 128, S, w1, acc, c, g, par);
      store_step(st);
    }
  } else {
    for (int st = step_begin; st < step_end; st += 2) {
      load_blk(st + 1, 0, w1);
      zero_acc();
      mma_block<DT, LAYOUT, NMS, false>(s_ar, S, w0, acc, c, g, par);
      store_step(st);
      load_blk(st + 2, 0, w0);
      if (st + 1 < step_end) {
        zero_acc();
        mma_block<DT, LAYOUT, NMS, false>(s_ar, S, w1, acc, c, g, par);
        store_step(st + 1);
      }
    }
  }
}

// Four waves per SIMD (two workgroups per CU): twice the weight requests in
// flight per CU; measured faster than one workgroup with more registers
// although the four-subtile path then keeps a few values in scratch.
// PART: the activations come from split-K partials (a separate instance, so
// that the plain kernel's register allocation is not affected).
template <int DT, int LAYOUT, int NKB, bool PART = false>
__global__ void __launch_bounds__(kTileThreads, 4)
down_resident_kernel(const GemmParams p) {
  __shared__ uint16_t s_ar[kTileRows * (NKB * 128 + 8)];
  __shared__ __align__(16) uint16_t s_out[kTileWaves][kTileRows * kOutStride];

  // same XCD-aware order as the streaming kernel (n_tiles = column chunks)
  const int L = blockIdx.x;
  if (p.fin_cnt != nullptr && L >= p.n_main) {  // fused combine: empty tokens' rows
    finalize_zero_rows(p, L - p.n_main);
    return;
  }
  int chunk;
  const int mt = tile_at(p, tile_position(p, L, chunk));
  if (mt < 0) return;  // position past the used tiles
  const int row_base = mt * kTileRows;
  // every index the workgroup needs comes in one batch of loads before the
  // first decision (see tile_gemm_kernel)
  const int rb = min(mt, p.tiles - 1) * kTileRows;
  const int total = p.offsets[p.E];
  const int e = p.tile_expert[rb / kTileRows];
  int first[kTileMs];
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) first[ms] = p.sorted[rb + 16 * ms];
  asm volatile("" : : "s"(total), "s"(e), "s"(first[0]), "s"(first[1]), "s"(first[2]), "s"(first[3]));
  if (row_base >= total) return;
  int nms = 0;
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) nms += first[ms] >= 0 ? 1 : 0;
  switch (nms) {
    case 1: down_resident_run<DT, LAYOUT, 1, NKB, PART>(p, row_base, e, chunk, s_ar,
                                                  s_out[threadIdx.x >> 6]); break;
    case 2: down_resident_run<DT, LAYOUT, 2, NKB, PART>(p, row_base, e, chunk, s_ar,
                                                  s_out[threadIdx.x >> 6]); break;
    case 3: down_resident_run<DT, LAYOUT, 3, NKB, PART>(p, row_base, e, chunk, s_ar,
                                                  s_out[threadIdx.x >> 6]); break;
    default: down_resident_run<DT, LAYOUT, 4, NKB, PART>(p, row_base, e, chunk, s_ar,
                                                  s_out[threadIdx.x >> 6]); break;
  }
  if (p.fin_cnt != nullptr) {
    const int c0 = chunk * p.col_steps * kTileColsPlain;
    const int c1 = min(p.n_cols, c0 + p.col_steps * kTileColsPlain);
    if (c0 < c1) finalize_arrivals<DT>(p, row_base, chunk, c0, c1);
  }
}

// down_resident_run with the exact fp16 route (bf16 activations and scales,
// group layout; the per-group form stays a function of its own so that its
// register allocation is untouched): the activation rows are staged as
// fp16; returns false, with nothing stored, if one of them has magnitude
// 2^16 or more (or is not finite).
template <int DT, int LAYOUT, int NMS, int NKB, bool X16 = true>
__device__ __forceinline__ bool down_resident_run_x16(const GemmParams& p, const int row_base,
                                                  const int e, const int chunk, uint16_t* s_ar,
                                                  uint16_t* s_out) {
  static_assert(!X16 || (DT == DT_BF16 && LAYOUT == Q_GROUP_K), "fp16 route");
  constexpr int S = NKB * 128 + 8;   // row stride of the resident tile
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4, par = c & 1;

  // stage the tile's activation rows once (padding rows and columns past K
  // read zeros)
  {
    constexpr int kPerRow = NKB * 16;                       // 16-byte chunks per row
    constexpr int kIters = kTileRows * kPerRow / kTileThreads;
    static_assert(kTileRows * kPerRow % kTileThreads == 0, "staging covers the tile");
    const auto ra = make_rsrc(p.a + static_cast<int64_t>(row_base) * p.lda,
                              static_cast<uint32_t>(2 * kTileRows * p.lda));
    u32x4 v[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int idx = tid + i * kTileThreads;
      const int row = idx / kPerRow, ch = idx % kPerRow;
      const bool ok = p.sorted[row_base + row] >= 0 && 8 * ch < p.K;
      v[i] = bload16(ra, 2u * static_cast<uint32_t>(row * p.lda + 8 * ch), ok);
    }
    [[maybe_unused]] bool big = false;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int idx = tid + i * kTileThreads;
      const int row = idx / kPerRow, ch = idx % kPerRow;
      if constexpr (X16) {
        // bf16 exponent field 127 + 16 or more (Inf and NaN included)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          big |= (v[i][k] & 0x7FFFu) >= 0x4780u || (v[i][k] & 0x7FFF0000u) >= 0x47800000u;
        *reinterpret_cast<u32x4*>(s_ar + row * S + 8 * ch) = bf16x8_to_f16x8(v[i]);
      } else {
        *reinterpret_cast<u32x4*>(s_ar + row * S + 8 * ch) = v[i];
      }
    }
    if constexpr (X16) {
      if (__syncthreads_or(big)) return false;
    } else {
      __syncthreads();
    }
  }

  const int step_begin = chunk * p.col_steps;
  const int step_end = min(step_begin + p.col_steps, (p.n_cols + kTileColsPlain - 1) / kTileColsPlain);

  const WExpert wx = make_wexpert(p, e);
  const uint32_t vmask = valid_rows<NMS>(p, row_base, g);
  // wave w's columns in step st: st * 256 + 32 w + 16 k + c (k = subtile)
  auto step_src = [&](int st, int (&col)[kNsub], bool (&on)[kNsub]) {
    const int n0 = st * kTileColsPlain + w * 32;
#pragma unroll
    for (int k = 0; k < kNsub; ++k) {
      col[k] = n0 + 16 * k + c;
      on[k] = st < step_end && n0 + 16 * k < p.n_cols;
    }
    return make_wsrc<LAYOUT>(p.K, col, on);
  };
  // two register sets: the next block's weights are requested while the
  // current block is computed
  auto load_blk = [&](int st, int kb, WBlk<LAYOUT> (&wb)[kNsub]) {
    int col[kNsub];
    bool on[kNsub];
    const WSrc<> ws = step_src(st, col, on);
    if constexpr (NKB == 1) load_wblk<LAYOUT, kNsub, SC_SINGLE>(wx, ws, 128 * kb, p.K, g, wb);
    else if (kb == 0) load_wblk<LAYOUT, kNsub, SC_PAIR_FIRST>(wx, ws, 0, p.K, g, wb);
    else load_wblk<LAYOUT, kNsub, SC_PAIR_SECOND>(wx, ws, 128, p.K, g, wb);
  };
  f32x4 acc[NMS][kNsub];
  auto zero_acc = [&]() {
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
      for (int k = 0; k < kNsub; ++k) acc[ms][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // rows of the tile holding a route (bit r: tile row r)
  const uint64_t rows_valid = __ballot(p.sorted[row_base + lane] >= 0);
  const bool vec_out = (p.n_cols & 7) == 0;  // a 16-byte chunk is all in or all out
  // route index of the row each lane stores in the vectorized epilogue
  int route[NMS];
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) route[ms] = p.sorted[row_base + 16 * ms + (lane >> 2)];
  bool sbad = false;  // X16: a group scale outside the route's exact range
  auto mma = [&](const uint16_t* sa, const WBlk<LAYOUT> (&wb)[kNsub]) {
    if constexpr (X16) mma_block_x<NMS, false>(sa, S, wb, acc, c, g, sbad);
    else mma_block<DT, LAYOUT, NMS, false>(sa, S, wb, acc, c, g, par);
  };
  auto store_step = [&](int st) {
    int col[kNsub];
    bool on[kNsub];
    step_src(st, col, on);
    if constexpr (X16) {
      // the stores apply the per-group form's factor 16 (exact)
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
        for (int k = 0; k < kNsub; ++k) acc[ms][k] *= 0.0625f;
    }
    if (!vec_out) {
      store_outputs<DT, MODE_DOWN, NMS>(p, row_base, acc, col, on, g, vmask);
      return;
    }
    // lane (c, g) holds rows 16 ms + 4 g + i of columns 16 s + c
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
      for (int s = 0; s < kNsub; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_out[(16 * ms + 4 * g + i) * kOutStride + 16 * s + c] =
              H16<DT>::from_f32(16.0f * acc[ms][s][i]);
    // lane l: row 16 ms + l / 4, columns 8 (l % 4) .. + 8 of the wave's 32
    const int n0 = st * kTileColsPlain + w * 32 + 8 * (lane & 3);
    const bool col_ok = st < step_end && n0 < p.n_cols;
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms) {
      const int r = 16 * ms + (lane >> 2);
      const u32x4 v = *reinterpret_cast<const u32x4*>(s_out + r * kOutStride + 8 * (lane & 3));
      const bool ok = col_ok && ((rows_valid >> r) & 1u);
      // Y rows by route index
      if (ok) *reinterpret_cast<u32x4*>(p.out + static_cast<int64_t>(route[ms]) * p.ldo + n0) = v;
    }
  };

  static_assert(NKB == 1 || NKB == 2, "one or two 128-blocks per step");
  // tiles of one or two subtiles hold few accumulators: their weights stream
  // through a ring of four blocks, two column steps ahead (the register
  // count of the kernel is set by the larger tiles)
  constexpr bool kDeep = NKB == 2 && NMS <= 2;
  if constexpr (kDeep) {
    WBlk<LAYOUT> w[4][kNsub];
    load_blk(step_begin, 0, w[0]);
    load_blk(step_begin, 1, w[1]);
    load_blk(step_begin + 1, 0, w[2]);
    load_blk(step_begin + 1, 1, w[3]);
    for (int st = step_begin; st < step_end; st += 2) {
      zero_acc();
      pass_scales<LAYOUT, kNsub>(w[0], w[1]);
      mma(s_ar, w[0]);
      mma(s_ar + 128, w[1]);
      store_step(st);
      load_blk(st + 2, 0, w[0]);
      load_blk(st + 2, 1, w[1]);
      if (st + 1 < step_end) {
        zero_acc();
        pass_scales<LAYOUT, kNsub>(w[2], w[3]);
        mma(s_ar, w[2]);
        mma(s_ar + 128, w[3]);
        store_step(st + 1);
      }
      load_blk(st + 3, 0, w[2]);
      load_blk(st + 3, 1, w[3]);
    }
    return !__syncthreads_or(sbad);  // stored outputs get rewritten by the rerun
  }
  WBlk<LAYOUT> w0[kNsub], w1[kNsub];
  load_blk(step_begin, 0, w0);
  if constexpr (NKB == 2) {
    for (int st = step_begin; st < step_end; ++st) {
      load_blk(st, 1, w1);
      zero_acc();
      mma(s_ar, w0);
      pass_scales<LAYOUT, kNsub>(w0, w1);
      load_blk(st + 1, 0, w0);
      mma(s_ar + 128, w1);
      store_step(st);
    }
  } else {
    for (int st = step_begin; st < step_end; st += 2) {
      load_blk(st + 1, 0, w1);
      zero_acc();
      mma(s_ar, w0);
      store_step(st);
      load_blk(st + 2, 0, w0);
      if (st + 1 < step_end) {
        zero_acc();
        mma(s_ar, w1);
        store_step(st + 1);
      }
    }
  }
  return !__syncthreads_or(sbad);  // stored outputs get rewritten by the rerun
}

// The work of resident-kernel workgroup L on the fp16 route (false: rerun).
template <int DT, int LAYOUT, int NKB>
__device__ __forceinline__ bool down_work_x16(const GemmParams& p, const int L, uint16_t* s_ar,
                                          uint16_t* s_out) {
  // same XCD-aware order as the streaming kernel (n_tiles = column chunks)
  int chunk;
  const int mt = tile_at(p, tile_position(p, L, chunk));
  if (mt < 0) return true;  // position past the used tiles
  const int row_base = mt * kTileRows;
  // every index the workgroup needs comes in one batch of loads before the
  // first decision (see tile_work)
  const int rb = min(mt, p.tiles - 1) * kTileRows;
  const int total = p.offsets[p.E];
  const int e = p.tile_expert[rb / kTileRows];
  int first[kTileMs];
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) first[ms] = p.sorted[rb + 16 * ms];
  asm volatile("" : : "s"(total), "s"(e), "s"(first[0]), "s"(first[1]), "s"(first[2]), "s"(first[3]));
  if (row_base >= total) return true;
  int nms = 0;
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) nms += first[ms] >= 0 ? 1 : 0;
  switch (nms) {
    case 1: return down_resident_run_x16<DT, LAYOUT, 1, NKB>(p, row_base, e, chunk, s_ar, s_out);
    case 2: return down_resident_run_x16<DT, LAYOUT, 2, NKB>(p, row_base, e, chunk, s_ar, s_out);
    case 3: return down_resident_run_x16<DT, LAYOUT, 3, NKB>(p, row_base, e, chunk, s_ar, s_out);
    default: return down_resident_run_x16<DT, LAYOUT, 4, NKB>(p, row_base, e, chunk, s_ar, s_out);
  }
}

// The work of resident-kernel workgroup L on the per-group form (for the
// rerun of flagged workgroups).
template <int DT, int LAYOUT, int NKB>
__device__ __forceinline__ void down_work_pg(const GemmParams& p, const int L, uint16_t* s_ar,
                                             uint16_t* s_out) {
  int chunk;
  const int mt = tile_at(p, tile_position(p, L, chunk));
  if (mt < 0) return;  // position past the used tiles
  const int row_base = mt * kTileRows;
  if (row_base >= p.offsets[p.E]) return;
  int nms = 0;
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) nms += p.sorted[row_base + 16 * ms] >= 0 ? 1 : 0;
  const int e = p.tile_expert[mt];
  switch (nms) {
    case 1: down_resident_run<DT, LAYOUT, 1, NKB>(p, row_base, e, chunk, s_ar, s_out); break;
    case 2: down_resident_run<DT, LAYOUT, 2, NKB>(p, row_base, e, chunk, s_ar, s_out); break;
    case 3: down_resident_run<DT, LAYOUT, 3, NKB>(p, row_base, e, chunk, s_ar, s_out); break;
    default: down_resident_run<DT, LAYOUT, 4, NKB>(p, row_base, e, chunk, s_ar, s_out); break;
  }
}

// The fp16-route resident kernel: every workgroup records whether it must be
// rerun (the flag array needs no clearing).
template <int DT, int LAYOUT, int NKB>
__global__ void __launch_bounds__(kTileThreads, 4)
down_resident_x16_kernel(const GemmParams p) {
  __shared__ uint16_t s_ar[kTileRows * (NKB * 128 + 8)];
  __shared__ __align__(16) uint16_t s_out[kTileWaves][kTileRows * kOutStride];
  const bool done = down_work_x16<DT, LAYOUT, NKB>(p, static_cast<int>(blockIdx.x), s_ar,
                                                  s_out[threadIdx.x >> 6]);
  if (threadIdx.x == 0) p.redo[blockIdx.x] = done ? 0 : 1;
}

// Reruns, with the per-group form, the workgroups of a fp16-route resident
// launch of n_wg workgroups that found an activation outside fp16's range
// (flag scan as in tile_redo_kernel).
template <int DT, int LAYOUT, int NKB>
__global__ void __launch_bounds__(kTileThreads)
down_redo_kernel(const GemmParams p, const int n_wg) {
  __shared__ uint16_t s_ar[kTileRows * (NKB * 128 + 8)];
  __shared__ __align__(16) uint16_t s_out[kTileWaves][kTileRows * kOutStride];
  const int G = static_cast<int>(gridDim.x);
  for (int base = static_cast<int>(blockIdx.x); base < n_wg; base += G * kTileThreads) {
    const int L = base + G * static_cast<int>(threadIdx.x);
    const bool f = L < n_wg && p.redo[L] != 0;
    if (!__syncthreads_or(f)) continue;
    for (int i = 0; i < kTileThreads; ++i) {
      const int Li = base + G * i;
      if (Li >= n_wg) break;
      if (p.redo[Li] == 0) continue;  // uniform
      down_work_pg<DT, LAYOUT, NKB>(p, Li, s_ar, s_out[threadIdx.x >> 6]);
      __syncthreads();  // LDS reuse by the next workgroup's tile
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K gate/up GEMM for tiles of few rows ([P1] Modification: small-batch
// split-K).  Workgroup (tile, K chunk): the tile's x rows over the chunk stay
// in LDS (one 16-row subtile at a time), and each wave streams its NSUB
// subtiles of every weight row of the chunk, with no barrier inside the
// stream.  FP32 partial pre-activations go to part[chunk][route][N1]; the
// activation kernel below sums the chunks in order.
// ---------------------------------------------------------------------------

template <int DT, int LAYOUT, int NSUB>
__global__ void __launch_bounds__(kTileThreads)
up_splitk_kernel(const GemmParams p) {
  extern __shared__ uint16_t s_x[];   // [16][cb * 128 + 8], then per wave [32][4 * cb] scales
  // workgroup = (tile, reduction chunk, column chunk of p.col_steps passes)
  const int nchunk = p.n_tiles;
  const int mt = blockIdx.x / (p.S * nchunk);
  const int kc = (blockIdx.x / nchunk) % p.S;
  const int cc = blockIdx.x % nchunk;
  const int row_base = mt * kTileRows;
  // every index the workgroup needs comes in one batch of loads before the
  // first decision (see tile_gemm_kernel)
  const int rb = min(mt, p.tiles - 1) * kTileRows;
  const int total = p.offsets[p.E];
  const int e = p.tile_expert[rb / kTileRows];
  int first[kTileMs];
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) first[ms] = p.sorted[rb + 16 * ms];
  const int my_r0 = p.sorted[rb + (threadIdx.x & 15)];  // subtile 0: route of row l % 16
  asm volatile("" : : "s"(total), "s"(e), "s"(first[0]), "s"(first[1]), "s"(first[2]), "s"(first[3]),
               "v"(my_r0));
  if (row_base >= total) return;  // whole workgroup: tile past the padded total
  const int nblk = (p.K + 127) >> 7;
  const int b0 = kc * p.cb;
  const int b1 = min(nblk, b0 + p.cb);
  if (b0 >= b1) return;
  const int kend = min(p.K, 128 * b1);
  int nms = 0;
#pragma unroll
  for (int ms = 0; ms < kTileMs; ++ms) nms += first[ms] >= 0 ? 1 : 0;
  const int stride = p.cb * 128 + 8;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4, par = c & 1;
  const WExpert wx = make_wexpert(p, e);
  const auto xr = make_rsrc(p.a, p.a_bytes);
  constexpr int kPassRows = kTileWaves * 16 * NSUB;  // weight rows per column pass

  for (int rp = 0; rp < nms; ++rp) {
    if (rp > 0) __syncthreads();  // the previous subtile's rows are no longer read
    // stage x rows of subtile rp over the chunk, in A operand order: the
    // token of each of the 16 rows (lane l: row l % 16), then every x chunk
    // in flight at once, then the LDS stores
    const int nch = (b1 - b0) * 16;
    const int my_r = rp == 0 ? my_r0 : p.sorted[row_base + 16 * rp + c];
    // a subtile of at most 4 routes (valid rows are a prefix) puts route q
    // on MFMA row 4q: each lane's element 0 then carries one route, and the
    // group scale is applied to that element alone (the other rows stay
    // zero and their products are dropped)
    const bool row4 = __ballot(lane < 16 && my_r >= 0) < 16;  // routes on rows 0..3 only
    // the route of each chunk's row, read per chunk (one batch, no lane
    // exchange chain), then the chunks
    int rr[kSplitkXLoads];
#pragma unroll
    for (int i = 0; i < kSplitkXLoads; ++i) {
      const int idx = tid + kTileThreads * i;
      const int row = min(idx / nch, 15);
      const int src = row4 ? ((row & 3) == 0 ? row >> 2 : -1) : row;
      rr[i] = src >= 0 ? p.sorted[row_base + 16 * rp + src] : -1;
    }
    u32x4 xv[kSplitkXLoads];
#pragma unroll
    for (int i = 0; i < kSplitkXLoads; ++i) {
      const int idx = tid + kTileThreads * i;
      const int row = idx / nch, ch = idx - row * nch;
      const bool ok = idx < 16 * nch && rr[i] >= 0 && 128 * b0 + 8 * ch < p.K;
      xv[i] = bload16(xr, 2u * static_cast<uint32_t>((ok ? rr[i] / p.top_k : 0) * p.lda + 128 * b0 + 8 * ch),
                      ok);
    }
#pragma unroll
    for (int i = 0; i < kSplitkXLoads; ++i) {
      const int idx = tid + kTileThreads * i;
      const int row = idx / nch, ch = idx - row * nch;
      if (idx < 16 * nch) *reinterpret_cast<u32x4*>(s_x + row * stride + 8 * ch) = permute_a(xv[i]);
    }
    __syncthreads();
    // the route of each accumulator element (element i of lane row g: tile
    // row 4g + i; with row4 only element 0 is used, for row g)
    int rts[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rts[i] = __shfl(my_r, row4 ? g : 4 * g + i);

    // the column passes, with NI accumulator elements per lane scaled
    auto stream = [&](auto ni_tag) {
      constexpr int NI = decltype(ni_tag)::value;
      const int n_end = min(p.n_cols, (cc + 1) * p.col_steps * kPassRows);
      for (int n0 = cc * p.col_steps * kPassRows; n0 < n_end; n0 += kPassRows) {
        int wrow[NSUB];
        bool on[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          const int r0 = n0 + (w * NSUB + s) * 16;
          wrow[s] = r0 + c;
          on[s] = r0 < p.n_cols;
        }
        const WSrc<NSUB> ws = make_wsrc<LAYOUT, NSUB>(p.K, wrow, on);
        f32x4 acc[1][NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) acc[0][s] = f32x4{0.f, 0.f, 0.f, 0.f};
        static_assert(kSplitkRing % 2 == 0, "block pairs must not straddle the ring");
        WBlk<LAYOUT> wr[kSplitkRing][NSUB];
        if constexpr (is_group(LAYOUT)) {
          // group scales of the wave's 32 rows over the chunk, staged in the
          // wave's own LDS region (read back only by the wave: no barrier);
          // 8 bytes (4 groups) per row and block
          const int nb = b1 - b0;
          uint16_t* my_sc = s_x + 16 * stride + w * 32 * 4 * p.cb;  // [32 rows][4 * cb]
          {
            u32x2 sv[kSplitkScLoads];
#pragma unroll
            for (int i = 0; i < kSplitkScLoads; ++i) {
              const int idx = lane + 64 * i;           // (row, block) = (idx / nb, idx % nb)
              const int row = idx / nb, blk = idx - row * nb;
              const int grow = n0 + 16 * w * NSUB + row;  // weight row
              const bool ok = row < 32 && grow < p.n_cols;
              const uint32_t so = 2u * (static_cast<uint32_t>(grow) * (p.K >> 5) + 4 * (b0 + blk));
              sv[i] = __builtin_bit_cast(
                  u32x2, __builtin_amdgcn_raw_buffer_load_b64(wx.rs, ok ? so : kOob, 0, 0));
            }
            // the first weight blocks go out before the scales are stored
#pragma unroll
            for (int i = 0; i < kSplitkRing - 1; ++i)
              load_wblk<LAYOUT, NSUB, SC_NONE>(wx, ws, 128 * (b0 + i), kend, g, wr[i]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kSplitkScLoads; ++i) {
              const int idx = lane + 64 * i;
              const int row = idx / nb, blk = idx - row * nb;
              if (row < 32) *reinterpret_cast<u32x2*>(my_sc + row * 4 * p.cb + 4 * blk) = sv[i];
            }
          }
          for (int b = b0; b < b1; b += kSplitkRing) {
#pragma unroll
            for (int u = 0; u < kSplitkRing; ++u) {
              load_wblk<LAYOUT, NSUB, SC_NONE>(wx, ws, 128 * (b + u + kSplitkRing - 1), kend, g,
                                               wr[(u + kSplitkRing - 1) % kSplitkRing]);
              if (b + u < b1) {
#pragma unroll
                for (int s2 = 0; s2 < NSUB; ++s2) {
                  const u32x2 sp = *reinterpret_cast<const u32x2*>(
                      my_sc + (16 * s2 + c) * 4 * p.cb + 4 * (b + u - b0));
                  wr[u][s2].s0 = sp[0];
                  wr[u][s2].s1 = sp[1];
                }
                mma_block<DT, LAYOUT, 1, true, NSUB, NI>(s_x + 128 * (b + u - b0), stride, wr[u],
                                                         acc, c, g, par);
              }
            }
          }
        } else {
          // ring of kSplitkRing register sets: block b + kSplitkRing - 1 is
          // requested while block b is computed (loads past the chunk are
          // masked); block b0 + i into wr[slot], `first` = i is even
          auto load_i = [&](int i, int slot, bool first) {
            if (first)
              load_wblk<LAYOUT, NSUB, SC_PAIR_FIRST>(wx, ws, 128 * (b0 + i), kend, g, wr[slot]);
            else
              load_wblk<LAYOUT, NSUB, SC_PAIR_SECOND>(wx, ws, 128 * (b0 + i), kend, g, wr[slot]);
          };
#pragma unroll
          for (int i = 0; i < kSplitkRing - 1; ++i) load_i(i, i, i % 2 == 0);
          for (int b = b0; b < b1; b += kSplitkRing) {
#pragma unroll
            for (int u = 0; u < kSplitkRing; ++u) {
              // the second block of a pair reads its scales from the first
              // block's registers, so the load that refills that slot (the
              // next pair's first block) is issued after it
              if (u % 2 == 0)
                load_i(b - b0 + u + kSplitkRing - 1, (u + kSplitkRing - 1) % kSplitkRing, false);
              if (b + u < b1)
                mma_block2<DT, LAYOUT, 1, NSUB, NI>(s_x + 128 * (b + u - b0), stride, wr[u],
                                                    wr[u & ~1], u % 2, acc, c, g, par);
              if (u % 2 == 1)
                load_i(b - b0 + u + kSplitkRing - 1, (u + kSplitkRing - 1) % kSplitkRing, true);
            }
          }
        }
        // FP32 partials of valid rows: lane (c, g) element i holds route
        // rts[i], weight row wrow[s]
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (rts[i] < 0) continue;
          float* prow = p.part + (static_cast<int64_t>(kc) * p.R + rts[i]) * p.n_cols;
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            if (on[s]) prow[wrow[s]] = 16.0f * acc[0][s][i];
        }
      }
    };
    if (row4) stream(std::integral_constant<int, 1>{});
    else stream(std::integral_constant<int, 4>{});
  }
}

// act[slot[r]] for route r from its split-K partials (act_from_partials).
// One thread per 8 consecutive activation columns.
template <int DT, bool GATED>
__global__ void __launch_bounds__(256)
splitk_act_kernel(const GemmParams p) {
  const int I = p.ldo;
  const int per_row = I / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int r = static_cast<int>(idx / per_row);
  const int i0 = 8 * static_cast<int>(idx % per_row);
  if (r >= p.R) return;
  const int pos = p.slot[r];
  if (pos < 0) return;  // invalid route: no position, nothing reads it
  *reinterpret_cast<u32x4*>(p.out + static_cast<int64_t>(pos) * I + i0) =
      act_from_partials<DT>(p.part, p.S, p.R, p.n_cols, GATED ? I : 0, r, i0);
}

template <typename F>
static hipError_t allow_lds_tile(F* kernel, size_t lds, size_t static_lds = 0) {
  if (lds + static_lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}

template <int DT, int LAYOUT>
static hipError_t launch_splitk_dl(const GemmParams& p, int max_tiles, hipStream_t st) {
  // x slice [16][cb * 128 + 8], then (group layout) per wave [32][4 * cb] scales
  const size_t lds = sizeof(uint16_t) * (16 * (static_cast<size_t>(p.cb) * 128 + 8) +
                                         (is_group(LAYOUT) ? kTileWaves * 32 * 4 * p.cb : 0));
  const hipError_t err = allow_lds_tile(up_splitk_kernel<DT, LAYOUT, kSplitkNsub>, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((up_splitk_kernel<DT, LAYOUT, kSplitkNsub>),
                     dim3(max_tiles * p.S * p.n_tiles), dim3(kTileThreads), lds, st, p);
  return hipGetLastError();
}

hipError_t launch_up_splitk(const GemmParams& p, int dtype, int layout, int max_tiles,
                            hipStream_t stream) {
  if (p.S < 1 || p.cb < 1 || p.n_tiles < 1 || p.col_steps < 1 ||
      16 * (p.cb * 128 + 8) * 2 > kSplitkMaxLds || 16 * 16 * p.cb > kSplitkXLoads * kTileThreads ||
      32 * p.cb > 64 * kSplitkScLoads ||
      static_cast<int64_t>(max_tiles) * p.S * p.n_tiles > 0x7fffffff)
    return hipErrorInvalidValue;
  if (dtype == DT_BF16)
    return layout == Q_GROUP_K ? launch_splitk_dl<DT_BF16, Q_GROUP_K>(p, max_tiles, stream)
         : layout == Q_FP4_GROUP_K ? launch_splitk_dl<DT_BF16, Q_FP4_GROUP_K>(p, max_tiles, stream)
                               : launch_splitk_dl<DT_BF16, Q_PER_CHANNEL>(p, max_tiles, stream);
  return layout == Q_GROUP_K ? launch_splitk_dl<DT_FP16, Q_GROUP_K>(p, max_tiles, stream)
       : layout == Q_FP4_GROUP_K ? launch_splitk_dl<DT_FP16, Q_FP4_GROUP_K>(p, max_tiles, stream)
                             : launch_splitk_dl<DT_FP16, Q_PER_CHANNEL>(p, max_tiles, stream);
}

hipError_t launch_splitk_act(const GemmParams& p, int dtype, bool gated, hipStream_t stream) {
  if (p.ldo % 8 != 0 || p.R < 1) return hipErrorInvalidValue;
  const int64_t threads = static_cast<int64_t>(p.R) * (p.ldo / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (dtype == DT_BF16) {
    if (gated) hipLaunchKernelGGL((splitk_act_kernel<DT_BF16, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((splitk_act_kernel<DT_BF16, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (gated) hipLaunchKernelGGL((splitk_act_kernel<DT_FP16, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((splitk_act_kernel<DT_FP16, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <int DT, int LAYOUT, int MODE, bool X16>
static hipError_t launch_tile_kx(const GemmParams& p, dim3 grid, hipStream_t st) {
  if constexpr (is_group(LAYOUT)) {
    if (tile_scales_in_lds(LAYOUT, p.K)) {
      const size_t lds = tile_lds_bytes(true, p.K);
      const hipError_t err = allow_lds_tile(tile_gemm_kernel<DT, LAYOUT, MODE, true, X16>, lds);
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL((tile_gemm_kernel<DT, LAYOUT, MODE, true, X16>), grid, dim3(kTileThreads),
                         lds, st, p);
      return hipGetLastError();
    }
  }
  // per-channel scales, or group scales that neither fit whole nor split
  // into phases: fetched with the weights, per block pair
  const size_t lds = tile_lds_bytes(false, p.K);
  const hipError_t err = allow_lds_tile(tile_gemm_kernel<DT, LAYOUT, MODE, false, X16>, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((tile_gemm_kernel<DT, LAYOUT, MODE, false, X16>), grid, dim3(kTileThreads), lds,
                     st, p);
  return hipGetLastError();
}

template <int DT, int LAYOUT, int MODE>
static hipError_t launch_tile_k(const GemmParams& p, dim3 grid, hipStream_t st) {
  if constexpr (DT == DT_BF16 && LAYOUT == Q_GROUP_K) {
    if (p.redo != nullptr) {
      // fp16 route, then the rerun of flagged tiles (a few workgroups that
      // each scan a share of the flags)
      hipError_t err = launch_tile_kx<DT, LAYOUT, MODE, true>(p, grid, st);
      if (err != hipSuccess) return err;
      const size_t lds = tile_lds_bytes(false, p.K);
      err = allow_lds_tile(tile_redo_kernel<DT, LAYOUT, MODE>, lds);
      if (err != hipSuccess) return err;
      const int n_wg = static_cast<int>(grid.x);
      const dim3 rgrid(static_cast<unsigned>(std::min(n_wg, kTileRedoWorkgroups)));
      hipLaunchKernelGGL((tile_redo_kernel<DT, LAYOUT, MODE>), rgrid, dim3(kTileThreads), lds, st,
                         p, n_wg);
      return hipGetLastError();
    }
  }
  return launch_tile_kx<DT, LAYOUT, MODE, false>(p, grid, st);
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

template <int DT, int LAYOUT, int NKB>
static hipError_t launch_resident_k(const GemmParams& p, dim3 grid, hipStream_t st) {
  if constexpr (DT == DT_BF16 && LAYOUT == Q_GROUP_K) {
    if (p.redo != nullptr) {
      // fp16 route, then the rerun of flagged workgroups
      hipLaunchKernelGGL((down_resident_x16_kernel<DT, LAYOUT, NKB>), grid, dim3(kTileThreads), 0,
                         st, p);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      const int n_wg = static_cast<int>(grid.x);
      const dim3 rgrid(static_cast<unsigned>(std::min(n_wg, kTileRedoWorkgroups)));
      hipLaunchKernelGGL((down_redo_kernel<DT, LAYOUT, NKB>), rgrid, dim3(kTileThreads), 0, st, p,
                         n_wg);
      return hipGetLastError();
    }
  }
  if (p.part != nullptr)
    hipLaunchKernelGGL((down_resident_kernel<DT, LAYOUT, NKB, true>), grid, dim3(kTileThreads), 0,
                       st, p);
  else
    hipLaunchKernelGGL((down_resident_kernel<DT, LAYOUT, NKB>), grid, dim3(kTileThreads), 0, st,
                       p);
  return hipGetLastError();
}

template <int DT, int LAYOUT>
static hipError_t launch_resident_dl(const GemmParams& p, dim3 grid, hipStream_t st) {
  return p.K <= 128 ? launch_resident_k<DT, LAYOUT, 1>(p, grid, st)
                    : launch_resident_k<DT, LAYOUT, 2>(p, grid, st);
}

hipError_t launch_down_resident(const GemmParams& p, int dtype, int layout, int max_tiles,
                                hipStream_t stream) {
  if (p.K > kResidentK || p.col_steps < 1) return hipErrorInvalidValue;
  // activations from split-K partials: whole 8-value chunks inside a partial
  // row, and not with the fp16 route (whose rerun reads the activations)
  if (p.part != nullptr &&
      (p.redo != nullptr || p.S < 1 || p.R < 1 || p.K % 8 != 0 || p.up_rows < 0 ||
       p.up_rows + p.K > p.part_ld || (p.up_rows > 0 && p.up_rows < p.K)))
    return hipErrorInvalidValue;
  const int n_main = kXcds * p.n_tiles * ((max_tiles + kXcds - 1) / kXcds);
  if (p.fin_cnt != nullptr && (p.n_main != n_main || p.redo != nullptr)) return hipErrorInvalidValue;
  const dim3 grid(n_main + (p.fin_cnt != nullptr ? fin_zero_workgroups(p.T) : 0));
  if (dtype == DT_BF16)
    return layout == Q_GROUP_K ? launch_resident_dl<DT_BF16, Q_GROUP_K>(p, grid, stream)
         : layout == Q_FP4_GROUP_K ? launch_resident_dl<DT_BF16, Q_FP4_GROUP_K>(p, grid, stream)
                               : launch_resident_dl<DT_BF16, Q_PER_CHANNEL>(p, grid, stream);
  return layout == Q_GROUP_K ? launch_resident_dl<DT_FP16, Q_GROUP_K>(p, grid, stream)
       : layout == Q_FP4_GROUP_K ? launch_resident_dl<DT_FP16, Q_FP4_GROUP_K>(p, grid, stream)
                             : launch_resident_dl<DT_FP16, Q_PER_CHANNEL>(p, grid, stream);
}

hipError_t launch_tile_gemm(const GemmParams& p, int dtype, int layout, int mode, int max_tiles,
                            hipStream_t stream) {
  const int n_main = kXcds * p.n_tiles * ((max_tiles + kXcds - 1) / kXcds);
  const bool fin = mode == MODE_DOWN && p.fin_cnt != nullptr;
  if (p.fin_cnt != nullptr && (mode != MODE_DOWN || p.n_main != n_main || p.redo != nullptr))
    return hipErrorInvalidValue;
  const dim3 grid(n_main + (fin ? fin_zero_workgroups(p.T) : 0));
  if (dtype == DT_BF16)
    return layout == Q_GROUP_K ? launch_tile_mode<DT_BF16, Q_GROUP_K>(p, mode, grid, stream)
         : layout == Q_FP4_GROUP_K ? launch_tile_mode<DT_BF16, Q_FP4_GROUP_K>(p, mode, grid, stream)
                               : launch_tile_mode<DT_BF16, Q_PER_CHANNEL>(p, mode, grid, stream);
  return layout == Q_GROUP_K ? launch_tile_mode<DT_FP16, Q_GROUP_K>(p, mode, grid, stream)
       : layout == Q_FP4_GROUP_K ? launch_tile_mode<DT_FP16, Q_FP4_GROUP_K>(p, mode, grid, stream)
                             : launch_tile_mode<DT_FP16, Q_PER_CHANNEL>(p, mode, grid, stream);
}

}  // namespace w4moe
