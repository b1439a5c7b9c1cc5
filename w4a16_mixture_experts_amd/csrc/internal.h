// internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4moe {

enum : int { MODE_UP_GATED = 0, MODE_UP_RELU2 = 1, MODE_DOWN = 2 };

// Columns of the output one workgroup covers (4 waves).
//   gated gate/up: 16 logical columns per wave (a gate and an up subtile)
//   otherwise:     32 columns per wave (two subtiles)
constexpr int kWgColsGated = 64;
constexpr int kWgColsPlain = 128;
constexpr int kFusedCols = 32;  // per-token down kernel: one wave, two subtiles
constexpr int kCombineCols = 2048;

struct GemmParams {
  const uint16_t* a;          // UP: x [T][lda]; DOWN: act [P][lda] (A operand order)
  int lda;
  const int32_t* sorted;      // [P] route index or -1 (padding)
  int top_k;
  const uint8_t* wq;          // packed weights, expert 0
  const uint16_t* ws;         // scales, expert 0
  int64_t wq_expert_bytes;
  int64_t ws_expert_elems;
  int K;                      // reduction length
  int n_cols;                 // logical output columns (I for gated UP)
  int up_rows;                // gated: row offset of the up weights (= I)
  const int32_t* tile_expert; // [max tiles]
  const int32_t* offsets;     // [E+1]; offsets[E] = padded total
  int E;
  int bm;
  int split;
  int kchunk;
  float* partial;             // [split][P][n_total]
  int32_t* counters;          // [max tiles][n_tiles]
  int64_t P;
  int n_total;                // partial row length (N1)
  uint16_t* out;              // UP: act [P][ldo]; DOWN: Y [P][ldo]
  int ldo;
  int n_tiles;
};

struct FusedDownParams {
  const uint16_t* act;        // [P][I] (A operand order)
  const uint8_t* wq;
  const uint16_t* ws;
  int64_t wq_expert_bytes;
  int64_t ws_expert_elems;
  const int32_t* ids;         // [T][K]
  const float* wts;           // [T][K]
  const int32_t* slot;        // [T*K]
  int top_k, E, off;
  int I, H;
  uint16_t* out;              // [T][H]
};

struct CombineParams {
  const uint16_t* y;          // [P][H]
  const int32_t* slot;        // [T*K]
  const float* wts;           // [T][K]
  int top_k, H;
  uint16_t* out;              // [T][H]
};

hipError_t launch_route_prep(const int32_t* ids, int R, int E, int off, int bm, int32_t* counts,
                             int32_t* offsets, int32_t* sorted, int32_t* slot,
                             int32_t* tile_expert, int32_t* zero_buf, int zero_n,
                             hipStream_t stream);

hipError_t launch_grouped_gemm(const GemmParams& p, int dtype, int layout, int ms, int mode,
                               int max_tiles, hipStream_t stream);

hipError_t launch_fused_down(const FusedDownParams& p, int dtype, int layout, int T,
                             hipStream_t stream);

hipError_t launch_combine(const CombineParams& p, int dtype, int T, hipStream_t stream);

hipError_t launch_unpack(const uint8_t* packed, int64_t n_bytes, int8_t* out, hipStream_t stream);

}  // namespace w4moe
