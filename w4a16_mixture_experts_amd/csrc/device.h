// device.h -- gfx950 device helpers shared by the W4A16 MoE kernels.
//
// Sources (web pages, cited by tag and section):
//   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
//   [P3] TensorRT-LLM PR #18313, "Add W4A16 per-channel weight-only support
//        for Cutlass fused MoE"
//
// Exact INT4 dequantization on the matrix cores.
//   A packed nibble v (two's complement q in [-8, 7], [P3] Checkpoint format)
//   becomes the 16-bit float (24 + q) / 16 with two bit operations: the
//   nibble, with its top bit flipped (v ^ 8 = q + 8), is placed in the top four
//   mantissa bits of 1.0.  Every such value is exact in bf16 and fp16.
//   For one 32-wide quantization group the matrix core then computes
//       sum_k a_k (24 + q_k) / 16  +  c   with   c = -1.5 * sum_k a_k
//   (c itself comes from one MFMA against a constant -1.5 operand), which is
//   sum_k a_k q_k / 16 with FP32 accumulation; the group's scale is applied
//   to that FP32 result (acc += s * tmp) and the factor 16 once at the end.
//   The weights are therefore never rounded to 16 bits: dequantization is
//   exact up to FP32 accumulation order ([P1] Modification: register-side
//   INT4 dequantization, FP32 accumulation).
//
// Operand order.  The bit trick produces, from one dword of eight nibbles
//   n0..n7, the 16-bit pairs (n0,n4) (n1,n5) (n2,n6) (n3,n7).  The reduction
//   order inside an MFMA is free as long as A and B agree, so A (activations)
//   is fed in the same order: 8 consecutive values x0..x7 are presented as
//   [x0,x4,x1,x5,x2,x6,x3,x7].  Intermediate activations written by the
//   gate/up kernel are stored already in that order.
//
// FP4 weights (E2M1 codes, the OCP microscaling element format): each code
//   becomes its exact value / 16 (e2m1_to_h16), so the MFMA computes
//   sum_k a_k v_k / 16 directly, with no correction term, and the same group
//   scale and final factor 16 apply.
//
// MFMA lane layout (v_mfma_f32_16x16x32_{bf16,f16}, wave64): lane l feeds
//   row/column l%16 of A/B with 8 reduction values of slice l/16, and holds
//   rows 4*(l/16) + i, column l%16 of the 16x16 FP32 result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

enum : int { DT_BF16 = 0, DT_FP16 = 1 };
enum : int { Q_GROUP_K = 0, Q_PER_CHANNEL = 1, Q_FP4_GROUP_K = 2 };

// Layouts with one scale per 32 values along K, packed along K (INT4 or FP4).
__host__ __device__ constexpr bool is_group(int layout) { return layout != Q_PER_CHANNEL; }

// Logical-to-storage position of value j (0..7) inside an 8-chunk of A.
__host__ __device__ constexpr int a_pos(int j) { return j < 4 ? 2 * j : 2 * (j - 4) + 1; }

template <int S>
__device__ __forceinline__ uint32_t shr_signed(uint32_t d) {
  if constexpr (S >= 0) return d >> S;
  else return d << (-S);
}

template <int DT>
struct H16;

template <>
struct H16<DT_BF16> {
  // (24 + q) / 16 = 1.0 + (q + 8) / 16: nibble in mantissa bits 3..6
  static constexpr int kShift = 3;
  static constexpr uint32_t kMask = 0x00780078u;
  static constexpr uint32_t kBias = 0x3FC03FC0u;  // 1.0 | (8 << 3): xor flips the nibble sign bit
  static constexpr uint32_t kNegOneHalf2 = 0xBFC0BFC0u;
  static __device__ __forceinline__ float to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    __bf16 b = static_cast<__bf16>(f);  // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
  }
  // c + h0 + h1 for the two values packed in one dword
  static __device__ __forceinline__ float dot2_ones(uint32_t pair, float c) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), c, false);
  }
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct H16<DT_FP16> {
  static constexpr int kShift = 6;
  static constexpr uint32_t kMask = 0x03C003C0u;
  static constexpr uint32_t kBias = 0x3E003E00u;  // 1.0 | (8 << 6)
  static constexpr uint32_t kNegOneHalf2 = 0xBE00BE00u;
  static __device__ __forceinline__ float to_f32(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
  }
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    _Float16 h = static_cast<_Float16>(f);  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
  }
  static __device__ __forceinline__ float dot2_ones(uint32_t pair, float c) {
    typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair),
                                  __builtin_bit_cast(f16x2, 0x3C003C00u), c, false);
  }
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// Eight nibbles (one dword, n_i at bits 4i..4i+3) -> four 16-bit pairs
// (n0,n4) (n1,n5) (n2,n6) (n3,n7), each value (24 + q) / 16.
template <int DT>
__device__ __forceinline__ u32x4 nibbles_to_h16(uint32_t d) {
  using T = H16<DT>;
  u32x4 r;
  r[0] = (shr_signed<0 - T::kShift>(d) & T::kMask) ^ T::kBias;
  r[1] = (shr_signed<4 - T::kShift>(d) & T::kMask) ^ T::kBias;
  r[2] = (shr_signed<8 - T::kShift>(d) & T::kMask) ^ T::kBias;
  r[3] = (shr_signed<12 - T::kShift>(d) & T::kMask) ^ T::kBias;
  return r;
}

// FP4 (E2M1) codes -> 16-bit value / 16 (OCP microscaling formats: 1 sign
// bit, 2 exponent bits with bias 1, 1 mantissa bit, exponent 0 subnormal).
// The magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 divided by 16 are exact in bf16
// and fp16; the division lets the FP4 layout share the INT4 layout's final
// factor 16 and needs no correction term.  One dword of eight codes n0..n7
// (byte b: n_2b in its low nibble, n_2b+1 in its high one) gives the same
// pairs as nibbles_to_h16: (n0,n4) (n1,n5) (n2,n6) (n3,n7).  gfx950 converts
// the two codes of a byte in one instruction (v_cvt_scalef32_pk_*_fp4, the
// value times an FP32 scale, here 1/16: exact); byte permutes then pair the
// codes four apart.
template <int DT>
__device__ __forceinline__ uint32_t fp4_byte_to_h16(uint32_t d, int b);
template <>
__device__ __forceinline__ uint32_t fp4_byte_to_h16<DT_BF16>(uint32_t d, int b) {
  switch (b) {  // the byte select is an immediate
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 0.0625f, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 0.0625f, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 0.0625f, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 0.0625f, 3));
  }
}
template <>
__device__ __forceinline__ uint32_t fp4_byte_to_h16<DT_FP16>(uint32_t d, int b) {
  switch (b) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 0.0625f, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 0.0625f, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 0.0625f, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 0.0625f, 3));
  }
}

template <int DT>
__device__ __forceinline__ u32x4 e2m1_to_h16(uint32_t d) {
  const uint32_t c0 = fp4_byte_to_h16<DT>(d, 0);  // (n0, n1)
  const uint32_t c1 = fp4_byte_to_h16<DT>(d, 1);  // (n2, n3)
  const uint32_t c2 = fp4_byte_to_h16<DT>(d, 2);  // (n4, n5)
  const uint32_t c3 = fp4_byte_to_h16<DT>(d, 3);  // (n6, n7)
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(c2, c0, 0x05040100u);  // (n0, n4)
  r[1] = __builtin_amdgcn_perm(c2, c0, 0x07060302u);  // (n1, n5)
  r[2] = __builtin_amdgcn_perm(c3, c1, 0x05040100u);  // (n2, n6)
  r[3] = __builtin_amdgcn_perm(c3, c1, 0x07060302u);  // (n3, n7)
  return r;
}

// B operand of one 32-value group in the group layouts (after the transpose).
template <int DT, int LAYOUT>
__device__ __forceinline__ u32x4 group_to_h16(uint32_t d) {
  if constexpr (LAYOUT == Q_FP4_GROUP_K) return e2m1_to_h16<DT>(d);
  else return nibbles_to_h16<DT>(d);
}

// Per-channel packing: bytes b0..b7 each hold the value of 8 consecutive
// reduction indices k0..k7 for this lane's output column in the low nibble
// (after the caller shifted odd columns' high nibbles down).  Returns the
// same pair order as nibbles_to_h16: (k0,k4) (k1,k5) (k2,k6) (k3,k7).
template <int DT>
__device__ __forceinline__ u32x4 bytes_to_h16(uint32_t lo4, uint32_t hi4) {
  using T = H16<DT>;
  const uint32_t x = __builtin_amdgcn_perm(hi4, lo4, 0x05040100u);  // [k0 k1 k4 k5]
  const uint32_t y = __builtin_amdgcn_perm(hi4, lo4, 0x07060302u);  // [k2 k3 k6 k7]
  u32x4 r;
  r[0] = (shr_signed<0 - T::kShift>(x) & T::kMask) ^ T::kBias;
  r[1] = (shr_signed<8 - T::kShift>(x) & T::kMask) ^ T::kBias;
  r[2] = (shr_signed<0 - T::kShift>(y) & T::kMask) ^ T::kBias;
  r[3] = (shr_signed<8 - T::kShift>(y) & T::kMask) ^ T::kBias;
  return r;
}

// 8 consecutive 16-bit values (4 dwords, natural order) -> A operand order.
__device__ __forceinline__ u32x4 permute_a(u32x4 v) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);  // (x0, x4)
  r[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);  // (x1, x5)
  r[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);  // (x2, x6)
  r[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);  // (x3, x7)
  return r;
}

// 4x4 transpose of dwords across the four 16-lane rows of a wave: on entry
// row r holds d[0..3] = (r,0..3); on exit row r holds (0..3, r).
__device__ __forceinline__ void transpose_rows4(uint32_t& d0, uint32_t& d1, uint32_t& d2,
                                                uint32_t& d3) {
  auto p02 = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
  auto p13 = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
  auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
  auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
  d0 = q01[0];
  d1 = q01[1];
  d2 = q23[0];
  d3 = q23[1];
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Loads that never sit inside a lane-divergent branch: a lane whose access
// is not wanted reads `safe` (any valid address) instead and gets zeros.  A
// load in a divergent branch makes the compiler wait for it at the branch's
// end, which would serialize every load of a wave.
__device__ __forceinline__ u32x4 load16_if(bool ok, const void* p, const void* safe) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(ok ? p : safe);
  u32x4 r;
  r[0] = ok ? v[0] : 0u;
  r[1] = ok ? v[1] : 0u;
  r[2] = ok ? v[2] : 0u;
  r[3] = ok ? v[3] : 0u;
  return r;
}

// Same with a wave-uniform base and a 32-bit per-lane byte offset (the base
// lives in scalar registers; an unwanted lane reads offset 0 and gets zeros).
__device__ __forceinline__ u32x4 load16_at(const void* base, uint32_t off, bool ok) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + (ok ? off : 0u));
  u32x4 r;
  r[0] = ok ? v[0] : 0u;
  r[1] = ok ? v[1] : 0u;
  r[2] = ok ? v[2] : 0u;
  r[3] = ok ? v[3] : 0u;
  return r;
}

// Raw buffer accesses.  A resource covers [base, base + bytes) with bytes
// below 2^31; a load at an offset at or past the end returns zeros without a
// memory access, so a masked lane simply uses kOob and needs no select after
// the load (a select right behind a load forces an early wait on it).
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ok ? off : kOob, 0, 0));
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, ok ? off : kOob, 0, 0);
}

// 16-bit store; a masked lane writes nothing (the store falls outside the
// resource and is dropped).
__device__ __forceinline__ void bstore2(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok,
                                        uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, ok ? off : kOob, 0, 0);
}

__device__ __forceinline__ uint32_t load4_if(bool ok, const void* p, const void* safe) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(ok ? p : safe);
  return ok ? v : 0u;
}

// Value of the neighbouring lane (lanes 2i and 2i+1 swap), one DPP move.
__device__ __forceinline__ float swap_lane_pairs(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace w4moe
