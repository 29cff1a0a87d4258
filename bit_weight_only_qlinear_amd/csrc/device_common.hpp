// Device-side helpers for the gfx950 kernels: scalar type conversions with
// explicit rounding, and wave64 cross-lane sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qp {

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// v_cvt_f16_f32: nearest-even, fp16 subnormals kept (default FP mode).
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Correctly rounded fp32 quotient: the fp64 quotient rounded to fp32.
// fp64 carries 53 >= 2*24 + 2 bits, so the double rounding is innocuous
// (Figueroa, "When is double rounding innocuous?", 1995).
__device__ __forceinline__ float div_rn(float a, float b) {
  return (float)((double)a / (double)b);
}

__device__ __forceinline__ float meta_to_f32(uint32_t bits, int meta_bf16) {
  return meta_bf16 ? bf16_to_f32(bits) : f16_to_f32(bits);
}

// DPP row/bank controls (gfx9 encodings).
#define QP_DPP_QUAD_1032 0xB1
#define QP_DPP_QUAD_2301 0x4E
#define QP_DPP_ROW_ROR4 0x124
#define QP_DPP_ROW_ROR8 0x128
#define QP_DPP_ROW_BCAST15 0x142
#define QP_DPP_ROW_BCAST31 0x143

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND = false>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                         __builtin_bit_cast(int, v), CTRL,
                                         ROW_MASK, BANK_MASK, BOUND));
}

#define QP_DPP_ROW_HALF_MIRROR 0x141

// Wave sums of R <= 8 per-lane values at once (a transposed reduction):
// permlane32 / permlane16 swaps pair the values up across lane halves, an
// xor-8 exchange and three DPP steps finish inside 8-lane groups.
// Afterwards the total of value v is in all 8 lanes of group (R, h),
// R = lane >> 4, h = (lane >> 3) & 1, where v = 4 h + ((R & 1) << 1 | R >> 1).
template <int R>
__device__ __forceinline__ float wave_sums8(const float (&v)[R], int lane) {
  static_assert(R >= 1 && R <= 8, "up to 8 values");
  float b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (2 * k >= R) { b[k] = 0.f; continue; }
    const float hi = 2 * k + 1 < R ? v[2 * k + 1] : 0.f;
    // lanes 0-31: value 2k over lanes (l, l + 32); lanes 32-63: value 2k + 1
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * k]), __float_as_uint(hi),
                                                    false, false);
    b[k] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  float c[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    // 16-lane rows 0..3: values 4k, 4k + 2, 4k + 1, 4k + 3 over 4 lanes each
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(b[2 * k]),
                                                    __float_as_uint(b[2 * k + 1]), false, false);
    c[k] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  const bool h = (lane & 8) != 0;
  float d = (h ? c[1] : c[0]) + dpp_f<QP_DPP_ROW_ROR8>(0.f, h ? c[0] : c[1]);
  d += dpp_f<QP_DPP_QUAD_1032>(0.f, d);
  d += dpp_f<QP_DPP_QUAD_2301>(0.f, d);
  d += dpp_f<QP_DPP_ROW_HALF_MIRROR>(0.f, d);
  return d;
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<QP_DPP_QUAD_1032>(0.f, v);
  v += dpp_f<QP_DPP_QUAD_2301>(0.f, v);
  v += dpp_f<QP_DPP_ROW_ROR4>(0.f, v);
  v += dpp_f<QP_DPP_ROW_ROR8>(0.f, v);
  return v;
}

// Sum over all 64 lanes; the total is valid in lane 63.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v = row16_sum(v);
  v += dpp_f<QP_DPP_ROW_BCAST15, 0xA>(0.f, v);
  v += dpp_f<QP_DPP_ROW_BCAST31, 0xC>(0.f, v);
  return v;
}

// Sum over the 32 lanes of each half-wave; valid in lanes 31 and 63.
__device__ __forceinline__ float half_sum_lane31(float v) {
  v = row16_sum(v);
  v += dpp_f<QP_DPP_ROW_BCAST15, 0xA>(0.f, v);
  return v;
}

__device__ __forceinline__ float wave_sum_all(float v) {
  v = wave_sum_lane63(v);
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max_all(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace qp
