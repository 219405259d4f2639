// device_math.hpp -- fp32 device helpers for the selective scan kernels (gfx950).
//
// Every function here is written from its mathematical definition on top of
// the hardware base-2 exponential / logarithm / reciprocal (v_exp_f32,
// v_log_f32, v_rcp_f32), with the error analysis stated next to it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mamba {

constexpr float kLog2e = 1.4426950408889634f;  // 1 / ln 2
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// bf16 <-> fp32.  Widening is exact (bf16 is the top half of an fp32 pattern);
// narrowing rounds to nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// softplus(x) = max(x, 0) + log(1 + e^-|x|).
// With e = e^-|x| in (0, 1] and w = fl(1 + e), the rounding error of the sum
// is c = e - (w - 1) exactly (w - 1 is exact by Sterbenz; |c| <= 2^-24), and
// log(1 + e) = log(w) + c / w + O(c^2) = ln2 * log2(w) + c - c (w - 1) / w.
// Dropping the last term costs at most c * e <= 2^-24 * e, a relative error
// of 2^-24 of the result, so small arguments (where w rounds to 1) keep full
// relative precision instead of losing it to the 1 + e rounding.
__device__ __forceinline__ float softplus(float x) {
  const float e = hw_exp2(-__builtin_fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float c = e - (w - 1.0f);
  return __builtin_fmaxf(x, 0.0f) + __builtin_fmaf(hw_log2(w), kLn2, c);
}

// z * sigmoid(z) = z / (1 + e^-z).  For z -> -inf, e^-z -> +inf, the
// reciprocal -> 0 and the product -> -0 (the right limit); no NaN arises.
__device__ __forceinline__ float silu(float z) {
  return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

// e^y - 1 for y = x2 * ln2 given x2 (the exponent in base-2 units) and
// e2 = 2^x2 already evaluated.  For |y| < 1/8 the Taylor series to y^6 is used
// (truncation < y^7/5040 relative, below 2^-24 there); otherwise e2 - 1 has a
// relative error below 2^-24 / (1 - e^-1/8) < 2^-20.
__device__ __forceinline__ float expm1_from_exp2(float x2, float e2) {
  const float y = x2 * kLn2;
  float p = __builtin_fmaf(y, 1.0f / 720.0f, 1.0f / 120.0f);
  p = __builtin_fmaf(y, p, 1.0f / 24.0f);
  p = __builtin_fmaf(y, p, 1.0f / 6.0f);
  p = __builtin_fmaf(y, p, 0.5f);
  p = __builtin_fmaf(y, p, 1.0f);
  const float series = y * p;
  return (__builtin_fabsf(y) < 0.125f) ? series : (e2 - 1.0f);
}

}  // namespace mamba
