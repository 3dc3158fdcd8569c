// Element-level steps of the FP8 and int8 quantizers, shared by the quantize
// kernels and the fused small-M quantize + GEMM kernel (internal to the
// library).  Definitions: "[vLLM] Other quantization: FP8, ModelOpt, INC,
// TorchAO, Quark", section "FP8" (s = amax / 448, e4m3fn codes of x / s); the
// online-quantization guide's int8 path (s = amax / 127, integer codes).
#pragma once

#include "pql_device.hpp"

namespace pql {

// Scales at or above this use the reciprocal-and-correction quotient.
constexpr float kSmallestFastScale = 0x1p-80f;

// ---------------------------------------------------------------- FP8 casts
// fp32 scale of the FP8 schemes: s = fp32(amax / 448), 1 if that is 0.
__device__ __forceinline__ float fp8_scale(float amax) {
  float s = __fdiv_rn(amax, 448.0f);
  return s == 0.0f ? 1.0f : s;
}

// fp32(x / s), correctly rounded.  FAST (s >= 2^-80): one reciprocal per
// scale and a Markstein correction per element; the correction turns -0 / s
// into +0, so the sign is taken from x (s > 0).
template <bool FAST>
__device__ __forceinline__ float quot(float x, float s, float rcp) {
  if constexpr (FAST) return __builtin_copysignf(div_rn_markstein(x, s, rcp), x);
  else return __fdiv_rn(x, s);
}

// Four fp32 values -> four e4m3fn codes (byte j = value j) with the hardware
// convert, which rounds to nearest even and keeps the sign of zero.  It agrees
// with the saturating definition for every |v| < 464 (checked on the device for
// all fp32 values) and returns NaN above: FP8 quotients are at most
// 448 (1 + 2^-24) by construction, MX callers clamp to +-448 first.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// 8 bf16 -> 8 e4m3fn codes of fp32(x / s).
template <bool FAST>
__device__ __forceinline__ uint2 fp8_chunk(uint4 c, float s, float rcp) {
  float f[8];
  chunk_to_f32(c, f);
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = quot<FAST>(f[j], s, rcp);
  return make_uint2(fp8x4(f[0], f[1], f[2], f[3]), fp8x4(f[4], f[5], f[6], f[7]));
}

// Static scales: the quotient can exceed 448 (a calibrated scale may be below
// amax / 448) and even overflow fp32 (then the corrected quotient is inf or
// NaN), so every quotient outside [-448, 448] becomes 448 with the sign of x
// before the convert, which is exact inside; zeros keep their sign.
template <bool FAST>
__device__ __forceinline__ uint2 fp8_chunk_sat(uint4 c, float s, float rcp) {
  float f[8];
  chunk_to_f32(c, f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q = quot<FAST>(f[j], s, rcp);
    f[j] = __builtin_fabsf(q) <= 448.0f ? q : __builtin_copysignf(448.0f, f[j]);
  }
  return make_uint2(fp8x4(f[0], f[1], f[2], f[3]), fp8x4(f[4], f[5], f[6], f[7]));
}

// int8 scale: s = fp32(amax / 127), 1 if that is 0.
__device__ __forceinline__ float int8_scale(float amax) {
  float s = __fdiv_rn(amax, 127.0f);
  return s == 0.0f ? 1.0f : s;
}

// 8 bf16 -> 8 int8 codes clamp(rne(fp32(x / s)), -128, 127), byte j = element j.
template <bool FAST>
__device__ __forceinline__ uint2 int8_chunk(uint4 c, float s, float rcp) {
  float f[8];
  chunk_to_f32(c, f);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = __builtin_rintf(quot<FAST>(f[j], s, rcp));   // round half to even
    const int q = (int)__builtin_fminf(__builtin_fmaxf(r, -128.0f), 127.0f);
    w[j >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (j & 3));
  }
  return make_uint2(w[0], w[1]);
}

}  // namespace pql
