// Device-side helpers shared by the libpql kernels (gfx950 / CDNA4).
//
// Element formats (OCP definitions; the pages name the dtypes float8_e4m3fn,
// float8_e8m0fnu and float4_e2m1fn_x2 in "vLLM-Omni Online Quantization
// complete guide", section "How online quantization works underneath"):
//   e4m3fn  sign | 4 exponent bits (bias 7) | 3 mantissa bits, max 448, no inf
//   e2m1    sign | 2 exponent bits (bias 1) | 1 mantissa bit, max 6
//   e8m0    biased exponent only, 2^(c-127)
// Every cast rounds to nearest even, saturates at the largest finite value and
// keeps the sign of zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pql {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------------------ division
// Correctly rounded fp32 x / s from rcp = RN(1/s): q0 = x*rcp is within one
// ulp, the remainder x - s*q0 is exact under fma, and one correction step
// gives the correctly rounded quotient (Markstein's theorem for
// round-to-nearest).  Valid while s is a normal number >= 2^-80; callers fall
// back to the IEEE division outside that range.
__device__ __forceinline__ float div_rn_markstein(float x, float s, float rcp) {
  float q0 = x * rcp;
  float r = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(r, rcp, q0);
}

// ------------------------------------------------------------------ e4m3fn
// RNE, saturating encode of a finite fp32 value.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {                 // |v| >= 448
    code = 0x7eu;
  } else if (a < 0x3c800000u) {           // |v| < 2^-6: subnormal grid, spacing 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {                                // round the fp32 mantissa to 3 bits
    uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    code = r - (120u << 3);               // rebias 127 -> 7
  }
  return sign | code;
}

// ------------------------------------------------------------------ e2m1
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 28) & 0x8u;
  uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x40c00000u) {                 // |v| >= 6
    code = 0x7u;
  } else if (a < 0x3f800000u) {           // |v| < 1: spacing 0.5
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
  } else {                                // round the fp32 mantissa to 1 bit
    uint32_t r = (a + 0x1fffffu + ((a >> 22) & 1u)) >> 22;
    code = r - (126u << 1);               // rebias 127 -> 1
  }
  return sign | code;
}

// ------------------------------------------------------------------ MX exponent
// floor(log2 amax) for amax > 0 from the fp32 bits (subnormals included).
__device__ __forceinline__ int floor_log2_f32(float amax) {
  uint32_t u = __float_as_uint(amax);
  int e = (int)(u >> 23);
  if (e == 0) return -118 - (int)__builtin_clz(u & 0x7fffffu);   // subnormal: m * 2^-149
  return e - 127;
}

// Shared exponent X = clamp(floor(log2 amax) - emax, -127, 127); amax = 0 -> -127.
__device__ __forceinline__ int mx_shared_exponent(float amax, int emax) {
  if (!(amax > 0.0f)) return -127;
  int X = floor_log2_f32(amax) - emax;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// 2^n as fp32 for n in [-126, 127].
__device__ __forceinline__ float exp2i(int n) { return __uint_as_float((uint32_t)(n + 127) << 23); }

// ------------------------------------------------------------------ reductions
// Max over aligned groups of 4 / 16 consecutive lanes, result in every lane
// of the group (DPP quad permutes and row mirrors stay inside the group).
__device__ __forceinline__ float dpp_max_xor1(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_max_xor2(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_max_half_mirror(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_max_mirror(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_min_xor1(float v) {
  return fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_min_xor2(float v) {
  return fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_min_half_mirror(float v) {
  return fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_min_mirror(float v) {
  return fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
}

__device__ __forceinline__ float group4_max(float v) { return dpp_max_xor2(dpp_max_xor1(v)); }
__device__ __forceinline__ float group16_max(float v) {
  return dpp_max_mirror(dpp_max_half_mirror(dpp_max_xor2(dpp_max_xor1(v))));
}
__device__ __forceinline__ float group16_min(float v) {
  return dpp_min_mirror(dpp_min_half_mirror(dpp_min_xor2(dpp_min_xor1(v))));
}
__device__ __forceinline__ float wave_max(float v) {
  v = group16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// ------------------------------------------------------------------ loads / stores
__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void stg8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

// Non-temporal variants for streaming data that is touched exactly once.
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// |x| max of the 8 bf16 values packed in a 16-byte chunk.
__device__ __forceinline__ float chunk_absmax(uint4 c) {
  uint32_t w0 = c.x, w1 = c.y, w2 = c.z, w3 = c.w;
  float m = fmaxf(fabsf(bf16lo(w0)), fabsf(bf16hi(w0)));
  m = fmaxf(m, fmaxf(fabsf(bf16lo(w1)), fabsf(bf16hi(w1))));
  m = fmaxf(m, fmaxf(fabsf(bf16lo(w2)), fabsf(bf16hi(w2))));
  m = fmaxf(m, fmaxf(fabsf(bf16lo(w3)), fabsf(bf16hi(w3))));
  return m;
}

__device__ __forceinline__ void chunk_to_f32(uint4 c, float (&f)[8]) {
  f[0] = bf16lo(c.x); f[1] = bf16hi(c.x);
  f[2] = bf16lo(c.y); f[3] = bf16hi(c.y);
  f[4] = bf16lo(c.z); f[5] = bf16hi(c.z);
  f[6] = bf16lo(c.w); f[7] = bf16hi(c.w);
}

}  // namespace pql
