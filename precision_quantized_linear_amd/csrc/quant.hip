// Online quantization and dequantization kernels (gfx950).
//
// Every kernel reads bf16 in 16-byte chunks (8 elements) with lanes on
// consecutive chunks, so a wave's load covers 1 KB of contiguous memory, and
// writes its codes the same way.  The scale unit decides the reduction:
//   per tensor      two launches: per-block partial maxima, then quantize
//   per row         one wave per row, the row held in registers
//   1x128 group     16 lanes, DPP max inside the 16-lane row
//   128x128 block   one 256-thread workgroup per block
//   32-element MX   4 lanes, DPP quad max
// Scheme definitions: "[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO,
// Quark", section "FP8" (tensor / token / 128x128 dynamic symmetric scales);
// "vLLM-Omni Online Quantization complete guide", section "How online
// quantization works underneath", steps 2-3 (MX: e8m0 per 32 K-elements);
// "vLLM-Omni accelerates inference with AutoRound quantization", section
// "Usage" (int4, group 128, round-to-nearest).
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

constexpr float kSmallestFastScale = 0x1p-80f;

// fp32 scale of the FP8 schemes: s = fp32(amax / 448), 1 if that is 0.
__device__ __forceinline__ float fp8_scale(float amax) {
  float s = __fdiv_rn(amax, 448.0f);
  return s == 0.0f ? 1.0f : s;
}

struct Fp8Div {
  float s, rcp;
  bool fast;
  __device__ __forceinline__ explicit Fp8Div(float s_) : s(s_) {
    rcp = __fdiv_rn(1.0f, s_);
    fast = s_ >= kSmallestFastScale;
  }
  // The correction step turns -0 / s into +0; the quotient's sign is x's (s > 0).
  __device__ __forceinline__ float operator()(float x) const {
    return fast ? __builtin_copysignf(div_rn_markstein(x, s, rcp), x) : __fdiv_rn(x, s);
  }
};

// 8 bf16 -> 8 e4m3fn codes of fp32(x / s).
__device__ __forceinline__ uint2 fp8_chunk(uint4 c, const Fp8Div& d) {
  float f[8];
  chunk_to_f32(c, f);
  uint32_t b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = e4m3_encode(d(f[j]));
  return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                    b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

// ---------------------------------------------------------------- per tensor
// Pass 1: partial[b] = max |x| over the chunks block b visits.
__global__ __launch_bounds__(256) void k_amax_partial(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ldx,
                                                      float* __restrict__ partial) {
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    int64_t r = i / cpr, c = i - r * cpr;
    m = fmaxf(m, chunk_absmax(ldg16(x + r * ldx + c * 8)));
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Pass 2: every block folds the partials into amax, then quantizes its chunks.
__global__ __launch_bounds__(256) void k_fp8_tensor(const uint16_t* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ldx,
                                                    const float* __restrict__ partial, int npartial,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ scale) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < npartial; i += 256) m = fmaxf(m, partial[i]);
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const Fp8Div d(fp8_scale(amax));
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = d.s;
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    int64_t r = i / cpr, c = i - r * cpr;
    stg8(codes + r * cols + c * 8, fp8_chunk(ldg16(x + r * ldx + c * 8), d));
  }
}

// ---------------------------------------------------------------- per row
// One wave per row.  CH > 0: the row (at most 64*CH chunks) stays in
// registers between the max and the cast.  CH == 0: rows too long for that
// are read twice.
template <int CH>
__global__ __launch_bounds__(256) void k_fp8_row(const uint16_t* __restrict__ x, int64_t rows,
                                                 int64_t cols, int64_t ldx,
                                                 uint8_t* __restrict__ codes,
                                                 float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * ldx;
  uint8_t* cr = codes + row * cols;
  const int nch = (int)(cols >> 3);
  if constexpr (CH > 0) {
    uint4 c[CH];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = i * 64 + lane;
      if (ch < nch) {
        c[i] = ldg16(xr + ch * 8);
        m = fmaxf(m, chunk_absmax(c[i]));
      }
    }
    const Fp8Div d(fp8_scale(wave_max(m)));
    if (lane == 0) scales[row] = d.s;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = i * 64 + lane;
      if (ch < nch) stg8(cr + ch * 8, fp8_chunk(c[i], d));
    }
  } else {
    float m = 0.0f;
    for (int ch = lane; ch < nch; ch += 64) m = fmaxf(m, chunk_absmax(ldg16(xr + ch * 8)));
    const Fp8Div d(fp8_scale(wave_max(m)));
    if (lane == 0) scales[row] = d.s;
    for (int ch = lane; ch < nch; ch += 64) stg8(cr + ch * 8, fp8_chunk(ldg16(xr + ch * 8), d));
  }
}

// ---------------------------------------------------------------- 1x128 groups
// One chunk per thread; the 16 chunks of a group sit in one 16-lane DPP row.
__global__ __launch_bounds__(256) void k_fp8_block_act(const uint16_t* __restrict__ x, int64_t rows,
                                                       int64_t cols, int64_t ldx,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
  const int64_t cpr = cols >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = i < rows * cpr;      // whole groups are valid or invalid together
  const int64_t r = valid ? i / cpr : 0, c = valid ? i - r * cpr : 0;
  uint4 v = valid ? ldg16(x + r * ldx + c * 8) : make_uint4(0, 0, 0, 0);
  const Fp8Div d(fp8_scale(group16_max(chunk_absmax(v))));
  if (!valid) return;
  if ((c & 15) == 0) scales[r * (cols >> 7) + (c >> 4)] = d.s;
  stg8(codes + r * cols + c * 8, fp8_chunk(v, d));
}

// ---------------------------------------------------------------- 128x128 blocks
// One workgroup per block: thread t owns chunk (t % 16) of rows t/16 + 16 j.
__global__ __launch_bounds__(256) void k_fp8_block_wt(const uint16_t* __restrict__ x, int64_t cols,
                                                      int64_t ldx, uint8_t* __restrict__ codes,
                                                      float* __restrict__ scales) {
  const int64_t gb = cols >> 7;
  const int64_t rb = blockIdx.x / gb, kb = blockIdx.x - rb * gb;
  const int t = threadIdx.x, cc = t & 15, r0 = t >> 4;
  const uint16_t* xb = x + (rb * 128) * ldx + kb * 128 + cc * 8;
  uint4 v[8];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = ldg16(xb + (int64_t)(r0 + 16 * j) * ldx);
    m = fmaxf(m, chunk_absmax(v[j]));
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  const Fp8Div d(fp8_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
  if (t == 0) scales[blockIdx.x] = d.s;
  uint8_t* cb = codes + (rb * 128) * cols + kb * 128 + cc * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) stg8(cb + (int64_t)(r0 + 16 * j) * cols, fp8_chunk(v[j], d));
}

// ---------------------------------------------------------------- MX
// One chunk per thread; the 4 chunks of a 32-element block share a DPP quad.
template <bool FP4>
__global__ __launch_bounds__(256) void k_mx(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                            int64_t ldx, uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales) {
  const int64_t cpr = cols >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = i < rows * cpr;
  const int64_t r = valid ? i / cpr : 0, c = valid ? i - r * cpr : 0;
  uint4 v = valid ? ldg16(x + r * ldx + c * 8) : make_uint4(0, 0, 0, 0);
  const int X = mx_shared_exponent(group4_max(chunk_absmax(v)), FP4 ? 2 : 8);
  if (!valid) return;
  if ((c & 3) == 0) scales[r * (cols >> 5) + (c >> 2)] = (uint8_t)(X + 127);
  const float inv = exp2i(-X);             // exact scaling: x * 2^-X
  float f[8];
  chunk_to_f32(v, f);
  if constexpr (FP4) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= e2m1_encode(f[j] * inv) << (4 * j);
    *reinterpret_cast<uint32_t*>(codes + r * (cols >> 1) + c * 4) = w;
  } else {
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = e4m3_encode(f[j] * inv);
    stg8(codes + r * cols + c * 8, make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                                              b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)));
  }
}

// ---------------------------------------------------------------- int4 round-to-nearest
// One chunk (= one u32 of codes) per thread; a 128-group is a 16-lane DPP row.
template <bool SYM>
__global__ __launch_bounds__(256) void k_int4(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                              int64_t ldx, uint32_t* __restrict__ codes,
                                              uint16_t* __restrict__ scales,
                                              uint8_t* __restrict__ zeros) {
  const int64_t cpr = cols >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = i < rows * cpr;
  const int64_t r = valid ? i / cpr : 0, c = valid ? i - r * cpr : 0;
  uint4 v = valid ? ldg16(x + r * ldx + c * 8) : make_uint4(0, 0, 0, 0);
  float f[8];
  chunk_to_f32(v, f);
  float s, z;
  if constexpr (SYM) {
    const float amax = group16_max(chunk_absmax(v));
    s = __uint_as_float(f32_to_bf16_rne(__fdiv_rn(amax, 7.0f)) << 16);
    z = 8.0f;
    if (s == 0.0f) s = 1.0f;
  } else {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) { lo = fminf(lo, f[j]); hi = fmaxf(hi, f[j]); }
    lo = group16_min(lo);
    hi = group16_max(hi);
    s = __uint_as_float(f32_to_bf16_rne(__fdiv_rn(hi - lo, 15.0f)) << 16);
    if (s == 0.0f) {
      s = 1.0f;
      z = 0.0f;
    } else {
      z = fminf(fmaxf(__builtin_rintf(__fdiv_rn(-lo, s)), 0.0f), 15.0f);
    }
  }
  if (!valid) return;
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float q = fminf(fmaxf(__builtin_rintf(__fdiv_rn(f[j], s)) + z, 0.0f), 15.0f);
    w |= (uint32_t)q << (4 * j);
  }
  codes[r * cpr + c] = w;
  if ((c & 15) == 0) {
    const int64_t g = r * (cols >> 7) + (c >> 4);
    scales[g] = (uint16_t)(__float_as_uint(s) >> 16);
    zeros[g] = (uint8_t)z;
  }
}

// ---------------------------------------------------------------- dequantize
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t E = (c >> 3) & 0xF, m = c & 7;
  float mag = E == 0 ? (float)m * 0x1p-9f : __uint_as_float(((E + 120u) << 23) | (m << 20));
  if (E == 15 && m == 7) mag = __uint_as_float(0x7fc00000u);
  return (c & 0x80) ? -mag : mag;
}

__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  const uint32_t E = (c >> 1) & 3, m = c & 1;
  float mag = E == 0 ? (float)m * 0.5f : __uint_as_float(((E + 126u) << 23) | (m << 22));
  return (c & 8) ? -mag : mag;
}

// 2^X for X in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float e8m0_value(uint32_t code) {
  if (code == 0) return __uint_as_float(0x00400000u);
  if (code == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(code << 23);
}

__global__ __launch_bounds__(256) void k_dequant(int kind, const uint8_t* __restrict__ codes,
                                                 const void* __restrict__ scales,
                                                 const uint8_t* __restrict__ zeros, int64_t rows,
                                                 int64_t cols, uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t cpr = cols >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cpr) return;
  const int64_t r = i / cpr, c = i - r * cpr;
  float v[8];
  if (kind <= 5) {
    if (kind == 5) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * (cols >> 1) + c * 4);
      const float sc = e8m0_value(static_cast<const uint8_t*>(scales)[r * (cols >> 5) + (c >> 2)]);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e2m1_decode((w >> (4 * j)) & 0xF) * sc;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(codes + r * cols + c * 8);
      float sc;
      const float* sf = static_cast<const float*>(scales);
      switch (kind) {
        case 0: sc = sf[0]; break;
        case 1: sc = sf[r]; break;
        case 2: sc = sf[r * (cols >> 7) + (c >> 4)]; break;
        case 3: sc = sf[(r >> 7) * (cols >> 7) + (c >> 4)]; break;
        default: sc = e8m0_value(static_cast<const uint8_t*>(scales)[r * (cols >> 5) + (c >> 2)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = e4m3_decode((w.x >> (8 * j)) & 0xFF) * sc;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 + j] = e4m3_decode((w.y >> (8 * j)) & 0xFF) * sc;
    }
  } else {
    const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[r * cpr + c];
    const int64_t g = r * (cols >> 7) + (c >> 4);
    const float s = __uint_as_float((uint32_t)static_cast<const uint16_t*>(scales)[g] << 16);
    const float z = (float)zeros[g];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ((float)((w >> (4 * j)) & 0xF) - z) * s;
  }
  uint4 o;
  o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
  o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
  o.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
  o.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
  stg16(y + r * ldy + c * 8, o);
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_quant_fp8_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, float* scale, float* ws_partials, hipStream_t st) {
  const int64_t chunks = rows * (cols >> 3);
  int np = (int)std::min<int64_t>(kTensorAmaxBlocks, std::max<int64_t>(1, blocks_for(chunks)));
  hipLaunchKernelGGL(k_amax_partial, dim3(np), dim3(256), 0, st, x, rows, cols, ldx, ws_partials);
  unsigned nb = (unsigned)std::min<int64_t>(8192, std::max<int64_t>(1, blocks_for(chunks)));
  hipLaunchKernelGGL(k_fp8_tensor, dim3(nb), dim3(256), 0, st, x, rows, cols, ldx, ws_partials, np,
                     codes, scale);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* codes, float* scales, hipStream_t st) {
  const int64_t nch = cols >> 3;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (nch <= 64) hipLaunchKernelGGL(k_fp8_row<1>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 128) hipLaunchKernelGGL(k_fp8_row<2>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 256) hipLaunchKernelGGL(k_fp8_row<4>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 512) hipLaunchKernelGGL(k_fp8_row<8>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 1024) hipLaunchKernelGGL(k_fp8_row<16>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else hipLaunchKernelGGL(k_fp8_row<0>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_block_act(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t* codes, float* scales, hipStream_t st) {
  hipLaunchKernelGGL(k_fp8_block_act, dim3(blocks_for(rows * (cols >> 3))), dim3(256), 0, st, x, rows,
                     cols, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_block_wt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                     uint8_t* codes, float* scales, hipStream_t st) {
  hipLaunchKernelGGL(k_fp8_block_wt, dim3((unsigned)((rows >> 7) * (cols >> 7))), dim3(256), 0, st, x,
                     cols, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mx(bool fp4, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const dim3 grid(blocks_for(rows * (cols >> 3))), block(256);
  if (fp4) hipLaunchKernelGGL(k_mx<true>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else hipLaunchKernelGGL(k_mx<false>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_int4(bool sym, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint32_t* codes, uint16_t* scales, uint8_t* zeros, hipStream_t st) {
  const dim3 grid(blocks_for(rows * (cols >> 3))), block(256);
  if (sym) hipLaunchKernelGGL(k_int4<true>, grid, block, 0, st, x, rows, cols, ldx, codes, scales, zeros);
  else hipLaunchKernelGGL(k_int4<false>, grid, block, 0, st, x, rows, cols, ldx, codes, scales, zeros);
  return hipGetLastError();
}

hipError_t launch_dequant(int kind, const void* codes, const void* scales, const uint8_t* zeros,
                          int64_t rows, int64_t cols, uint16_t* y, int64_t ldy, hipStream_t st) {
  hipLaunchKernelGGL(k_dequant, dim3(blocks_for(rows * (cols >> 3))), dim3(256), 0, st, kind,
                     static_cast<const uint8_t*>(codes), scales, zeros, rows, cols, y, ldy);
  return hipGetLastError();
}

}  // namespace pql
