// Online quantization and dequantization kernels (gfx950).
//
// Every kernel reads bf16 in 16-byte chunks (8 elements) with lanes on
// consecutive chunks, so a wave's load covers 1 KB of contiguous memory, and
// writes its codes the same way.  Inputs read exactly once are loaded
// non-temporally: a 100-200 MB activation would otherwise push the GEMM's
// operands out of the 256 MB Infinity Cache (measured: the C4 MXFP8 step's
// GEMM 481 -> 455 us, its quantize 58 -> 54 us); the per-tensor scheme and the
// two-pass long-row path read their input twice and keep it cached.  The scale unit decides the reduction:
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
// "Usage" (int4, group 128, round-to-nearest).  Static FP8 scales (supplied per
// tensor or per 128-block) from the FP8 section's scheme keys; int8 per-row
// dynamic scales from the online-quantization guide's int8 path (sections "Key
// parameters in detail" and "How online quantization works underneath").
#include "pql_device.hpp"
#include "pql_internal.hpp"
#include "quant_common.hpp"

namespace pql {

namespace {

// ---------------------------------------------------------------- geometry
// Chunk-parallel kernels use row segments: a workgroup is 4 waves, wave w works
// on row 4 * blockIdx.x + w and lane l on chunks (8 bf16 = 16 bytes)
// 64 U blockIdx.y + 64 u + l, u < U, of that row.  No index division, and
// every wave-wide load is 1 KB of one row.  Scale groups (4, 16 or 64 lanes)
// never straddle a 64-chunk slice because K is a multiple of the group.
constexpr int kSegU = 4;
struct Seg {
  int64_t row;
  int lane;
  int64_t c0;   // first chunk of this lane (add 64 u)
  __device__ __forceinline__ Seg() {
    lane = threadIdx.x & 63;
    row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    c0 = (int64_t)blockIdx.y * 64 * kSegU + lane;
  }
};
inline dim3 seg_grid(int64_t rows, int64_t cols) {
  const int64_t cpr = cols >> 3;
  return dim3((unsigned)((rows + 3) / 4), (unsigned)((cpr + 64 * kSegU - 1) / (64 * kSegU)));
}

// ---------------------------------------------------------------- per tensor
// Pass 1: partial[b] = max |x| over the row segments workgroup b visits.
__global__ __launch_bounds__(256) void k_amax_partial(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ldx,
                                                      float* __restrict__ partial) {
  const int64_t cpr = cols >> 3;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t segs = (cpr + 63) >> 6;
  const int64_t units = rows * segs;         // (row, 64-chunk segment) pairs
  float m = 0.0f;
  for (int64_t u = (int64_t)blockIdx.x * 4 + wave; u < units; u += (int64_t)gridDim.x * 4) {
    const int64_t r = u / segs, c = (u - r * segs) * 64 + lane;
    if (c < cpr) m = fmaxf(m, chunk_absmax(ldg16(x + r * ldx + c * 8)));
  }
  m = wave_max(m);
  __shared__ float red[4];
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Pass 2: every workgroup folds the partials into amax, then quantizes its segment.
template <bool FAST>
__device__ __forceinline__ void fp8_tensor_seg(const Seg& g, const uint16_t* xr, uint8_t* cr, int64_t cpr,
                                               float s, float rcp) {
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    if (c < cpr) stg8(cr + c * 8, fp8_chunk<FAST>(ldg16(xr + c * 8), s, rcp));
  }
}
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
  const float s = fp8_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) scale[0] = s;
  const Seg g;
  if (g.row >= rows) return;
  const int64_t cpr = cols >> 3;
  const uint16_t* xr = x + g.row * ldx;
  uint8_t* cr = codes + g.row * cols;
  if (s >= kSmallestFastScale) fp8_tensor_seg<true>(g, xr, cr, cpr, s, __fdiv_rn(1.0f, s));
  else fp8_tensor_seg<false>(g, xr, cr, cpr, s, 0.0f);
}

// ---------------------------------------------------------------- per row
// One wave per row.  CH > 0: the row (at most 64*CH chunks) stays in
// registers between the max and the cast.  CH == 0: rows too long for that
// are read twice.  INT8: the int8 scheme (s = amax / 127, integer codes)
// instead of FP8.
template <bool INT8, bool FAST>
__device__ __forceinline__ uint2 row_chunk(uint4 c, float s, float rcp) {
  if constexpr (INT8) return int8_chunk<FAST>(c, s, rcp);
  else return fp8_chunk<FAST>(c, s, rcp);
}
template <int CH, bool INT8, bool FAST>
__device__ __forceinline__ void fp8_row_cast(const uint4 (&c)[CH > 0 ? CH : 1], const uint16_t* xr, uint8_t* cr,
                                             int nch, int lane, float s, float rcp) {
  if constexpr (CH > 0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = i * 64 + lane;
      if (ch < nch) stg8(cr + ch * 8, row_chunk<INT8, FAST>(c[i], s, rcp));
    }
  } else {
    for (int ch = lane; ch < nch; ch += 64) stg8(cr + ch * 8, row_chunk<INT8, FAST>(ldg16(xr + ch * 8), s, rcp));
  }
}
template <int CH, bool INT8>
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
  uint4 c[CH > 0 ? CH : 1];
  float m = 0.0f;
  if constexpr (CH > 0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = i * 64 + lane;
      c[i] = ch < nch ? ldg16_nt(xr + ch * 8) : make_uint4(0, 0, 0, 0);
      m = fmaxf(m, chunk_absmax(c[i]));
    }
  } else {
    for (int ch = lane; ch < nch; ch += 64) m = fmaxf(m, chunk_absmax(ldg16(xr + ch * 8)));
  }
  const float amax = wave_max(m);
  const float s = INT8 ? int8_scale(amax) : fp8_scale(amax);
  if (lane == 0) scales[row] = s;
  if (s >= kSmallestFastScale) fp8_row_cast<CH, INT8, true>(c, xr, cr, nch, lane, s, __fdiv_rn(1.0f, s));
  else fp8_row_cast<CH, INT8, false>(c, xr, cr, nch, lane, s, 0.0f);
}

// ---------------------------------------------------------------- static FP8 scales
// Row segments; every chunk looks its scale up: MODE 0 one scale per tensor,
// 1 one per (row, 128-group) (activations), 2 one per 128x128 block (weights).
template <int MODE>
__global__ __launch_bounds__(256) void k_fp8_static(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ldx, const float* __restrict__ scales,
                                                    uint8_t* __restrict__ codes) {
  const Seg g;
  if (g.row >= rows) return;
  const int64_t cpr = cols >> 3, gpr = cols >> 7;
  const uint16_t* xr = x + g.row * ldx;
  uint8_t* cr = codes + g.row * cols;
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    if (c >= cpr) continue;
    const float s = MODE == 0 ? scales[0]
                    : MODE == 1 ? scales[g.row * gpr + (c >> 4)]
                                : scales[(g.row >> 7) * gpr + (c >> 4)];
    const uint4 v = ldg16_nt(xr + c * 8);
    uint2 q;
    if (s >= kSmallestFastScale) q = fp8_chunk_sat<true>(v, s, __fdiv_rn(1.0f, s));
    else q = fp8_chunk_sat<false>(v, s, 0.0f);
    stg8(cr + c * 8, q);
  }
}

// ---------------------------------------------------------------- 1x128 groups
// Row segments; the 16 chunks of a group sit in one 16-lane DPP row.
__global__ __launch_bounds__(256) void k_fp8_block_act(const uint16_t* __restrict__ x, int64_t rows,
                                                       int64_t cols, int64_t ldx,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
  const Seg g;
  if (g.row >= rows) return;
  const int64_t cpr = cols >> 3;
  const uint16_t* xr = x + g.row * ldx;
  uint4 v[kSegU];
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    v[u] = c < cpr ? ldg16_nt(xr + c * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    const float s = fp8_scale(group16_max(chunk_absmax(v[u])));   // whole groups are in or out of range
    if (c >= cpr) continue;
    if ((c & 15) == 0) scales[g.row * (cols >> 7) + (c >> 4)] = s;
    uint2 q;
    if (s >= kSmallestFastScale) q = fp8_chunk<true>(v[u], s, __fdiv_rn(1.0f, s));
    else q = fp8_chunk<false>(v[u], s, 0.0f);
    stg8(codes + g.row * cols + c * 8, q);
  }
}

// ---------------------------------------------------------------- 128x128 blocks
// One workgroup per block: thread t owns chunk (t % 16) of rows t/16 + 16 j.
template <bool FAST>
__device__ __forceinline__ void fp8_block_wt_cast(const uint4 (&v)[8], uint8_t* cb, int64_t cols, int r0, float s,
                                                  float rcp) {
#pragma unroll
  for (int j = 0; j < 8; ++j) stg8(cb + (int64_t)(r0 + 16 * j) * cols, fp8_chunk<FAST>(v[j], s, rcp));
}
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
    v[j] = ldg16_nt(xb + (int64_t)(r0 + 16 * j) * ldx);
    m = fmaxf(m, chunk_absmax(v[j]));
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  const float s = fp8_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  if (t == 0) scales[blockIdx.x] = s;
  uint8_t* cb = codes + (rb * 128) * cols + kb * 128 + cc * 8;
  if (s >= kSmallestFastScale) fp8_block_wt_cast<true>(v, cb, cols, r0, s, __fdiv_rn(1.0f, s));
  else fp8_block_wt_cast<false>(v, cb, cols, r0, s, 0.0f);
}

// ---------------------------------------------------------------- MX
// Row segments; the 4 chunks of a 32-element block share a DPP quad.  The
// scaling x * 2^-X is exact; e4m3 values in (448, 512) saturate (clamped before
// the hardware convert), e2m1 values above 6 saturate in the convert itself
// (which agrees with the definition for every fp32 value at unit scale).
template <bool FP4>
__global__ __launch_bounds__(256) void k_mx(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                            int64_t ldx, uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales) {
  const Seg g;
  if (g.row >= rows) return;
  const int64_t cpr = cols >> 3;
  const uint16_t* xr = x + g.row * ldx;
  uint4 v[kSegU];
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    v[u] = c < cpr ? ldg16_nt(xr + c * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    const int X = mx_shared_exponent(group4_max(chunk_absmax(v[u])), FP4 ? 2 : 8);
    if (c >= cpr) continue;
    if ((c & 3) == 0) {   // packed exponent layout: [chunk][row][kC]
      constexpr int kC = mx_chunk(FP4);
      const int64_t b = c >> 2;
      uint8_t* sp = scales + ((b / kC) * rows + g.row) * kC + (b % kC);
      sp[0] = (uint8_t)(X + 127);
      if (b == (cols >> 5) - 1)   // the row's last block fills the rest of its chunk
        for (int p = 1; p < kC - (int)(b % kC); ++p) sp[p] = 127;
    }
    const float inv = exp2i(-X);
    float f[8];
    chunk_to_f32(v[u], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] *= inv;
    if constexpr (FP4) {
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0], f[1], 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], 1.0f, 3);
      *reinterpret_cast<uint32_t*>(codes + g.row * (cols >> 1) + c * 4) = w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = __builtin_amdgcn_fmed3f(f[j], -448.0f, 448.0f);
      stg8(codes + g.row * cols + c * 8, make_uint2(fp8x4(f[0], f[1], f[2], f[3]), fp8x4(f[4], f[5], f[6], f[7])));
    }
  }
}

// ---------------------------------------------------------------- dual-scale MXFP4
// Two online scale levels: a coarse fp32 scale per 512 K-elements and a fine
// e8m0 exponent per 32 ("vLLM-Omni Online Quantization complete guide",
// section "How online quantization works underneath", MXFP4 paragraph; the
// calibrated multiplier of offline checkpoints is all ones online, so x is
// used as it is).  s_c = fp32(amax_512 / 6) (1 if 0); v = fp32(x / s_c),
// correctly rounded like the FP8 quotient; then MX on v: X = floor(log2
// max|v|) - 2 per 32-block, code = e2m1 RNE_sat(v * 2^-X).
// Row segments: with K % 512 == 0 a lane slice of 64 chunks is exactly one
// coarse block, so its amax is a wave reduction (every lane of a wave shares
// the row and the slice); a fine block is a DPP quad.  Fine exponents go to the
// packed MXFP4 layout [G, rows, 8] (K % 512 == 0: no pad bytes), coarse scales
// group-major [K / 512, rows].
__global__ __launch_bounds__(256) void k_mx4_dual(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                  int64_t ldx, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ fine, float* __restrict__ coarse) {
  const Seg g;
  if (g.row >= rows) return;   // wave-uniform: a wave is one row
  const int64_t cpr = cols >> 3;
  const uint16_t* xr = x + g.row * ldx;
  const int64_t slice0 = g.c0 - g.lane;   // first chunk of the wave's first slice
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    if (slice0 + 64 * u >= cpr) break;    // wave-uniform (cpr is a multiple of 64)
    const int64_t c = g.c0 + 64 * u;
    const uint4 v = ldg16_nt(xr + c * 8);
    const float amax = wave_max(chunk_absmax(v));
    float sc = __fdiv_rn(amax, 6.0f);
    sc = sc == 0.0f ? 1.0f : sc;
    const int64_t cb = (slice0 + 64 * u) >> 6;   // coarse block of this slice
    if (g.lane == 0) coarse[cb * rows + g.row] = sc;
    float f[8];
    chunk_to_f32(v, f);
    if (sc >= kSmallestFastScale) {
      const float rcp = __fdiv_rn(1.0f, sc);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = quot<true>(f[j], sc, rcp);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = quot<false>(f[j], sc, 0.0f);
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(f[j]));
    const int X = mx_shared_exponent(group4_max(m), 2);
    if ((c & 3) == 0) {
      const int64_t b = c >> 2;
      fine[((b >> 3) * rows + g.row) * 8 + (b & 7)] = (uint8_t)(X + 127);
    }
    const float inv = exp2i(-X);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] *= inv;
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0], f[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], 1.0f, 3);
    *reinterpret_cast<uint32_t*>(codes + g.row * (cols >> 1) + c * 4) = w;
  }
}

// ---------------------------------------------------------------- int4 round-to-nearest
// Row segments; a 128-group is a 16-lane DPP row.  One chunk = one u32 of codes.
template <bool SYM>
__global__ __launch_bounds__(256) void k_int4(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                              int64_t ldx, uint32_t* __restrict__ codes,
                                              uint16_t* __restrict__ scales,
                                              uint8_t* __restrict__ zeros) {
  const Seg g;
  if (g.row >= rows) return;
  const int64_t cpr = cols >> 3;
  const uint16_t* xr = x + g.row * ldx;
  uint4 v[kSegU];
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    v[u] = c < cpr ? ldg16_nt(xr + c * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    float f[8];
    chunk_to_f32(v[u], f);
    // The group's range over its fixed divisor (7 or 15) and -lo / s are correctly rounded
    // quotients: by reciprocal and one correction where the quotient is a normal number (a
    // finite dividend of at least 2^-100), by the IEEE division otherwise.
    auto by_const = [](float d, float den, float rcp_den) {
      return d >= 0x1p-100f && d <= 0x1.fffffep127f ? div_rn_markstein(d, den, rcp_den) : __fdiv_rn(d, den);
    };
    float s, z, lo = 0.0f, hi = 0.0f;
    if constexpr (SYM) {
      const float amax = group16_max(chunk_absmax(v[u]));
      s = __uint_as_float(f32_to_bf16_rne(by_const(amax, 7.0f, 1.0f / 7.0f)) << 16);
      z = 8.0f;
      if (s == 0.0f) s = 1.0f;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) { lo = fminf(lo, f[j]); hi = fmaxf(hi, f[j]); }
      lo = group16_min(lo);
      hi = group16_max(hi);
      s = __uint_as_float(f32_to_bf16_rne(by_const(hi - lo, 15.0f, 1.0f / 15.0f)) << 16);
      z = 0.0f;
      if (s == 0.0f) s = 1.0f;
    }
    if (c >= cpr) continue;
    // Element quotients x / s (and -lo / s): a zero quotient's sign cannot change a code
    // (rint(+-0) + z = z), so the correction's +0 for -0 needs no sign fix-up.
    const bool fast = s >= kSmallestFastScale;
    const float rcp = fast ? __fdiv_rn(1.0f, s) : 0.0f;
    if constexpr (!SYM) {
      if (hi - lo > 0.0f)   // s == 1 from a zero range keeps z = 0
        z = fminf(fmaxf(__builtin_rintf(fast ? div_rn_markstein(-lo, s, rcp) : __fdiv_rn(-lo, s)), 0.0f), 15.0f);
    }
    float q[8];
    if (fast) {
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = div_rn_markstein(f[j], s, rcp);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = __fdiv_rn(f[j], s);
    }
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= (uint32_t)fminf(fmaxf(__builtin_rintf(q[j]) + z, 0.0f), 15.0f) << (4 * j);
    codes[g.row * cpr + c] = w;
    if ((c & 15) == 0) {
      const int64_t gi = (c >> 4) * rows + g.row;   // group-major
      scales[gi] = (uint16_t)(__float_as_uint(s) >> 16);
      zeros[gi] = (uint8_t)z;
    }
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Dequantize, one instance per code layout (KIND as numbered by the launcher):
// every chunk's codes and scales are loaded before any is converted (a chunk
// past the row repeats the row's last and is not stored), so the loads of a
// lane are in flight together.
template <int KIND>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
                                                 const uint8_t* __restrict__ zeros, int64_t rows, int64_t cols,
                                                 uint16_t* __restrict__ y, int64_t ldy) {
  constexpr bool kFp4 = KIND == 5 || KIND == 8;   // MXFP4, dual-scale MXFP4: 4 code bytes per chunk
  constexpr bool kInt4 = KIND == 6;               // W4A16: 4 code bytes, bf16 scale and zero-point per group
  const Seg g;
  if (g.row >= rows) return;
  const int64_t cpr = cols >> 3, r = g.row;
  const float* sf = static_cast<const float*>(scales);
  const uint8_t* sb = static_cast<const uint8_t*>(scales);
  uint2 w8[kSegU];
  uint32_t w4[kSegU];
  float sc[kSegU], aux[kSegU];   // aux: the int4 zero-point, or the dual-scale coarse scale
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u < cpr ? g.c0 + 64 * u : cpr - 1;
    if constexpr (kFp4) {
      w4[u] = *reinterpret_cast<const uint32_t*>(codes + r * (cols >> 1) + c * 4);
      const int64_t b = c >> 2;
      sc[u] = e8m0_value(sb[((b >> 3) * rows + r) * 8 + (b & 7)]);
      if constexpr (KIND == 8) aux[u] = reinterpret_cast<const float*>(zeros)[(c >> 6) * rows + r];
    } else if constexpr (kInt4) {
      w4[u] = reinterpret_cast<const uint32_t*>(codes)[r * cpr + c];
      const int64_t gi = (c >> 4) * rows + r;   // group-major
      sc[u] = __uint_as_float((uint32_t)static_cast<const uint16_t*>(scales)[gi] << 16);
      aux[u] = (float)zeros[gi];
    } else {
      w8[u] = *reinterpret_cast<const uint2*>(codes + r * cols + c * 8);
      if constexpr (KIND == 0) sc[u] = sf[0];
      else if constexpr (KIND == 1 || KIND == 7) sc[u] = sf[r];
      else if constexpr (KIND == 2) sc[u] = sf[r * (cols >> 7) + (c >> 4)];
      else if constexpr (KIND == 3) sc[u] = sf[(r >> 7) * (cols >> 7) + (c >> 4)];
      else {   // MXFP8
        const int64_t b = c >> 2;
        sc[u] = e8m0_value(sb[((b >> 2) * rows + r) * 4 + (b & 3)]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const int64_t c = g.c0 + 64 * u;
    float v[8];
    if constexpr (kFp4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e2m1_decode((w4[u] >> (4 * j)) & 0xF) * sc[u];   // exact
      if constexpr (KIND == 8) {   // dual-scale: times the coarse scale, one rounding
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= aux[u];
      }
    } else if constexpr (kInt4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ((float)((w4[u] >> (4 * j)) & 0xF) - aux[u]) * sc[u];
    } else if constexpr (KIND == 7) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = (float)(int8_t)(((j < 4 ? w8[u].x : w8[u].y) >> (8 * (j & 3))) & 0xFF) * sc[u];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = e4m3_decode((w8[u].x >> (8 * j)) & 0xFF) * sc[u];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 + j] = e4m3_decode((w8[u].y >> (8 * j)) & 0xFF) * sc[u];
    }
    if (c < cpr)
      stg16(y + r * ldy + c * 8, make_uint4(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]), bf16x2_rne(v[4], v[5]),
                                            bf16x2_rne(v[6], v[7])));
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_quant_fp8_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, float* scale, float* ws_partials, hipStream_t st) {
  const int64_t units = rows * (((cols >> 3) + 63) >> 6);
  const int np = (int)std::min<int64_t>(kTensorAmaxBlocks, std::max<int64_t>(1, (units + 3) / 4));
  hipLaunchKernelGGL(k_amax_partial, dim3(np), dim3(256), 0, st, x, rows, cols, ldx, ws_partials);
  hipLaunchKernelGGL(k_fp8_tensor, seg_grid(rows, cols), dim3(256), 0, st, x, rows, cols, ldx, ws_partials, np,
                     codes, scale);
  return hipGetLastError();
}

template <bool INT8>
hipError_t launch_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes, float* scales,
                      hipStream_t st) {
  const int64_t nch = cols >> 3;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (nch <= 64) hipLaunchKernelGGL((k_fp8_row<1, INT8>), grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 128) hipLaunchKernelGGL((k_fp8_row<2, INT8>), grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 256) hipLaunchKernelGGL((k_fp8_row<4, INT8>), grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 384) hipLaunchKernelGGL((k_fp8_row<6, INT8>), grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 512) hipLaunchKernelGGL((k_fp8_row<8, INT8>), grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else if (nch <= 1024) hipLaunchKernelGGL((k_fp8_row<16, INT8>), grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else hipLaunchKernelGGL((k_fp8_row<0, INT8>), grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* codes, float* scales, hipStream_t st) {
  return launch_row<false>(x, rows, cols, ldx, codes, scales, st);
}

hipError_t launch_quant_int8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* codes, float* scales, hipStream_t st) {
  return launch_row<true>(x, rows, cols, ldx, codes, scales, st);
}

hipError_t launch_quant_fp8_static(int mode, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   const float* scales, uint8_t* codes, hipStream_t st) {
  const dim3 grid = seg_grid(rows, cols), block(256);
  if (mode == 0) hipLaunchKernelGGL(k_fp8_static<0>, grid, block, 0, st, x, rows, cols, ldx, scales, codes);
  else if (mode == 1) hipLaunchKernelGGL(k_fp8_static<1>, grid, block, 0, st, x, rows, cols, ldx, scales, codes);
  else hipLaunchKernelGGL(k_fp8_static<2>, grid, block, 0, st, x, rows, cols, ldx, scales, codes);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_block_act(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t* codes, float* scales, hipStream_t st) {
  hipLaunchKernelGGL(k_fp8_block_act, seg_grid(rows, cols), dim3(256), 0, st, x, rows, cols, ldx, codes, scales);
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
  const dim3 grid = seg_grid(rows, cols), block(256);
  if (fp4) hipLaunchKernelGGL(k_mx<true>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  else hipLaunchKernelGGL(k_mx<false>, grid, block, 0, st, x, rows, cols, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mx4_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                                uint8_t* fine, float* coarse, hipStream_t st) {
  hipLaunchKernelGGL(k_mx4_dual, seg_grid(rows, cols), dim3(256), 0, st, x, rows, cols, ldx, codes, fine, coarse);
  return hipGetLastError();
}

hipError_t launch_quant_int4(bool sym, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint32_t* codes, uint16_t* scales, uint8_t* zeros, hipStream_t st) {
  const dim3 grid = seg_grid(rows, cols), block(256);
  if (sym) hipLaunchKernelGGL(k_int4<true>, grid, block, 0, st, x, rows, cols, ldx, codes, scales, zeros);
  else hipLaunchKernelGGL(k_int4<false>, grid, block, 0, st, x, rows, cols, ldx, codes, scales, zeros);
  return hipGetLastError();
}

hipError_t launch_dequant(int kind, const void* codes, const void* scales, const uint8_t* zeros,
                          int64_t rows, int64_t cols, uint16_t* y, int64_t ldy, hipStream_t st) {
  const dim3 grid = seg_grid(rows, cols), block(256);
  const uint8_t* cb = static_cast<const uint8_t*>(codes);
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_dequant<0>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 1: hipLaunchKernelGGL(k_dequant<1>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 2: hipLaunchKernelGGL(k_dequant<2>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 3: hipLaunchKernelGGL(k_dequant<3>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 4: hipLaunchKernelGGL(k_dequant<4>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 5: hipLaunchKernelGGL(k_dequant<5>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 6: hipLaunchKernelGGL(k_dequant<6>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 7: hipLaunchKernelGGL(k_dequant<7>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    case 8: hipLaunchKernelGGL(k_dequant<8>, grid, block, 0, st, cb, scales, zeros, rows, cols, y, ldy); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pql
