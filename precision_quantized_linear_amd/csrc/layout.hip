// Scale-layout conversion between the library's packed (device) layout and the
// canonical one (gfx950).
//
// Codes are the same bytes in both layouts.  Scales and zero-points differ for
// two schemes:
//   MX (e8m0 per 32 K-elements; "vLLM-Omni Online Quantization complete
//   guide", section "How online quantization works underneath", steps 2-3):
//     canonical u8 [rows, nblk]; packed u8 [G, rows, c] with c = 4 (MXFP8) or
//     8 (MXFP4) exponents per 128 bytes of codes, G = ceil(nblk / c), byte
//     [g, r, b] = canonical [r, c g + b], bytes past a row's last block 127.
//   W4A16 (bf16 scale and 4-bit zero-point per 128-element K-group; "vLLM-Omni
//     accelerates inference with AutoRound quantization", section "Usage"):
//     canonical [rows, groups]; packed group-major [groups, rows].
// Both conversions are bijections on the bytes that carry values (the MX pad
// bytes are rebuilt), so packing an unpacked tensor gives back the same bytes.
#include <algorithm>

#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

constexpr int kThreads = 256;

inline unsigned blocks_for(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (unsigned)std::min<int64_t>(b, 1 << 20);   // grid-stride loops cover the rest
}

// packed [G, rows, c] <- canonical [rows, nblk]; one thread per packed byte.
__global__ __launch_bounds__(kThreads) void k_mx_pack(const uint8_t* __restrict__ canon, int64_t rows, int64_t nblk,
                                                      int c, uint8_t* __restrict__ packed) {
  const int64_t G = (nblk + c - 1) / c;
  const int64_t n = G * rows * c;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t b = i % c, r = (i / c) % rows, g = i / (c * rows);
    const int64_t j = g * c + b;
    packed[i] = j < nblk ? canon[r * nblk + j] : (uint8_t)127;
  }
}

// canonical [rows, nblk] <- packed [G, rows, c]; one thread per canonical byte.
__global__ __launch_bounds__(kThreads) void k_mx_unpack(const uint8_t* __restrict__ packed, int64_t rows,
                                                        int64_t nblk, int c, uint8_t* __restrict__ canon) {
  const int64_t n = rows * nblk;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / nblk, j = i % nblk;
    canon[i] = packed[((j / c) * rows + r) * c + j % c];
  }
}

// out[C, R] = in[R, C]^T through a 32 x 33 LDS tile (coalesced on both sides);
// a 1-D grid walks the tiles, so neither dimension is limited by a grid axis.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_transpose(const T* __restrict__ in, int64_t R, int64_t C,
                                                        T* __restrict__ out) {
  __shared__ T tile[32][33];
  const int64_t tiles_c = (C + 31) / 32, ntiles = ((R + 31) / 32) * tiles_c;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8 threads
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t r0 = (t / tiles_c) * 32, c0 = (t % tiles_c) * 32;
    for (int k = ty; k < 32; k += 8) {
      const int64_t r = r0 + k, c = c0 + tx;
      if (r < R && c < C) tile[k][tx] = in[r * C + c];
    }
    __syncthreads();
    for (int k = ty; k < 32; k += 8) {
      const int64_t c = c0 + k, r = r0 + tx;
      if (r < R && c < C) out[c * R + r] = tile[tx][k];
    }
    __syncthreads();
  }
}

template <typename T>
hipError_t transpose(const void* in, int64_t R, int64_t C, void* out, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  const int64_t ntiles = ((R + 31) / 32) * ((C + 31) / 32);
  const unsigned grid = (unsigned)std::min<int64_t>(ntiles, 1 << 20);
  hipLaunchKernelGGL(k_transpose<T>, dim3(grid), dim3(kThreads), 0, st, static_cast<const T*>(in), R, C,
                     static_cast<T*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_repack(bool to_packed, bool fp4, const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out,
                            hipStream_t st) {
  const int c = mx_chunk(fp4);
  const int64_t nblk = cols / 32;
  if (rows == 0) return hipSuccess;
  if (to_packed) {
    const int64_t n = mx_chunks(cols, fp4) * rows * c;
    hipLaunchKernelGGL(k_mx_pack, dim3(blocks_for(n)), dim3(kThreads), 0, st, in, rows, nblk, c, out);
  } else {
    hipLaunchKernelGGL(k_mx_unpack, dim3(blocks_for(rows * nblk)), dim3(kThreads), 0, st, in, rows, nblk, c, out);
  }
  return hipGetLastError();
}

hipError_t launch_transpose_f32(const float* in, int64_t R, int64_t C, float* out, hipStream_t st) {
  return transpose<uint32_t>(in, R, C, out, st);
}

hipError_t launch_group_repack(bool to_packed, const uint16_t* scales_in, const uint8_t* zeros_in, int64_t rows,
                               int64_t groups, uint16_t* scales_out, uint8_t* zeros_out, hipStream_t st) {
  // canonical [rows, groups] -> packed [groups, rows] and back: a transpose either way
  const int64_t R = to_packed ? rows : groups, C = to_packed ? groups : rows;
  hipError_t e = transpose<uint16_t>(scales_in, R, C, scales_out, st);
  if (e != hipSuccess || !zeros_in) return e;
  return transpose<uint8_t>(zeros_in, R, C, zeros_out, st);
}

}  // namespace pql
