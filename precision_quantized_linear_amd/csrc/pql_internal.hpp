// Host-side interface between the C ABI (abi.cpp) and the kernel launchers.
// Launchers assume their arguments were validated by the ABI layer and return
// the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pql {

// Number of per-block partial maxima the per-tensor amax pass writes.
constexpr int kTensorAmaxBlocks = 1024;

// Packed MX exponents: the e8m0 bytes of a [rows, cols] operand are stored as
// [ceil(cols / (32 c)), rows, c] with c = 4 (MXFP8) or 8 (MXFP4) -- byte b of
// chunk g of row r is the exponent of 32-block c g + b, and bytes past the
// row's last block hold 127.  One chunk covers the 128 K-bytes of codes that
// the GEMM stages per step, so a step's exponents for consecutive rows are
// consecutive bytes.
constexpr int mx_chunk(bool fp4) { return fp4 ? 8 : 4; }
constexpr int64_t mx_chunks(int64_t cols, bool fp4) { return (cols / 32 + mx_chunk(fp4) - 1) / mx_chunk(fp4); }
constexpr int64_t mx_packed_row_bytes(int64_t cols, bool fp4) { return mx_chunks(cols, fp4) * mx_chunk(fp4); }

// ---------------------------------------------------------------- quantize
hipError_t launch_quant_fp8_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, float* scale, float* ws_partials, hipStream_t st);
hipError_t launch_quant_fp8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_quant_int8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* codes, float* scales, hipStream_t st);
// Static (supplied) FP8 scales: mode 0 per tensor, 1 per (row, 128-group), 2 per 128x128 block.
hipError_t launch_quant_fp8_static(int mode, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   const float* scales, uint8_t* codes, hipStream_t st);
hipError_t launch_quant_fp8_block_act(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_quant_fp8_block_wt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                     uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_quant_mx(bool fp4, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, hipStream_t st);
// Dual-scale MXFP4 (K % 512 == 0): codes [rows, K/2], fine exponents packed [K/256, rows, 8],
// coarse fp32 scales group-major [K/512, rows].
hipError_t launch_quant_mx4_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                                uint8_t* fine, float* coarse, hipStream_t st);
hipError_t launch_quant_int4(bool sym, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint32_t* codes, uint16_t* scales, uint8_t* zeros, hipStream_t st);

// ---------------------------------------------------------------- dequantize
// kind: 0 fp8 tensor, 1 fp8 row, 2 fp8 block act, 3 fp8 block weight, 4 mxfp8,
//       5 mxfp4, 6 int4, 7 int8 row, 8 dual-scale mxfp4 (zeros = its coarse fp32 scales)
hipError_t launch_dequant(int kind, const void* codes, const void* scales, const uint8_t* zeros,
                          int64_t rows, int64_t cols, uint16_t* y, int64_t ldy, hipStream_t st);

// ---------------------------------------------------------------- layouts
// MX exponents: canonical [rows, cols / 32] <-> packed [G, rows, c] (to_packed picks the direction).
hipError_t launch_mx_repack(bool to_packed, bool fp4, const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out,
                            hipStream_t st);
// W4A16 scales (and zero-points, if zeros_in is non-null): canonical [rows, groups] <-> group-major [groups, rows].
// fp32 [R, C] -> [C, R] (dual-scale MXFP4 coarse scales between canonical and group-major).
hipError_t launch_transpose_f32(const float* in, int64_t R, int64_t C, float* out, hipStream_t st);
hipError_t launch_group_repack(bool to_packed, const uint16_t* scales_in, const uint8_t* zeros_in, int64_t rows,
                               int64_t groups, uint16_t* scales_out, uint8_t* zeros_out, hipStream_t st);

// ---------------------------------------------------------------- GEMM
enum GemmKind { GEMM_FP8_ROWSCALE = 0, GEMM_FP8_BLOCK = 1, GEMM_MXFP8 = 2, GEMM_MXFP4 = 3, GEMM_INT8_ROW = 4 };

struct GemmArgs {
  const uint8_t* a;        // A codes [M, K] (fp4: [M, K/2])
  const uint8_t* w;        // W codes [N, K] (fp4: [N, K/2])
  const void* a_scales;    // fp32 or e8m0, per kind
  const void* w_scales;
  int64_t a_scale_stride;  // fp8 row-scale kind: 0 = one scale for all rows, 1 = per row
  int64_t w_scale_stride;
  int64_t M, N, K;
  uint16_t* c;             // bf16 [M, ldc]
  int64_t ldc;
  int vec_store;           // 1 if c and ldc allow 16-byte row stores
  float alpha;             // epilogue: C = alpha * (A_hat W_hat^T) + bias (FP8 and int8 kinds)
  const uint16_t* bias;    // bf16 [N], or null for none
};

hipError_t launch_gemm(GemmKind kind, const GemmArgs& g, hipStream_t st);
// Persistent 32x32x64 kernels: FP8 tensor / row scales, and MXFP8 / MXFP4
// (MXFP4 needs K % 256 == 0, MXFP8 K % 128 == 0).
hipError_t launch_gemm32_fp8(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm32_mx(bool fp4, const GemmArgs& g, hipStream_t st);
// Same kernel with the int8 matrix cores (int32 sums), per-row scales.
hipError_t launch_gemm32_int8(const GemmArgs& g, hipStream_t st);
// Persistent FP8 block-128 kernel (16x16x128 MFMA per K-group, FMA promotion; N % 128 == 0).
hipError_t launch_gemm_block(const GemmArgs& g, hipStream_t st);
// The block-128 GEMM runs 256 x 256 tiles on 8 waves when they fill at least
// one round of the 256 CUs, else 256 x 128 tiles on 4 waves.
inline bool gemm_block_uses_256(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256) >= 256; }
hipError_t launch_gemm_block256(const GemmArgs& g, hipStream_t st);
const char* gemm_kernel_name(GemmKind kind, int64_t M, int64_t N, int64_t K);
// Dual-scale MXFP4 (K % 512 == 0): g's a_scales / w_scales are the fine exponents (packed
// MXFP4 layout), a_coarse / w_coarse the coarse fp32 scales, group-major [K / 512, rows].
hipError_t launch_gemm_mx4_dual(const GemmArgs& g, const float* a_coarse, const float* w_coarse, hipStream_t st);

// Fused quantize + GEMM for M <= 16 tokens (qlinear only): the activation is quantized
// inside the GEMM with the scheme's activation rule.
enum SmallKindId { SMALL_TENSOR = 0, SMALL_ROW = 1, SMALL_INT8 = 2, SMALL_BLOCK = 3 };
struct SmallArgs {
  const uint16_t* a;        // bf16 [M, lda]
  int64_t M, K, lda;
  const float* a_static;    // static activation scales (TENSOR: [1], BLOCK: [M, K/128]) or null
  const uint8_t* w;         // weight codes [N, K]
  const float* w_scales;    // the weight's scales in its scheme's layout
  int64_t N;
  float alpha;
  const uint16_t* bias;     // bf16 [N] or null
  uint16_t* c;
  int64_t ldc;
};
inline bool qlinear_small_applies(int64_t M, int64_t K) { return M >= 1 && M <= 16 && K % 128 == 0; }
// The staged-activation variant: each thread quantizes one 8-element column-chunk of every
// staged row (two for a single row), so K <= 4096 (8192 for one token).
inline bool qlinear_few_applies(int64_t M, int64_t K) {
  return qlinear_small_applies(M, K) && K <= (M == 1 ? 8192 : 4096);
}
hipError_t launch_qlinear_small(int kind, const SmallArgs& s, hipStream_t st);

// W4A16: C = A (bf16) * dequant(Wq)^T
// W4A16, M > 64: pipelined 256 x 128 tile kernel (N % 4 == 0, K % 128 == 0).
bool w4a16_mm_supported(int64_t M, int64_t N, int64_t K);
// Whether the 256 x 64 tile shape is used (small M: 256 x 128 tiles would leave CUs idle).
bool w4a16_mm_narrow(int64_t M, int64_t N);
hipError_t launch_gemm_w4a16_mm(const uint16_t* a, const uint32_t* wq, const uint16_t* w_scales,
                                const uint8_t* w_zeros, int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc,
                                hipStream_t st);
hipError_t launch_gemm_w4a16(const uint16_t* a, const uint32_t* wq, const uint16_t* w_scales,
                             const uint8_t* w_zeros, int64_t M, int64_t N, int64_t K,
                             uint16_t* c, int64_t ldc, hipStream_t st);
const char* gemm_w4a16_kernel_name(int64_t M, int64_t N, int64_t K);

}  // namespace pql
