// MXFP4 GEMM for K % 256 == 128, gfx950, and the GEMM dispatch.
//
// C[m, n] = bf16( sum_b 2^(Xa[m, b] + Xw[n, b]) sum_{k in block b} qa[m, k] qw[n, k] )
// with e2m1 codes and one e8m0 exponent per 32 K-elements ("vLLM-Omni Online
// Quantization complete guide", section "How online quantization works
// underneath", steps 2-3).  The persistent 32x32x64 kernel (gemm32.hip)
// consumes 256 K-elements (128 code bytes) per region, two regions per LDS
// round; this kernel takes the shapes whose last 128-byte step is only half
// filled (K % 256 == 128), which that pipeline does not handle.
//
// The exponents ride the MFMA's own scale operands: in
// v_mfma_scale_f32_16x16x128_f8f6f4 with e2m1 operands lane l feeds row
// (l % 16) with the 32 K-elements 32 g .. 32 g + 31 (16 bytes, g = l / 16),
// and its scale byte is that row's exponent for the same 32 elements.  The
// accumulator lane l holds C[4 (l / 16) + r][l % 16], r = 0..3.
//
// Tiling: a 256-thread workgroup computes a 256 x 256 tile; each of its 4
// waves a 128 x 128 quarter (8 x 8 MFMA tiles, 256 fp32 accumulators per
// lane).  K advances 128 code bytes (256 elements) per step, two MFMAs per
// tile.  The A and W tiles (32 KB each) and the step's exponents are staged
// in LDS, double buffered, with the next step's global loads in flight while
// the current one computes.  LDS rows are 128 bytes with the 16-row-period
// chunk swizzle of the other GEMMs (swz128), so the 16 lanes that read one
// fragment hit distinct banks.  Workgroups are mapped to tiles so that the
// 32 concurrent workgroups of one XCD (dispatch is round-robin over the 8
// XCDs) cover a 4 x 8 patch of tiles and share its A and W rows in that
// XCD's L2.
#include <algorithm>
#include <atomic>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

using gemm::swz128;

constexpr int BM = 256, BN = 256, BKB = 128;   // tile rows, cols, code bytes per step
constexpr int kExpBytes = 2 * 256 * 8;         // a step's exponents: 8 per row, A then W
constexpr int kStageBytes = BM * BKB + BN * BKB + kExpBytes;
constexpr int kGroupM = 4;                     // tile rows per XCD patch
constexpr int kFmt = 4;                        // cbsz / blgp: e2m1

// XCD-aware tile order: block b runs on XCD b % 8; consecutive tiles of one
// XCD walk a kGroupM-tall patch column by column.
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, idx = b >> 3;
  const int per = T >> 3, rem = T & 7;
  const int L = xcd * per + min(xcd, rem) + idx;
  const int in_group = kGroupM * tiles_n;
  const int group = L / in_group;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int l = L - group * in_group;
  tm = first_m + l % gm;
  tn = l / gm;
}

__global__ __launch_bounds__(256, 1) void k_gemm_mx4_tail(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  int tm, tn;
  tile_of_block(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t Kb = g.K / 2;                  // code bytes per row
  const int nsteps = (int)((Kb + BKB - 1) / BKB);

  // ---- global -> register staging: thread t moves chunk (t & 7) of rows (t >> 3) + 32 i.
  // Buffer descriptors cover exactly the tile's valid rows, so rows past M / N read 0.
  const int ld_c = t & 7, ld_r = t >> 3;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a + m0 * Kb), (short)0, (int)(std::min<int64_t>(BM, g.M - m0) * Kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + n0 * Kb), (short)0, (int)(std::min<int64_t>(BN, g.N - n0) * Kb), 0x00020000);
  const int ld_off = ld_r * (int)Kb + ld_c * 16;
  uint4 ra_reg[8], rw_reg[8];
  // exponent staging: thread t fetches the 8 exponents of row t of the tile (A) and of W
  uint2 sa_reg = make_uint2(0, 0), sw_reg = make_uint2(0, 0);
  const int64_t sa_row = std::min<int64_t>(m0 + t, g.M - 1);
  const int64_t sw_row = std::min<int64_t>(n0 + t, g.N - 1);

  auto load_step = [&](int s) {
    const int kb0 = s * BKB;
    const bool inside = kb0 + ld_c * 16 < Kb;   // the last step is half filled
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = ld_off + 32 * i * (int)Kb + kb0;
      v4i va = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, off, 0, 0);
      v4i vw = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, off, 0, 0);
      ra_reg[i] = inside ? make_uint4(va.x, va.y, va.z, va.w) : make_uint4(0, 0, 0, 0);
      rw_reg[i] = inside ? make_uint4(vw.x, vw.y, vw.z, vw.w) : make_uint4(0, 0, 0, 0);
    }
    // packed exponents [G, rows, 8]: a step's 8 blocks are chunk s of the row (pads are 127)
    const uint8_t* sa = static_cast<const uint8_t*>(g.a_scales) + ((int64_t)s * g.M + sa_row) * 8;
    const uint8_t* sw = static_cast<const uint8_t*>(g.w_scales) + ((int64_t)s * g.N + sw_row) * 8;
    sa_reg = *reinterpret_cast<const uint2*>(sa);
    sw_reg = *reinterpret_cast<const uint2*>(sw);
  };
  auto store_step = [&](int stage) {
    uint8_t* A = smem + stage * kStageBytes;
    uint8_t* W = A + BM * BKB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = ld_r + 32 * i;
      *reinterpret_cast<uint4*>(A + swz128(r, ld_c)) = ra_reg[i];
      *reinterpret_cast<uint4*>(W + swz128(r, ld_c)) = rw_reg[i];
    }
    uint8_t* S = W + BN * BKB;   // [256 rows][8 bytes] for A, then the same for W
    *reinterpret_cast<uint2*>(S + t * 8) = sa_reg;
    *reinterpret_cast<uint2*>(S + BM * 8 + t * 8) = sw_reg;
  };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  load_step(0);
  store_step(0);
  __syncthreads();

  const int fr = lane & 15, fk = lane >> 4;   // fragment row and 32-element K slot
  for (int s = 0; s < nsteps; ++s) {
    const int stage = s & 1;
    // Order of one step: issue the next step's global loads, run this step's
    // MFMAs, then write the loaded tile to the other LDS buffer.  The
    // scheduling barriers keep the compiler from hoisting those LDS writes
    // (and their wait on the loads) above the MFMAs.
    if (s + 1 < nsteps) load_step(s + 1);
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* A = smem + stage * kStageBytes;
    const uint8_t* W = A + BM * BKB;
    const uint8_t* S = W + BN * BKB;

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i af[8];
      int asc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wm * 128 + i * 16 + fr;
        const uint4 lo = *reinterpret_cast<const uint4*>(A + swz128(r, 4 * h + fk));
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        asc[i] = S[r * 8 + 4 * h + fk];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = wn * 128 + j * 16 + fr;
        const uint4 lo = *reinterpret_cast<const uint4*>(W + swz128(c, 4 * h + fk));
        const v8i bf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        const int bsc = S[BM * 8 + c * 8 + 4 * h + fk];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[i][j], kFmt, kFmt, 0,
                                                                       asc[i], 0, bsc);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nsteps) store_step(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: round to bf16, masked stores
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t col = n0 + wn * 128 + j * 16 + fr;
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 128 + i * 16 + 4 * fk + r;
        if (row < g.M) g.c[row * g.ldc + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
      }
    }
  }
}

hipError_t launch_mx4_tail(const GemmArgs& g, hipStream_t st) {
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  const size_t lds = 2 * kStageBytes;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<bool> configured[64];   // the dynamic-LDS limit, raised once per device
  if (dev >= 64 || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mx4_tail),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev < 64) configured[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(k_gemm_mx4_tail, dim3(tiles), dim3(256), lds, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, const GemmArgs& g, hipStream_t st) {
  switch (kind) {
    case GEMM_FP8_ROWSCALE: return launch_gemm32_fp8(g, st);
    case GEMM_FP8_BLOCK: return launch_gemm_block(g, st);
    case GEMM_MXFP8: return launch_gemm32_mx(false, g, st);
    case GEMM_MXFP4: return g.K % 256 == 0 ? launch_gemm32_mx(true, g, st) : launch_mx4_tail(g, st);
    case GEMM_INT8_ROW: return launch_gemm32_int8(g, st);
  }
  return hipErrorInvalidValue;
}

const char* gemm_kernel_name(GemmKind kind, int64_t M, int64_t N, int64_t K) {
  switch (kind) {
    case GEMM_FP8_ROWSCALE: return "k_gemm32_fp8";
    case GEMM_FP8_BLOCK: return gemm_block_uses_256(M, N) ? "k_gemm_block256" : "k_gemm_block";
    case GEMM_MXFP8: return "k_gemm32<mxfp8>";
    case GEMM_MXFP4: return K % 256 == 0 ? "k_gemm32<mxfp4>" : "k_gemm<mxfp4>_256x256x256";
    case GEMM_INT8_ROW: return "k_gemm32<int8>";
  }
  return "";
}

}  // namespace pql
