// Dual-scale MXFP4 GEMM, gfx950:
//
//   C[m, n] = bf16( sum_b sa[m, b] sw[n, b] sum_{k in b} 2^(Xa[m, k/32] + Xw[n, k/32]) qa[m, k] qw[n, k] )
//
// with e2m1 codes q, fine e8m0 exponents X per 32 K-elements and coarse fp32
// scales per 512 K-elements b ("vLLM-Omni Online Quantization complete guide",
// section "How online quantization works underneath": the MXFP4 mode with
// fine per-32 and coarse per-512 scales computed online).
//
// The fine exponents ride the scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4,
// e2m1 operands): as in the single-scale MXFP4 GEMM, lane l feeds row l % 32
// of its operand with the 32 K-elements of chunk 2 h + l / 32 of the 128-byte
// region (slice h = 0..3), and its exponent is that 32-block's.  A coarse
// block is two regions (8 slices); each 32 x 32 block's MFMAs accumulate a
// partial sum P over them, which is then promoted into the fp32 sums:
// acc += P * (sa[m, b] * sw[n, b]).  The W fragment is the first MFMA
// operand, so lane l of P holds C[m = l % 32][n = 8 (r / 4) + 4 (l / 32) +
// r % 4]: one activation scale per lane and block row, four float4 reads of
// weight scales per block column.
//
// Shape: 128 x 128 tiles, 4 waves (64 x 64 parts: 2 x 2 blocks), two
// workgroups per CU so that one workgroup's promotion FMAs overlap the
// other's MFMAs.  Operands move through registers into a double-buffered LDS
// stage per 128-byte K region (codes in the 16-row-period swizzle, fine
// exponents packed [region][row][8 bytes], coarse scales per group).  Tiles
// are numbered XCD by XCD so that concurrent tiles share operand rows in an
// XCD's L2.
#include <algorithm>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

using namespace gemm;

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128;
constexpr int kRow = 128;                    // K bytes of a region per row (256 e2m1)
constexpr int kOp = BM * kRow;               // one operand's codes in a stage: 16 KB
constexpr int kExp = BM * 8;                 // one operand's fine exponents in a stage: 1 KB
constexpr int kStage = 2 * kOp + 2 * kExp + 2 * BM * 4;   // + coarse scales of A and W
constexpr int kLds = 2 * kStage;             // 71680 bytes: two workgroups per CU
constexpr int kGroupM = 4;

typedef float v16f __attribute__((ext_vector_type(16)));

// XCD-aware order: workgroup b runs on XCD b % 8; each XCD walks a contiguous
// range of a kGroupM-tall, column-by-column tile order.
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

__global__ __launch_bounds__(kThreads, 2) void k_gemm_mx4_dual(GemmArgs g, const float* __restrict__ a_coarse,
                                                               const float* __restrict__ w_coarse) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  int tm, tn;
  tile_of_block(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t Kb = g.K / 2;                  // code bytes per row
  const int nreg = (int)(Kb / kRow);           // regions; two per coarse block
  const uint8_t* a_exp = static_cast<const uint8_t*>(g.a_scales);
  const uint8_t* w_exp = static_cast<const uint8_t*>(g.w_scales);

  // ---- staging: thread t moves chunk t % 8 of rows t / 8 + 32 i (i < 4) of A and W,
  // the 8 exponent bytes of one row (t < 128: A row t, else W row t - 128) and, at a
  // coarse block's first region, that row's coarse scale.  Rows past M / N repeat the
  // last row (their sums are never stored).
  const int ld_c = t & 7, ld_r = t >> 3;
  const uint8_t* a_rows[4];
  const uint8_t* w_rows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_rows[i] = g.a + std::min<int64_t>(m0 + ld_r + 32 * i, g.M - 1) * Kb + ld_c * 16;
    w_rows[i] = g.w + std::min<int64_t>(n0 + ld_r + 32 * i, g.N - 1) * Kb + ld_c * 16;
  }
  const bool s_is_a = t < BM;
  const int64_t s_row = s_is_a ? std::min<int64_t>(m0 + t, g.M - 1) : std::min<int64_t>(n0 + t - BM, g.N - 1);
  const int64_t s_rows = s_is_a ? g.M : g.N;
  const uint8_t* s_exp = (s_is_a ? a_exp : w_exp) + s_row * 8;
  const float* s_coarse = (s_is_a ? a_coarse : w_coarse) + s_row;

  uint4 ra[4], rw[4];
  uint2 re;
  float rc = 0.f;
  auto load_region = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ldg16(a_rows[i] + (int64_t)r * kRow);
      rw[i] = ldg16(w_rows[i] + (int64_t)r * kRow);
    }
    re = *reinterpret_cast<const uint2*>(s_exp + (int64_t)r * s_rows * 8);
    if ((r & 1) == 0) rc = s_coarse[(int64_t)(r >> 1) * s_rows];   // an odd region keeps its block's value
  };
  auto store_region = [&](int stage) __attribute__((always_inline)) {
    uint8_t* A = smem + stage * kStage;
    uint8_t* W = A + kOp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(A + swz128(ld_r + 32 * i, ld_c)) = ra[i];
      *reinterpret_cast<uint4*>(W + swz128(ld_r + 32 * i, ld_c)) = rw[i];
    }
    *reinterpret_cast<uint2*>(W + kOp + t * 8) = re;             // [A rows | W rows] x 8 bytes
    reinterpret_cast<float*>(W + kOp + 2 * kExp)[t] = rc;        // [A rows | W rows] fp32, every stage
  };

  // ---- fragments and exponents of slice h, block i (A) / j (W)
  const int fr = lane & 31, fk = lane >> 5;
  v16f acc[2][2], P[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) P[i][j] = v16f{};
  load_region(0);
  store_region(0);
  __syncthreads();

  for (int r = 0; r < nreg; ++r) {
    const int stage = r & 1;
    if (r + 1 < nreg) load_region(r + 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* A = smem + stage * kStage;
    const uint8_t* W = A + kOp;
    const uint8_t* E = W + kOp;
    // exponents of the lane's rows: 8 bytes (the region's 8 blocks), shifted by fk
    // bytes so that byte 2 h' of dword d is this lane's block of slice 4 d + h'
    int ea[2][2], ew[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint2 va = *reinterpret_cast<const uint2*>(E + (wm * 64 + 32 * i + fr) * 8);
      const uint2 vw = *reinterpret_cast<const uint2*>(E + kExp + (wn * 64 + 32 * i + fr) * 8);
      ea[i][0] = (int)(va.x >> (8 * fk));
      ea[i][1] = (int)(va.y >> (8 * fk));
      ew[i][0] = (int)(vw.x >> (8 * fk));
      ew[i][1] = (int)(vw.y >> (8 * fk));
    }
    const bool first = (r & 1) == 0;   // the coarse block's first region starts P from zero
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint4 fa[2], fw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = lds16(A + swz128(wm * 64 + 32 * i + fr, 2 * h + fk));
        fw[i] = lds16(W + swz128(wn * 64 + 32 * i + fr, 2 * h + fk));
      }
      const int d = h >> 1;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const v16f c = (first && h == 0) ? v16f{} : P[i][j];
          if (h & 1)
            P[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(fw[j], uint4{0, 0, 0, 0}),
                                                                      cat(fa[i], uint4{0, 0, 0, 0}), c, 4, 4, 2,
                                                                      ew[j][d], 2, ea[i][d]);
          else
            P[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(fw[j], uint4{0, 0, 0, 0}),
                                                                      cat(fa[i], uint4{0, 0, 0, 0}), c, 4, 4, 0,
                                                                      ew[j][d], 0, ea[i][d]);
        }
    }
    if (!first) {   // end of a coarse block: acc += P * sa[m] * sw[n]
      const float* CA = reinterpret_cast<const float*>(E + 2 * kExp);
      const float* CW = CA + BM;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float sa = CA[wm * 64 + 32 * i + fr];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 sw = *reinterpret_cast<const float4*>(CW + wn * 64 + 32 * j + 8 * q + 4 * fk);
            acc[i][j][4 * q + 0] = __builtin_fmaf(P[i][j][4 * q + 0], sa * sw.x, acc[i][j][4 * q + 0]);
            acc[i][j][4 * q + 1] = __builtin_fmaf(P[i][j][4 * q + 1], sa * sw.y, acc[i][j][4 * q + 1]);
            acc[i][j][4 * q + 2] = __builtin_fmaf(P[i][j][4 * q + 2], sa * sw.z, acc[i][j][4 * q + 2]);
            acc[i][j][4 * q + 3] = __builtin_fmaf(P[i][j][4 * q + 3], sa * sw.w, acc[i][j][4 * q + 3]);
          }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (r + 1 < nreg) store_region(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: four consecutive columns per register quad, rounded to bf16
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t row = m0 + wm * 64 + 32 * i + fr;
    if (row >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wn * 64 + 32 * j + 8 * q + 4 * fk;
        uint16_t* dst = g.c + row * g.ldc + col;
        const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (g.vec_store && col + 4 <= g.N) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < g.N) dst[e] = (uint16_t)(pack_bf16x2(v[e], 0.f) & 0xFFFFu);
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_mx4_dual(const GemmArgs& g, const float* a_coarse, const float* w_coarse, hipStream_t st) {
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL(k_gemm_mx4_dual, dim3((unsigned)tiles), dim3(kThreads), 0, st, g, a_coarse, w_coarse);
  return hipGetLastError();
}

}  // namespace pql
