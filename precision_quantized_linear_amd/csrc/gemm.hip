// Block-scaled GEMM on gfx950 matrix cores: C[M, N] = A_hat * W_hat^T, bf16 out.
//
// A and W arrive as K-contiguous codes (e4m3fn bytes, or e2m1 pairs).  In
// v_mfma_scale_f32_16x16x128_f8f6f4 lane l feeds row (l % 16); with g = l / 16
// its operand holds, for fp4, the 32 K-elements 32 g .. 32 g + 31 (16 bytes),
// and for fp8 the 16 K-elements 16 g .. 16 g + 15 in bytes 0-15 and
// 64 + 16 g .. 64 + 16 g + 15 in bytes 16-31.  In both cases lane l's scale
// byte is row (l % 16)'s e8m0 exponent for K-elements 32 g .. 32 g + 31.  (The
// fp8 split was pinned with one-hot probes on the device.)  The accumulator
// lane l holds C[4 * (l / 16) + r][l % 16], r = 0..3.
//
// Scale handling per scheme ("[vLLM] Other quantization: FP8, ModelOpt, INC,
// TorchAO, Quark", section "FP8"; "vLLM-Omni Online Quantization complete
// guide", section "How online quantization works underneath", steps 2-3):
//   FP8 tensor / row   unit MFMA scales; C = acc * s_a[m] * s_w[n] at the end
//   FP8 block-128      each 128-K step is one K-group: the MFMA result of the
//                      step is promoted with s_a[m, g] * s_w[n / 128, g]
//   MXFP8 / MXFP4      the e8m0 exponents ride the MFMA's own scale operands
//
// Tiling: a 256-thread workgroup computes a 256 x 256 tile; each of its 4
// waves a 128 x 128 quarter (8 x 8 MFMA tiles, 256 fp32 accumulators per
// lane).  K advances 128 bytes per step (128 fp8 or 256 fp4 elements).  The
// A and W tiles (32 KB each) and the step's scales are staged in LDS, double
// buffered (130 KB of the 160 KB), with the next step's global loads in
// flight while the current one computes.  LDS rows are 128 bytes; 16-byte
// chunk c of row r is stored at chunk position c ^ (r & 7), so the 16 lanes
// that read one MFMA fragment hit distinct banks.  Workgroups are mapped to
// tiles so that the 32 concurrent workgroups of one XCD (dispatch is
// round-robin over the 8 XCDs) cover a 4 x 8 patch of tiles and share its A
// and W rows in that XCD's L2.
#include <algorithm>

#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

constexpr int BM = 256, BN = 256, BKB = 128;   // tile rows, cols, K bytes per step
constexpr int kScaleBytes = 4096;                          // per-row scales of A and W
constexpr int kStageBytes = BM * BKB + BN * BKB + kScaleBytes;
constexpr int kGroupM = 4;                     // tile rows per XCD patch

__device__ __forceinline__ int swz(int row, int chunk) { return row * BKB + ((chunk ^ (row & 7)) << 4); }

template <int KIND>
struct Traits {
  static constexpr bool kFp4 = KIND == GEMM_MXFP4;
  static constexpr bool kMx = KIND == GEMM_MXFP8 || KIND == GEMM_MXFP4;
  static constexpr bool kBlock = KIND == GEMM_FP8_BLOCK;
  static constexpr int kFmt = kFp4 ? 4 : 0;              // cbsz / blgp format code
  static constexpr int kKPerStep = kFp4 ? 256 : 128;     // K elements per 128-byte step
  static constexpr int kMfmaPerStep = kFp4 ? 2 : 1;      // 16x16x128 MFMAs per step
};

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

template <int KIND>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs g) {
  using T = Traits<KIND>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  int tm, tn;
  tile_of_block(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t Kb = T::kFp4 ? g.K / 2 : g.K;           // code bytes per row
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
  // scale staging: thread t fetches the scales of row t of the tile (A) and of W
  uint2 sa_reg = make_uint2(0, 0), sw_reg = make_uint2(0, 0);
  float sblk_reg = 0.0f;
  const int64_t sa_row = std::min<int64_t>(m0 + t, g.M - 1);
  const int64_t sw_row = std::min<int64_t>(n0 + t, g.N - 1);

  auto load_step = [&](int s) {
    const int kb0 = s * BKB;
    // only an fp4 operand with K % 256 == 128 has a half-filled last step
    const bool inside = !T::kFp4 || kb0 + ld_c * 16 < Kb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = ld_off + 32 * i * (int)Kb + kb0;
      v4i va = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, off, 0, 0);
      v4i vw = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, off, 0, 0);
      ra_reg[i] = inside ? make_uint4(va.x, va.y, va.z, va.w) : make_uint4(0, 0, 0, 0);
      rw_reg[i] = inside ? make_uint4(vw.x, vw.y, vw.z, vw.w) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (T::kMx) {
      // packed exponents: a step's kKPerStep / 32 blocks are chunk s of the row
      constexpr int kC = T::kKPerStep / 32;
      const uint8_t* sa = static_cast<const uint8_t*>(g.a_scales) + ((int64_t)s * g.M + sa_row) * kC;
      const uint8_t* sw = static_cast<const uint8_t*>(g.w_scales) + ((int64_t)s * g.N + sw_row) * kC;
      sa_reg.x = *reinterpret_cast<const uint32_t*>(sa);
      sw_reg.x = *reinterpret_cast<const uint32_t*>(sw);
      if constexpr (T::kFp4) {
        sa_reg.y = *reinterpret_cast<const uint32_t*>(sa + 4);
        sw_reg.y = *reinterpret_cast<const uint32_t*>(sw + 4);
      }
    } else if constexpr (T::kBlock) {
      const int64_t ng = g.K / 128;
      sblk_reg = static_cast<const float*>(g.a_scales)[sa_row * ng + s];
    }
  };
  auto store_step = [&](int stage) {
    uint8_t* A = smem + stage * kStageBytes;
    uint8_t* W = A + BM * BKB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = ld_r + 32 * i;
      *reinterpret_cast<uint4*>(A + swz(r, ld_c)) = ra_reg[i];
      *reinterpret_cast<uint4*>(W + swz(r, ld_c)) = rw_reg[i];
    }
    uint8_t* S = W + BN * BKB;
    if constexpr (T::kMx) {
      // [256 rows][8 bytes] for A, then the same for W
      *reinterpret_cast<uint2*>(S + t * 8) = sa_reg;
      *reinterpret_cast<uint2*>(S + BM * 8 + t * 8) = sw_reg;
    } else if constexpr (T::kBlock) {
      reinterpret_cast<float*>(S)[t] = sblk_reg;
    }
  };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // block-128 weight scale column: the wave's 128 columns share one 128-row W block
  const int64_t wblk = std::min<int64_t>((n0 + wn * 128) / 128, g.N / 128 - 1);

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
    for (int h = 0; h < T::kMfmaPerStep; ++h) {
      v8i af[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wm * 128 + i * 16 + fr;
        if constexpr (T::kFp4) {
          uint4 lo = *reinterpret_cast<const uint4*>(A + swz(r, 4 * h + fk));
          af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        } else {
          uint4 lo = *reinterpret_cast<const uint4*>(A + swz(r, fk));
          uint4 hi = *reinterpret_cast<const uint4*>(A + swz(r, 4 + fk));
          af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
      int asc[8];
      if constexpr (T::kMx) {
#pragma unroll
        for (int i = 0; i < 8; ++i) asc[i] = S[(wm * 128 + i * 16 + fr) * 8 + 4 * h + fk];
      }
      float ablk[8][4];
      if constexpr (T::kBlock) {
        const float swv = static_cast<const float*>(g.w_scales)[wblk * (g.K / 128) + s];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 v = *reinterpret_cast<const float4*>(
              reinterpret_cast<const float*>(S) + wm * 128 + i * 16 + 4 * fk);
          ablk[i][0] = v.x * swv; ablk[i][1] = v.y * swv; ablk[i][2] = v.z * swv; ablk[i][3] = v.w * swv;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = wn * 128 + j * 16 + fr;
        v8i bf;
        if constexpr (T::kFp4) {
          uint4 lo = *reinterpret_cast<const uint4*>(W + swz(c, 4 * h + fk));
          bf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        } else {
          uint4 lo = *reinterpret_cast<const uint4*>(W + swz(c, fk));
          uint4 hi = *reinterpret_cast<const uint4*>(W + swz(c, 4 + fk));
          bf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        int bsc = 127;
        if constexpr (T::kMx) bsc = S[BM * 8 + c * 8 + 4 * h + fk];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if constexpr (T::kMx) {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[i][j], T::kFmt,
                                                                         T::kFmt, 0, asc[i], 0, bsc);
          } else if constexpr (T::kBlock) {
            v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, v4f{0.f, 0.f, 0.f, 0.f},
                                                                     0, 0, 0, 127, 0, 127);
            acc[i][j][0] = __builtin_fmaf(p[0], ablk[i][0], acc[i][j][0]);
            acc[i][j][1] = __builtin_fmaf(p[1], ablk[i][1], acc[i][j][1]);
            acc[i][j][2] = __builtin_fmaf(p[2], ablk[i][2], acc[i][j][2]);
            acc[i][j][3] = __builtin_fmaf(p[3], ablk[i][3], acc[i][j][3]);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[i][j], 0, 0, 0,
                                                                         127, 0, 127);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nsteps) store_step(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: scale (FP8 tensor / row), round to bf16, masked stores
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float rs[4] = {1.f, 1.f, 1.f, 1.f};
    int64_t rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rows[r] = m0 + wm * 128 + i * 16 + 4 * fk + r;
      if constexpr (KIND == GEMM_FP8_ROWSCALE) {
        const int64_t rr = std::min<int64_t>(rows[r], g.M - 1);
        rs[r] = static_cast<const float*>(g.a_scales)[rr * g.a_scale_stride];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t col = n0 + wn * 128 + j * 16 + fr;
      if (col >= g.N) continue;
      float cs = 1.f;
      if constexpr (KIND == GEMM_FP8_ROWSCALE) cs = static_cast<const float*>(g.w_scales)[col * g.w_scale_stride];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (rows[r] < g.M) {
          float v = acc[i][j][r];
          if constexpr (KIND == GEMM_FP8_ROWSCALE) v = v * rs[r] * cs;
          g.c[rows[r] * g.ldc + col] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
  }
}

template <int KIND>
hipError_t launch_kind(const GemmArgs& g, hipStream_t st) {
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  const size_t lds = 2 * kStageBytes;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static bool configured[64] = {};
  if (dev < 64 && !configured[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<KIND>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured[dev] = true;
  }
  hipLaunchKernelGGL(k_gemm<KIND>, dim3(tiles), dim3(256), lds, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, const GemmArgs& g, hipStream_t st) {
  switch (kind) {
    case GEMM_FP8_ROWSCALE: return launch_gemm32_fp8(g, st);
    case GEMM_FP8_BLOCK: return launch_gemm_block(g, st);
    case GEMM_MXFP8: return launch_gemm32_mx(false, g, st);
    case GEMM_MXFP4: return g.K % 256 == 0 ? launch_gemm32_mx(true, g, st) : launch_kind<GEMM_MXFP4>(g, st);
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
