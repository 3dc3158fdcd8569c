// Fused quantize + GEMM for a few tokens (M <= 16), gfx950.
//
// For one or a few tokens the separate activation quantize is pure overhead
// ("vLLM-Omni Online Quantization complete guide", section "How online
// quantization works underneath": the activation-quantize prologue fusion;
// per-call quantize and dequant overhead dominating single requests on the
// quantization page for diffusion transformers) and a 256 x 256 output tile
// leaves most CUs idle.  This kernel streams the weight like a GEMV and
// quantizes the activation inside: every workgroup owns 32 output columns and
// all M <= 16 rows, reads the bf16 activation itself (it is tiny and stays in
// L2), quantizes each K-chunk with the scheme's activation rule exactly as the
// quantize kernels do (same scales, same codes) and feeds the codes straight
// to the matrix core.  Schemes:
//   TENSOR  FP8, one scale for the whole activation (max over its M rows)
//   ROW     FP8, one scale per token
//   INT8    int8 W8A8, one scale per token, int32 sums
//   BLOCK   FP8, one scale per (token, 128-wide K-group), computed per chunk
// with static (supplied) activation scales for TENSOR and BLOCK.  The weight
// keeps its own layout and scales (per tensor, per channel, per 128 x 128
// block) and the epilogue is the GEMMs' alpha * (...) + bias.
//
// Matrix core: v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (int8:
// v_mfma_i32_16x16x64_i8 twice).  Lane l feeds row l % 16 with, for g = l / 16,
// the 16 K-elements 16 g .. + 15 of a 128-element chunk in bytes 0-15 and
// 64 + 16 g .. + 15 in bytes 16-31, for the activation and the weight alike
// (so each K-element meets its partner whatever order the sums run in); lane l
// then holds C[4 g + r][l % 16], r = 0..3.  The 8 waves take the K-chunks
// round-robin, each with the loads of three chunks in flight before it uses
// any, and add their sums in LDS at the end.
//
// Two kernels share this.  k_qlinear_few (K up to 4096, 8192 for one token)
// quantizes the activation once per workgroup into LDS codes, while its first
// batch of weight loads is already in flight, and its main loop then holds
// only weight registers; for wide outputs its workgroups own 48 columns
// instead of 32 (256 workgroups at N = 12288, one per CU, rather than two on
// half of the CUs), since every workgroup repeats the cast and streams its own
// weight rows.
// k_qlinear_small (longer K) quantizes in its main loop: each lane casts its
// own row's 32 elements of every chunk.
#include <algorithm>
#include <atomic>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"
#include "quant_common.hpp"

namespace pql {

namespace {

constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kBatch = 3;   // K-chunks whose loads a wave has in flight at once
constexpr int kCols = 32;   // output columns per workgroup (two blocks of 16)
constexpr int64_t kFewMaxK = 8192;   // the longest K of the staged-activation kernel

typedef float v4f_t __attribute__((ext_vector_type(4)));

template <int KIND>
struct SmallKind {
  static constexpr bool kInt8 = KIND == SMALL_INT8;
  static constexpr bool kBlock = KIND == SMALL_BLOCK;
  static constexpr bool kTensor = KIND == SMALL_TENSOR;
};

// 32 bf16 of the lane's row for one chunk -> 32 codes (FP8 or int8), in MFMA byte order.
template <int KIND, bool STATIC>
__device__ __forceinline__ void cast_chunk(const uint4 (&x)[4], float s, uint32_t (&q)[8]) {
  const bool fast = s >= kSmallestFastScale;
  const float rcp = fast ? __fdiv_rn(1.0f, s) : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint2 v;
    if constexpr (KIND == SMALL_INT8) v = fast ? int8_chunk<true>(x[i], s, rcp) : int8_chunk<false>(x[i], s, rcp);
    else if constexpr (STATIC) v = fast ? fp8_chunk_sat<true>(x[i], s, rcp) : fp8_chunk_sat<false>(x[i], s, rcp);
    else v = fast ? fp8_chunk<true>(x[i], s, rcp) : fp8_chunk<false>(x[i], s, rcp);
    q[2 * i] = v.x;
    q[2 * i + 1] = v.y;
  }
}

template <int KIND, bool STATIC, bool EPI>
__global__ __launch_bounds__(kThreads) void k_qlinear_small(const uint16_t* __restrict__ a, int64_t M, int64_t K,
                                                          int64_t lda, const float* __restrict__ a_static,
                                                          const uint8_t* __restrict__ w,
                                                          const float* __restrict__ w_scales, int64_t N, float alpha,
                                                          const uint16_t* __restrict__ bias, uint16_t* __restrict__ c,
                                                          int64_t ldc) {
  using T = SmallKind<KIND>;
  __shared__ float red[kWaves][16];
  __shared__ float s_row[16];
  __shared__ float part[kWaves][16][kCols + 1];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kCols;
  const int nk = (int)(K / 128);
  const bool row_valid = r16 < M;
  const uint16_t* arow = a + (int64_t)std::min<int64_t>(r16, M - 1) * lda;

  // ---- per-token (or per-tensor) scales: the max of |x| over each row, from all threads
  if constexpr (!T::kBlock) {
    if constexpr (STATIC) {
      if (t < 16) s_row[t] = a_static[0];
    } else {
      float pm[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        pm[m] = 0.0f;
        if (m < M)
          for (int64_t ch = t; ch < K / 8; ch += kThreads)
            pm[m] = fmaxf(pm[m], chunk_absmax(ldg16(a + (int64_t)m * lda + ch * 8)));
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float v = wave_max(pm[m]);
        if (lane == 0) red[wave][m] = v;
      }
      __syncthreads();
      if (t < 16) {
        float amax = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, red[w][t]);
        if constexpr (T::kTensor) {   // one scale: the max over every row
          amax = 0.0f;
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, red[w][m]);
        }
        s_row[t] = T::kInt8 ? int8_scale(amax) : fp8_scale(amax);
      }
    }
    __syncthreads();
  }
  const float s_lane = T::kBlock ? 1.0f : s_row[r16];   // the lane's own row's scale

  const uint8_t* wrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wrow[j] = w + std::min<int64_t>(n0 + 16 * j + r16, N - 1) * K;
  const int64_t nblk = n0 / 128;   // block-128: the 32 columns lie in one weight block (N % 128 == 0)

  v4f_t acc[2] = {v4f_t{0.f, 0.f, 0.f, 0.f}, v4f_t{0.f, 0.f, 0.f, 0.f}};
  v4i acci[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
  // One chunk's work once its operands are in registers: scale (block-128: from the
  // chunk's own amax), cast to codes, matrix core.
  auto chunk = [&](int ck, const uint4 (&x)[4], const uint4 (&wv)[2][2]) __attribute__((always_inline)) {
    float s = s_lane;
    if constexpr (T::kBlock) {
      if constexpr (STATIC) {
        s = a_static[(int64_t)std::min<int64_t>(r16, M - 1) * nk + ck];
      } else {   // the chunk is the row's K-group ck: its 128 elements are spread over lanes r16 + 16 g'
        float m = fmaxf(fmaxf(chunk_absmax(x[0]), chunk_absmax(x[1])), fmaxf(chunk_absmax(x[2]), chunk_absmax(x[3])));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        s = fp8_scale(m);
      }
    }
    uint32_t q[8];
    cast_chunk<KIND, STATIC>(x, s, q);
    if constexpr (T::kInt8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acci[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]},
                                                        __builtin_bit_cast(v4i, wv[j][0]), acci[j], 0, 0, 0);
        acci[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]},
                                                        __builtin_bit_cast(v4i, wv[j][1]), acci[j], 0, 0, 0);
      }
    } else {
      const v8i qa = v8i{(int)q[0], (int)q[1], (int)q[2], (int)q[3], (int)q[4], (int)q[5], (int)q[6], (int)q[7]};
      if constexpr (T::kBlock) {
        // this chunk's partial sums, promoted with s_a[m, ck] s_w[block, ck]; the lane's
        // outputs are rows 4 g + r, whose scales sit in lanes 4 g + r
        float sr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sr[r] = __shfl(s, 4 * g + r);
        const float sw = w_scales[nblk * nk + ck];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const v4f_t P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, gemm::cat(wv[j][0], wv[j][1]),
                                                                          v4f_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0,
                                                                          127);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(P[r], sr[r] * sw, acc[j][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, gemm::cat(wv[j][0], wv[j][1]), acc[j], 0, 0, 0, 127,
                                                                    0, 127);
      }
    }
  };

  // Each wave takes chunks wave, wave + kWaves, ...; it issues the loads of kBatch of them
  // before using any, so that enough bytes are in flight to stream the weight.  (The
  // weight rows are read with ordinary loads: each load instruction covers half of 16
  // rows' 128-byte lines, and the other half, a second instruction's, then hits in L2.)
  for (int ck0 = wave; ck0 < nk; ck0 += kWaves * kBatch) {
    uint4 x[kBatch][4], wv[kBatch][2][2];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int ck = ck0 + u * kWaves;
      const int64_t k0 = (int64_t)ck * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[u][i] = uint4{0, 0, 0, 0};
      if (ck < nk) {   // wave-uniform
        if (row_valid) {
          x[u][0] = ldg16(arow + k0 + 16 * g);
          x[u][1] = ldg16(arow + k0 + 16 * g + 8);
          x[u][2] = ldg16(arow + k0 + 64 + 16 * g);
          x[u][3] = ldg16(arow + k0 + 64 + 16 * g + 8);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          wv[u][j][0] = ldg16(wrow[j] + k0 + 16 * g);
          wv[u][j][1] = ldg16(wrow[j] + k0 + 64 + 16 * g);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (ck0 + u * kWaves < nk) chunk(ck0 + u * kWaves, x[u], wv[u]);
  }

  // ---- sums of the waves, then the epilogue (the scales of the row / column GEMMs)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      part[wave][4 * g + r][16 * j + r16] = T::kInt8 ? __int_as_float(acci[j][r]) : acc[j][r];
  __syncthreads();
  for (int e = t; e < 16 * kCols; e += kThreads) {
    const int m = e / kCols, col = e - m * kCols;
    const int64_t n = n0 + col;
    if (m >= M || n >= N) continue;
    float v;
    if constexpr (T::kInt8) {
      int si = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) si += __float_as_int(part[w][m][col]);
      v = (float)si;
    } else {
      float p2[kWaves / 2];
#pragma unroll
      for (int w = 0; w < kWaves / 2; ++w) p2[w] = part[2 * w][m][col] + part[2 * w + 1][m][col];
      v = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves / 2; ++w) v += p2[w];
    }
    float out;
    if constexpr (T::kBlock) {
      out = EPI ? __builtin_fmaf(v, alpha, bias ? __uint_as_float((uint32_t)bias[n] << 16) : 0.0f) : v;
    } else {
      const float rs = alpha * s_row[m];
      const float cs = T::kTensor ? w_scales[0] : w_scales[n];
      out = EPI ? __builtin_fmaf(v * rs, cs, bias ? __uint_as_float((uint32_t)bias[n] << 16) : 0.0f) : v * rs * cs;
    }
    c[(int64_t)m * ldc + n] = (uint16_t)(gemm::pack_bf16x2(out, 0.0f) & 0xFFFFu);
  }
}


// ---------------------------------------------------------------- staged activation
// R rows of the activation are staged (R = 1, 4 or 16, the smallest that
// covers M; rows past M repeat row M - 1, and their outputs are never
// stored).  Thread t owns the 16-byte activation column-chunk j = t (+ 512 for
// R = 1 and K > 4096) of every staged row, so a row is a compile-time index.
// Work order:
//   1. the thread's activation loads, then the wave's first batch of weight
//      loads (and block-128 weight scales): loads retire in issue order, so the
//      activation is waited for while the weight loads stay in flight;
//   2. the activation scales: per row (or tensor) the max of |x| over the
//      workgroup (one barrier), or per 1 x 128 group the max over the 16
//      lanes that hold the group's chunks (no barrier).  With 16 rows and a
//      per-row or per-tensor scale the thread's 16 chunks are loaded twice:
//      once, before any weight load, for the maxima, and again beside the
//      weight batch for the cast, so that the chunks and the batch are not
//      held through the barrier together (the registers would cost the second
//      workgroup per CU);
//   3. the cast into LDS codes (K bytes per row plus 16 of padding) and a
//      barrier;
//   4. the main loop: each chunk's A codes come from LDS, its weight bytes
//      from the batch, computed as soon as the chunk's loads have landed; a
//      slot past the last chunk repeats the batch's first and adds zero.
// J: column-chunks per thread (K <= 4096 J); NB: 16-column blocks per workgroup
template <int KIND, bool STATIC, bool EPI, int R, int J, int NB>
__global__ __launch_bounds__(kThreads) void k_qlinear_few(const uint16_t* __restrict__ a, int64_t M, int64_t K,
                                                        int64_t lda, const float* __restrict__ a_static,
                                                        const uint8_t* __restrict__ w,
                                                        const float* __restrict__ w_scales, int64_t N, float alpha,
                                                        const uint16_t* __restrict__ bias, uint16_t* __restrict__ c,
                                                        int64_t ldc) {
  using T = SmallKind<KIND>;
  constexpr int kJ = J;
  constexpr int kC = 16 * NB;   // output columns of the workgroup
  // 16 rows in 32-column workgroups (two may share a CU): the dynamic row maxima are taken on
  // a first pass over the activation and the cast reloads it, so that its 16 chunks are not
  // live across the barrier; 48-column workgroups, one per CU, keep them.
  constexpr bool kTwoPass = R == 16 && NB == 2 && !T::kBlock && !STATIC;
  extern __shared__ __attribute__((aligned(16))) uint8_t few_lds[];
  const int nk = (int)(K / 128);
  float (*part)[16][kC + 1] = reinterpret_cast<float (*)[16][kC + 1]>(few_lds);
  float (*red)[R] = reinterpret_cast<float (*)[R]>(few_lds + sizeof(float) * kWaves * 16 * (kC + 1));
  float* s_row = &red[kWaves][0];                            // [R]
  float* sa = s_row + R;                                     // block-128: [nk][R]
  // [R][K + 16], 16-byte aligned for the 16-byte fragment reads
  uint8_t* codes = few_lds + ((reinterpret_cast<uint8_t*>(sa + (T::kBlock ? R * nk : 0)) - few_lds + 15) & ~15);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kC;
  const int cpr = (int)(K / 8);   // 16-byte activation chunks per row
  const int ldq = (int)K + 16;    // LDS bytes per row of codes
  const int mlast = (int)M - 1;

  // ---- 1. activation loads (a column past the row repeats the last), then the weight batch
  uint4 av[kJ][R];
  float ast[T::kBlock && STATIC ? kJ : 1][R];   // static block-128: the supplied scale of each chunk
  auto load_act = [&](const uint16_t* ap) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int j = std::min(t + kThreads * jj, cpr - 1);
#pragma unroll
      for (int m = 0; m < R; ++m) {
        av[jj][m] = ldg16(ap + (int64_t)std::min(m, mlast) * lda + 8 * j);
        if constexpr (T::kBlock && STATIC) ast[jj][m] = a_static[(int64_t)std::min(m, mlast) * nk + (j >> 4)];
      }
    }
  };
  const uint8_t* wrow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) wrow[j] = w + std::min<int64_t>(n0 + 16 * j + r16, N - 1) * K;
  // block-128 (N % 128 == 0): the weight block of each 16-column block, clamped inside N
  int64_t nblk[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) nblk[j] = std::min<int64_t>((n0 + 16 * j) / 128, N / 128 - 1);
  uint4 wv[kBatch][NB][2];
  float wsc[kBatch][NB];
  // slots u0 .. u1 - 1 of the batch starting at chunk ck0
  auto fetch = [&](int ck0, int u0 = 0, int u1 = kBatch) __attribute__((always_inline)) {
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int ck = ck0 + u * kWaves < nk ? ck0 + u * kWaves : ck0;   // wave-uniform
      const int64_t k0 = (int64_t)ck * 128;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (T::kBlock) wsc[u][j] = w_scales[nblk[j] * nk + ck];
        wv[u][j][0] = ldg16(wrow[j] + k0 + 16 * g);
        wv[u][j][1] = ldg16(wrow[j] + k0 + 64 + 16 * g);
      }
    }
  };

  // the scale of staged row m (per tensor: row 0 holds the tensor's max) from the maxima
  auto row_scale = [&](int m) __attribute__((always_inline)) {
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) amax = fmaxf(amax, red[q][m]);
    return T::kInt8 ? int8_scale(amax) : fp8_scale(amax);
  };
  // ---- 2. per-row / per-tensor maxima (dynamic, not block-128): thread m < R turns row m's
  // maximum (per tensor: the tensor's) into its scale in s_row; two barriers
  auto row_maxima = [&]() __attribute__((always_inline)) {
    float pm[R];
#pragma unroll
    for (int m = 0; m < R; ++m) pm[m] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
      for (int m = 0; m < R; ++m) pm[m] = fmaxf(pm[m], chunk_absmax(av[jj][m]));   // a repeat repeats a maximum
    if constexpr (T::kTensor) {   // rows past M repeat row M - 1: the max over all R rows is the tensor's
#pragma unroll
      for (int m = 1; m < R; ++m) pm[0] = fmaxf(pm[0], pm[m]);
      const float v = wave_max(pm[0]);
      if (lane == 0) red[wave][0] = v;
    } else {
#pragma unroll
      for (int m = 0; m < R; ++m) {
        const float v = wave_max(pm[m]);
        if (lane == 0) red[wave][m] = v;
      }
    }
    __syncthreads();
    if constexpr (R == 16) {   // one thread per row: 16 scales in every thread would cost registers
      if (t < R) s_row[t] = row_scale(T::kTensor ? 0 : t);   // rows past M: row M - 1's scale
      __syncthreads();
    }
  };

  // With 16 rows the cast holds two of the batch's three chunks: with 32 columns the 16
  // activation chunks beside a whole batch would cost the second workgroup per CU, and with 48
  // the third chunk's loads, issued before the cast, measured slower for block-128.
  constexpr int kEarly = R == 16 ? 2 : kBatch;
  const int ck_first = std::min(wave, nk - 1);   // a wave with no chunk (nk < 8) loads chunk nk - 1, unused
  load_act(a);
  if constexpr (kTwoPass) {
    row_maxima();
    // the same bytes again: an opaque zero offset makes them loads, where the compiler
    // would otherwise keep the first pass's registers live through the barrier (an opaque
    // pointer would lose its address space and turn them into flat loads)
    int zero = 0;
    asm volatile("" : "+s"(zero));
    load_act(a + zero);
  }
  __builtin_amdgcn_sched_barrier(0);   // every activation-side load goes out before the weight batch
  fetch(ck_first, 0, kEarly);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!T::kBlock && !STATIC && !kTwoPass) row_maxima();

  // ---- 3. scales and the cast into LDS codes: every staged row, with no branch on M (a
  // branch would make the compiler wait for the weight batch too); rows past M repeat row
  // M - 1 and are never read
#pragma unroll
  for (int m = 0; m < R; ++m) {
    __builtin_amdgcn_sched_barrier(0);   // one row's scale and cast at a time
    float s;
    if constexpr (T::kBlock || !STATIC) s = 0.0f;
    if constexpr (!T::kBlock) {
      if constexpr (STATIC) {
        s = a_static[0];
        if (t == 0) s_row[m] = s;
      } else if constexpr (R == 16) {
        s = s_row[m];
      } else {
        s = row_scale(T::kTensor ? 0 : m);
        if (t == 0) s_row[m] = s;   // rows past M: row M - 1's scale
      }
    }
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int j = t + kThreads * jj;
      float sj = s;
      if constexpr (T::kBlock) {   // the group's 16 chunks are 16 consecutive lanes
        const int grp = std::min(j, cpr - 1) >> 4;
        if constexpr (STATIC) {
          sj = ast[T::kBlock && STATIC ? jj : 0][m];
        } else {
          float mx = chunk_absmax(av[jj][m]);
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
          sj = fp8_scale(mx);
        }
        if ((lane & 15) == 0 && j < cpr) sa[grp * R + m] = sj;
      }
      // the cast is unconditional (a column past the row repeats the last one) and only the
      // store is not: a cast under the branch let the compiler sink the chunk's load into it,
      // behind the weight loads
      const bool fast = sj >= kSmallestFastScale;
      const float rcp = fast ? __fdiv_rn(1.0f, sj) : 0.0f;
      uint2 q;
      if constexpr (T::kInt8) q = fast ? int8_chunk<true>(av[jj][m], sj, rcp) : int8_chunk<false>(av[jj][m], sj, rcp);
      else if constexpr (STATIC) q = fast ? fp8_chunk_sat<true>(av[jj][m], sj, rcp) : fp8_chunk_sat<false>(av[jj][m], sj, rcp);
      else q = fast ? fp8_chunk<true>(av[jj][m], sj, rcp) : fp8_chunk<false>(av[jj][m], sj, rcp);
      if (j < cpr) *reinterpret_cast<uint2*>(codes + m * ldq + 8 * j) = q;
    }
  }
  if constexpr (kEarly < kBatch) fetch(ck_first, kEarly, kBatch);
  __syncthreads();

  // ---- 4. the main loop
  const uint8_t* qrow = codes + std::min(r16, mlast) * ldq + 16 * g;   // the lane's row, as a GEMM operand
  v4f_t acc[NB];
  v4i acci[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    acc[j] = v4f_t{0.f, 0.f, 0.f, 0.f};
    acci[j] = v4i{0, 0, 0, 0};
  }
  auto chunk = [&](int ck, bool live, const uint4 (&wvc)[NB][2], const float (&wscale)[NB]) __attribute__((always_inline)) {
    uint4 q0 = gemm::lds16(qrow + ck * 128), q1 = gemm::lds16(qrow + ck * 128 + 64);
    if constexpr (T::kInt8) {
      if (!live) q0 = q1 = uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        acci[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, q0), __builtin_bit_cast(v4i, wvc[j][0]),
                                                        acci[j], 0, 0, 0);
        acci[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, q1), __builtin_bit_cast(v4i, wvc[j][1]),
                                                        acci[j], 0, 0, 0);
      }
    } else if constexpr (T::kBlock) {
      // the chunk's partial sums, promoted with s_a[m, ck] s_w[block, ck]; the lane's outputs
      // are rows 4 g + r (past M: row M - 1)
      float sr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sr[r] = sa[ck * R + std::min(4 * g + r, mlast)];
      const v8i qa = gemm::cat(q0, q1);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float sw = live ? wscale[j] : 0.0f;
        const v4f_t P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, gemm::cat(wvc[j][0], wvc[j][1]),
                                                                        v4f_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(P[r], sr[r] * sw, acc[j][r]);
      }
    } else {
      if (!live) q0 = q1 = uint4{0u, 0u, 0u, 0u};
      const v8i qa = gemm::cat(q0, q1);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, gemm::cat(wvc[j][0], wvc[j][1]), acc[j], 0, 0, 0,
                                                                  127, 0, 127);
    }
  };
  for (int ck0 = wave; ck0 < nk; ck0 += kWaves * kBatch) {
    if (ck0 != wave) {
      fetch(ck0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool live = ck0 + u * kWaves < nk;
      chunk(live ? ck0 + u * kWaves : ck0, live, wv[u], wsc[u]);
    }
  }

  // ---- sums of the waves, then the epilogue (the scales of the row / column GEMMs)
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      part[wave][4 * g + r][16 * j + r16] = T::kInt8 ? __int_as_float(acci[j][r]) : acc[j][r];
  __syncthreads();
  for (int e = t; e < 16 * kC; e += kThreads) {
    const int m = e / kC, col = e - m * kC;
    const int64_t n = n0 + col;
    if (m >= M || n >= N) continue;
    float v;
    if constexpr (T::kInt8) {
      int si = 0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) si += __float_as_int(part[q][m][col]);
      v = (float)si;
    } else {
      float p2[kWaves / 2];
#pragma unroll
      for (int q = 0; q < kWaves / 2; ++q) p2[q] = part[2 * q][m][col] + part[2 * q + 1][m][col];
      v = 0.0f;
#pragma unroll
      for (int q = 0; q < kWaves / 2; ++q) v += p2[q];
    }
    float out;
    if constexpr (T::kBlock) {
      out = EPI ? __builtin_fmaf(v, alpha, bias ? __uint_as_float((uint32_t)bias[n] << 16) : 0.0f) : v;
    } else {
      const float rs = alpha * s_row[m];
      const float cs = T::kTensor ? w_scales[0] : w_scales[n];
      out = EPI ? __builtin_fmaf(v * rs, cs, bias ? __uint_as_float((uint32_t)bias[n] << 16) : 0.0f) : v * rs * cs;
    }
    c[(int64_t)m * ldc + n] = (uint16_t)(gemm::pack_bf16x2(out, 0.0f) & 0xFFFFu);
  }
}

size_t few_lds_bytes(int R, int NB, bool block, int64_t K) {
  const size_t head = sizeof(float) * (kWaves * 16 * (16 * NB + 1) + (kWaves + 1) * R + (block ? R * (K / 128) : 0));
  return (head + 15) / 16 * 16 + (size_t)R * (size_t)(K + 16);
}

template <int KIND, bool STATIC, bool EPI, int R, int J, int NB>
hipError_t launch_few_epi(const SmallArgs& s, hipStream_t st) {
  const size_t lds = few_lds_bytes(R, NB, KIND == SMALL_BLOCK, s.K);
  if (lds > 64 * 1024) {   // above the default dynamic-LDS limit: raise it once per device
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::atomic<bool> configured[64] = {};
    if (dev >= 64) return hipErrorInvalidDevice;
    if (!configured[dev].load()) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_qlinear_few<KIND, STATIC, EPI, R, J, NB>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)few_lds_bytes(R, NB, true, kFewMaxK));
      if (e != hipSuccess) return e;
      configured[dev].store(true);
    }
  }
  hipLaunchKernelGGL((k_qlinear_few<KIND, STATIC, EPI, R, J, NB>), dim3((unsigned)((s.N + 16 * NB - 1) / (16 * NB))),
                     dim3(kThreads), lds, st, s.a, s.M, s.K, s.lda, s.a_static, s.w, s.w_scales, s.N, s.alpha, s.bias,
                     s.c, s.ldc);
  return hipGetLastError();
}

// Workgroups of 48 columns instead of 32 when that leaves fewer columns on the busiest of the
// 256 CUs (N = 12288: 256 workgroups, one per CU, against 384, two on half of the CUs, each
// repeating the activation cast and streaming its own weight rows); 32 keeps more workgroups
// for narrower outputs.
inline bool few_wide(int64_t N) {
  constexpr int64_t kCUs = 256;
  const int64_t per_cu32 = ((N + 31) / 32 + kCUs - 1) / kCUs * 32;
  const int64_t per_cu48 = ((N + 47) / 48 + kCUs - 1) / kCUs * 48;
  return per_cu48 < per_cu32;
}

template <int KIND, bool STATIC, int R, int J = 1>
hipError_t launch_few(const SmallArgs& s, hipStream_t st) {
  const bool epi = s.alpha != 1.0f || s.bias;
  if (few_wide(s.N))
    return epi ? launch_few_epi<KIND, STATIC, true, R, J, 3>(s, st)
               : launch_few_epi<KIND, STATIC, false, R, J, 3>(s, st);
  return epi ? launch_few_epi<KIND, STATIC, true, R, J, 2>(s, st) : launch_few_epi<KIND, STATIC, false, R, J, 2>(s, st);
}

template <int KIND, bool STATIC>
hipError_t launch_kind(const SmallArgs& s, hipStream_t st) {
  if (qlinear_few_applies(s.M, s.K))
    return s.M == 1   ? (s.K <= 4096 ? launch_few<KIND, STATIC, 1>(s, st) : launch_few<KIND, STATIC, 1, 2>(s, st))
           : s.M <= 4 ? launch_few<KIND, STATIC, 4>(s, st)
                      : launch_few<KIND, STATIC, 16>(s, st);
  const dim3 grid((unsigned)((s.N + kCols - 1) / kCols)), block(kThreads);
  if (s.alpha != 1.0f || s.bias)
    hipLaunchKernelGGL((k_qlinear_small<KIND, STATIC, true>), grid, block, 0, st, s.a, s.M, s.K, s.lda, s.a_static,
                       s.w, s.w_scales, s.N, s.alpha, s.bias, s.c, s.ldc);
  else
    hipLaunchKernelGGL((k_qlinear_small<KIND, STATIC, false>), grid, block, 0, st, s.a, s.M, s.K, s.lda, s.a_static,
                       s.w, s.w_scales, s.N, s.alpha, s.bias, s.c, s.ldc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qlinear_small(int kind, const SmallArgs& s, hipStream_t st) {
  const bool stat = s.a_static != nullptr;
  switch (kind) {
    case SMALL_TENSOR: return stat ? launch_kind<SMALL_TENSOR, true>(s, st) : launch_kind<SMALL_TENSOR, false>(s, st);
    case SMALL_ROW: return launch_kind<SMALL_ROW, false>(s, st);
    case SMALL_INT8: return launch_kind<SMALL_INT8, false>(s, st);
    case SMALL_BLOCK: return stat ? launch_kind<SMALL_BLOCK, true>(s, st) : launch_kind<SMALL_BLOCK, false>(s, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pql
