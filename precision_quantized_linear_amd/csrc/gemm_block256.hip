// Persistent FP8 block-128 GEMM for large outputs, gfx950 (256 x 256 tiles, 8 waves).
//
// C[m, n] = bf16( sum_g s_a[m, g] * s_w[n / 128, g] * sum_{k in group g} qa[m, k] qw[n, k] )
// ("[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO, Quark", section
// "FP8": activations with one scale per 1x128 K-group, weights with one scale
// per 128x128 block), optionally as alpha * (...) + bias[n] (the fused
// epilogue of "vLLM-Omni Online Quantization complete guide", section "How
// online quantization works underneath"), applied to the fp32 sums before
// the one rounding to bf16.
//
// A 128-wide K-group is two v_mfma_scale_f32_32x32x64_f8f6f4 (unit MFMA
// scales) per 32 x 32 output block, so every group's partial product P comes
// out of the matrix core on its own and is promoted into the fp32 sums with
// one FMA per element: acc += P * (s_a[m, g] * s_w[nb, g]).  The sums are VALU
// operands, so they live in VGPRs: 128 per lane for a wave's 128 x 64 part
// (4 x 2 blocks).  The W fragment is the MFMA's first operand, so lane l's P
// holds C[m = l % 32][n = 8 (r / 4) + 4 (l / 32) + r % 4] for r = 0..15: one
// row per lane (one activation scale per 32-row block) and four quads of
// consecutive columns; a wave's 64 columns lie in one 128-wide weight block,
// so its weight scale is uniform.
//
// Shape: a 256 x 256 tile per workgroup of 8 waves, two per SIMD; wave w owns
// the 128 x 64 part (w / 4, w % 4).  The two waves of a SIMD take turns on
// its matrix core: one wave's promotion FMAs and LDS reads run while the
// other's MFMAs do, which a single wave cannot do (its own VALU and MFMA
// instructions do not overlap), and the 256 x 256 tile needs 1.5x fewer
// operand bytes per flop than a 256 x 128 one.
//
// Pipeline: LDS holds two K-groups ("regions": A and W, 256 rows of 128 bytes
// each, 64 KB, with each row's 16-byte chunk c at c ^ ((r / 2) % 8), plus the
// group's activation scales and each wave's weight scale).  At the start of
// region R every wave waits for its own loads of R and meets the others at a
// barrier; slot (R + 1) % 2 is then free and each wave issues its share of
// region R + 1 into it (direct-to-LDS loads of whole 128-byte lines: A and W
// rows 32 w .. + 31, waves 0-3 the activation scales of 64 rows, every wave
// its weight scale), which have the whole region to land.  Within a region a
// wave reads its W fragments and the first A block, then per block (i, j)
// issues the two MFMAs, prefetches the next A block and promotes the previous
// block (whose MFMAs have finished behind the other wave's work); the last
// block is promoted at the start of the next region, or before the epilogue.
// The grid is persistent, one workgroup per CU, with the XCD-aware tile order
// of the other GEMMs.
#include <algorithm>
#include <type_traits>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

using namespace gemm;

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int BM = 256, BN = 256;
constexpr int kRow = 128;                          // bytes of one K-group per row
constexpr int kOp = 256 * kRow;                    // 32 KB: one operand's rows of a region
constexpr int kRegion = 2 * kOp;                   // A then W
constexpr int kSlots = 2;
constexpr int kSaBytes = BM * 4;                   // activation scales of one group
constexpr int kSwBytes = 256;                      // a wave's weight scale, one copy per lane
constexpr int kEpiRow = 144;                       // staged output row: 64 bf16 + 16 bytes of padding
constexpr int kEpiBytes = 16 * kEpiRow;            // per wave: 16 output rows
constexpr int kLds = kSlots * kRegion + kSlots * kSaBytes + kSlots * kWaves * kSwBytes + kWaves * kEpiBytes;
constexpr int kPersistentCap = 256;

typedef float v16f __attribute__((ext_vector_type(16)));

// EPI: apply alpha * (...) + bias in the epilogue (a separate instance, so the
// plain kernel's code is unchanged).
template <bool EPI>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_block256(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];

  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  Sched sched;
  sched.init(tiles_m * tiles_n, tiles_m, tiles_n);
  const int my_tiles = __builtin_amdgcn_readfirstlane(sched.count);
  if (my_tiles == 0) return;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int Kb = (int)g.K;
  const int G = Kb / kRow;                         // K-groups = regions per tile
  const int nblocks = (int)(g.N / 128);            // weight-scale blocks along N
  const float* sa_g = static_cast<const float*>(g.a_scales);
  const float* sw_g = static_cast<const float*>(g.w_scales);

  uint8_t* const sa_lds = smem + kSlots * kRegion;                             // [slot][256] floats
  uint8_t* const sw_lds = sa_lds + kSlots * kSaBytes;                          // [slot][wave][64] floats
  uint8_t* const epi = sw_lds + kSlots * kWaves * kSwBytes + wave * kEpiBytes; // this wave's output staging

  // ---- load stream (see the file comment).  One buffer descriptor per operand
  // and tile covers the tile's valid rows; each load's per-lane offset (fixed
  // for the whole kernel) holds its row and swizzled chunk, so rows past M / N
  // fall outside the descriptor and read 0, and the region's K offset rides in
  // the scalar offset, which stays inside a row.  Load p of a wave covers rows
  // 32 w + 8 p .. + 7 of A and of W (row group 4 w + p has the parity of p).
  int voff[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) voff[p] = (wave * 32 + 8 * p + (lane >> 3)) * Kb + (dma_chunk(lane, p & 1) << 4);
  const int voff_sa = ((wave & 3) * 64 + lane) * G * 4;   // waves 0-3: activation scales of rows 64 w .. + 63
  struct TileRsrc {
    v4i a, w, sa, sw;   // codes, activation scales, this wave's row of weight scales
  };
  auto tile_rsrc = [&](int k, TileRsrc& tr) __attribute__((always_inline)) {
    int tm, tn;
    sched.coords(std::min(k, my_tiles - 1), tm, tn);
    tm = __builtin_amdgcn_readfirstlane(tm);
    tn = __builtin_amdgcn_readfirstlane(tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int mr = (int)std::min<int64_t>(BM, g.M - m0), nr = (int)std::min<int64_t>(BN, g.N - n0);
    // the wave's weight block; a wave wholly past N takes the last one (its sums are never stored)
    const int nb = std::min((int)(n0 / 128) + (wn >> 1), nblocks - 1);
    tr.a = make_rsrc(g.a + m0 * Kb, mr * Kb);
    tr.w = make_rsrc(g.w + n0 * Kb, nr * Kb);
    tr.sa = make_rsrc(sa_g + m0 * G, mr * G * 4);
    tr.sw = make_rsrc(sw_g + (int64_t)nb * G, G * 4);
  };
  TileRsrc cur, nxt;
  tile_rsrc(0, cur);
  tile_rsrc(1, nxt);
  // Local region `lr` counts from the current tile's start; lr == G is the
  // next tile's first (past the workgroup's last tile: its last tile again,
  // into a slot that is never read).
  auto issue_region = [&](int lr, int slot) __attribute__((always_inline)) {
    const bool here = lr < G;
    const int rg = here ? lr : 0;
    const TileRsrc tr = here ? cur : nxt;   // by value: a select of the (scalar) fields
    uint8_t* const base = smem + slot * kRegion;
    // the scales first: the activation scales are a gather (one cache line per row), and
    // issued ahead of the code lines they no longer finish last
    if (wave < 4) lds_load4_so(tr.sa, sa_lds + slot * kSaBytes + wave * 256, voff_sa, rg * 4);
    lds_load4_so(tr.sw, sw_lds + (slot * kWaves + wave) * kSwBytes, 0, rg * 4);
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_load16_so(tr.a, base + (wave * 32 + 8 * p) * kRow, voff[p], rg * kRow);
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_load16_so(tr.w, base + kOp + (wave * 32 + 8 * p) * kRow, voff[p], rg * kRow);
  };

  // ---- fragments: 32x32x64 operands, lane row l % 32; slice h (bytes 64 h ..
  // + 63 of the group) takes chunks 4 h + c and 4 h + 2 + c (c = l / 32) of the
  // row, for A and W alike; rows + 32 i keep the swizzle.
  const int r32 = lane & 31, c32 = lane >> 5;
  int a_off[2][2], w_off[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      a_off[h][q] = swz128(wm * 128 + r32, 4 * h + 2 * q + c32);
      w_off[h][q] = kOp + swz128(wn * 64 + r32, 4 * h + 2 * q + c32);
    }
  uint4 fw[2][2][2];   // [j][slice][chunk]
  uint4 fa[2][2][2];   // [buffer][slice][chunk]: A block i in buffer i % 2
  auto read_w = [&](const uint8_t* region) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 2; ++q) fw[j][h][q] = lds16(region + w_off[h][q] + j * 32 * kRow);
  };
  auto read_a = [&](const uint8_t* region, int i) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 2; ++q) fa[i & 1][h][q] = lds16(region + a_off[h][q] + i * 32 * kRow);
  };
  float sc[4], scp[4];   // s_a * s_w per 32-row block: this region's, the previous region's
  auto read_scales = [&](int slot) __attribute__((always_inline)) {
    const float* sa = reinterpret_cast<const float*>(sa_lds + slot * kSaBytes) + wm * 128 + r32;
    const float sw = reinterpret_cast<const float*>(sw_lds + (slot * kWaves + wave) * kSwBytes)[lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sa[i * 32] * sw;
  };

  v16f acc[4][2];
  v16f P[2];   // partial products of consecutive blocks, alternating
  // acc(block b) += P[b % 2] * s, elements 8 half .. + 7
  auto promote = [&](int b, int half, float s) __attribute__((always_inline)) {
    const int i = b >> 1, j = b & 1;
#pragma unroll
    for (int e = 8 * half; e < 8 * half + 8; ++e) acc[i][j][e] = __builtin_fmaf(P[b & 1][e], s, acc[i][j][e]);
  };

  // One region (local index lr, global R): the next region's loads, this
  // region's fragments and scales, the carried promotion of the previous
  // region's last block (carry), then the 8 blocks.
  auto region = [&](int R, int lr, bool carry) __attribute__((always_inline)) {
    const int slot = R & 1;
    const uint8_t* rgn = smem + slot * kRegion;
    issue_region(lr + 1, slot ^ 1);
    read_w(rgn);
    read_a(rgn, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) scp[i] = sc[i];
    read_scales(slot);
    if (carry) {
      promote(7, 0, scp[3]);
      promote(7, 1, scp[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int i = b >> 1, j = b & 1;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        P[b & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(fw[j][h][0], fw[j][h][1]),
                                                                   cat(fa[i & 1][h][0], fa[i & 1][h][1]),
                                                                   h ? P[b & 1] : v16f{}, 0, 0, 0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
      if (j == 0 && i < 3) read_a(rgn, i + 1);
      if (b > 0) {
        promote(b - 1, 0, sc[(b - 1) >> 1]);
        promote(b - 1, 1, sc[(b - 1) >> 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- epilogue.  In block (i, j) lane (r, c) = (l % 32, l / 32) holds, per
  // register quad rq, columns 8 rq + 4 c .. + 3 of row 32 i + r.  One
  // v_permlane32_swap per packed dword trades quad 2 h + 1 of the lower half
  // for quad 2 h of the upper half, after which the lane holds the 8
  // consecutive columns 32 j + 16 h + 8 c .. + 7 (16 bytes).  Interior blocks
  // are staged 16 rows at a time in padded LDS rows and written as whole
  // 128-byte row segments (8 lanes per row), which keeps the number of cache
  // lines per store instruction at 8 (the vector memory path also carries the
  // operand stream); edge blocks (and C without 16-byte rows) store the pieces
  // directly, masking rows past M and columns past N.
  auto epilogue = [&](int k) __attribute__((always_inline)) {
    int tm, tn;
    sched.coords(k, tm, tn);
    const int64_t m0 = (int64_t)tm * BM + wm * 128, n0 = (int64_t)tn * BN + wn * 64;
    const bool interior = g.vec_store && m0 + 128 <= g.M && n0 + 64 <= g.N;   // wave-uniform
    const int el = fresh_lane();
    const int fr = el & 31, fk = el >> 5;
    const int rr = el >> 3, rc = el & 7;   // staged read-back: row rr (+ 8), 16-byte piece rc
    const int64_t voff_c = (int64_t)rr * g.ldc * 2 + rc * 16;   // bytes; 64-bit for any ldc
    float bs[2][4][4];   // bias of the lane's columns (EPI)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        uint2 bw = uint2{0u, 0u};
        if constexpr (EPI) {   // a wave's 64 columns lie wholly inside or outside N (N % 128 == 0)
          if (g.bias && n0 < g.N) bw = *reinterpret_cast<const uint2*>(g.bias + n0 + j * 32 + rq * 8 + fk * 4);
        }
        bs[j][rq][0] = __uint_as_float(bw.x << 16);
        bs[j][rq][1] = __uint_as_float(bw.x & 0xFFFF0000u);
        bs[j][rq][2] = __uint_as_float(bw.y << 16);
        bs[j][rq][3] = __uint_as_float(bw.y & 0xFFFF0000u);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 u[2][2];   // [j][h]
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
          v[e] = EPI ? __builtin_fmaf(acc[i][j][e], g.alpha, bs[j][e >> 2][e & 3]) : acc[i][j][e];
        uint32_t d[4][2];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          d[rq][0] = pack_bf16x2(v[4 * rq + 0], v[4 * rq + 1]);
          d[rq][1] = pack_bf16x2(v[4 * rq + 2], v[4 * rq + 3]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto s0 = __builtin_amdgcn_permlane32_swap(d[2 * h][0], d[2 * h + 1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(d[2 * h][1], d[2 * h + 1][1], false, false);
          u[j][h] = uint4{s0[0], s1[0], s0[1], s1[1]};
        }
      }
      if (interior) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {   // rows 16 p .. + 15 of the block
          if ((fr >> 4) == p) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int h = 0; h < 2; ++h)
                *reinterpret_cast<uint4*>(epi + (fr & 15) * kEpiRow + (j * 32 + h * 16 + 8 * fk) * 2) = u[j][h];
          }
          // The rows pass between lanes of the wave (LDS runs one wave's
          // accesses in order): the compiler must neither reuse the previous
          // pass's reads for lanes that did not write nor move the next pass's
          // writes above these reads.
          asm volatile("" ::: "memory");
          uint4 w[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) w[q] = lds16(epi + (rr + 8 * q) * kEpiRow + rc * 16);
          asm volatile("" ::: "memory");
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            char* base = reinterpret_cast<char*>(g.c + (m0 + i * 32 + 16 * p + 8 * q) * g.ldc + n0);
            *reinterpret_cast<uint4*>(base + voff_c) = w[q];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int64_t row = m0 + i * 32 + fr, col = n0 + j * 32 + h * 16 + 8 * fk;
            if (row < g.M) {
              uint16_t* dst = g.c + row * g.ldc + col;
              if (g.vec_store && col + 8 <= g.N) {
                *reinterpret_cast<uint4*>(dst) = u[j][h];
              } else {
                const uint32_t wds[4] = {u[j][h].x, u[j][h].y, u[j][h].z, u[j][h].w};
#pragma unroll
                for (int c = 0; c < 8; ++c)
                  if (col + c < g.N) dst[c] = (uint16_t)(wds[c >> 1] >> (16 * (c & 1)));
              }
            }
          }
      }
      __builtin_amdgcn_sched_barrier(0);   // one accumulator block at a time
    }
  };

  // ---- the stream.  R counts regions over all tiles; region R uses slot R % 2.
  issue_region(0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = 0.f;
  int R = 0;
  for (int k = 0; k < my_tiles; ++k) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
    for (int r = 0; r < G; ++r, ++R) {
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // this wave's loads of region R (and older work)
      __builtin_amdgcn_s_barrier();                    // everyone's; slot (R + 1) % 2 is free
      __builtin_amdgcn_sched_barrier(0);
      region(R, r, r > 0);
    }
    promote(7, 0, sc[3]);   // the tile's last block
    promote(7, 1, sc[3]);
    epilogue(k);
    cur = nxt;
    tile_rsrc(k + 2, nxt);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

hipError_t launch_gemm_block256(const GemmArgs& g, hipStream_t st) {
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  const int grid = std::min(tiles, kPersistentCap);
  if (g.alpha != 1.0f || g.bias) hipLaunchKernelGGL(k_gemm_block256<true>, dim3(grid), dim3(kThreads), 0, st, g);
  else hipLaunchKernelGGL(k_gemm_block256<false>, dim3(grid), dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace pql
