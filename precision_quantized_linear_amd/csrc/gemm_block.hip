// Persistent FP8 block-128 GEMM, gfx950.
//
// C[m, n] = bf16( sum_g s_a[m, g] * s_w[n / 128, g] * sum_{k in group g} qa[m, k] qw[n, k] )
// ("[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO, Quark", section
// "FP8": activations with one scale per 1x128 K-group, weights with one scale
// per 128x128 block), optionally as alpha * (...) + bias[n] (the fused
// epilogue of "vLLM-Omni Online Quantization complete guide", section "How
// online quantization works underneath"), applied to the fp32 sums before
// the one rounding to bf16.
//
// A 128-wide K-group is exactly one v_mfma_scale_f32_16x16x128_f8f6f4 (unit
// MFMA scales), so every group's partial product P comes out of the matrix
// core on its own and is promoted into the fp32 sums with one FMA per element:
// acc += P * (s_a[m, g] * s_w[nb, g]).  The sums are VALU operands, so they
// live in VGPRs; that caps a wave at a 128 x 64 output block (128 sums per
// lane) and a workgroup of 4 waves at a 256 x 128 tile.  The W fragment is the
// MFMA's first operand, so lane l's P holds C[m = l % 16][n = 4 (l / 16) + r]:
// one row per lane (one activation scale per 16-row block) and four
// consecutive columns; the weight scale is uniform over the tile.
//
// Pipeline: one 128-byte K-group per "region"; LDS holds three regions
// (A 256 rows + W 128 rows of 128 bytes, the A scales of the group, and the W
// scale), filled by direct-to-LDS loads of whole 128-byte lines (lane i of an
// 8-row load fetches the chunk of row i / 8 whose swizzled position is i % 8, which is the
// swizzled position: chunk c of row r at c ^ ((r / 2) % 8)).  Before region R the
// waves wait for region R + 1 and meet at a barrier; region R's 32 MFMAs are
// interleaved with the LDS reads of region R + 1's fragments and with the loads
// of region R + 3 into region R's slot.  The grid is persistent, one
// workgroup per CU, with the XCD-aware tile order of the other GEMMs.
#include <algorithm>
#include <type_traits>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

using namespace gemm;

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 128;
constexpr int kRow = 128;                          // bytes of one K-group per row
constexpr int kAOp = BM * kRow;                    // 32 KB
constexpr int kWOp = BN * kRow;                    // 16 KB
constexpr int kRegion = kAOp + kWOp;               // 48 KB
constexpr int kSlots = 3;                          // regions in the ring
constexpr int kSaBytes = BM * 4;                   // A scales of one group
constexpr int kSwBytes = 256;                      // W scale of one group, one copy per lane of a wave
constexpr int kEpiRow = 136;                       // staged output row: 64 bf16 + 8 bytes of padding
constexpr int kEpiBytes = 16 * kEpiRow;            // per wave: 16 output rows
constexpr int kLoads = 8 + 4 + 1 + 1;              // per wave and region: A rows, W rows, A scales, W scale
constexpr int kLds = kSlots * kRegion + kSlots * kSaBytes + kSlots * 4 * kSwBytes + 4 * kEpiBytes;
constexpr int kPersistentCap = 256;

typedef float v4f_t __attribute__((ext_vector_type(4)));

// EPI: apply alpha * (...) + bias in the epilogue (a separate instance, so the
// plain kernel's code is unchanged).
template <bool EPI>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_block(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];

  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  Sched sched;
  sched.init(tiles_m * tiles_n, tiles_m, tiles_n);
  const int my_tiles = __builtin_amdgcn_readfirstlane(sched.count);
  if (my_tiles == 0) return;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int Kb = (int)g.K;
  const int G = Kb / kRow;                         // K-groups = regions per tile
  const float* sa_g = static_cast<const float*>(g.a_scales);
  const float* sw_g = static_cast<const float*>(g.w_scales);

  uint8_t* const sa_lds = smem + kSlots * kRegion;                       // [slot][256] floats
  uint8_t* const sw_lds = sa_lds + kSlots * kSaBytes;                    // [slot][wave][64] floats
  uint8_t* const epi = sw_lds + kSlots * 4 * kSwBytes + wave * kEpiBytes;

  // ---- load stream (see the file comment).  One buffer descriptor per operand
  // and tile covers the tile's valid rows; each load's per-lane offset (fixed
  // for the whole kernel) holds its row and swizzled chunk, so rows past M / N
  // fall outside the descriptor and read 0, and the region's K offset rides in
  // the scalar offset, which stays inside a row.  Code part p of A is rows
  // 64 wave + 8 p .. + 7 of the tile, of W rows 32 wave + 8 p .. + 7; the
  // activation scales are rows 64 wave .. + 63, one lane per row.
  int voff_a[8], voff_w[4];
#pragma unroll
  for (int p = 0; p < 8; ++p) voff_a[p] = (wave * 64 + 8 * p + (lane >> 3)) * Kb + (dma_chunk(lane, p & 1) << 4);
#pragma unroll
  for (int p = 0; p < 4; ++p) voff_w[p] = (wave * 32 + 8 * p + (lane >> 3)) * Kb + (dma_chunk(lane, p & 1) << 4);
  const int voff_sa = (wave * 64 + lane) * G * 4;
  struct TileRsrc {
    v4i a, w, sa, sw;   // codes, activation scales, this tile's row of weight scales
  };
  auto tile_rsrc = [&](int k, TileRsrc& tr) __attribute__((always_inline)) {
    int tm, tn;
    sched.coords(std::min(k, my_tiles - 1), tm, tn);
    tm = __builtin_amdgcn_readfirstlane(tm);
    tn = __builtin_amdgcn_readfirstlane(tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int mr = (int)std::min<int64_t>(BM, g.M - m0), nr = (int)std::min<int64_t>(BN, g.N - n0);
    tr.a = make_rsrc(g.a + m0 * Kb, mr * Kb);
    tr.w = make_rsrc(g.w + n0 * Kb, nr * Kb);
    tr.sa = make_rsrc(sa_g + m0 * G, mr * G * 4);
    tr.sw = make_rsrc(sw_g + (n0 / 128) * G, G * 4);
  };
  TileRsrc cur, nxt;
  tile_rsrc(0, cur);
  tile_rsrc(1, nxt);
  // Part `part` (0..13) of K-group `rg` of tile `tr` into slot `slot`.
  auto issue_part = [&](const TileRsrc& tr, int rg, int slot, int part) __attribute__((always_inline)) {
    uint8_t* const base = smem + slot * kRegion;
    if (part < 8)
      lds_load16_so(tr.a, base + (wave * 64 + 8 * part) * kRow, voff_a[part], rg * kRow);
    else if (part < 12)
      lds_load16_so(tr.w, base + kAOp + (wave * 32 + 8 * (part - 8)) * kRow, voff_w[part - 8], rg * kRow);
    else if (part == 12)
      lds_load4_so(tr.sa, sa_lds + slot * kSaBytes + wave * 256, voff_sa, rg * 4);
    else   // the W scale, to every lane's slot
      lds_load4_so(tr.sw, sw_lds + (slot * 4 + wave) * kSwBytes, 0, rg * 4);
  };
  // Local region `lr` counts from the current tile's start; past G it is the
  // next tile's.  Past the next tile's end (only when G < 3, one tile per
  // workgroup) the group is clamped: those slots are never read.
  auto region_src = [&](int lr, int& rg) __attribute__((always_inline)) -> TileRsrc {
    const bool here = lr < G;
    rg = std::min(here ? lr : lr - G, G - 1);
    return here ? cur : nxt;   // by value: a select of the (scalar) fields
  };

  // ---- fragments: 16x16x128 operands, lane row l % 16, chunks g4 and 4 + g4.
  const int r16 = lane & 15, g4 = lane >> 4;
  const int a_lo = swz128(wm * 128 + r16, g4), a_hi = swz128(wm * 128 + r16, 4 + g4);
  const int w_lo = kAOp + swz128(wn * 64 + r16, g4), w_hi = kAOp + swz128(wn * 64 + r16, 4 + g4);
  uint4 fa0[8][2], fw0[4][2], fa1[8][2], fw1[4][2];
  float sc0[8], sc1[8];                              // s_a * s_w per 16-row block
  // LDS reads of one region's fragment number idx (0..23: 16 A halves, then 8 W halves).
  auto read_one = [&](uint4 (&fa)[8][2], uint4 (&fw)[4][2], const uint8_t* region, int idx)
                      __attribute__((always_inline)) {
    if (idx < 16) {
      const int i = idx >> 1, q = idx & 1;
      fa[i][q] = lds16(region + (q ? a_hi : a_lo) + i * 16 * kRow);
    } else {
      const int j = (idx - 16) >> 1, q = idx & 1;
      fw[j][q] = lds16(region + (q ? w_hi : w_lo) + j * 16 * kRow);
    }
  };
  auto read_scales = [&](float (&sc)[8], int slot) __attribute__((always_inline)) {
    const float* sa = reinterpret_cast<const float*>(sa_lds + slot * kSaBytes) + wm * 128 + r16;
    const float sw = reinterpret_cast<const float*>(sw_lds + (slot * 4 + wave) * kSwBytes)[lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[i] = sa[i * 16] * sw;
  };
  auto read_all = [&](uint4 (&fa)[8][2], uint4 (&fw)[4][2], float (&sc)[8], int slot)
                      __attribute__((always_inline)) {
#pragma unroll
    for (int idx = 0; idx < 24; ++idx) read_one(fa, fw, smem + slot * kRegion, idx);
    read_scales(sc, slot);
  };

  v4f_t acc[8][4];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.f, 0.f, 0.f, 0.f};
  };

  // One region: 32 MFMAs (block (i, j) = slot 4 i + j); slot s also promotes
  // the partial product of slot s - 2 (the MFMA result is ready by then), reads
  // one fragment of the next region (slots 0..23) and issues one load of region
  // lr + 3 (even slots 0..26).
  auto region = [&](auto reads_c, const uint4 (&fa)[8][2], const uint4 (&fw)[4][2], const float (&sc)[8],
                    uint4 (&na)[8][2], uint4 (&nw)[4][2], float (&nsc)[8], int R, int lr)
                    __attribute__((always_inline)) {
    constexpr bool reads = decltype(reads_c)::value;
    const uint8_t* next = smem + ((R + 1) % kSlots) * kRegion;
    const int load_slot = R % kSlots;
    int load_rg;
    const TileRsrc load_tr = region_src(lr + 3, load_rg);
    v4f_t P[4];
#pragma unroll
    for (int s = 0; s < 34; ++s) {
      if (s < 32) {
        const int i = s >> 2, j = s & 3;
        P[s & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat(fw[j][0], fw[j][1]), cat(fa[i][0], fa[i][1]),
                                                                    v4f_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0,
                                                                    127);
      }
      if (s >= 2) {
        const int p = s - 2, i = p >> 2, j = p & 3;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(P[p & 3][e], sc[i], acc[i][j][e]);
      }
      if (reads && s < 24) read_one(na, nw, next, s);
      if ((s & 1) == 0 && s < 2 * kLoads) issue_part(load_tr, load_rg, load_slot, s >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (reads) read_scales(nsc, (R + 1) % kSlots);
  };
  auto barrier_next = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 0));   // region R + 1 landed (R + 2 may be in flight)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- epilogue: per 16-row block i, the 4 column quads of each lane are staged
  // in padded LDS rows, then written as whole 128-byte lines.
  auto epilogue = [&](int k) __attribute__((always_inline)) {
    int tm, tn;
    sched.coords(k, tm, tn);
    const int64_t m0 = (int64_t)tm * BM + wm * 128, n0 = (int64_t)tn * BN + wn * 64;
    if constexpr (EPI) {   // N % 128 == 0, so every column exists
      float b[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 bw = uint2{0u, 0u};
        if (g.bias) bw = *reinterpret_cast<const uint2*>(g.bias + n0 + j * 16 + g4 * 4);
        b[j][0] = __uint_as_float(bw.x << 16);
        b[j][1] = __uint_as_float(bw.x & 0xFFFF0000u);
        b[j][2] = __uint_as_float(bw.y << 16);
        b[j][3] = __uint_as_float(bw.y & 0xFFFF0000u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(acc[i][j][e], g.alpha, b[j][e]);
    }
    const bool interior = g.vec_store && m0 + 128 <= g.M && n0 + 64 <= g.N;   // wave-uniform
    if (interior) {
      const int rr = lane >> 3, rc = lane & 7;
      uint8_t* wr = epi + r16 * kEpiRow + g4 * 8;
      const uint8_t* rd = epi + rr * kEpiRow + rc * 16;
      const uint32_t voff_c = (uint32_t)(rr * g.ldc * 2 + rc * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(wr + j * 32) =
              uint2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint2 lo = *reinterpret_cast<const uint2*>(rd + q * 8 * kEpiRow);
          const uint2 hi = *reinterpret_cast<const uint2*>(rd + q * 8 * kEpiRow + 8);
          char* base = reinterpret_cast<char*>(g.c + (m0 + i * 16 + 8 * q) * g.ldc + n0);
          *reinterpret_cast<uint4*>(base + voff_c) = uint4{lo.x, lo.y, hi.x, hi.y};
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = m0 + i * 16 + r16;
      if (row >= g.M) continue;
      uint16_t* dst_row = g.c + row * g.ldc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + j * 16 + g4 * 4;
        const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]), hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        if (g.vec_store && col + 4 <= g.N) {
          *reinterpret_cast<uint2*>(dst_row + col) = uint2{lo, hi};
        } else {
          const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (col + c < g.N) dst_row[col + c] = e[c];
        }
      }
    }
  };

  // ---- prologue: regions 0, 1, 2 in flight; then region 0's fragments.
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    int rg;
    const TileRsrc tr = region_src(s, rg);
#pragma unroll
    for (int part = 0; part < kLoads; ++part) issue_part(tr, rg, s, part);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoads, 0));   // region 0 landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_all(fa0, fw0, sc0, 0);

  // ---- the stream.  R counts regions over all tiles; sets 0 / 1 alternate per
  // region (pairs of regions per loop trip; G may be odd, then the tile's last
  // region is handled on its own).
  using RD = std::true_type;
  using NORD = std::false_type;
  int R = 0;
  for (int k = 0; k < my_tiles; ++k) {
    zero_acc();
    int r = 0;
    // Regions r, r + 1 with set 0 then set 1, while at least one more follows.
    for (; r + 2 < G; r += 2) {
      barrier_next();
      region(RD{}, fa0, fw0, sc0, fa1, fw1, sc1, R, r);
      ++R;
      barrier_next();
      region(RD{}, fa1, fw1, sc1, fa0, fw0, sc0, R, r + 1);
      ++R;
    }
    if (r + 1 < G) {   // two regions left: the second ends the tile
      barrier_next();
      region(RD{}, fa0, fw0, sc0, fa1, fw1, sc1, R, r);
      ++R;
      barrier_next();
      region(NORD{}, fa1, fw1, sc1, fa0, fw0, sc0, R, r + 1);
      ++R;
    } else {           // one region left
      barrier_next();
      region(NORD{}, fa0, fw0, sc0, fa1, fw1, sc1, R, r);
      ++R;
    }
    epilogue(k);
    // The next tile starts with set 0: its first region's fragments and scales
    // (complete: the last barrier waited for region R).
    read_all(fa0, fw0, sc0, R % kSlots);
    cur = nxt;
    tile_rsrc(k + 2, nxt);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

hipError_t launch_gemm_block(const GemmArgs& g, hipStream_t st) {
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  // The stream loads three regions ahead; when a tile has fewer than three
  // K-groups those loads would reach past the next tile, so short K gets one
  // tile per workgroup (its look-ahead loads land in slots that are never read).
  const int grid = (g.K / kRow >= kSlots) ? std::min(tiles, kPersistentCap) : tiles;
  if (g.alpha != 1.0f || g.bias) hipLaunchKernelGGL(k_gemm_block<true>, dim3(grid), dim3(kThreads), 0, st, g);
  else hipLaunchKernelGGL(k_gemm_block<false>, dim3(grid), dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace pql
