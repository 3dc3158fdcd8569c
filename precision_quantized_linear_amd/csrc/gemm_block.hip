// Persistent FP8 block-128 GEMM, gfx950.  Outputs with at least 256 tiles of
// 256 x 256 run the 8-wave kernel of gemm_block256.hip instead.
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
// operands, so they live in VGPRs; that caps a wave at a 128 x 64 output block
// (128 sums per lane) and a workgroup of 4 waves at a 256 x 128 tile.  The W
// fragment is the MFMA's first operand, so lane l's P holds
// C[m = l % 32][n = 8 (r / 4) + 4 (l / 32) + r % 4] for r = 0..15: one row per
// lane (one activation scale per 32-row block) and four quads of consecutive
// columns; the weight scale is uniform over the tile.  Each block's 16
// promotion FMAs are issued after the next block's MFMAs, by which time the
// block's own result is complete.
//
// Pipeline: one 128-byte K-group per "region"; LDS holds three regions
// (A 256 rows + W 128 rows of 128 bytes, the A scales of the group, and the W
// scale), filled by direct-to-LDS loads of whole 128-byte lines (lane i of an
// 8-row load fetches the chunk of row i / 8 whose swizzled position is i % 8;
// chunk c of row r sits at c ^ ((r / 2) % 8)).  Before region R the waves
// wait for region R + 1 and meet at a barrier; region R's 16 MFMAs are
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
constexpr int kLoads = 8 + 4 + 1 + 1;              // per wave and region: A rows, W rows, A scales, W scale
constexpr int kEpiRow = 144;                       // staged output row: 64 bf16 + 16 bytes of padding
constexpr int kEpiBytes = 16 * kEpiRow;            // per wave: 16 output rows
constexpr int kLds = kSlots * kRegion + kSlots * kSaBytes + kSlots * 4 * kSwBytes + 4 * kEpiBytes;
constexpr int kPersistentCap = 256;

typedef float v16f __attribute__((ext_vector_type(16)));

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
  uint8_t* const epi = sw_lds + kSlots * 4 * kSwBytes + wave * kEpiBytes; // this wave's output staging

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
      w_off[h][q] = kAOp + swz128(wn * 64 + r32, 4 * h + 2 * q + c32);
    }
  uint4 fa0[4][2][2], fw0[2][2][2], fa1[4][2][2], fw1[2][2][2];   // [block][slice][chunk]
  float sc0[4], sc1[4];                                          // s_a * s_w per 32-row block
  // LDS read of one region's fragment number idx (0..23: 16 A, then 8 W).
  auto read_one = [&](uint4 (&fa)[4][2][2], uint4 (&fw)[2][2][2], const uint8_t* region, int idx)
                      __attribute__((always_inline)) {
    const int h = (idx >> 1) & 1, q = idx & 1;
    if (idx < 16) {
      const int i = idx >> 2;
      fa[i][h][q] = lds16(region + a_off[h][q] + i * 32 * kRow);
    } else {
      const int j = (idx - 16) >> 2;
      fw[j][h][q] = lds16(region + w_off[h][q] + j * 32 * kRow);
    }
  };
  auto read_scales = [&](float (&sc)[4], int slot) __attribute__((always_inline)) {
    const float* sa = reinterpret_cast<const float*>(sa_lds + slot * kSaBytes) + wm * 128 + r32;
    const float sw = reinterpret_cast<const float*>(sw_lds + (slot * 4 + wave) * kSwBytes)[lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sa[i * 32] * sw;
  };
  auto read_all = [&](uint4 (&fa)[4][2][2], uint4 (&fw)[2][2][2], float (&sc)[4], int slot)
                      __attribute__((always_inline)) {
#pragma unroll
    for (int idx = 0; idx < 24; ++idx) read_one(fa, fw, smem + slot * kRegion, idx);
    read_scales(sc, slot);
  };

  v16f acc[4][2];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  };
  // Partial products of the 32 x 32 blocks, alternating between two buffers.
  v16f P[2];
  // acc(block b) += P[b % 2] * s for elements 8 half .. + 7.
  auto promote = [&](int b, int half, float s) __attribute__((always_inline)) {
    const int i = b >> 1, j = b & 1;
#pragma unroll
    for (int e = 8 * half; e < 8 * half + 8; ++e) acc[i][j][e] = __builtin_fmaf(P[b & 1][e], s, acc[i][j][e]);
  };

  // One region: 16 MFMAs, block b = (i, j) = (b / 2, b % 2) takes slots 2 b
  // (slice 0, from zero) and 2 b + 1 (slice 1, accumulating).  Block b is
  // promoted over slots 2 b + 2 and 2 b + 3, behind the next block's MFMAs;
  // the last block's promotion is carried into the next region's slots 0 and
  // 1 (CARRY: with the previous region's scales, which are still in `nsc`), or
  // done after the tile's last region (flush).  Slot s also reads fragments of
  // the next region (A part s, and W part s for s < 8; a tile's last region
  // reads the next tile's first one, which has landed too) and issues load
  // part s (s < 14) of region lr + 3.
  auto region = [&](auto carry_c, const uint4 (&fa)[4][2][2], const uint4 (&fw)[2][2][2], const float (&sc)[4],
                    uint4 (&na)[4][2][2], uint4 (&nw)[2][2][2], float (&nsc)[4], int R, int lr)
                    __attribute__((always_inline)) {
    constexpr bool carry = decltype(carry_c)::value;
    const uint8_t* next = smem + ((R + 1) % kSlots) * kRegion;
    const int load_slot = R % kSlots;
    int load_rg;
    const TileRsrc load_tr = region_src(lr + 3, load_rg);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int b = s >> 1, h = s & 1, i = b >> 1, j = b & 1;
      P[b & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(fw[j][h][0], fw[j][h][1]),
                                                                 cat(fa[i][h][0], fa[i][h][1]),
                                                                 h ? P[b & 1] : v16f{}, 0, 0, 0, 127, 0, 127);
      // In each slot the MFMA goes first, then the reads and the load (which
      // cover the wait for the previous slot's result), then the FMAs.
      __builtin_amdgcn_sched_barrier(0);
      read_one(na, nw, next, s);
      if (s < 8) read_one(na, nw, next, 16 + s);
      if (s < kLoads) issue_part(load_tr, load_rg, load_slot, s);
      __builtin_amdgcn_sched_barrier(0);
      if (s < 2) {
        if constexpr (carry) promote(7, s, nsc[3]);
      } else {
        promote((s - 2) >> 1, s & 1, sc[(s - 2) >> 2]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    read_scales(nsc, (R + 1) % kSlots);
  };
  auto barrier_next = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 0));   // region R + 1 landed (R + 2 may be in flight)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
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
    float bs[2][4][4];   // bias of the lane's columns (EPI; N % 128 == 0, so every column exists)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        uint2 bw = uint2{0u, 0u};
        if constexpr (EPI) {
          if (g.bias) bw = *reinterpret_cast<const uint2*>(g.bias + n0 + j * 32 + rq * 8 + fk * 4);
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

  // ---- the stream.  R counts regions over all tiles.  A tile's first region
  // uses register set 0 and carries nothing in; the sets then alternate (pairs
  // of regions per loop trip), and the last block of the tile's last region is
  // promoted after it, with that region's scales.  (The tail has no code of
  // its own that repeats a region: identical MFMA chains on both sides of a
  // branch get hoisted above it, all live at once.)
  using T_ = std::true_type;
  using F_ = std::false_type;
  int R = 0;
  for (int k = 0; k < my_tiles; ++k) {
    zero_acc();
    barrier_next();
    region(F_{}, fa0, fw0, sc0, fa1, fw1, sc1, R, 0);
    ++R;
    int r = 1;
    for (; r + 1 < G; r += 2) {
      barrier_next();
      region(T_{}, fa1, fw1, sc1, fa0, fw0, sc0, R, r);
      ++R;
      barrier_next();
      region(T_{}, fa0, fw0, sc0, fa1, fw1, sc1, R, r + 1);
      ++R;
    }
    if (r < G) {   // G even: region G - 1 runs on set 1
      barrier_next();
      region(T_{}, fa1, fw1, sc1, fa0, fw0, sc0, R, r);
      ++R;
    }
    const float s_last = (G & 1) ? sc0[3] : sc1[3];
    promote(7, 0, s_last);
    promote(7, 1, s_last);
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
  if (gemm_block_uses_256(g.M, g.N)) return launch_gemm_block256(g, st);
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
