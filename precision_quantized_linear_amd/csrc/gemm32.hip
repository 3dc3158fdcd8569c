// Persistent FP8 GEMM for the per-tensor / per-row scale schemes, gfx950.
//
// C[M, N] = alpha * s_a[m] * s_w[n] * sum_k e4m3(a[m, k]) * e4m3(w[n, k]) + bias[n],
// bf16 out ("[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO, Quark",
// section "FP8": tensor- and token-wise scales; the weight's per-output-channel
// scale is the token-wise rule applied to W's rows; the fused epilogue
// alpha * (A @ B) + bias from "vLLM-Omni Online Quantization complete guide",
// section "How online quantization works underneath").  The same kernel runs
// MXFP8 / MXFP4 (scaled MFMA, no epilogue scales) and int8 with per-row
// scales (the guide's int8 online path): v_mfma_i32_32x32x32_i8 twice per
// 64-byte K slice, int32 sums converted to fp32 in the epilogue.
//
// Matrix core: v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales.  Lane l
// feeds row (l % 32) of its operand; with g = l / 32 its 32 operand bytes are
// K-elements 16 g .. 16 g + 15 (bytes 0-15) and 32 + 16 g .. 32 + 16 g + 15
// (bytes 16-31) of a 64-element K slice -- pinned with one-hot probes on the
// device.  The W fragment is the first operand and the A fragment the second,
// so accumulator register r of lane l holds C[m = l % 32][n = 8 (r / 4) +
// 4 (l / 32) + r % 4]: four consecutive output columns per register quad.
//
// Shape: one 256 x 256 output tile at a time per workgroup of 4 waves (one per
// SIMD); each wave owns a 128 x 128 quarter as 4 x 4 MFMA blocks (256
// accumulators per lane).  The grid is persistent (one workgroup per CU) and
// each workgroup walks its tiles as one continuous stream of K slices.
//
// Operands move global -> LDS with direct-to-LDS buffer loads, one full
// 128-byte line per row and instruction (8 rows x 128 bytes per wave-wide
// load): half-line loads cost about 40 % more L2 bandwidth, the limit of this
// kernel.  A line holds two 64-byte K slices, so LDS holds operands in two
// 64 KB regions, each with both slices of a K pair for all 256 A and 256 W
// rows.  With slices numbered t over the whole stream and pair j = slices
// (2 j, 2 j + 1) in region j % 2:
//   * fragments of slice t are read from LDS while slice t - 1 computes, into
//     the other of two register sets;
//   * before odd slice 2 j + 1 the waves meet at a barrier, having waited for
//     all their loads: pair j + 1 is then complete and region j % 2 (read up
//     to slice 2 j) is free;
//   * slice 2 j + 1 interleaves its 16 MFMAs with the 16 LDS reads of slice
//     2 j + 2 and with the 16 loads of pair j + 2 into region j % 2.
// Loads therefore have one to two slices to land.  The loads are inline asm:
// the compiler's alias tracking cannot tell the regions of one LDS array
// apart and would order every LDS read behind them; all waits on them are the
// explicit counts below.  Rows are 128 bytes (eight 16-byte chunks); chunk c
// of row r sits at position c ^ ((r / 2) % 8), which keeps each 16-lane group of a
// fragment read on distinct banks.
#include <algorithm>
#include <tuple>
#include <type_traits>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

using namespace gemm;

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256;
constexpr int kSlice = 64;                       // K bytes per MFMA slice
constexpr int kRow = 128;                        // K bytes per LDS row: one pair of slices
constexpr int kOpBytes = BM * kRow;              // one operand's rows in a region (32 KB)
constexpr int kRegionBytes = 2 * kOpBytes;       // A then W
constexpr int kScaleBytes = 1280;                // per wave: 128 row scales, 128 column scales, 128 bf16 biases
constexpr int kPersistentCap = 256;              // one workgroup per CU

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));


// BIAS: the FP8 / int8 epilogue adds a per-column bias (a separate instance,
// so the plain path carries no bias loads; alpha rides in the row scale).
template <int KIND, bool BIAS>
struct Kind {
  static constexpr bool kMx = KIND == GEMM_MXFP8 || KIND == GEMM_MXFP4;
  static constexpr bool kBias = BIAS && !kMx;
  static constexpr bool kFp4 = KIND == GEMM_MXFP4;
  static constexpr bool kInt8 = KIND == GEMM_INT8_ROW;
  static constexpr int kSpr = kFp4 ? 4 : 2;                // MFMA slices per 128-byte row of a region
  static constexpr int kLogSpr = kFp4 ? 2 : 1;
  static constexpr int kQ = kFp4 ? 1 : 2;                  // 16-byte fragment reads per block and slice
  static constexpr int kFmt = kFp4 ? 4 : 0;                // MFMA operand format: e2m1 or e4m3
  static constexpr int kSB = kFp4 ? 8 : 4;                 // e8m0 bytes per row and region
  static constexpr int kMxRegionBytes = kMx ? 2 * BM * kSB : 0;
  static constexpr int kWaveBytes = kMx ? 0 : kScaleBytes;
  static constexpr int kScLoads = kMx ? 0 : kBias ? 5 : 4;  // scale and bias loads per wave and tile
  static constexpr int kLdsBytes = 2 * kRegionBytes + 2 * kMxRegionBytes + 4 * kWaveBytes;
};

template <int KIND, bool BIAS>
__global__ __launch_bounds__(kThreads, 1) void k_gemm32(GemmArgs g) {
  using T = Kind<KIND, BIAS>;
  constexpr int kSpr = T::kSpr, kQ = T::kQ;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::kLdsBytes];

  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  Sched sched;
  sched.init(tiles_m * tiles_n, tiles_m, tiles_n);
  const int my_tiles = __builtin_amdgcn_readfirstlane(sched.count);
  if (my_tiles == 0) return;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int Kb = (int)(T::kFp4 ? g.K / 2 : g.K);   // bytes per operand row
  const int nreg = Kb / kRow;                      // regions (128-byte K spans) per tile
  // MX exponents are packed [region][row][kSB] (kSB = exponent bytes per row
  // and 128-byte region): one region's exponents for consecutive rows are
  // consecutive bytes, so each exponent load reads 256 contiguous bytes.
  const int64_t plane_a = g.M * T::kSB, plane_w = g.N * T::kSB;   // bytes per region of exponents

  // ---- load stream.  Wave w moves A rows and W rows 64 w .. 64 w + 63 of a tile
  // for one K region, 8 rows per instruction: lane i fetches chunk
  // dma_chunk(i) of row i / 8 of the group, which lands at LDS offset 16 i,
  // the swizzled position.  One buffer descriptor per operand and tile covers
  // the tile's valid rows; the per-lane offset of row group p (fixed for the
  // whole kernel, shared by A and W) holds the row, so rows past M / N fall
  // outside the descriptor and read 0, and the region's K offset rides in the
  // scalar offset, which stays inside a row.  Regions past a tile's end come
  // from the next tile, whose descriptors are kept beside the current ones;
  // past this workgroup's last tile the stream refetches its last tile into a
  // region that is never read.  MX scales ride the same stream: per region,
  // each row's kSB exponent bytes.
  int voff_p[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) voff_p[p] = (wave * 64 + 8 * p + (lane >> 3)) * Kb + (dma_chunk(lane, p & 1) << 4);
  const int voff_sc = lane * 4;
  struct Span {
    uint64_t base;
    int bytes;
  };
  struct TileSpans {
    v4i a, w;      // codes
    Span sa, sw;   // MX exponents
  };
  auto tile_spans = [&](int k, TileSpans& ts) __attribute__((always_inline)) {
    int tm, tn;
    sched.coords(std::min(k, my_tiles - 1), tm, tn);
    tm = __builtin_amdgcn_readfirstlane(tm);
    tn = __builtin_amdgcn_readfirstlane(tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int mr = (int)std::min<int64_t>(BM, g.M - m0), nr = (int)std::min<int64_t>(BN, g.N - n0);
    ts.a = make_rsrc(g.a + m0 * Kb, mr * Kb);
    ts.w = make_rsrc(g.w + n0 * Kb, nr * Kb);
    if constexpr (T::kMx) {
      ts.sa = Span{reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(g.a_scales) + m0 * T::kSB), mr * T::kSB};
      ts.sw = Span{reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(g.w_scales) + n0 * T::kSB), nr * T::kSB};
    }
  };
  TileSpans cur, nxt;
  tile_spans(0, cur);
  tile_spans(1, nxt);
  uint8_t* const mx_sc = smem + 2 * kRegionBytes;   // two slots of MX scales
  // Load part `part` of local region `lr` (counted from the current tile's
  // start; past nreg it is the next tile's) into LDS slot `slot`.  Parts 0..15
  // are code rows (row group part / 2 of A for even parts, of W for odd ones);
  // MX parts 16.. are the exponent rows (A, then W; 256 / kSB rows each).
  // `ts` / `rg` are the tile and its region, from load_src().
  auto issue_part = [&](const TileSpans& ts, int rg, int slot, int part) __attribute__((always_inline)) {
    if (part < 16) {
      const int rows = wave * 64 + 8 * (part >> 1);
      const uint8_t* dst = smem + (slot & 1) * kRegionBytes + (part & 1) * kOpBytes + rows * kRow;
      lds_load16_so((part & 1) ? ts.w : ts.a, dst, voff_p[part >> 1], rg * kRow);
    } else if constexpr (T::kMx) {
      constexpr int kRowsPer = 256 / T::kSB;                     // exponent rows per instruction
      const int q = part - 16, per_op = 64 / kRowsPer;
      const bool wop = q >= per_op;
      const Span& sp = wop ? ts.sw : ts.sa;
      const int rows = wave * 64 + kRowsPer * (wop ? q - per_op : q);
      const uint8_t* dst = mx_sc + (slot & 1) * T::kMxRegionBytes + (wop ? BM * T::kSB : 0) + rows * T::kSB;
      const int off = rows * T::kSB;
      lds_load4(make_rsrc(reinterpret_cast<const void*>(sp.base + (uint64_t)(rg * (wop ? plane_w : plane_a) + off)),
                          std::max(sp.bytes - off, 0)),
                dst, voff_sc);
    }
  };
  constexpr int kParts = 16 + (T::kMx ? 2 * (64 * T::kSB / 256) : 0);   // loads per wave and region
  // Local region `lr` counts from the current tile's start; past nreg it is the
  // next tile's, and past the next tile's end (nreg = 1: one tile per
  // workgroup) it is clamped into a region that is never read.
  auto load_src = [&](int lr, int& rg) __attribute__((always_inline)) -> TileSpans {
    const bool here = lr < nreg;
    rg = std::min(here ? lr : lr - nreg, nreg - 1);
    return here ? cur : nxt;   // by value: a select of the (scalar) fields
  };

  // Fragment offsets within a region for slice h: fp8 uses chunks 4 h + g and
  // 4 h + 2 + g (g = lane / 32), fp4 chunk 2 h + g; rows + 32 i keep the swizzle.
  const int fr = lane & 31, fk = lane >> 5;
  // They are recomputed after every epilogue from a fresh lane index, so that
  // they are not live across it: under the epilogue's register pressure they
  // would be spilled, and the reload's wait would also wait for the epilogue's
  // stores and the loads in flight.
  int a_off[kSpr][kQ], w_off[kSpr][kQ];
  auto compute_offsets = [&]() __attribute__((always_inline)) {
    const int l = fresh_lane();
    const int r = l & 31, c = l >> 5;
#pragma unroll
    for (int h = 0; h < kSpr; ++h)
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int chunk = T::kFp4 ? 2 * h + c : 4 * h + 2 * q + c;
        a_off[h][q] = swz128(wm * 128 + r, chunk);
        w_off[h][q] = kOpBytes + swz128(wn * 128 + r, chunk);
      }
  };
  compute_offsets();
  // MX exponents of a region: lane l holds, for each of its 4 A (and W) row
  // blocks, the kSB bytes of row 32 i + l % 32, shifted down by l / 32 bytes so
  // that byte 2 h' of dword d is the exponent of the K-block this lane's
  // operand covers in slice 4 d + h' (the slice's two 32-blocks go to the two
  // lane halves).
  const int sa_off = (wm * 128 + fr) * T::kSB, sw_off = BM * T::kSB + (wn * 128 + fr) * T::kSB;
  constexpr int kSD = T::kSB / 4;   // exponent dwords per row and region

  v16f acc[4][4];   // each tile's first slice starts the sums from zero

  uint4 fa0[4][kQ], fw0[4][kQ], fa1[4][kQ], fw1[4][kQ];   // two register sets of fragments
  int eca[4][kSD], ecw[4][kSD], ena[4][kSD], enw[4][kSD];  // MX exponents: current and next region
  auto read_frags = [&](uint4 (&fa)[4][kQ], uint4 (&fw)[4][kQ], const uint8_t* region, auto hc) __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        fa[i][q] = lds16(region + a_off[h][q] + i * 32 * kRow);
        fw[i][q] = lds16(region + w_off[h][q] + i * 32 * kRow);
      }
  };
  auto read_exps = [&](int (&ea)[4][kSD], int (&ew)[4][kSD], int slot) __attribute__((always_inline)) {
    if constexpr (T::kMx) {
      const uint8_t* base = mx_sc + (slot & 1) * T::kMxRegionBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < kSD; ++d) {
          ea[i][d] = *reinterpret_cast<const int*>(base + sa_off + i * 32 * T::kSB + 4 * d);
          ew[i][d] = *reinterpret_cast<const int*>(base + sw_off + i * 32 * T::kSB + 4 * d);
        }
    }
  };
  auto shift_exps = [&](int (&ea)[4][kSD], int (&ew)[4][kSD]) __attribute__((always_inline)) {
    if constexpr (T::kMx) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < kSD; ++d) {
          ea[i][d] = (int)((uint32_t)ea[i][d] >> (8 * fk));
          ew[i][d] = (int)((uint32_t)ew[i][d] >> (8 * fk));
        }
    }
  };
  auto operand = [](const uint4 (&f)[kQ]) __attribute__((always_inline)) {
    if constexpr (kQ == 2) return cat(f[0], f[kQ - 1]);
    else return cat(f[0], uint4{0, 0, 0, 0});
  };
  // One slice (slice h of its region): its 16 MFMAs, interleaved with the LDS
  // reads of the next slice's fragments (slice hn of `next_region`), with the
  // next region's exponents when the next slice starts a region, and, for the
  // last slice of a region, with the loads of local region `load_lr` into LDS
  // slot `load_slot` (scheduling barriers pin this order).
  auto slice = [&](auto hc, auto flags, const uint4 (&fa)[4][kQ], const uint4 (&fw)[4][kQ], uint4 (&na)[4][kQ],
                   uint4 (&nw)[4][kQ], const uint8_t* next_region, int next_slot, int load_lr, int load_slot) __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
    constexpr int fl = decltype(flags)::value;
    constexpr bool reads = fl & 1, loads = fl & 2, first = fl & 4;
    constexpr int hn = (h + 1) & (kSpr - 1);
    constexpr bool region_end = h == kSpr - 1;
    constexpr int d = T::kFp4 ? (h >> 1) : 0;
    constexpr int opsel = T::kFp4 ? 2 * (h & 1) : 2 * h;
    int load_rg = 0;
    const TileSpans load_ts = load_src(load_lr, load_rg);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v16f c = first ? v16f{} : acc[i][j];   // compile-time choice
        if constexpr (T::kInt8) {
          // K-elements 0-31 of the slice from chunk g of every lane, 32-63 from
          // chunk 2 + g: both operands use the same assignment, so each K-element
          // meets its partner whatever order the MFMA sums in.
          v16i ci = __builtin_bit_cast(v16i, c);
          ci = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, fw[j][0]), __builtin_bit_cast(v4i, fa[i][0]),
                                                    ci, 0, 0, 0);
          ci = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, fw[j][1]), __builtin_bit_cast(v4i, fa[i][1]),
                                                    ci, 0, 0, 0);
          acc[i][j] = __builtin_bit_cast(v16f, ci);
        } else if constexpr (T::kMx)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(operand(fw[j]), operand(fa[i]), c, T::kFmt,
                                                                      T::kFmt, opsel, ecw[j][d], opsel, eca[i][d]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(operand(fw[j]), operand(fa[i]), c, 0, 0, 0,
                                                                      127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
        const int k = j * 4 + i;
        if constexpr (reads) {
          if constexpr (kQ == 2) {
            const int blk = (k >> 1) & 3, q = k & 1;
            if (k < 8) na[blk][q] = lds16(next_region + a_off[hn][q] + blk * 32 * kRow);
            else nw[blk][q] = lds16(next_region + w_off[hn][q] + blk * 32 * kRow);
          } else if ((k & 1) == 0) {
            const int idx = k >> 1;
            if (idx < 4) na[idx][0] = lds16(next_region + a_off[hn][0] + idx * 32 * kRow);
            else nw[idx - 4][0] = lds16(next_region + w_off[hn][0] + (idx - 4) * 32 * kRow);
          }
          if constexpr (T::kMx && region_end) {
            if (k == 15) read_exps(ena, enw, next_slot);
          }
        }
        if constexpr (loads) {
          issue_part(load_ts, load_rg, load_slot, k);
          if (k < kParts - 16) issue_part(load_ts, load_rg, load_slot, 16 + k);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  auto region_ptr = [&](int R) __attribute__((always_inline)) { return smem + (R & 1) * kRegionBytes; };
  // Barrier before a region's last slice: this wave's loads of the next region
  // have landed, and so have every other wave's.
  auto barrier_all_loads = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The first such barrier of a tile has younger operations from the tile
  // change behind the loads it needs: vector memory operations retire in
  // issue order, so it waits only until `pend` of them are left (the previous
  // epilogue's 32 stores and the scale loads), which lets the stores drain
  // under the next slices; -1 (their number is not fixed: edge tiles) waits
  // for everything.
  auto barrier_tile_start = [&](int pend) __attribute__((always_inline)) {
    if (pend == 32 + T::kScLoads)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(32 + T::kScLoads, 0));
    else if (pend == T::kScLoads)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(T::kScLoads, 0));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- FP8 / int8 row and column scales and the bias.  Each wave keeps its 128
  // row and 128 column scales and 128 bf16 biases in its own 1.25 KB of LDS,
  // fetched by direct-to-LDS loads right after the previous tile's epilogue;
  // the next barrier's wait retires them.  Per-tensor scales have stride 0:
  // every lane then reads the one scale.  Without a bias the descriptor is
  // empty and the loads write zeros.
  uint8_t* wave_lds = smem + 2 * kRegionBytes + 2 * T::kMxRegionBytes + wave * T::kWaveBytes;
  const float* sc_rows = reinterpret_cast<const float*>(wave_lds);
  const float* sc_cols = sc_rows + 128;
  auto prefetch_scales = [&](int k) __attribute__((always_inline)) {
    if constexpr (!T::kMx) {
      int tm, tn;
      sched.coords(std::min(k, my_tiles - 1), tm, tn);
      const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane(tm) * BM + wm * 128;
      const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane(tn) * BN + wn * 128;
      const int64_t sa_first = g.a_scale_stride ? m0 : 0, sw_first = g.w_scale_stride ? n0 : 0;
      const int64_t sa_rows = g.a_scale_stride ? std::max<int64_t>(0, std::min<int64_t>(128, g.M - m0)) : 1;
      const int64_t sw_rows = g.w_scale_stride ? std::max<int64_t>(0, std::min<int64_t>(128, g.N - n0)) : 1;
      const v4i ra = make_rsrc(static_cast<const float*>(g.a_scales) + sa_first, (int)(sa_rows * 4));
      const v4i rw = make_rsrc(static_cast<const float*>(g.w_scales) + sw_first, (int)(sw_rows * 4));
      const int va = (int)g.a_scale_stride * lane * 4, vw = (int)g.w_scale_stride * lane * 4;
      uint8_t* scr = wave_lds;
      lds_load4(ra, scr, va);
      lds_load4(ra, scr + 256, va + (int)g.a_scale_stride * 256);
      lds_load4(rw, scr + 512, vw);
      lds_load4(rw, scr + 768, vw + (int)g.w_scale_stride * 256);
      if constexpr (T::kBias) {
        const int64_t nb = std::max<int64_t>(0, std::min<int64_t>(128, g.N - n0));
        lds_load4(make_rsrc(g.bias + n0, (int)(nb * 2)), scr + 1024, lane * 4);
      }
    }
  };
  const uint16_t* bias_cols = reinterpret_cast<const uint16_t*>(wave_lds + 1024);
  // Value of accumulator element (i, j, r) as written to C: rs carries alpha
  // (alpha * s_a[m]), cs is s_w[n], b the bias; int8 sums are converted first.
  auto out_val = [&](float a, float rs, float cs, float b) __attribute__((always_inline)) {
    const float v = T::kInt8 ? (float)__builtin_bit_cast(int, a) : a;
    if constexpr (T::kMx) return a;
    else if constexpr (T::kBias) return __builtin_fmaf(v * rs, cs, b);
    else return v * rs * cs;
  };

  // ---- epilogue of tile k: each lane owns output row m = 32 i + l % 32 of block
  // i and, per accumulator quad, four consecutive columns.  Returns whether
  // the wave's quarter took the interior path (exactly 32 stores).
  auto epilogue = [&](int k) __attribute__((always_inline)) -> bool {
    int tm, tn;
    sched.coords(k, tm, tn);
    const int64_t m0 = (int64_t)tm * BM + wm * 128, n0 = (int64_t)tn * BN + wn * 128;
    const bool interior = g.vec_store && m0 + 128 <= g.M && n0 + 128 <= g.N;   // wave-uniform
    // Per-lane addresses come from a fresh lane index: hoisted out of the tile
    // loop they would be spilled, and their reload would wait for the loads in
    // flight.
    const int el = fresh_lane();
    const int fr = el & 31, fk = el >> 5;
    // Stores go straight from registers.  In block (i, j) lane (fr, fk) holds,
    // per register quad rq, columns 8 rq + 4 fk .. + 3 of row 32 i + fr.  One
    // v_permlane32_swap per packed dword trades quad 2 h + 1 of the lower half
    // (fk = 0) for quad 2 h of the upper half, after which lane (fr, fk) holds
    // the 8 consecutive columns 16 h + 8 fk .. + 7: one 16-byte store, and each
    // instruction writes 32 contiguous bytes of 32 rows.  Interior quarters
    // store every piece; edge quarters (and C without 16-byte rows) mask rows
    // past M and columns past N.
    const float4* cs4 = static_cast<const float4*>(__builtin_assume_aligned(sc_cols, 16));
    const int64_t lane_off = (int64_t)fr * g.ldc + 8 * fk;   // elements from the block's first row and column
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float rs = T::kMx ? 1.0f : sc_rows[i * 32 + fr] * g.alpha;
      uint16_t* blk = g.c + (m0 + i * 32) * g.ldc + n0;   // wave-uniform
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float4 cs[4], bs[4];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          cs[rq] = T::kMx ? float4{1.f, 1.f, 1.f, 1.f} : cs4[j * 8 + rq * 2 + fk];
          bs[rq] = float4{0.f, 0.f, 0.f, 0.f};
          if constexpr (T::kBias) {
            const uint2 bw = *reinterpret_cast<const uint2*>(bias_cols + j * 32 + rq * 8 + fk * 4);
            bs[rq] = float4{__uint_as_float(bw.x << 16), __uint_as_float(bw.x & 0xFFFF0000u),
                            __uint_as_float(bw.y << 16), __uint_as_float(bw.y & 0xFFFF0000u)};
          }
        }
        const v16f a = acc[i][j];
        uint32_t d[4][2];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          d[rq][0] = pack_bf16x2(out_val(a[4 * rq + 0], rs, cs[rq].x, bs[rq].x),
                                 out_val(a[4 * rq + 1], rs, cs[rq].y, bs[rq].y));
          d[rq][1] = pack_bf16x2(out_val(a[4 * rq + 2], rs, cs[rq].z, bs[rq].z),
                                 out_val(a[4 * rq + 3], rs, cs[rq].w, bs[rq].w));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto s0 = __builtin_amdgcn_permlane32_swap(d[2 * h][0], d[2 * h + 1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(d[2 * h][1], d[2 * h + 1][1], false, false);
          const uint4 v = uint4{s0[0], s1[0], s0[1], s1[1]};
          if (interior) {
            *reinterpret_cast<uint4*>(blk + lane_off + j * 32 + h * 16) = v;
          } else {
            const int64_t row = m0 + i * 32 + fr, col = n0 + j * 32 + h * 16 + 8 * fk;
            if (row < g.M) {
              uint16_t* dst = g.c + row * g.ldc + col;
              if (g.vec_store && col + 8 <= g.N) {
                *reinterpret_cast<uint4*>(dst) = v;
              } else {
                const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int c = 0; c < 8; ++c)
                  if (col + c < g.N) dst[c] = (uint16_t)(wds[c >> 1] >> (16 * (c & 1)));
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // one accumulator block at a time
      }
    }
    return interior;
  };

  using H0 = std::integral_constant<int, 0>;
  // ---- prologue: regions 0 and 1 in flight, then slice 0's fragments.
#pragma unroll
  for (int part = 0; part < kParts; ++part) {
    int rg;
    const TileSpans ts = load_src(0, rg);
    issue_part(ts, rg, 0, part);
  }
#pragma unroll
  for (int part = 0; part < kParts; ++part) {
    int rg;
    const TileSpans ts = load_src(1, rg);
    issue_part(ts, rg, 1, part);
  }
  prefetch_scales(0);
  constexpr int kPend0 = T::kScLoads;   // issued after region 1's loads
  int pend = kPend0;
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(kParts + kPend0, 0));   // region 0 landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_frags(fa0, fw0, smem, H0{});
  read_exps(eca, ecw, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  shift_exps(eca, ecw);

  // ---- the stream.  R counts regions over all tiles.  Within a region the
  // slices alternate register sets 0 / 1 (kSpr is even, so a region and a tile
  // always start with set 0); the last slice of a region waits for all loads
  // and meets the other waves first, then refills the region two ahead and
  // reads the next region's exponents, which become current after it.
  // Flags: 1 = read the next slice's fragments, 2 = issue loads, 4 = first
  // slice of a tile (its sums start from zero).
  using F_FIRST = std::integral_constant<int, 5>;
  using F_MID = std::integral_constant<int, 1>;
  using F_LOAD = std::integral_constant<int, 3>;
  using F_END = std::integral_constant<int, 2>;
  auto adopt_exps = [&]() __attribute__((always_inline)) {
    if constexpr (T::kMx) {
      shift_exps(ena, enw);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int dd = 0; dd < kSD; ++dd) {
          eca[i][dd] = ena[i][dd];
          ecw[i][dd] = enw[i][dd];
        }
    }
  };
  // Slices 1 .. kSpr - 2 of region R (fp4 only), all in the region.
  auto inner_slices = [&](int R) __attribute__((always_inline)) {
    if constexpr (kSpr == 4) {
      slice(std::integral_constant<int, 1>{}, F_MID{}, fa1, fw1, fa0, fw0, region_ptr(R), R + 1, 0, 0);
      slice(std::integral_constant<int, 2>{}, F_MID{}, fa0, fw0, fa1, fw1, region_ptr(R), R + 1, 0, 0);
    }
  };
  int R = 0;   // regions over all tiles
  for (int k = 0; k < my_tiles; ++k) {
    slice(H0{}, F_FIRST{}, fa0, fw0, fa1, fw1, region_ptr(R), R + 1, 0, 0);
    inner_slices(R);
    barrier_tile_start(pend);
    for (int r = 0; r + 1 < nreg; ++r, ++R) {
      slice(std::integral_constant<int, kSpr - 1>{}, F_LOAD{}, fa1, fw1, fa0, fw0, region_ptr(R + 1), R + 1, r + 2,
            R);
      adopt_exps();
      slice(H0{}, F_MID{}, fa0, fw0, fa1, fw1, region_ptr(R + 1), R + 2, 0, 0);
      inner_slices(R + 1);
      barrier_all_loads();
    }
    // The tile's last slice: the next tile's first fragments are read after
    // the epilogue, which keeps their registers free while it runs.
    slice(std::integral_constant<int, kSpr - 1>{}, F_END{}, fa1, fw1, fa0, fw0, region_ptr(R + 1), R + 1, nreg + 1,
          R);
    ++R;
    pend = epilogue(k) ? 32 + T::kScLoads : -1;
    compute_offsets();
    read_frags(fa0, fw0, region_ptr(R), H0{});
    read_exps(eca, ecw, R);
    cur = nxt;
    tile_spans(k + 2, nxt);
    // The epilogue's LDS reads of the scales are done before the next tile's
    // scales may overwrite them.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    shift_exps(eca, ecw);
    prefetch_scales(k + 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

template <int KIND>
hipError_t launch_kind32(const GemmArgs& g, hipStream_t st) {
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  const int64_t row_bytes = Kind<KIND, false>::kFp4 ? g.K / 2 : g.K;
  // The load stream runs two regions ahead, into the next tile, which is the
  // next tile's own first regions only when a tile has at least two regions;
  // shorter K gets one tile per workgroup (its look-ahead loads then land in a
  // region that is never read).
  const int grid = (row_bytes / kRow >= 2) ? std::min(tiles, kPersistentCap) : tiles;
  if constexpr (!Kind<KIND, false>::kMx) {
    if (g.bias) {
      hipLaunchKernelGGL((k_gemm32<KIND, true>), dim3(grid), dim3(kThreads), 0, st, g);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gemm32<KIND, false>), dim3(grid), dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm32_fp8(const GemmArgs& g, hipStream_t st) { return launch_kind32<GEMM_FP8_ROWSCALE>(g, st); }
hipError_t launch_gemm32_int8(const GemmArgs& g, hipStream_t st) { return launch_kind32<GEMM_INT8_ROW>(g, st); }
hipError_t launch_gemm32_mx(bool fp4, const GemmArgs& g, hipStream_t st) {
  return fp4 ? launch_kind32<GEMM_MXFP4>(g, st) : launch_kind32<GEMM_MXFP8>(g, st);
}

}  // namespace pql
