// Deep-pipelined FP8 GEMM for the per-tensor / per-row scale schemes, gfx950.
//
// C[M, N] = s_a[m] * s_w[n] * sum_k e4m3(a[m, k]) * e4m3(w[n, k]), bf16 out
// ("[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO, Quark", section
// "FP8": tensor- and token-wise dynamic scales; the weight's per-output-channel
// scale is the token-wise rule applied to W's rows).
//
// Matrix core: v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales.  Lane l
// feeds row (l % 32); with g = l / 32 its 32 operand bytes are K-elements
// 16 g .. 16 g + 15 (bytes 0-15) and 32 + 16 g .. 32 + 16 g + 15 (bytes
// 16-31) of a 64-element K block -- the same split as the 16x16x128 form,
// pinned with one-hot probes on the device.  Accumulator register r of lane l
// holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// Shape: one 256 x 256 output tile per workgroup of 4 waves (one per SIMD);
// each wave owns a 128 x 128 quarter as 4 x 4 MFMA blocks (256 accumulators
// per lane).  Large wave tiles keep LDS read traffic at 64 bytes per clock
// per CU at the matrix-core peak (each wave reads 16 KB of operands per
// 64-wide K step for 16 MFMAs).
//
// Pipeline: K advances 64 bytes per step; a stage (A and W tiles) is 32 KB
// and four stages rotate through one 128 KB LDS array.  At step
// s a wave
//   1. waits for its own loads of stage s + 1 and for its LDS reads, then
//      meets the other waves at s_barrier (after which stage s + 1 is
//      complete and stage s, read during step s - 1, is free);
//   2. refills stage s with step s + 4 (global -> LDS, buffer_load ... lds);
//   3. issues the 16 MFMAs of step s on fragments already in registers,
//      interleaved one-to-one with the 16 LDS reads that fetch step s + 1's
//      fragments into the other register set.
// Loads therefore run three steps ahead of their use, and LDS latency hides
// behind the matrix core.  The direct-to-LDS loads are inline asm so that
// the compiler does not order the LDS reads behind them (its alias tracking
// cannot tell the stages of one LDS array apart); all waits on them are the
// explicit vmcnt values below.  LDS rows are 64 bytes (four 16-byte chunks); chunk c of row
// r sits at position c ^ ((r >> 1) & 3), which keeps each 8-lane group of a
// fragment read on distinct banks.  Tiles are assigned XCD by XCD in 4 x 8
// patches so that concurrent workgroups share A and W rows in L2.
#include <algorithm>

#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BKB = 64;      // tile rows, cols, K bytes per step
constexpr int kOpBytes = BM * BKB;               // one operand's tile per stage (16 KB)
constexpr int kStageBytes = 2 * kOpBytes;        // A then W
constexpr int kGroupM = 4;
constexpr int kLoadsPerStep = 8;                 // direct-to-LDS instructions per wave per step
constexpr int kEpiBytes = 32 * 128 * 2;          // per wave: 32 output rows x 128 bf16
constexpr int kPersistentCap = 256;              // one workgroup per CU

typedef float v16f __attribute__((ext_vector_type(16)));

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt 6:4
// left at its maximum, lgkmcnt in bits 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

__device__ __forceinline__ int swz64(int row, int chunk) { return row * BKB + ((chunk ^ ((row >> 1) & 3)) << 4); }

// Persistent schedule.  Workgroup b runs on XCD b % 8 (dispatch is round-robin
// over the XCDs).  Each XCD owns a contiguous range of the tile order, and its
// workgroups take consecutive tiles of that range round by round, so the
// tiles in flight on one XCD form 4 x 8 patches that share A and W rows in
// its L2.  The tile order walks 4-tile-tall groups column by column.
struct Sched {
  int tiles_m, tiles_n, first, stride, count;   // this workgroup's tiles: first + k * stride, k < count
  __device__ void init(int T, int tm_, int tn_) {
    tiles_m = tm_;
    tiles_n = tn_;
    const int G = gridDim.x, b = blockIdx.x;
    const int xcd = b & 7, slot = b >> 3;
    const int nslots = (G - xcd + 7) >> 3;                       // workgroups on this XCD
    const int per = T >> 3, rem = T & 7;
    const int start = xcd * per + min(xcd, rem), len = per + (xcd < rem ? 1 : 0);
    first = start + slot;
    stride = nslots;
    count = slot < len ? (len - slot + nslots - 1) / nslots : 0;
  }
  __device__ void coords(int k, int& tm, int& tn) const {
    const int L = first + k * stride;
    const int in_group = kGroupM * tiles_n;
    const int group = L / in_group;
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int l = L - group * in_group;
    tm = first_m + l % gm;
    tn = l / gm;
  }
};

// Buffer descriptor for bytes [base, base + nbytes); loads beyond nbytes read 0.
__device__ __forceinline__ v4i make_rsrc(const void* base, int nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)p), __builtin_amdgcn_readfirstlane((int)(p >> 32) & 0xffff),
             __builtin_amdgcn_readfirstlane(nbytes), 0x00020000};
}

// One direct-to-LDS load: 16 bytes per lane from rsrc + voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void lds_load16(v4i rsrc, const uint8_t* lds, int voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ v8i cat(uint4 lo, uint4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm32_fp8(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kStageBytes + 4 * kEpiBytes];

  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  Sched sched;
  sched.init(tiles_m * tiles_n, tiles_m, tiles_n);
  const int my_tiles = __builtin_amdgcn_readfirstlane(sched.count);
  if (my_tiles == 0) return;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int Kb = (int)g.K;
  const int nsteps = Kb / BKB;

  // ---- load stream.  Wave w moves A rows and W rows 64 w .. 64 w + 63 of a tile,
  // 16 rows (1 KB) per instruction; lane i fetches chunk (i % 4) ^ f(row) of row
  // i / 4 of the group, which lands at LDS offset 16 i.  Descriptors cover only
  // the tile's valid rows, so rows past M / N (and offsets past the end) read 0.
  // Loads run four steps ahead; the steps past a tile's end come from the next
  // tile, whose descriptors are kept beside the current ones so the choice is a
  // scalar select rather than a branch.  Past this workgroup's last tile the
  // stream refetches its last tile into stages that are never read.
  const int dl_row = wave * 64 + (lane >> 2);
  const int dl_off = dl_row * Kb + (((lane & 3) ^ ((dl_row >> 1) & 3)) << 4);   // rows + 16 q keep f(row)
  // A tile operand as a scalar (base, byte count) pair.  Each load gets a
  // descriptor whose base is moved forward by the row group and K offset (and
  // whose byte count shrinks by as much), so the per-lane offset is the one
  // loop-invariant register dl_off and the loop writes no VGPR for its loads.
  struct Span {
    uint64_t base;
    int bytes;
  };
  auto tile_spans = [&](int k, Span& as, Span& ws) {
    int tm, tn;
    sched.coords(std::min(k, my_tiles - 1), tm, tn);
    tm = __builtin_amdgcn_readfirstlane(tm);
    tn = __builtin_amdgcn_readfirstlane(tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    as = Span{reinterpret_cast<uint64_t>(g.a + m0 * Kb), (int)(std::min<int64_t>(BM, g.M - m0) * Kb)};
    ws = Span{reinterpret_cast<uint64_t>(g.w + n0 * Kb), (int)(std::min<int64_t>(BN, g.N - n0) * Kb)};
  };
  auto rsrc_at = [](const Span& sp, int off) {
    return make_rsrc(reinterpret_cast<const void*>(sp.base + (uint64_t)off), std::max(sp.bytes - off, 0));
  };
  Span a_cur, w_cur, a_nxt, w_nxt;
  tile_spans(0, a_cur, w_cur);
  tile_spans(1, a_nxt, w_nxt);
  // Load step `ls` (counted from the current tile's start) into stage `slot`.
  auto issue = [&](int ls, int slot) {
    const bool here = ls < nsteps;
    const Span as = here ? a_cur : a_nxt, ws = here ? w_cur : w_nxt;
    const int koff = (here ? ls : ls - nsteps) * BKB + wave * 64 * Kb;
    const uint8_t* stage = smem + (slot & 3) * kStageBytes + wave * 64 * BKB;
    const int voff = dl_off - wave * 64 * Kb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lds_load16(rsrc_at(as, koff + 16 * q * Kb), stage + 16 * q * BKB, voff);
      lds_load16(rsrc_at(ws, koff + 16 * q * Kb), stage + kOpBytes + 16 * q * BKB, voff);
    }
  };

  // Fragment offsets within a stage (blocks of 32 rows; rows + 32 i keep f(row)).
  const int fr = lane & 31, fk = lane >> 5;
  const int a_lo = swz64(wm * 128 + fr, fk), a_hi = swz64(wm * 128 + fr, 2 + fk);
  const int w_lo = kOpBytes + swz64(wn * 128 + fr, fk), w_hi = kOpBytes + swz64(wn * 128 + fr, 2 + fk);

  v16f acc[4][4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  zero_acc();

  uint4 fa0[4][2], fw0[4][2], fa1[4][2], fw1[4][2];   // two register sets of fragment halves
  auto read_frags = [&](uint4 (&fa)[4][2], uint4 (&fw)[4][2], int slot) {
    const uint8_t* stage = smem + (slot & 3) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i][0] = lds16(stage + a_lo + i * 32 * BKB);
      fa[i][1] = lds16(stage + a_hi + i * 32 * BKB);
      fw[i][0] = lds16(stage + w_lo + i * 32 * BKB);
      fw[i][1] = lds16(stage + w_hi + i * 32 * BKB);
    }
  };
  // The step's 16 MFMAs, each followed by one of the 16 LDS reads that fetch the
  // next step's fragments (scheduling barriers pin this order).
  auto mfmas_and_reads = [&](const uint4 (&fa)[4][2], const uint4 (&fw)[4][2], uint4 (&na)[4][2],
                             uint4 (&nw)[4][2], const uint8_t* next_stage) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(fa[i][0], fa[i][1]), cat(fw[j][0], fw[j][1]),
                                                                    acc[i][j], 0, 0, 0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
        const int k = j * 4 + i;
        const int blk = (k >> 1) & 3, half = k & 1;
        if (k < 8) na[blk][half] = lds16(next_stage + (half ? a_hi : a_lo) + blk * 32 * BKB);
        else nw[blk][half] = lds16(next_stage + (half ? w_hi : w_lo) + blk * 32 * BKB);
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // ---- epilogue of tile k: scales, bf16, 16-byte row stores.  Each wave stages 32
  // output rows at a time in its own 8 KB region (not part of the stage ring, which
  // already holds the next tile's first steps).
  uint16_t* ep = reinterpret_cast<uint16_t*>(smem + 4 * kStageBytes + wave * kEpiBytes);
  const float* sa = static_cast<const float*>(g.a_scales);
  const float* sw = static_cast<const float*>(g.w_scales);
  auto epilogue = [&](int k) {
    int tm, tn;
    sched.coords(k, tm, tn);
    const int64_t m0 = (int64_t)tm * BM + wm * 128, n0 = (int64_t)tn * BN + wn * 128;
    float cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cs[j] = sw[std::min<int64_t>(n0 + j * 32 + fr, g.N - 1) * g.w_scale_stride];
    const int64_t col0 = n0 + (lane & 15) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = 8 * (r >> 2) + 4 * fk + (r & 3);
        const float rs = sa[std::min<int64_t>(m0 + i * 32 + lr, g.M - 1) * g.a_scale_stride];
#pragma unroll
        for (int j = 0; j < 4; ++j) ep[lr * 128 + j * 32 + fr] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] * rs * cs[j]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int lr = q * 4 + (lane >> 4);
        const int64_t row = m0 + i * 32 + lr;
        const uint4 v = *reinterpret_cast<const uint4*>(ep + lr * 128 + (lane & 15) * 8);
        if (row >= g.M) continue;
        uint16_t* dst = g.c + row * g.ldc + col0;
        if (g.vec_store && col0 + 8 <= g.N) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
          const uint16_t e[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                                 (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8)
            if (col0 + e8 < g.N) dst[e8] = e[e8];
        }
      }
    }
    zero_acc();
  };

  // ---- prologue: steps 0..3 in flight; wait for stage 0 and read step 0's fragments.
#pragma unroll
  for (int s = 0; s < 4; ++s) issue(s, s);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * kLoadsPerStep, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_frags(fa0, fw0, 0);

  // ---- step s of the current tile (G counts steps over all tiles): fragments of
  // the step are in (fa, fw); stage G % 4 was read at step G - 1 and is refilled
  // with the load four steps ahead.  The look-ahead reads of the very last step
  // fetch a stage whose values are never used.  nsteps is even (K % 128 == 0), so
  // tiles end after the second step of a pair.
  auto step = [&](int s, int G, const uint4 (&fa)[4][2], const uint4 (&fw)[4][2], uint4 (&na)[4][2],
                  uint4 (&nw)[4][2]) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsPerStep, 0));   // stage G + 1 complete
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(s + 4, G);
    __builtin_amdgcn_sched_barrier(0);
    mfmas_and_reads(fa, fw, na, nw, smem + ((G + 1) & 3) * kStageBytes);
  };
  int G = 0;
  for (int k = 0; k < my_tiles; ++k) {
    for (int s = 0; s < nsteps; s += 2, G += 2) {
      step(s, G, fa0, fw0, fa1, fw1);
      step(s + 1, G + 1, fa1, fw1, fa0, fw0);
    }
    epilogue(k);
    a_cur = a_nxt;
    w_cur = w_nxt;
    tile_spans(k + 2, a_nxt, w_nxt);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

hipError_t launch_gemm32_fp8(const GemmArgs& g, hipStream_t st) {
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  // The load stream runs four K steps ahead, which stays within the next tile
  // only when a tile has at least four steps; shorter K gets one tile per
  // workgroup (its look-ahead loads then land in stages that are never read).
  const int grid = (g.K / BKB >= 4) ? std::min(tiles, kPersistentCap) : tiles;
  hipLaunchKernelGGL(k_gemm32_fp8, dim3(grid), dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace pql
