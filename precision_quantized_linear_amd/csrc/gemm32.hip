// Persistent FP8 GEMM for the per-tensor / per-row scale schemes, gfx950.
//
// C[M, N] = s_a[m] * s_w[n] * sum_k e4m3(a[m, k]) * e4m3(w[n, k]), bf16 out
// ("[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO, Quark", section
// "FP8": tensor- and token-wise dynamic scales; the weight's per-output-channel
// scale is the token-wise rule applied to W's rows).
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
// of row r sits at position c ^ (r % 8), which keeps each 8-lane group of a
// fragment read on distinct banks.
#include <algorithm>

#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256;
constexpr int kSlice = 64;                       // K bytes per MFMA slice
constexpr int kRow = 128;                        // K bytes per LDS row: one pair of slices
constexpr int kOpBytes = BM * kRow;              // one operand's rows in a region (32 KB)
constexpr int kRegionBytes = 2 * kOpBytes;       // A then W
constexpr int kScaleBytes = 1024;                // per wave: 128 row scales, then 128 column scales
constexpr int kEpiRow = 136;                     // staged output row: 64 bf16 + 8 bytes of padding
constexpr int kEpiBytes = 32 * kEpiRow;          // per wave: 32 output rows staged for row stores
constexpr int kWaveBytes = kScaleBytes + kEpiBytes;
constexpr int kGroupM = 4;
constexpr int kPersistentCap = 256;              // one workgroup per CU

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt 6:4
// left at its maximum, lgkmcnt in bits 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

__device__ __forceinline__ int swz128(int row, int chunk) { return row * kRow + ((chunk ^ (row & 7)) << 4); }

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
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff),
               "s"(rsrc)
               : "memory", "m0");
}

// One direct-to-LDS load of 4 bytes per lane: rsrc + voff into LDS at lds + 4 * lane.
__device__ __forceinline__ void lds_load4(v4i rsrc, const uint8_t* lds, int voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff),
               "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ v8i cat(uint4 lo, uint4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm32_fp8(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kRegionBytes + 4 * kWaveBytes];

  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  Sched sched;
  sched.init(tiles_m * tiles_n, tiles_m, tiles_n);
  const int my_tiles = __builtin_amdgcn_readfirstlane(sched.count);
  if (my_tiles == 0) return;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int Kb = (int)g.K;
  const int nsteps = Kb / kSlice;               // slices per tile (even: K % 128 == 0)

  // ---- load stream.  Wave w moves A rows and W rows 64 w .. 64 w + 63 of a tile
  // for one K pair, 8 rows per instruction: lane i fetches chunk (i % 8) ^ (i / 8)
  // of row i / 8 of the group, which lands at LDS offset 16 i, the swizzled
  // position.  Each load's descriptor starts at its row group and K pair and
  // covers only the tile's valid rows (rows past M / N read 0), so the per-lane
  // offset is the one loop-invariant register `voff`.  Pairs past a tile's end
  // come from the next tile, whose (base, bytes) pairs are kept beside the
  // current ones; past this workgroup's last tile the stream refetches its last
  // tile into a region that is never read.
  const int voff = (lane >> 3) * Kb + (((lane & 7) ^ (lane >> 3)) << 4);
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
  // Load part `part` (0..15: row group part / 2 of A for even parts, of W for odd
  // ones) of the pair starting at local slice `ls` (even; counted from the
  // current tile's start) into region `region`.
  auto issue_part = [&](int ls, int region, int part) {
    const bool here = ls < nsteps;
    const Span sp = (part & 1) ? (here ? w_cur : w_nxt) : (here ? a_cur : a_nxt);
    const int rows = wave * 64 + 8 * (part >> 1);
    const int off = (here ? ls : ls - nsteps) * kSlice + rows * Kb;
    const uint8_t* dst = smem + (region & 1) * kRegionBytes + (part & 1) * kOpBytes + rows * kRow;
    lds_load16(rsrc_at(sp, off), dst, voff);
  };

  // Fragment offsets within a region: slice half h of the pair uses chunks
  // 4 h + g and 4 h + 2 + g (g = lane / 32); rows + 32 i keep the swizzle.
  const int fr = lane & 31, fk = lane >> 5;
  int a_off[2][2], w_off[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      a_off[h][q] = swz128(wm * 128 + fr, 4 * h + 2 * q + fk);
      w_off[h][q] = kOpBytes + swz128(wn * 128 + fr, 4 * h + 2 * q + fk);
    }

  v16f acc[4][4];   // each tile's first slice starts the sums from zero

  uint4 fa0[4][2], fw0[4][2], fa1[4][2], fw1[4][2];   // two register sets of fragment halves
  auto read_frags = [&](uint4 (&fa)[4][2], uint4 (&fw)[4][2], const uint8_t* region, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        fa[i][q] = lds16(region + a_off[h][q] + i * 32 * kRow);
        fw[i][q] = lds16(region + w_off[h][q] + i * 32 * kRow);
      }
  };
  // One slice: its 16 MFMAs, each followed by one of the 16 LDS reads that fetch
  // the next slice's fragments (half h of `next_region`) and, for the first
  // slice of a pair, by one of the 16 loads of the pair starting at local slice
  // `ls` into `load_region` (scheduling barriers pin this order).
  auto slice = [&](const uint4 (&fa)[4][2], const uint4 (&fw)[4][2], uint4 (&na)[4][2], uint4 (&nw)[4][2],
                   const uint8_t* next_region, int h, bool loads, int ls, int load_region, bool reads = true,
                   bool first = false) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            cat(fw[j][0], fw[j][1]), cat(fa[i][0], fa[i][1]), first ? v16f{} : acc[i][j], 0, 0, 0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
        const int k = j * 4 + i;
        const int blk = (k >> 1) & 3, q = k & 1;
        if (reads) {
          if (k < 8) na[blk][q] = lds16(next_region + a_off[h][q] + blk * 32 * kRow);
          else nw[blk][q] = lds16(next_region + w_off[h][q] + blk * 32 * kRow);
        }
        if (loads) issue_part(ls, load_region, k);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  auto region_of = [&](int G) { return smem + ((G >> 1) & 1) * kRegionBytes; };   // slice G's pair region
  auto barrier_all_loads = [&]() {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- scales.  Each wave keeps its 128 row and 128 column scales in its own
  // 1 KB of LDS, fetched by direct-to-LDS loads right after the previous tile's
  // epilogue; the next barrier's wait retires them.  Per-tensor scales have
  // stride 0: every lane then reads the one scale.
  uint8_t* scr = smem + 2 * kRegionBytes + wave * kWaveBytes;
  const float* sc_rows = reinterpret_cast<const float*>(scr);
  const float* sc_cols = sc_rows + 128;
  auto prefetch_scales = [&](int k) {
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
    lds_load4(ra, scr, va);
    lds_load4(ra, scr + 256, va + (int)g.a_scale_stride * 256);
    lds_load4(rw, scr + 512, vw);
    lds_load4(rw, scr + 768, vw + (int)g.w_scale_stride * 256);
  };

  // ---- epilogue of tile k: each lane owns output row m = 32 i + l % 32 of block
  // i and, per accumulator quad, four consecutive columns: scale, round to bf16,
  // store 8 bytes (the two lane halves of a row fill 16 contiguous bytes).
  auto epilogue = [&](int k) {
    int tm, tn;
    sched.coords(k, tm, tn);
    const int64_t m0 = (int64_t)tm * BM + wm * 128, n0 = (int64_t)tn * BN + wn * 128;
    const bool interior = g.vec_store && m0 + 128 <= g.M && n0 + 128 <= g.N;   // wave-uniform
    if (interior) {
      // The wave's 128 x 128 quarter is inside C.  Rows go out through LDS so
      // that each store writes whole 128-byte lines: per 32-row block i and
      // 64-column half p, lanes write their scaled bf16 quads (8 bytes) into a
      // 32-row staging block, then read it back as 16-byte row pieces (8 lanes
      // per row, 8 rows per instruction).  Staged rows are padded to 136 bytes,
      // which keeps both the quad writes and the row reads on distinct banks
      // with constant offsets from one per-lane address.
      uint8_t* stg = scr + kScaleBytes;
      const float4* cs4 = static_cast<const float4*>(__builtin_assume_aligned(sc_cols, 16));
      const int rr = lane >> 3, rc = lane & 7;             // read-back: row rr + 8 q, 16-byte piece rc
      uint8_t* wr = stg + fr * kEpiRow + fk * 8;
      const uint8_t* rd = stg + rr * kEpiRow + rc * 16;
      const uint32_t voff = (uint32_t)(rr * g.ldc * 2 + rc * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float rs = sc_rows[i * 32 + fr];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * p + jj;
            float4 cs[4];
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) cs[rq] = cs4[j * 8 + rq * 2 + fk];
            const v16f a = acc[i][j];
#pragma unroll
            for (int rq = 0; rq < 4; ++rq)
              *reinterpret_cast<uint2*>(wr + (jj * 8 + rq * 2) * 8) =
                  uint2{pack_bf16x2(a[4 * rq + 0] * rs * cs[rq].x, a[4 * rq + 1] * rs * cs[rq].y),
                        pack_bf16x2(a[4 * rq + 2] * rs * cs[rq].z, a[4 * rq + 3] * rs * cs[rq].w)};
            __builtin_amdgcn_sched_barrier(0);   // one accumulator block at a time
          }
#pragma unroll
          for (int qr = 0; qr < 4; ++qr) {
            const uint2 lo = *reinterpret_cast<const uint2*>(rd + qr * 8 * kEpiRow);
            const uint2 hi = *reinterpret_cast<const uint2*>(rd + qr * 8 * kEpiRow + 8);
            char* base = reinterpret_cast<char*>(g.c + (m0 + i * 32 + 8 * qr) * g.ldc + n0 + p * 64);
            *reinterpret_cast<uint4*>(base + voff) = uint4{lo.x, lo.y, hi.x, hi.y};
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + i * 32 + fr;
      const float rs = sc_rows[i * 32 + fr];
      uint16_t* dst_row = g.c + row * g.ldc;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int cl = j * 32 + rq * 8 + fk * 4;
          const float4 cs = *reinterpret_cast<const float4*>(sc_cols + cl);
          const uint32_t lo = pack_bf16x2(acc[i][j][4 * rq + 0] * rs * cs.x, acc[i][j][4 * rq + 1] * rs * cs.y);
          const uint32_t hi = pack_bf16x2(acc[i][j][4 * rq + 2] * rs * cs.z, acc[i][j][4 * rq + 3] * rs * cs.w);
          const int64_t col = n0 + cl;
          if (row < g.M) {
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
    }
  };

  // ---- prologue: pairs 0 and 1 in flight, then slice 0's fragments.
#pragma unroll
  for (int part = 0; part < 16; ++part) issue_part(0, 0, part);
#pragma unroll
  for (int part = 0; part < 16; ++part) issue_part(2, 1, part);
  prefetch_scales(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(16 + 4, 0));   // pair 0 landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_frags(fa0, fw0, smem, 0);

  // ---- the stream.  G counts slices over all tiles; nsteps is even, so a
  // tile's slice s has the parity of G, even slices use register set 0 and odd
  // slices set 1, and a tile ends with the first slice of a pair.
  int G = 0;
  for (int k = 0; k < my_tiles; ++k) {
    slice(fa0, fw0, fa1, fw1, region_of(G), 1, false, 0, 0, true, true);     // s = 0 starts the sums
    int s = 1;
    for (; s < nsteps - 1; s += 2) {
      barrier_all_loads();
      slice(fa1, fw1, fa0, fw0, region_of(G + s + 1), 0, true, s + 3, (G + s) >> 1);
      slice(fa0, fw0, fa1, fw1, region_of(G + s + 1), 1, false, 0, 0);
    }
    // s = nsteps - 1: the next tile's first fragments are read after the
    // epilogue, which keeps their registers free while it runs.
    barrier_all_loads();
    slice(fa1, fw1, fa0, fw0, region_of(G + s + 1), 0, true, s + 3, (G + s) >> 1, false);
    G += nsteps;
    epilogue(k);
    read_frags(fa0, fw0, region_of(G), 0);
    a_cur = a_nxt;
    w_cur = w_nxt;
    tile_spans(k + 2, a_nxt, w_nxt);
    // The epilogue's LDS reads of the scales are done before the next tile's
    // scales may overwrite them.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    prefetch_scales(k + 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

hipError_t launch_gemm32_fp8(const GemmArgs& g, hipStream_t st) {
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  // The load stream runs one pair (two slices) ahead into the next tile, which
  // is the next tile's own first pair only when a tile has at least two pairs;
  // K = 128 gets one tile per workgroup (its look-ahead loads then land in a
  // region that is never read).
  const int grid = (g.K / kRow >= 2) ? std::min(tiles, kPersistentCap) : tiles;
  hipLaunchKernelGGL(k_gemm32_fp8, dim3(grid), dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace pql
