// W4A16 GEMM for M > 64 on gfx950: C[M, N] = A (bf16) * W_hat^T with
// W_hat[n, k] = bf16((q[n, k] - z[g, n]) * s[g, n]), g = k / 128 (int4 codes, a bf16
// scale and a 4-bit zero-point per 128-element K-group: "vLLM-Omni accelerates
// inference with AutoRound quantization", section "Usage").  The product
// (q - z) * s is exact in fp32, so W_hat equals the library's dequantize.
//
// One 256 x 128 output tile per workgroup of 8 waves, specialized by role.
// Waves 0-3 (one per SIMD) only read LDS and run the matrix core: a 2 x 2
// grid of 128 x 64 quarters, each 4 x 2 blocks of v_mfma_f32_32x32x16_bf16.
// Waves 4-7 (the second wave on each SIMD) issue every global load and expand
// the int4 codes into bf16, so that VALU work runs beside the other wave's
// MFMAs instead of between them (a wave's own VALU and MFMA instructions do
// not overlap).  K advances in steps of 64 elements.  Per step the workgroup
// needs A (256 rows x 128 bytes, bf16) and the codes of its 128 weight rows
// (32 bytes each); both arrive by direct-to-LDS loads (A in 128-byte rows with
// chunk c of row r at c ^ ((r / 2) % 8), lane i of an 8-row load fetching the
// chunk of row i / 8 that lands at position i % 8; codes row-major).  Each
// step's codes are expanded once per workgroup into a bf16 weight tile in LDS
// (same swizzle), read by all 4 MFMA waves: every weight element is
// converted once per 256 output rows.
//
// Pipeline (one barrier B(s) per step, shared by all 8 waves): during step s
// the MFMA waves run step s's 4 quarter steps (the barrier sits before the
// last, after every read of step s's buffers has been issued), while the
// helper waves issue the loads of A for step s + 2 (3-slot ring) and of codes
// for step s + 5 (6-slot ring), plus, when step s + 5 starts a group, that
// group's scales and zero-points for the tile's rows (group-major in memory,
// so one 256-byte and one 128-byte load; 3 slots), and expand step s + 1's
// codes into the other weight buffer.  The weight stream comes from HBM and
// gets the longer lead.  Before B(s) a helper waits for the A loads issued one
// step earlier and everything before them (loads retire in issue order),
// leaving that step's younger code and scale loads in flight.
#include <algorithm>
#include <type_traits>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

using namespace gemm;

constexpr int BM = 256;
constexpr int kARow = 128;                         // A bytes per row per step (64 bf16)
constexpr int kAStage = BM * kARow;                // 32 KB
constexpr int kCRow = 32;                          // code bytes per weight row per step
constexpr int kLead = 5;                           // codes (and scales) run this many steps ahead
constexpr int kCStages = kLead + 1;
constexpr int kSZSlots = 3;
constexpr int kWRow = 128;                         // expanded bf16 bytes per weight row per step
constexpr int kSZ = 512;                           // per group slot: up to 128 bf16 scales, then the zero-points
constexpr int kEpiRow = 136;                       // staged output row: 64 bf16 + 8 bytes of padding
constexpr int kEpiBytes = 32 * kEpiRow;            // per wave, inside the (idle) A stages at the end

// Tile shape: 256 x BN.  BN = 128: each MFMA wave owns 128 x 64 (the large-M
// shape); BN = 64: each owns 64 x 64, which doubles the number of tiles when
// M is small and 256 x 128 tiles leave CUs idle, while every weight element is
// still expanded once per 256 output rows.
template <int BN>
struct Shape {
  // A stages: the loads of step s + kAStages - 1 are issued during step s, so
  // they have kAStages - 2 steps to land.  (A fourth stage, which the narrow
  // shape has the LDS for, measured the same: its steps are bounded by the
  // rate at which each CU takes in the tile's 32 KB of A, not by latency.)
  static constexpr int kAStages = 3;
  static constexpr int kCStage = BN * kCRow;                 // codes of one step
  static constexpr int kWBuf = BN * kWRow;                   // expanded weights of one step
  static constexpr int kOffC = kAStages * kAStage;
  static constexpr int kOffW = kOffC + kCStages * kCStage;
  static constexpr int kOffSZ = kOffW + 2 * kWBuf;
  static constexpr int kLds = kOffSZ + kSZSlots * kSZ;     // 153.5 KB (BN 128), 125.5 KB (BN 64)
  static constexpr int kCodeWaves = BN / 32;               // helper waves that load codes (32 rows each)
  static constexpr int kThreadsPerRow = 256 / BN;          // helper threads expanding one weight row
  static constexpr int kWaveM = BN == 128 ? 128 : 64;      // MFMA wave tile: kWaveM x 64
  static constexpr int NI = kWaveM / 32;                   // 32-row blocks per MFMA wave
};

typedef float v16f __attribute__((ext_vector_type(16)));

template <int BN>
__global__ __launch_bounds__(512, 1) void k_w4a16_mm(const uint16_t* __restrict__ a, const uint32_t* __restrict__ wq,
                                                    const uint16_t* __restrict__ w_scales,
                                                    const uint8_t* __restrict__ w_zeros, int64_t M, int64_t N,
                                                    int64_t K, uint16_t* __restrict__ c, int64_t ldc) {
  using S = Shape<BN>;
  constexpr int kCStage = S::kCStage, kWBuf = S::kWBuf, kOffC = S::kOffC, kOffW = S::kOffW, kOffSZ = S::kOffSZ;
  constexpr int kAStages = S::kAStages;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::kLds];

  // XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD takes a
  // contiguous range of tiles, walked in 4-tile-tall column groups.
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  int tm, tn;
  {
    const int T = tiles_m * tiles_n, b = blockIdx.x;
    const int xcd = b & 7, idx = b >> 3, per = T >> 3, rem = T & 7;
    const int L = xcd * per + min(xcd, rem) + idx;
    constexpr int kGroupM = 4;
    const int group = L / (kGroupM * tiles_n), first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM), l = L - group * kGroupM * tiles_n;
    tm = __builtin_amdgcn_readfirstlane(first_m + l % gm);
    tn = __builtin_amdgcn_readfirstlane(l / gm);
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int mr = (int)std::min<int64_t>(BM, M - m0), nr = (int)std::min<int64_t>(BN, N - n0);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nsteps = (int)(K / 64), ng = (int)(K / 128);

  if (wave >= 4) {
    // ================= helper waves: loads and weight expansion =================
    const int hw = wave - 4, ht = t - 256;
    const int Ab = (int)(K * 2), Wb = (int)(K / 2);   // bytes per A row, per code row
    // Per-tile descriptors cover the tile's valid rows (rows past M / N read
    // 0); lane offsets carry the row, the step's K offset rides in the scalar
    // offset.  Helper wave h moves A rows 64 h .. + 63 (8 loads of 8 rows) and,
    // for h < BN / 32, the codes of weight rows 32 h .. + 31 (one load).
    const v4i a_rsrc = make_rsrc(a + m0 * K, mr * Ab);
    const v4i w_rsrc = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + n0 * Wb, nr * Wb);
    int voff_a[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) voff_a[p] = (hw * 64 + 8 * p + (lane >> 3)) * Ab + (dma_chunk(lane, p & 1) << 4);
    const int voff_c = (hw * 32 + (lane >> 1)) * Wb + (lane & 1) * 16;
    auto load_a = [&](int s, int stage, int p) __attribute__((always_inline)) {
      lds_load16_so(a_rsrc, smem + stage * kAStage + (hw * 64 + 8 * p) * kARow, voff_a[p],
                    std::min(s, nsteps - 1) * kARow);
    };
    auto load_codes = [&](int s) __attribute__((always_inline)) {
      if (hw < S::kCodeWaves)
        lds_load16_so(w_rsrc, smem + kOffC + (s % kCStages) * kCStage + hw * 32 * kCRow, voff_c,
                      std::min(s, nsteps - 1) * kCRow);
    };
    auto load_group = [&](int g) __attribute__((always_inline)) {   // waves 0 and 1 of the helpers
      const int gc = std::min(g, ng - 1);
      uint8_t* slot = smem + kOffSZ + (g % kSZSlots) * kSZ;
      if (hw == 0) lds_load4(make_rsrc(w_scales + (int64_t)gc * N + n0, nr * 2), slot, lane * 4);
      else lds_load4(make_rsrc(w_zeros + (int64_t)gc * N + n0, nr), slot + 256, lane * 4);
    };

    // Expansion of step s's codes into weight buffer s & 1: with T = 256 / BN
    // helper threads per weight row, thread h owns row h / T and its part
    // h % T of the step's 8 code words (chunks 8 / T (h % T) .. of the row);
    // even and odd nibbles are spread into the bytes of two words, so each
    // code converts with one byte-to-float instruction.
    constexpr int kWords = 8 / S::kThreadsPerRow;   // code words (8 elements each) per thread
    const int er = ht / S::kThreadsPerRow, eh = ht % S::kThreadsPerRow;
    auto expand = [&](int s) __attribute__((always_inline)) {
      const uint8_t* cs = smem + kOffC + (s % kCStages) * kCStage;
      uint32_t code[kWords];
      if constexpr (kWords == 4) {
        const uint4 c4 = *reinterpret_cast<const uint4*>(cs + er * kCRow + eh * 16);
        code[0] = c4.x, code[1] = c4.y, code[2] = c4.z, code[3] = c4.w;
      } else {
        const uint2 c2 = *reinterpret_cast<const uint2*>(cs + er * kCRow + eh * 8);
        code[0] = c2.x, code[1] = c2.y;
      }
      const uint8_t* sz = smem + kOffSZ + ((s >> 1) % kSZSlots) * kSZ;
      const uint32_t sb = *reinterpret_cast<const uint16_t*>(sz + er * 2);
      const uint32_t zb = sz[256 + er];
      const float sc = __uint_as_float(sb << 16);
      const float zs = -(float)zb * sc;   // exact: z * s fits in fp32
      uint8_t* wb = smem + kOffW + (s & 1) * kWBuf;
#pragma unroll
      for (int q = 0; q < kWords; ++q) {
        const uint32_t w = code[q];
        uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
        asm volatile("" : "+v"(ev), "+v"(od));   // keep the byte planes
        uint32_t pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pr[j] = pack_bf16x2(__builtin_fmaf((float)((ev >> (8 * j)) & 0xFF), sc, zs),
                              __builtin_fmaf((float)((od >> (8 * j)) & 0xFF), sc, zs));
        *reinterpret_cast<uint4*>(wb + swz128(er, kWords * eh + q)) = uint4{pr[0], pr[1], pr[2], pr[3]};
      }
    };

    // Prologue: A of steps 0 .. kAStages - 2; codes of steps 0 .. kLead - 1; groups 0 .. 2.
#pragma unroll
    for (int st = 0; st + 1 < kAStages; ++st)
#pragma unroll
      for (int p = 0; p < 8; ++p) load_a(st, st, p);
#pragma unroll
    for (int s = 0; s < kLead; ++s) load_codes(s);
    if (hw < 2) {
#pragma unroll
      for (int g = 0; g < kSZSlots; ++g) load_group(g);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    expand(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();
    // Step s (between barriers B(s - 1) and B(s)): loads of A for step
    // s + kAStages - 1 (its stage was last read before B(s - 1)), of codes for
    // step s + kLead and, when that step starts a group, of the group's
    // scales; then the expansion of step s + 1 (codes and scales landed
    // before B(s - 1)).  B(s) needs A of step s + 1, issued during step
    // s - kAStages + 2, and everything older; younger are that step's code
    // load and everything issued in the kAStages - 2 steps after it.  Per step
    // a wave issues 8 A loads, a code load if h < BN / 32, and, if h < 2, a
    // scale load on every other step, so the younger count is
    //   A only:          8 (kAStages - 2)
    //   A + codes:       1 + 9 (kAStages - 2)
    //   A + codes + scales: 1 + 9 (kAStages - 2) + the scale loads among
    //                    kAStages - 1 consecutive steps, at least
    //                    (kAStages - 1) / 2 rounded down
    // (waiting for fewer outstanding loads than that only waits longer).
    constexpr int kYoungA = 8 * (kAStages - 2);
    constexpr int kYoungAC = 1 + 9 * (kAStages - 2);
    constexpr int kYoungACS = kYoungAC + (kAStages - 1) / 2;
    for (int s = 0; s < nsteps; ++s) {
#pragma unroll
      for (int p = 0; p < 8; ++p) load_a(s + kAStages - 1, (s + kAStages - 1) % kAStages, p);
      load_codes(s + kLead);
      if (((s + kLead) & 1) == 0 && hw < 2) load_group((s + kLead) >> 1);
      expand(s + 1);   // the last step expands a clamped step that is never read
      if (hw < 2) __builtin_amdgcn_s_waitcnt(waitcnt_imm(kYoungACS, 0));   // hw < 2 <= BN / 32: codes too
      else if (hw < S::kCodeWaves) __builtin_amdgcn_s_waitcnt(waitcnt_imm(kYoungAC, 0));
      else __builtin_amdgcn_s_waitcnt(waitcnt_imm(kYoungA, 0));
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // every load has landed before LDS is reused
    __builtin_amdgcn_s_barrier();
    return;
  }

  // ================= MFMA waves: a kWaveM x 64 part of the tile each =================
  // v_mfma_f32_32x32x16_bf16 (the form that runs at the full bf16 rate on
  // gfx950): lane l feeds row l % 32 and, with g = l / 32, K-elements
  // 8 g .. 8 g + 7 of a 16-element quarter step kq, i.e. chunk 2 kq + g of the
  // 128-byte row; the same assignment for both operands pairs every K-element
  // with itself.  The weight fragment is the first operand, so accumulator
  // register r of lane l holds C[m = l % 32][n = 8 (r / 4) + 4 (l / 32) + r % 4]:
  // four consecutive columns per register quad.
  // BN = 128: waves form 2 x 2 parts of 128 x 64; BN = 64: 4 x 1 parts of 64 x 64.
  constexpr int NI = S::NI, kWaveM = S::kWaveM;
  const int wm = BN == 128 ? wave >> 1 : wave, wn = BN == 128 ? wave & 1 : 0;
  const int fr = lane & 31, fg = lane >> 5;
  int aoff[4], woff[4];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    aoff[kq] = swz128(wm * kWaveM + fr, 2 * kq + fg);
    woff[kq] = swz128(wn * 64 + fr, 2 * kq + fg);
  }
  v16f acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  uint4 fa[2][NI], fw[2][2];   // two register sets, alternating by quarter step
  auto read_quarter = [&](int s, int kq, int set) __attribute__((always_inline)) {
    const uint8_t* As = smem + (s % kAStages) * kAStage;
    const uint8_t* Ws = smem + kOffW + (s & 1) * kWBuf;
#pragma unroll
    for (int i = 0; i < NI; ++i) fa[set][i] = lds16(As + aoff[kq] + i * 32 * kARow);
#pragma unroll
    for (int j = 0; j < 2; ++j) fw[set][j] = lds16(Ws + woff[kq] + j * 32 * kWRow);
  };
  __builtin_amdgcn_s_barrier();   // the helpers' prologue loads have landed
  __builtin_amdgcn_s_barrier();   // step 0's weights are expanded
  __builtin_amdgcn_sched_barrier(0);
  read_quarter(0, 0, 0);
  // Step s: quarter steps kq = 0..3 of NI x 2 MFMAs each, register set kq & 1,
  // the next quarter's NI + 2 fragment reads interleaved.  Every read of step s's
  // stage and weight buffer is issued before quarter 3, so B(s) comes there;
  // past it, step s + 1's A and weights are complete, and its first quarter
  // is read under quarter 3's MFMAs.
  auto quarter = [&](int s, auto kqc) __attribute__((always_inline)) {
    constexpr int kq = decltype(kqc)::value, cs = kq & 1, ns = cs ^ 1;
    if constexpr (kq == 3) {
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fw[cs][j]),
                                                            __builtin_bit_cast(v8bf, fa[cs][i]), acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        const int e = j * NI + i;
        if (e < NI + 2) {
          const int sn = kq == 3 ? s + 1 : s, kn = (kq + 1) & 3;
          const uint8_t* As = smem + (sn % kAStages) * kAStage;
          const uint8_t* Ws = smem + kOffW + (sn & 1) * kWBuf;
          if (e < NI) fa[ns][e] = lds16(As + aoff[kn] + e * 32 * kARow);
          else fw[ns][e - NI] = lds16(Ws + woff[kn] + (e - NI) * 32 * kWRow);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  for (int s = 0; s < nsteps; ++s) {
    quarter(s, std::integral_constant<int, 0>{});
    quarter(s, std::integral_constant<int, 1>{});
    quarter(s, std::integral_constant<int, 2>{});
    quarter(s, std::integral_constant<int, 3>{});
  }

  // ---- epilogue: every load has landed (the helpers wait) before the A
  // stages are reused for staging.  Per 32-row block i the wave stages its
  // 32 x 64 outputs (bf16 quads of consecutive columns) and writes them as
  // 16-byte row pieces (8 lanes per row, 8 rows per instruction).
  __builtin_amdgcn_s_barrier();
  uint8_t* stg = smem + wave * kEpiBytes;
  const int rr = lane >> 3, rc = lane & 7;
  const int64_t wrow0 = m0 + wm * kWaveM, wcol0 = n0 + wn * 64;
  const bool vec = (ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(c) & 15) == 0;
  const bool interior = vec && wrow0 + kWaveM <= M && wcol0 + 64 <= N;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const v16f& v = acc[i][j];
        *reinterpret_cast<uint2*>(stg + fr * kEpiRow + (j * 32 + 8 * rq + 4 * fg) * 2) =
            uint2{pack_bf16x2(v[4 * rq + 0], v[4 * rq + 1]), pack_bf16x2(v[4 * rq + 2], v[4 * rq + 3])};
      }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    // Rows pass between lanes of the wave: no compiler reordering or reuse of
    // LDS accesses across the exchange (the hardware keeps one wave's LDS
    // accesses in order).
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint8_t* src = stg + (q * 8 + rr) * kEpiRow + rc * 16;   // 8-byte aligned (136-byte rows)
      const uint2 lo = *reinterpret_cast<const uint2*>(src), hi = *reinterpret_cast<const uint2*>(src + 8);
      const uint4 v = uint4{lo.x, lo.y, hi.x, hi.y};
      const int64_t row = wrow0 + i * 32 + q * 8 + rr, col = wcol0 + rc * 8;
      uint16_t* dst = c + row * ldc + col;
      if (interior) {
        *reinterpret_cast<uint4*>(dst) = v;
      } else if (row < M) {
        if (vec && col + 8 <= N) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
          const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < N) dst[e] = (uint16_t)(wds[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));   // staging block read before it is rewritten
    asm volatile("" ::: "memory");
  }
}

}  // namespace

bool w4a16_mm_supported(int64_t M, int64_t N, int64_t K) {
  // group-major scale / zero loads of a tile's 128 rows are dword loads
  return M > 0 && N % 4 == 0 && K % 128 == 0 && K / 64 >= 1 && K * 2 * 256 < (int64_t)1 << 31;
}

// 256 x 64 tiles when 256 x 128 tiles would fill at most half of the CUs: twice
// the workgroups, each weight element still expanded once per 256 rows.
bool w4a16_mm_narrow(int64_t M, int64_t N) { return ((M + BM - 1) / BM) * ((N + 127) / 128) <= 128; }

hipError_t launch_gemm_w4a16_mm(const uint16_t* a, const uint32_t* wq, const uint16_t* w_scales,
                                const uint8_t* w_zeros, int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc,
                                hipStream_t st) {
  if (w4a16_mm_narrow(M, N)) {
    const int tiles = (int)(((M + BM - 1) / BM) * ((N + 63) / 64));
    hipLaunchKernelGGL(k_w4a16_mm<64>, dim3(tiles), dim3(512), 0, st, a, wq, w_scales, w_zeros, M, N, K, c, ldc);
  } else {
    const int tiles = (int)(((M + BM - 1) / BM) * ((N + 127) / 128));
    hipLaunchKernelGGL(k_w4a16_mm<128>, dim3(tiles), dim3(512), 0, st, a, wq, w_scales, w_zeros, M, N, K, c, ldc);
  }
  return hipGetLastError();
}

}  // namespace pql
