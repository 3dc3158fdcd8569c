// W4A16 GEMM on gfx950: C[M, N] = A (bf16) * W_hat^T, W_hat = bf16((q - z) * s).
//
// The weight is int4 with a bf16 scale and a 4-bit zero-point per 128-element
// K-group ("vLLM-Omni accelerates inference with AutoRound quantization",
// section "Usage": bits 4, group size 128).  Each weight element is expanded
// to bf16((q - z) * s) -- the product is exact in fp32, so this equals the
// library's own dequantize -- and multiplied on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16: lane l feeds row l % 16 with K-elements
// 8 * (l / 16) .. +7; accumulator lane l holds C[4 * (l / 16) + r][l % 16]).
//
// Dispatch by M:
//   * M <= 16 (activation rows fit the LDS stage): k_w4a16_gemv, weight-
//     bandwidth-bound; codes stay integers on the bf16 MFMA and each group is
//     promoted with its scale and zero-point (below).
//   * M <= 64: k_w4a16_small, weight-bandwidth-bound.  A workgroup owns 32
//     output columns; its 4 waves split the K-groups, each wave streams 16-byte
//     code chunks straight into registers (no LDS staging), and the partial
//     sums of the 4 waves are added in LDS.
//   * M > 64: compute-bound; the wave-specialized kernel of gemm_w4a16_mm.hip
//     when N % 4 == 0, else k_w4a16_tile here: 256 x 256 output tile per
//     256-thread workgroup, K steps of 64, A (bf16, 32 KB) and the expanded W
//     tile (bf16, 32 KB) double-buffered in LDS, each thread expanding one W
//     row-slice of 64 codes (128-byte rows, chunk c at c ^ (row & 7)).
#include <algorithm>
#include <atomic>

#include "gemm_common.hpp"
#include "pql_device.hpp"
#include "pql_internal.hpp"

namespace pql {

namespace {

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return bf16_bits(lo) | (bf16_bits(hi) << 16); }

// 8 int4 codes (element j at bits 4j) -> 8 bf16 of (q - z) * s, packed in pairs.
__device__ __forceinline__ uint4 expand8(uint32_t w, float s, float zs) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf((float)((w >> (4 * j)) & 0xF), s, zs);
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

constexpr int BM = 256, BN = 256, BKB = 128;    // BKB bytes = 64 bf16 per row per step
constexpr int kStageBytes = BM * BKB + BN * BKB;
constexpr int kGroupM = 4;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BKB + ((chunk ^ (row & 7)) << 4); }

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

// ---------------------------------------------------------------- large M
__global__ __launch_bounds__(256, 1) void k_w4a16_tile(const uint16_t* __restrict__ a,
                                                      const uint32_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ w_scales,
                                                      const uint8_t* __restrict__ w_zeros, int64_t M,
                                                      int64_t N, int64_t K, uint16_t* __restrict__ c,
                                                      int64_t ldc) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  int tm, tn;
  tile_of_block(tiles_m, tiles_n, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);   // computed with VALU division; keep it scalar so
  tn = __builtin_amdgcn_readfirstlane(tn);   // the buffer descriptors live in SGPRs
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t Ab = K * 2;                 // A bytes per row
  const int64_t Wb = K / 2;                 // code bytes per row
  const int nsteps = (int)(K / 64);
  const int64_t ngroups = K / 128;

  const int ld_c = t & 7, ld_r = t >> 3;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a + m0 * K), (short)0, (int)(std::min<int64_t>(BM, M - m0) * Ab), 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const uint8_t*>(wq) + n0 * Wb), (short)0,
      (int)(std::min<int64_t>(BN, N - n0) * Wb), 0x00020000);
  const int64_t wrow = std::min<int64_t>(n0 + t, N - 1);   // the W row this thread expands

  uint4 ra[8];
  uint4 rw[2];
  float s_reg = 0.f, zs_reg = 0.f;
  auto load_step = [&](int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v4i v = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, (ld_r + 32 * i) * (int)Ab + s * BKB + ld_c * 16, 0, 0);
      ra[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i v = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, t * (int)Wb + s * 32 + h * 16, 0, 0);
      rw[h] = make_uint4(v.x, v.y, v.z, v.w);
    }
    const int64_t gi = (s >> 1) * N + wrow;   // group-major
    s_reg = __uint_as_float((uint32_t)w_scales[gi] << 16);
    zs_reg = -(float)w_zeros[gi] * s_reg;      // exact: z * s fits in fp32
  };
  auto store_step = [&](int stage) {
    uint8_t* A = smem + stage * kStageBytes;
    uint8_t* W = A + BM * BKB;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(A + swz(ld_r + 32 * i, ld_c)) = ra[i];
    const uint32_t words[8] = {rw[0].x, rw[0].y, rw[0].z, rw[0].w, rw[1].x, rw[1].y, rw[1].z, rw[1].w};
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<uint4*>(W + swz(t, q)) = expand8(words[q], s_reg, zs_reg);
  };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  load_step(0);
  store_step(0);
  __syncthreads();
  const int fr = lane & 15, fk = lane >> 4;
  for (int s = 0; s < nsteps; ++s) {
    const int stage = s & 1;
    if (s + 1 < nsteps) load_step(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* A = smem + stage * kStageBytes;
    const uint8_t* W = A + BM * BKB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v8bf af[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        af[i] = as_v8bf(*reinterpret_cast<const uint4*>(A + swz(wm * 128 + i * 16 + fr, 4 * kk + fk)));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const v8bf bf = as_v8bf(*reinterpret_cast<const uint4*>(W + swz(wn * 128 + j * 16 + fr, 4 * kk + fk)));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf, acc[i][j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nsteps) store_step(stage ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t col = n0 + wn * 128 + j * 16 + fr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 128 + i * 16 + 4 * fk + r;
        if (row < M) c[row * ldc + col] = (uint16_t)bf16_bits(acc[i][j][r]);
      }
    }
  }
}

// ---------------------------------------------------------------- small M
// Workgroup: 32 columns (two 16-column MFMA blocks), 4 waves splitting the
// K-groups round-robin.  Within a 128-group, lane slot g = l / 16 owns the 32
// consecutive K-elements 32 g .. 32 g + 31 (one 16-byte code load), and MFMA
// step t consumes elements 32 g + 8 t .. + 7 from every slot; A is read with
// the same assignment, so the contraction still covers each k exactly once.
template <int MB>   // row blocks of 16
__global__ __launch_bounds__(256) void k_w4a16_small(const uint16_t* __restrict__ a,
                                                    const uint32_t* __restrict__ wq,
                                                    const uint16_t* __restrict__ w_scales,
                                                    const uint8_t* __restrict__ w_zeros, int64_t M,
                                                    int64_t N, int64_t K, uint16_t* __restrict__ c,
                                                    int64_t ldc) {
  __shared__ float part[4][MB * 16][33];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int fr = lane & 15, g4 = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int64_t ngroups = K / 128;
  const int64_t wpr = K / 8;                        // code words per row

  v4f acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i][0] = acc[i][1] = v4f{0.f, 0.f, 0.f, 0.f};

  int64_t wrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wrow[j] = std::min<int64_t>(n0 + j * 16 + fr, N - 1);

  for (int64_t gidx = wave; gidx < ngroups; gidx += 4) {
    uint4 code[2];
    float s[2], zs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      code[j] = ldg16_nt(wq + wrow[j] * wpr + gidx * 16 + g4 * 4);
      const int64_t gi = gidx * N + wrow[j];   // group-major scales / zero-points
      s[j] = __uint_as_float((uint32_t)w_scales[gi] << 16);
      zs[j] = -(float)w_zeros[gi] * s[j];
    }
    const uint32_t cw[2][4] = {{code[0].x, code[0].y, code[0].z, code[0].w},
                               {code[1].x, code[1].y, code[1].z, code[1].w}};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      v8bf bf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = as_v8bf(expand8(cw[j][st], s[j], zs[j]));
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int64_t row = (int64_t)i * 16 + fr;
        uint4 av = make_uint4(0, 0, 0, 0);
        if (row < M) av = ldg16(a + row * K + gidx * 128 + g4 * 32 + st * 8);
        const v8bf af = as_v8bf(av);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][i * 16 + 4 * g4 + r][j * 16 + fr] = acc[i][j][r];
  __syncthreads();
  for (int e = t; e < MB * 16 * 32; e += 256) {
    const int row = e >> 5, col = e & 31;
    const int64_t gc = n0 + col;
    if (row < M && gc < N) {
      const float v = part[0][row][col] + part[1][row][col] + part[2][row][col] + part[3][row][col];
      c[(int64_t)row * ldc + gc] = (uint16_t)bf16_bits(v);
    }
  }
}

// ---------------------------------------------------------------- M <= 16
// Weight-bandwidth-bound GEMV-like path.  Codes stay integers: each 16-byte
// chunk (32 codes of one row) is spread into bf16 pairs 128 + q with one AND-OR
// per pair (bf16 represents 128..143 exactly), and the zero-point is removed
// per group after the matrix core:
//   sum_k a_k (q_k - z) = sum_k a_k (128 + q_k) - (128 + z) sum_k a_k,
// with sum_k a_k from a second MFMA against a bf16 ones operand, so the
// dequantized weight is never rounded.  Each K-group's sums are promoted with
// the group's scale: acc += s (P - (128 + z) Q).
//
// A workgroup owns 16 NB output columns; its 8 waves split the K-groups.  Lane
// (n = l % 16, g = l / 16) streams chunk 4 G + g of weight row n for its
// wave's groups G (the 4 lanes of a row read 64 contiguous bytes per group).
// Because the nibbles of a code word come out as pairs (k, k + 4), the A
// operand of a lane holds a[m, k0 + {0, 4, 1, 5, 2, 6, 3, 7}] (one v_perm per
// pair); the matrix core's sum over K does not care about the order.
//
// Order of work in a wave: loads of its share of the activation rows, then
// every code, scale and zero-point load of its first batch of groups; it
// writes the activation rows to LDS (the compiler's wait for them leaves the
// younger weight loads in flight, since loads retire in issue order), meets
// the other waves, then computes each group as soon as that group's loads
// have landed.  The whole weight is requested at the start, so a wave that
// waited for all of its loads would leave every group's arithmetic to the end
// of the stream; this way it runs under the stream.  Every wait here is the
// compiler's own: the activation rows are staged with ordinary loads and LDS
// writes, not direct-to-LDS loads, whose completion the compiler cannot see.
// nibble j of w -> bf16 128 + q_j; dword i holds elements (i, i + 4).  `low`
// (0x000F000F, in an SGPR) and `base` (0x43004300, bf16 128 in both halves, in
// a VGPR) come in as opaque registers: with literal constants the compiler
// emits a separate AND and OR per dword, since a VOP3 instruction such as
// v_and_or_b32 takes no literal.
__device__ __forceinline__ uint4 spread_codes(uint32_t w, uint32_t low, uint32_t base) {
  return make_uint4((w & low) | base, ((w >> 4) & low) | base, ((w >> 8) & low) | base, ((w >> 12) & low) | base);
}
// 8 bf16 a0..a7 (pairs per dword) -> pairs (a0, a4), (a1, a5), (a2, a6), (a3, a7):
// the order of the spread codes.
__device__ __forceinline__ uint4 pair_k_k4(uint4 a) {
  return make_uint4(__builtin_amdgcn_perm(a.z, a.x, 0x05040100u), __builtin_amdgcn_perm(a.z, a.x, 0x07060302u),
                    __builtin_amdgcn_perm(a.w, a.y, 0x05040100u), __builtin_amdgcn_perm(a.w, a.y, 0x07060302u));
}

// Waves per workgroup, splitting the K-groups: 8, or 12 for the 48-column variant, whose
// 256 workgroups for N = 12288 put one workgroup on each CU.
__host__ __device__ constexpr int gemv_waves(int NB) { return NB == 1 ? 8 : 12; }
constexpr int kGemvStageMax = 128 * 1024;  // LDS bytes for the staged activation rows
// LDS bytes per staged activation row: K bf16 plus 16 bytes, which spreads the
// 16 rows of a fragment read over the banks (K % 128 == 0).
__host__ __device__ constexpr int64_t gemv_a_row_bytes(int64_t K) { return K * 2 + 16; }


// NB column blocks of 16 per workgroup: every A fragment feeds NB weight row
// blocks.  With NB = 1 (M <= 4) the activation rows are staged once per
// workgroup in LDS, every 8 elements already in the order of the spread codes;
// with NB = 3 (up to 16 rows, 6 KB each at K = 3072) staging every row costs
// more than each wave loading the fragments of its own groups, which it does
// beside the codes (from L2: every workgroup reads the same rows).  MFMA rows
// past M read row M - 1: their sums are never stored.
// BATCH groups' loads are in flight per wave, every one of them issued
// unconditionally (past the wave's last group they reload that group, and its
// arithmetic is skipped), so the compiler's wait for each group counts exactly
// the younger loads and nothing waits for the whole batch.
template <int NB, int BATCH>
__global__ __launch_bounds__(64 * gemv_waves(NB)) void k_w4a16_gemv(const uint16_t* __restrict__ a,
                                                               const uint32_t* __restrict__ wq,
                                                               const uint16_t* __restrict__ w_scales,
                                                               const uint8_t* __restrict__ w_zeros, int64_t M,
                                                               int64_t N, int64_t K, uint16_t* __restrict__ c,
                                                               int64_t ldc) {
  constexpr int kGemvWaves = gemv_waves(NB);
  static_assert(BATCH * 3 * NB <= 63, "the loads of one batch must fit the vmcnt counter");
  extern __shared__ __attribute__((aligned(16))) uint8_t gemv_lds[];
  float (*part)[16][16 * NB + 1] = reinterpret_cast<float (*)[16][16 * NB + 1]>(gemv_lds);
  uint8_t* a_lds = gemv_lds + sizeof(float) * kGemvWaves * 16 * (16 * NB + 1);
  const int a_row_bytes = (int)gemv_a_row_bytes(K);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // the K-group loop is uniform per wave
  const int n16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * NB;
  const int ng = (int)(K / 128);
  const int per = (ng + kGemvWaves - 1) / kGemvWaves;
  const int gbeg = std::min(ng, wave * per), gend = std::min(ng, gbeg + per);
  const uint32_t* wrow[NB];
  int64_t nrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    nrow[nb] = std::min<int64_t>(n0 + nb * 16 + n16, N - 1);   // weight row of this lane (clamped)
    wrow[nb] = wq + nrow[nb] * (K / 8);
  }
  constexpr bool kDirectA = NB > 1;
  const int am = std::min<int>(n16, (int)M - 1);                  // A row of this lane
  const uint8_t* arow = a_lds + am * a_row_bytes + g * 64;       // staged
  const uint16_t* agl = a + (int64_t)am * K + 32 * g;            // direct
  // Constants made opaque by empty asm statements (the moves that set them
  // are the compiler's own): the bf16 ones stay in registers instead of being
  // rebuilt before every use, and the spread's operands stay registers.
  uint32_t one2 = 0x3f803f80u, low = 0x000F000Fu, base = 0x43004300u;
  asm volatile("" : "+v"(one2));
  asm volatile("" : "+s"(low));
  asm volatile("" : "+v"(base));
  const v8bf ones = as_v8bf(make_uint4(one2, one2, one2, one2));

  // Activation chunks (16 bytes) of this thread: the first kEarly rounds are
  // loaded before the weight loads; rows beyond those (long K) are staged
  // after them.
  constexpr int kEarly = 4;   // covers M x K = 4 x 4096
  const int cpr = (int)(K / 8);   // 16-byte chunks per row
  const int chunks = (int)M * cpr;
  auto a_chunk = [&](int idx) __attribute__((always_inline)) {
    const int m = idx / cpr, j = idx - m * cpr;
    return ldg16(a + (int64_t)m * K + 8 * j);
  };
  auto a_store = [&](int idx, uint4 v) __attribute__((always_inline)) {
    const int m = idx / cpr, j = idx - m * cpr;
    *reinterpret_cast<uint4*>(a_lds + m * a_row_bytes + 16 * j) = pair_k_k4(v);
  };
  uint4 achunk[kEarly];
  if constexpr (!kDirectA) {
#pragma unroll
    for (int i = 0; i < kEarly; ++i) {
      const int idx = t + i * 64 * kGemvWaves;
      if (idx < chunks) achunk[i] = a_chunk(idx);
    }
  }
  // Codes, scales and zero-points of a batch of groups; the scale and zero
  // bytes stay raw until used, so that no load waits for another.
  uint4 code[BATCH][NB];
  uint4 afr[kDirectA ? BATCH : 1][4];   // direct A fragments, raw order
  uint32_t sraw[BATCH][NB], zraw[BATCH][NB];
  const int glast = std::max(gend - 1, 0);   // a valid group, also for a wave with none
  auto fetch = [&](int b0) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int G = std::min(b0 + u, glast);
      if constexpr (kDirectA) {
#pragma unroll
        for (int d = 0; d < 4; ++d) afr[u][d] = ldg16(agl + (int64_t)G * 128 + 8 * d);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        code[u][nb] = ldg16(wrow[nb] + (int64_t)G * 16 + g * 4);
        const int64_t gi = (int64_t)G * N + nrow[nb];   // group-major
        sraw[u][nb] = w_scales[gi];
        zraw[u][nb] = w_zeros[gi];
      }
    }
  };
  v4f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int b0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      // A slot past the wave's last group (its loads repeat that group) adds
      // its finite sums times a zero scale.  No branch: a conditional group
      // would let the compiler sink that group's loads into it, behind the
      // previous group's arithmetic.
      const int G = std::min(b0 + u, glast);
      const bool live = b0 + u < gend;
      // one group's spread codes at a time: computed ahead, every group's would be live together
      __builtin_amdgcn_sched_barrier(0);
      v4f P[NB], Q;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const v8bf af = as_v8bf(kDirectA ? pair_k_k4(afr[kDirectA ? u : 0][d])
                                         : *reinterpret_cast<const uint4*>(arow + G * 256 + d * 16));
        Q = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, ones, d ? Q : v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t cw = d == 0 ? code[u][nb].x : d == 1 ? code[u][nb].y : d == 2 ? code[u][nb].z : code[u][nb].w;
          P[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, as_v8bf(spread_codes(cw, low, base)),
                                                          d ? P[nb] : v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
      }
      // lane (n = l % 16, g) holds rows m = 4 g + r of column n
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float s = live ? __uint_as_float(sraw[u][nb] << 16) : 0.f;
        const float zq = -(128.0f + (float)zraw[u][nb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nb][r] = __builtin_fmaf(s, __builtin_fmaf(zq, Q[r], P[nb][r]), acc[nb][r]);
      }
    }
  };
  if constexpr (kDirectA) {
    for (int b0 = gbeg; b0 < gend; b0 += BATCH) {
      fetch(b0);
      compute(b0);
    }
  } else {
    // The first batch's loads go out before the staging waits for the
    // activation loads; the barrier is reached by every wave, also one with
    // no groups.
    fetch(gbeg);
#pragma unroll
    for (int i = 0; i < kEarly; ++i) {
      const int idx = t + i * 64 * kGemvWaves;
      if (idx < chunks) a_store(idx, achunk[i]);
    }
    for (int idx = t + kEarly * 64 * kGemvWaves; idx < chunks; idx += 64 * kGemvWaves) a_store(idx, a_chunk(idx));
    __syncthreads();
    for (int b0 = gbeg; b0 < gend; b0 += BATCH) {
      if (b0 != gbeg) fetch(b0);
      compute(b0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][4 * g + r][nb * 16 + n16] = acc[nb][r];
  __syncthreads();
  for (int e = t; e < 16 * 16 * NB; e += 64 * kGemvWaves) {
    const int m = e / (16 * NB), nn = e - m * (16 * NB);
    const int64_t col = n0 + nn;
    if (m < M && col < N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kGemvWaves; ++w) v += part[w][m][nn];
      c[(int64_t)m * ldc + col] = (uint16_t)bf16_bits(v);
    }
  }
}

template <int NB>
size_t gemv_lds_bytes(int64_t M, int64_t K) {   // the partial sums, then (NB = 1) the staged rows
  return sizeof(float) * gemv_waves(NB) * 16 * (16 * NB + 1) + (NB == 1 ? (size_t)M * (size_t)gemv_a_row_bytes(K) : 0);
}

template <int NB, int BATCH>
hipError_t launch_gemv_batch(const uint16_t* a, const uint32_t* wq, const uint16_t* w_scales, const uint8_t* w_zeros,
                             int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc, hipStream_t st) {
  const size_t lds = gemv_lds_bytes<NB>(M, K);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<bool> configured[64] = {};
  if (NB == 1 && dev < 64 && !configured[dev].load()) {   // only the staged variant passes 64 KB
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_w4a16_gemv<NB, BATCH>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(gemv_lds_bytes<NB>(0, 0) + kGemvStageMax));
    if (e != hipSuccess) return e;
    configured[dev].store(true);
  }
  hipLaunchKernelGGL((k_w4a16_gemv<NB, BATCH>), dim3((unsigned)((N + 16 * NB - 1) / (16 * NB))), dim3(64 * gemv_waves(NB)),
                     lds, st, a, wq, w_scales, w_zeros, M, N, K, c, ldc);
  return hipGetLastError();
}

// The batch is the number of groups each wave owns (K / 128 split over the
// waves), up to 4 (3 for the 48-column variant, whose 12 waves leave 168
// registers per lane); longer K loops over batches.
template <int NB>
hipError_t launch_gemv(const uint16_t* a, const uint32_t* wq, const uint16_t* w_scales, const uint8_t* w_zeros,
                       int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc, hipStream_t st) {
  const int64_t per = (K / 128 + gemv_waves(NB) - 1) / gemv_waves(NB);
  const int64_t most = NB == 1 ? 4 : 3;
  switch (per <= 1 ? 1 : per >= most ? (int)most : (int)per) {
    case 1: return launch_gemv_batch<NB, 1>(a, wq, w_scales, w_zeros, M, N, K, c, ldc, st);
    case 2: return launch_gemv_batch<NB, 2>(a, wq, w_scales, w_zeros, M, N, K, c, ldc, st);
    case 3: return launch_gemv_batch<NB, 3>(a, wq, w_scales, w_zeros, M, N, K, c, ldc, st);
    default: return launch_gemv_batch<NB, NB == 1 ? 4 : 3>(a, wq, w_scales, w_zeros, M, N, K, c, ldc, st);
  }
}

}  // namespace

hipError_t launch_gemm_w4a16(const uint16_t* a, const uint32_t* wq, const uint16_t* w_scales,
                             const uint8_t* w_zeros, int64_t M, int64_t N, int64_t K, uint16_t* c,
                             int64_t ldc, hipStream_t st) {
  // Small M: the GEMV kernel when the activation rows fit its LDS stage.
  if (M <= 16 && M * gemv_a_row_bytes(K) <= kGemvStageMax) {
    return M <= 4 ? launch_gemv<1>(a, wq, w_scales, w_zeros, M, N, K, c, ldc, st)
                  : launch_gemv<3>(a, wq, w_scales, w_zeros, M, N, K, c, ldc, st);
  }
  if (M <= 64) {
    const dim3 grid((unsigned)((N + 31) / 32)), block(256);
    if (M <= 16) hipLaunchKernelGGL(k_w4a16_small<1>, grid, block, 0, st, a, wq, w_scales, w_zeros, M, N, K, c, ldc);
    else if (M <= 32) hipLaunchKernelGGL(k_w4a16_small<2>, grid, block, 0, st, a, wq, w_scales, w_zeros, M, N, K, c, ldc);
    else hipLaunchKernelGGL(k_w4a16_small<4>, grid, block, 0, st, a, wq, w_scales, w_zeros, M, N, K, c, ldc);
    return hipGetLastError();
  }
  if (w4a16_mm_supported(M, N, K)) return launch_gemm_w4a16_mm(a, wq, w_scales, w_zeros, M, N, K, c, ldc, st);
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  const size_t lds = 2 * kStageBytes;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<bool> configured[64] = {};
  if (dev < 64 && !configured[dev].load()) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_w4a16_tile),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured[dev].store(true);
  }
  hipLaunchKernelGGL(k_w4a16_tile, dim3(tiles), dim3(256), lds, st, a, wq, w_scales, w_zeros, M, N, K, c, ldc);
  return hipGetLastError();
}

const char* gemm_w4a16_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 && M * gemv_a_row_bytes(K) <= kGemvStageMax) return M <= 4 ? "k_w4a16_gemv<16 cols>" : "k_w4a16_gemv<48 cols>";
  if (M <= 16) return "k_w4a16_small<16>";
  if (M <= 32) return "k_w4a16_small<32>";
  if (M <= 64) return "k_w4a16_small<64>";
  if (w4a16_mm_supported(M, N, K)) return w4a16_mm_narrow(M, N) ? "k_w4a16_mm_256x64x64" : "k_w4a16_mm_256x128x64";
  return "k_w4a16_tile_256x256x64";
}

}  // namespace pql
