// Building blocks shared by the persistent GEMM kernels (gfx950): the
// XCD-aware persistent tile schedule, buffer descriptors, direct-to-LDS
// loads and the LDS swizzle.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pql_device.hpp"

namespace pql {
namespace gemm {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt 6:4
// left at its maximum, lgkmcnt in bits 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// 128-byte LDS rows: 16-byte chunk c of row r sits at chunk position
// c ^ ((r / 2) % 8).  gfx950's LDS serves 16 lanes of a 16-byte read per
// cycle from 64 banks (256 bytes, two rows): a fragment read, whose 16 lanes
// take the same chunk of 16 consecutive rows, then finds the even rows on
// distinct positions of one bank half and the odd rows on the other.  (A
// period of 8 rows would put rows r and r + 8 on the same banks.)
__device__ __forceinline__ int swz128(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Chunk that lane i fetches in an 8-row direct-to-LDS load (8 lanes per
// 128-byte row, lane i landing at LDS byte 16 i): the one whose swizzled
// position is i % 8 in row i / 8 of the group.  `odd_group` is the parity of
// the group's index (row / 8), which sets bit 2 of (row / 2) % 8.
__device__ __forceinline__ int dma_chunk(int lane, int odd_group) {
  return (lane & 7) ^ ((odd_group << 2) | ((lane >> 4) & 3));
}

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
    constexpr int kGroupM = 4;
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

// The same with a scalar offset: 16 bytes per lane from rsrc + voff + soff.
// Only voff is checked against the descriptor's byte count, so voff must carry
// everything that can leave the valid range (the row) and soff only offsets
// that stay inside a valid row.
// The operands are uniform; readfirstlane keeps them in SGPRs (free when the
// compiler already holds them there, a move when register pressure parked
// them in VGPRs).
__device__ __forceinline__ v4i uniform4(v4i r) {
  return v4i{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
             __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}

__device__ __forceinline__ void lds_load16_so(v4i rsrc, const uint8_t* lds, int voff, int soff) {
  rsrc = uniform4(rsrc);
  soff = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff),
               "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ void lds_load4_so(v4i rsrc, const uint8_t* lds, int voff, int soff) {
  rsrc = uniform4(rsrc);
  soff = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(m0), "v"(voff),
               "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// One direct-to-LDS load of 4 bytes per lane: rsrc + voff into LDS at lds + 4 * lane.
__device__ __forceinline__ void lds_load4(v4i rsrc, const uint8_t* lds, int voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff),
               "s"(rsrc)
               : "memory", "m0");
}

// The lane index, computed afresh where it is called: the compiler can neither
// merge it with an earlier copy nor keep one live across the code in between,
// so values derived from it are rematerialised instead of being spilled.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ v8i cat(uint4 lo, uint4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace gemm
}  // namespace pql
