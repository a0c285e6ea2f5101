// Device helpers shared by the grouped-GEMM kernels (bf16 and MXFP8): the
// device-side segment lookup, the tile order, buffer descriptors, LDS-direct
// loads and explicit wait / barrier primitives.
#pragma once

#include "common.h"

namespace moe {

// M-tiles per group of the tile order: consecutive workgroups sweep the
// N-tiles of kGroupM M-tiles, so a group's A rows and the swept B columns
// are re-read from L2 rather than HBM.
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 4
#endif
constexpr int kGroupM = MOE_GEMM_GROUP_M;

// Finds the segment of global M-tile `mt`.  Wave-uniform result (every wave
// of the workgroup computes the same), so an early exit is workgroup-uniform.
template <int TM>
__device__ __forceinline__ bool find_segment(const int32_t* __restrict__ offsets, int G,
                                             int fixed_rows, int mt, int& seg, int& row0,
                                             int& rows) {
  if (!offsets) {
    const int r0 = mt * TM;
    if (r0 >= fixed_rows) return false;
    seg = 0;
    row0 = r0;
    rows = min(TM, fixed_rows - r0);
    return true;
  }
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int st = 0, cnt = 0;
    if (g < G) {
      st = offsets[g];
      cnt = offsets[g + 1] - st;
    }
    const int tiles = (cnt + TM - 1) / TM;
    const int incl = wave_inclusive_scan(tiles);
    const int total = __shfl(incl, 63, kWave);
    if (mt < carry + total) {
      const unsigned long long m = __ballot(carry + incl > mt);
      const int first = __ffsll((long long)m) - 1;
      const int excl = carry + __shfl(incl - tiles, first, kWave);
      const int st_g = __shfl(st, first, kWave);
      const int cnt_g = __shfl(cnt, first, kWave);
      const int ml = mt - excl;
      seg = g0 + first;
      row0 = st_g + ml * TM;
      rows = min(TM, cnt_g - ml * TM);
      return true;
    }
    carry += total;
  }
  return false;
}

__device__ __forceinline__ void decode_tile(int tile, int mt_bound, int nt_count, int& mt,
                                            int& nt) {
  const int group = tile / (kGroupM * nt_count);
  const int first_mt = group * kGroupM;
  const int gsize = min(kGroupM, mt_bound - first_mt);
  const int in_g = tile - group * kGroupM * nt_count;
  mt = first_mt + in_g % gsize;
  nt = in_g / gsize;
}

// Tile order across the XCDs.  Workgroups are dealt to the eight XCDs in
// turn (workgroup b runs on XCD b % 8), and each XCD has its own L2.  With
// chunk C > 0, each super-group of 8C workgroups hands XCD x the C
// consecutive logical tiles [8Cq + Cx, 8Cq + Cx + C) of super-group q: the
// tiles one XCD runs at once are neighbours in the group order above and
// share their A rows and B columns in that XCD's L2, while the eight XCDs
// still sweep the tile order side by side.  Workgroups past the last whole
// super-group, and chunk 0, keep their own index (a bijection on the grid).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int b, int grid, int chunk) {
  if (chunk <= 0) return b;
  const int span = kXcds * chunk;
  if (b >= grid / span * span) return b;
  return b / span * span + (b % kXcds) * chunk + (b / kXcds) % chunk;
}
// The chunk a launch uses: 16 tiles for outputs at least 32 tiles wide.
// Measured on the expert GEMMs (equal 8192-row segments): +4% (row-major and
// transposed-weight forms) and +5% (weight gradients) for 14336 output
// columns, within -1.5..+0.4% for 4096, so narrower outputs keep the plain
// order.
inline int xcd_chunk_for(int nt_count) { return nt_count >= 32 ? 16 : 0; }

constexpr uint32_t kOob = 0x80000000u;  // an offset past any num_records

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Raw buffer descriptor (dwords: base lo, base hi, num_records, format) for
// the inline-asm LDS-DMA load below; base and size must be wave-uniform.
__device__ __forceinline__ u32x4 make_rsrc_words(const void* base, long long bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t n = bytes > 0x7ffffff0LL ? 0x7ffffff0u : (bytes < 0 ? 0u : (uint32_t)bytes);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, n, 0x00020000u};
}

// 16 bytes per lane from buffer offset `voff` straight into LDS at
// lds_addr + 16 * lane (wave-uniform lds_addr).  Issued as inline asm so the
// compiler does not treat it as an LDS store that every later LDS read must
// wait for: the ring's explicit vmcnt waits and barriers order it instead.
// The LDS address is the asm's m0 operand, so that the compiler writes m0
// itself, straight from the address arithmetic (one s_add_i32 m0, ... per
// load rather than an add and a move).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_load16(uint32_t lds_addr, uint32_t voff, u32x4 rsrc) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// dma_load16 with the buffer's scalar offset as well: the 16 bytes at
// voff + soff (soff wave-uniform).  A loop that advances every lane's
// offset by the same amount each step passes that advance here, with no
// per-lane add.
__device__ __forceinline__ void dma_load16_s(uint32_t lds_addr, uint32_t voff, uint32_t soff,
                                             u32x4 rsrc) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}

// 4 bytes per lane from buffer offset `voff` straight into LDS at
// lds_addr + 4 * lane (the dword form of dma_load16).
__device__ __forceinline__ void dma_load4(uint32_t lds_addr, uint32_t voff, u32x4 rsrc) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}
#pragma clang diagnostic pop

}  // namespace moe
