// Capacity drop in token order, packed expert-major row map, and the dispatch
// copy of token rows into per-expert contiguous segments.
//
// Method: capacity and token drop of the cf-1.com page "Dissecting the MoE
// communication bottleneck", section 3.1 (capacity = ceil(cf * assignments /
// experts), later tokens dropped first), expert counts of the dpshk.com "MoE
// module infra notes" section 4.2 listing, and dispatch of section 1.1 step 2
// of the cf-1.com page.
//
// The rank of assignment (t,k) among the assignments to e = ids[t,k] is
//   base[e][block(t)] + lrank[t,k],
// where lrank (from the router) is its rank inside its route block and
// base[e][b] is the exclusive prefix sum over route blocks of the per-block
// histograms (moe_aux_loss's kernel computes it, with the per-expert
// totals).  Everything is integer arithmetic in a fixed order: the row map
// is bit-exact and deterministic, with no atomics.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {

// The packed rows of token t's K assignments (-1 when dropped).  t is
// wave-uniform, so ids, lrank, base and the segment offsets are read with
// scalar loads, which wait on their own counter (lgkmcnt): the caller issues
// the token row's vector loads first, and the two latencies overlap.  The
// checks keep a permutation run on stale or foreign routing results inside
// the row buffers (from this forward's router and aux-loss calls they always
// hold: 0 <= e < E, r >= 0, offset + r < the kept total).
// K is a compile-time constant so that the two rounds of loads (ids and
// lrank, then base and offsets) are 2K scalar loads each with no branch
// between them; expert ids are clamped for addressing, then masked.
template <int K>
__device__ __forceinline__ void token_rows(int t, const int32_t* __restrict__ ids,
                                           const int32_t* __restrict__ lrank,
                                           const int32_t* __restrict__ base,
                                           const int32_t* __restrict__ seg, int T, int E, int C,
                                           int nblk, int (&rows)[8]) {
  const long long max_rows = min((long long)T * K, (long long)E * C);
  const int blk = t / kRouteBlock;
  int e[K], lr[K], b[K], o[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    e[k] = ids[(size_t)t * K + k];
    lr[k] = lrank[(size_t)t * K + k];
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int ec = min(max(e[k], 0), E - 1);
    b[k] = base[(size_t)ec * nblk + blk];
    o[k] = seg[ec];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    rows[k] = -1;
    if (k < K) {
      const int r = b[k] + lr[k];
      const bool ok = e[k] >= 0 && e[k] < E && r >= 0 && r < C && (long long)o[k] + r < max_rows;
      rows[k] = ok ? o[k] + r : -1;
    }
  }
}

// Lane k < K writes row_of[t, k] and, for a kept row, token_of; the wave of
// token 0 also copies the per-expert counts and the segments (offsets, kept,
// n_dropped) from the workspace to the caller's arrays.
__device__ __forceinline__ void publish_rows(
    int t, const int (&rows)[8], const int32_t* __restrict__ cnt, const int32_t* __restrict__ seg,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_dropped, int32_t* __restrict__ row_of, int32_t* __restrict__ token_of,
    int E, int K) {
  const int lane = threadIdx.x & 63;
  int my = -1;
#pragma unroll
  for (int k = 0; k < 8; ++k) my = lane == k ? rows[k] : my;
  if (lane < K) {
    row_of[(size_t)t * K + lane] = my;
    if (my >= 0) token_of[my] = t;
  }
  if (t == 0) {
    for (int e = lane; e < E; e += kWave) {
      counts[e] = cnt[e];
      offsets[e] = seg[e];
      kept[e] = seg[E + 1 + e];
    }
    if (lane == 0) {
      offsets[E] = seg[E];
      *n_dropped = seg[2 * E + 1];
    }
  }
}

// One wave per token: the copy of its row to each kept destination, and its
// row map entries.  The row is read from HBM once, in 16-byte vectors, VPL
// per lane per chunk, with non-temporal loads (the dispatch is the last
// reader of x); the first chunk's loads are issued before the index loads
// (token_rows), so the row's latency and the indices' overlap.  Measured at
// T=32768, H=4096, E=8, top-2 (stage times): 154 us with the block scan as a
// launch of its own and vector index loads, 133 us with the scan in the
// aux-loss kernel and scalar index loads, 124 us with the non-temporal row
// loads.  Non-temporal stores of xp were no faster (the grouped GEMM reads
// xp next).
template <int VPL, int K>
__global__ __launch_bounds__(256) void k_permute(
    const u32x4* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ seg,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_dropped, int32_t* __restrict__ row_of,
    int32_t* __restrict__ token_of, u32x4* __restrict__ xp, int T, int nvec, int E, int C,
    int nblk) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= T) return;  // wave-uniform; the kernel has no barrier (token 0 always runs)
  const int lane = threadIdx.x & 63;
  const u32x4* src = x + (size_t)t * nvec;
  u32x4 v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = lane + 64 * j;
    if (c < nvec) v[j] = __builtin_nontemporal_load(src + c);
  }
  int rows[8];
  token_rows<K>(t, ids, lrank, base, seg, T, E, C, nblk, rows);
  publish_rows(t, rows, cnt, seg, counts, kept, offsets, n_dropped, row_of, token_of, E, K);
  for (int c0 = 0;;) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (rows[k] >= 0) {
        u32x4* dst = xp + (size_t)rows[k] * nvec;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nvec) dst[c] = v[j];
        }
      }
    }
    c0 += 64 * VPL;
    if (c0 >= nvec) break;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c < nvec) v[j] = __builtin_nontemporal_load(src + c);
    }
  }
}

// The same row map, with the copy quantising each bf16 token row to MXFP8
// (mx.h) on the way: lane l of chunk j holds 8 values (16 bytes), four
// consecutive lanes one block of 32.  The block maximum is a max over the
// lane quad; each destination gets 8 code bytes per lane and, from the first
// lane of every 16, one 4-byte word of four block scales (operand layout,
// leading dimension xp_ld).  With x_q set the token's own quantised row is
// also written (row t, leading dimension T), for the shared expert.
template <int VPL, int K>
__global__ __launch_bounds__(256) void k_permute_mx8(
    const u32x4* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ seg,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_dropped, int32_t* __restrict__ row_of,
    int32_t* __restrict__ token_of, u32x2* __restrict__ xp_q, uint8_t* __restrict__ xp_s,
    int xp_ld, u32x2* __restrict__ x_q, uint8_t* __restrict__ x_s, int T, int nvec, int E,
    int C, int nblk) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= T) return;  // wave-uniform; no barrier in this kernel
  const int lane = threadIdx.x & 63;
  const u32x4* src = x + (size_t)t * nvec;
  // the first chunk of the row before the index loads, as in k_permute
  u32x4 v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = lane + 64 * j;
    v[j] = c < nvec ? src[c] : u32x4{0u, 0u, 0u, 0u};
  }
  int rows[9];
  token_rows<K>(t, ids, lrank, base, seg, T, E, C, nblk, (int(&)[8])rows);
  publish_rows(t, (int(&)[8])rows, cnt, seg, counts, kept, offsets, n_dropped, row_of, token_of,
               E, K);
  rows[8] = x_q ? t : -1;  // the shared expert's copy
  for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
    if (c0 > 0) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int c = c0 + lane + 64 * j;
        v[j] = c < nvec ? src[c] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    u32x2 q[VPL];
    uint32_t sw[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_bits_to_f32(v[j][i] & 0xffffu);
        f[2 * i + 1] = bf16_bits_to_f32(v[j][i] >> 16);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
      const uint32_t code = mx_scale_code(amax);
      const float inv = mx_inv_scale(code);
      q[j] = u32x2{mx_encode4(f[0], f[1], f[2], f[3], inv), mx_encode4(f[4], f[5], f[6], f[7], inv)};
      // scale word of the 16-lane group (blocks of lanes +0, +4, +8, +12)
      const uint32_t c4 = __shfl_down(code, 4, kWave), c8 = __shfl_down(code, 8, kWave);
      const uint32_t c12 = __shfl_down(code, 12, kWave);
      sw[j] = code | (c4 << 8) | (c8 << 16) | (c12 << 24);
    }
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      if (rows[k] >= 0) {
        const int r = rows[k];
        u32x2* dq = k < 8 ? xp_q : x_q;
        uint8_t* ds = k < 8 ? xp_s : x_s;
        const int ld = k < 8 ? xp_ld : T;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;  // 16-byte input chunk = 8 values
          if (c < nvec) {
            dq[(size_t)r * nvec + c] = q[j];
            if ((lane & 15) == 0)
              *(uint32_t*)(ds + ((size_t)(c >> 4) * ld + r) * 4) = sw[j];
          }
        }
      }
    }
  }
}

template <int K>
static void launch_permute_k(const PermuteArgs& a, int nvec, int nblk, hipStream_t st) {
  k_permute<8, K><<<(a.T + 3) / 4, 256, 0, st>>>(
      (const u32x4*)a.x, a.topk_ids, a.lrank, a.base, a.cnt, a.seg, a.counts, a.kept, a.offsets,
      a.n_dropped, a.row_of, a.token_of, (u32x4*)a.xp, a.T, nvec, a.E, a.C, nblk);
}

template <int K>
static void launch_permute_mx8_k(const PermuteMx8Args& a, int nvec, int nblk, hipStream_t st) {
  k_permute_mx8<4, K><<<(a.T + 3) / 4, 256, 0, st>>>(
      (const u32x4*)a.x, a.topk_ids, a.lrank, a.base, a.cnt, a.seg, a.counts, a.kept, a.offsets,
      a.n_dropped, a.row_of, a.token_of, (u32x2*)a.xp_q, a.xp_s, a.xp_ld, (u32x2*)a.x_q, a.x_s,
      a.T, nvec, a.E, a.C, nblk);
}

#define MOE_PERMUTE_BY_K(LAUNCH, ...)          \
  switch (a.K) {                              \
    case 1: LAUNCH<1>(a, __VA_ARGS__); break; \
    case 2: LAUNCH<2>(a, __VA_ARGS__); break; \
    case 3: LAUNCH<3>(a, __VA_ARGS__); break; \
    case 4: LAUNCH<4>(a, __VA_ARGS__); break; \
    case 5: LAUNCH<5>(a, __VA_ARGS__); break; \
    case 6: LAUNCH<6>(a, __VA_ARGS__); break; \
    case 7: LAUNCH<7>(a, __VA_ARGS__); break; \
    case 8: LAUNCH<8>(a, __VA_ARGS__); break; \
    default: return hipErrorInvalidValue;     \
  }

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int nblk = (a.T + kRouteBlock - 1) / kRouteBlock;
  const int nvec = a.H * (a.bf16 ? 2 : 4) / 16;
  MOE_PERMUTE_BY_K(launch_permute_k, nvec, nblk, st)
  return hipGetLastError();
}

hipError_t launch_permute_mx8(const PermuteMx8Args& a, hipStream_t st) {
  const int nblk = (a.T + kRouteBlock - 1) / kRouteBlock;
  const int nvec = a.H / 8;  // 16-byte bf16 chunks per row
  MOE_PERMUTE_BY_K(launch_permute_mx8_k, nvec, nblk, st)
  return hipGetLastError();
}
#undef MOE_PERMUTE_BY_K

}  // namespace moe
