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
// histograms.  Everything is integer arithmetic in a fixed order: the row
// map is bit-exact and deterministic, with no atomics.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {

// One workgroup per expert: base[e][b] = sum_{b' < b} hist[e][b'], counts[e].
__global__ __launch_bounds__(256) void k_scan_blocks(const int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ base,
                                                     int32_t* __restrict__ counts, int nblk) {
  __shared__ int s_wave[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t* h = hist + (size_t)e * nblk;
  int32_t* bo = base + (size_t)e * nblk;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + tid;
    const int v = b < nblk ? h[b] : 0;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += w < wave ? s_wave[w] : 0;
      total += s_wave[w];
    }
    if (b < nblk) bo[b] = carry + before + incl - v;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) counts[e] = carry;
}

// Segment offsets from the per-expert counts, computed by every permute wave
// (E <= 256: lane l holds experts 4l .. 4l+3): kept = min(counts, C),
// offsets = exclusive scan of kept.  Returns this lane's four offsets and the
// wave-uniform total; the counts are integers, so every wave gets the same.
__device__ __forceinline__ void segment_offsets(const int32_t* __restrict__ counts, int E, int C,
                                                int (&off4)[4], int (&kept4)[4], int& drop4,
                                                int& total) {
  const int lane = threadIdx.x & 63;
  int run = 0;
  drop4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    const int c = e < E ? counts[e] : 0;
    kept4[i] = min(c, C);
    drop4 += c - kept4[i];
    off4[i] = run;  // exclusive within the lane
    run += kept4[i];
  }
  const int incl = wave_inclusive_scan(run);
  const int before = incl - run;
#pragma unroll
  for (int i = 0; i < 4; ++i) off4[i] += before;
  total = __shfl(incl, 63, kWave);
}

// The row map of token t, computed by its wave: lane k < K returns the packed
// row of assignment (t, k) (-1 when dropped) and writes row_of / token_of;
// other lanes return -1.  The wave of token 0 also publishes kept, offsets
// and n_dropped.  Index loads come first (the counts load independently of
// ids and lrank, so two dependent round trips precede any row traffic).
__device__ __forceinline__ int permute_row_map(
    int t, const int32_t* __restrict__ ids, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ kept, int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of, int E, int K, int C, int nblk) {
  const int lane = threadIdx.x & 63;
  int e = 0, lr = 0;
  if (lane < K) {
    e = ids[(size_t)t * K + lane];
    lr = lrank[(size_t)t * K + lane];
  }
  int off4[4], kept4[4], drop4, total;
  segment_offsets(counts, E, C, off4, kept4, drop4, total);
  if (t == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = 4 * lane + i;
      if (ee < E) {
        kept[ee] = kept4[i];
        offsets[ee] = off4[i];
      }
    }
    const int dropped = wave_sum(drop4);
    if (lane == 0) {
      offsets[E] = total;
      *n_dropped = dropped;
    }
  }
  int row = -1;
  // offsets[e] lives in lane e/4, slot e%4 (all lanes take part in the shuffles)
  const int o0 = __shfl(off4[0], e >> 2, kWave), o1 = __shfl(off4[1], e >> 2, kWave);
  const int o2 = __shfl(off4[2], e >> 2, kWave), o3 = __shfl(off4[3], e >> 2, kWave);
  const int oe = (e & 3) == 0 ? o0 : (e & 3) == 1 ? o1 : (e & 3) == 2 ? o2 : o3;
  if (lane < K) {
    const int r = base[(size_t)e * nblk + t / kRouteBlock] + lr;
    row = r < C ? oe + r : -1;
    row_of[(size_t)t * K + lane] = row;
    if (row >= 0) token_of[row] = t;
  }
  return row;
}

// One wave per token: its row map entries, then the copy of its row to each
// kept destination.  The row is read from HBM once (16-byte vectors, VPL per
// lane per chunk, all loads of a chunk issued before its stores; vmcnt waits
// are in issue order, so the row loads come after the index loads).
template <int VPL>
__global__ __launch_bounds__(256) void k_permute(
    const u32x4* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ counts, int32_t* __restrict__ kept,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped, int32_t* __restrict__ row_of,
    int32_t* __restrict__ token_of, u32x4* __restrict__ xp, int T, int nvec, int E, int K, int C,
    int nblk) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; the kernel has no barrier (token 0 always runs)
  const int lane = threadIdx.x & 63;
  const int row = permute_row_map(t, ids, lrank, base, counts, kept, offsets, n_dropped, row_of,
                                  token_of, E, K, C, nblk);
  const u32x4* src = x + (size_t)t * nvec;
  u32x4 v[VPL];
  int rows[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rows[k] = __shfl(row, k, kWave);
  for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c < nvec) v[j] = src[c];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K && rows[k] >= 0) {
        u32x4* dst = xp + (size_t)rows[k] * nvec;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nvec) dst[c] = v[j];
        }
      }
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
template <int VPL>
__global__ __launch_bounds__(256) void k_permute_mx8(
    const u32x4* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ counts, int32_t* __restrict__ kept,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped, int32_t* __restrict__ row_of,
    int32_t* __restrict__ token_of, u32x2* __restrict__ xp_q, uint8_t* __restrict__ xp_s,
    int xp_ld, u32x2* __restrict__ x_q, uint8_t* __restrict__ x_s, int T, int nvec, int E,
    int K, int C, int nblk) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barrier in this kernel
  const int lane = threadIdx.x & 63;
  const int row = permute_row_map(t, ids, lrank, base, counts, kept, offsets, n_dropped, row_of,
                                  token_of, E, K, C, nblk);
  const u32x4* src = x + (size_t)t * nvec;
  int rows[9];
#pragma unroll
  for (int k = 0; k < 8; ++k) rows[k] = k < K ? __shfl(row, k, kWave) : -1;
  rows[8] = x_q ? t : -1;  // the shared expert's copy
  for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
    u32x4 v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = c0 + lane + 64 * j;
      v[j] = c < nvec ? src[c] : u32x4{0u, 0u, 0u, 0u};
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

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int nblk = (a.T + kRouteBlock - 1) / kRouteBlock;
  k_scan_blocks<<<a.E, 256, 0, st>>>(a.hist, a.base, a.counts, nblk);
  const int elem = a.bf16 ? 2 : 4;
  const int nvec = a.H * elem / 16;
  const int grid = (a.T + 3) / 4;
  k_permute<8><<<grid, 256, 0, st>>>((const u32x4*)a.x, a.topk_ids, a.lrank, a.base, a.counts,
                                     a.kept, a.offsets, a.n_dropped, a.row_of, a.token_of,
                                     (u32x4*)a.xp, a.T, nvec, a.E, a.K, a.C, nblk);
  return hipGetLastError();
}

hipError_t launch_permute_mx8(const PermuteMx8Args& a, hipStream_t st) {
  const int nblk = (a.T + kRouteBlock - 1) / kRouteBlock;
  k_scan_blocks<<<a.E, 256, 0, st>>>(a.hist, a.base, a.counts, nblk);
  const int nvec = a.H / 8;  // 16-byte bf16 chunks per row
  const int grid = (a.T + 3) / 4;
  k_permute_mx8<4><<<grid, 256, 0, st>>>((const u32x4*)a.x, a.topk_ids, a.lrank, a.base,
                                         a.counts, a.kept, a.offsets, a.n_dropped, a.row_of,
                                         a.token_of, (u32x2*)a.xp_q, a.xp_s, a.xp_ld,
                                         (u32x2*)a.x_q, a.x_s, a.T, nvec, a.E, a.K, a.C, nblk);
  return hipGetLastError();
}

}  // namespace moe
