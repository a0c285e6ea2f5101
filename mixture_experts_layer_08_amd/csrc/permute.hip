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

// One workgroup: kept = min(counts, C), offsets = exclusive scan of kept,
// n_dropped = sum(counts - kept).  E <= 256.
__global__ __launch_bounds__(256) void k_offsets(const int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ kept,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ n_dropped, int E, int C) {
  __shared__ int s_wave[4];
  __shared__ int s_drop[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = tid < E ? counts[tid] : 0;
  const int kp = min(c, C);
  const int incl = wave_inclusive_scan(kp);
  const int drop = wave_sum(c - kp);
  if (lane == 63) s_wave[wave] = incl;
  if (lane == 0) s_drop[wave] = drop;
  __syncthreads();
  int before = 0, total = 0, dsum = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? s_wave[w] : 0;
    total += s_wave[w];
    dsum += s_drop[w];
  }
  if (tid < E) {
    kept[tid] = kp;
    offsets[tid] = before + incl - kp;
  }
  if (tid == 0) {
    offsets[E] = total;
    *n_dropped = dsum;
  }
}

// One wave per token: its row map entries, then the copy of its row to each
// kept destination.  The row is read from HBM once (16-byte vectors, VPL per
// lane per chunk, all loads of a chunk issued before its stores).
template <int VPL>
__global__ __launch_bounds__(256) void k_permute(
    const u32x4* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_of,
    int32_t* __restrict__ token_of, u32x4* __restrict__ xp, int T, int nvec, int K, int C,
    int nblk) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; the kernel has no barrier
  const int lane = threadIdx.x & 63;
  int row = -1;
  if (lane < K) {
    const int e = ids[(size_t)t * K + lane];
    const int r = base[(size_t)e * nblk + t / kRouteBlock] + lrank[(size_t)t * K + lane];
    row = r < C ? offsets[e] + r : -1;
    row_of[(size_t)t * K + lane] = row;
    if (row >= 0) token_of[row] = t;
  }
  int rows[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rows[k] = __shfl(row, k, kWave);
  const u32x4* src = x + (size_t)t * nvec;
  for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
    u32x4 v[VPL];
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

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int nblk = (a.T + kRouteBlock - 1) / kRouteBlock;
  k_scan_blocks<<<a.E, 256, 0, st>>>(a.hist, a.base, a.counts, nblk);
  k_offsets<<<1, 256, 0, st>>>(a.counts, a.kept, a.offsets, a.n_dropped, a.E, a.C);
  const int elem = a.bf16 ? 2 : 4;
  const int nvec = a.H * elem / 16;
  const int grid = (a.T + 3) / 4;
  k_permute<8><<<grid, 256, 0, st>>>((const u32x4*)a.x, a.topk_ids, a.lrank, a.base, a.offsets,
                                     a.row_of, a.token_of, (u32x4*)a.xp, a.T, nvec, a.K, a.C,
                                     nblk);
  return hipGetLastError();
}

}  // namespace moe
