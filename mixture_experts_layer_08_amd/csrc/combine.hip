// Combine (weighted un-permute back to token order) and the aux loss.
//
// Combine: section 1.1 step 4 of the cf-1.com page "Dissecting the MoE
// communication bottleneck" (expert outputs weighted by the routing weights
// and returned to each token's position); the aux loss is the N * sum f_i P_i
// formula of section 3.2 of the same page.
#include "common.h"
#include "kernels.h"

namespace moe {

// One wave per token.  y[t] = sum_k w[t,k] out[row_of[t,k]] over kept slots,
// accumulated in fp32 in slot order (fused multiply-add), then + shared[t],
// then rounded to the output dtype.  Each expert-output row is read once,
// each token row written once, in 16-byte vectors.  Both streams are
// non-temporal: the expert outputs are read once and y is not read again
// by this forward.  Measured at T=32768, H=4096, E=8, top-2: 144 -> 131 us,
// and the next router call, which reads x right after this kernel, 82 ->
// 65 us, since y no longer leaves dirty lines in the caches for it to evict.
// (Non-temporal stores alone: 150 us.)
template <bool BF16, int VPL>
__global__ __launch_bounds__(256) void k_combine(const u32x4* __restrict__ out,
                                                 const int32_t* __restrict__ row_of,
                                                 const float* __restrict__ topk_w,
                                                 const u32x4* __restrict__ shared,
                                                 u32x4* __restrict__ y, int T, int nvec, int K) {
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barrier in this kernel
  const int lane = threadIdx.x & 63;
  int row = -1;
  float wt = 0.0f;
  if (lane < K) {
    row = row_of[(size_t)t * K + lane];
    wt = topk_w[(size_t)t * K + lane];
  }
  int rows[8];
  float ws[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    rows[k] = __shfl(row, k, kWave);
    ws[k] = __shfl(wt, k, kWave);
  }
  for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
    float acc[VPL][EPV];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
#pragma unroll
      for (int i = 0; i < EPV; ++i) acc[j][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K && rows[k] >= 0) {
        const u32x4* src = out + (size_t)rows[k] * nvec;
        u32x4 v[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nvec) v[j] = __builtin_nontemporal_load(src + c);
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
#pragma unroll
          for (int i = 0; i < EPV; ++i) {
            float f;
            if (BF16)
              f = bf16_bits_to_f32(i & 1 ? (v[j][i >> 1] >> 16) : (v[j][i >> 1] & 0xffffu));
            else
              f = __uint_as_float(v[j][i]);
            acc[j][i] = fmaf(ws[k], f, acc[j][i]);
          }
        }
      }
    }
    if (shared) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c < nvec) {
          const u32x4 v = shared[(size_t)t * nvec + c];
#pragma unroll
          for (int i = 0; i < EPV; ++i) {
            const float f = BF16 ? bf16_bits_to_f32(i & 1 ? (v[i >> 1] >> 16)
                                                          : (v[i >> 1] & 0xffffu))
                                 : __uint_as_float(v[i]);
            acc[j][i] += f;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c < nvec) {
        u32x4 o;
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[j][2 * q], acc[j][2 * q + 1]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[j][q]);
        }
        __builtin_nontemporal_store(o, y + (size_t)t * nvec + c);
      }
    }
  }
}

#ifndef MOE_COMBINE_VPL
#define MOE_COMBINE_VPL 8
#endif

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int nvec = a.H * (a.bf16 ? 2 : 4) / 16;
  const int grid = (a.T + 3) / 4;
  if (a.bf16)
    k_combine<true, MOE_COMBINE_VPL><<<grid, 256, 0, st>>>(
        (const u32x4*)a.out, a.row_of, a.topk_w, (const u32x4*)a.shared_out, (u32x4*)a.y, a.T,
        nvec, a.K);
  else
    k_combine<false, 4><<<grid, 256, 0, st>>>((const u32x4*)a.out, a.row_of, a.topk_w,
                                              (const u32x4*)a.shared_out, (u32x4*)a.y, a.T,
                                              nvec, a.K);
  return hipGetLastError();
}

// aux = E * sum_e (count_e / (T K)) (P_e) with P_e = (1/T) sum_t p[t,e],
// and the permutation's block scan, in one workgroup of kAuxThreads threads
// that reads each per-block partial once.  Wave w takes experts w, w + 16,
// ..., two at a time with all their loads in flight together; per expert,
// in chunks of 512 route blocks, lane l holds blocks b0 + 64 i + l (i < 8),
// so every load and store is one coalesced 256-byte row:
//   - counts (integers: exact, any order): base[e][b] = sum_{b' < b}
//     hist[e][b'] by one wave scan (DPP) per 64 blocks, cnt[e] = the total;
//   - P (fp64, a fixed order): each lane sums its 8 blocks in block order,
//     a fixed butterfly over the 64 lanes sums the lanes, chunks add in
//     chunk order.
// Thread 0 then adds the per-expert terms in expert order, and wave 0
// derives the segments: kept[e] = min(cnt[e], C), offsets = exclusive scan
// of kept (E+1 entries), and the number of dropped assignments, into seg =
// [offsets (E+1) | kept (E) | n_dropped].  Everything has a fixed order, so
// the results are deterministic.  Doing the scan and the segments here saves
// moe_permute dependent launches and leaves it one load per index.
constexpr int kAuxThreads = 1024;

// Inclusive prefix sum over the 64 lanes with DPP moves (gfx9): four
// row_shr steps scan each row of 16 lanes (lanes shifted in from outside the
// row read 0), then row_bcast:15 adds row 0's total to row 1 and row 2's to
// row 3, and row_bcast:31 adds the total of rows 0-1 to rows 2 and 3.  No
// LDS round trips, unlike a shuffle-based scan.
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Block scan of expert e's per-block histogram (the block bases) and its
// totals: the count and the sum of its per-block probability sums, in a fixed
// order.  One wave; kPer slices of 64 blocks in flight per lane.
__device__ __forceinline__ void aux_expert(const int32_t* __restrict__ hist,
                                           const float* __restrict__ psum,
                                           int32_t* __restrict__ base, int e, int nblk, int lane,
                                           int& count, double& p_sum) {
  constexpr int kPer = 8;
  int carry = 0;
  double P = 0.0;
  const int32_t* h = hist + (size_t)e * nblk;
  const float* ps = psum + (size_t)e * nblk;
  int32_t* bo = base + (size_t)e * nblk;
  for (int b0 = 0; b0 < nblk; b0 += 64 * kPer) {
    int v[kPer];
    float pv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = b0 + 64 * i + lane;
      v[i] = b < nblk ? h[b] : 0;
      pv[i] = b < nblk ? ps[b] : 0.0f;
    }
    // the kPer wave scans are independent (their DPP steps overlap); the
    // carries from slice to slice are added afterwards
    int incl[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) incl[i] = wave_scan_dpp(v[i]);
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      part += (double)pv[i];
      const int b = b0 + 64 * i + lane;
      if (b < nblk) bo[b] = carry + incl[i] - v[i];
      carry += __builtin_amdgcn_readlane(incl[i], 63);
    }
    P += wave_sum_f64(part);
  }
  count = carry;
  p_sum = P;
}

// aux = E sum_e (count_e / (T K)) (P_e / T), by one wave: lane l adds
// experts 4l .. 4l+3 in order, then a fixed shuffle tree (deterministic).
// The segments from the counts, by another wave (E <= 256: lane l holds
// experts 4l .. 4l+3).
__device__ __forceinline__ void aux_finish(const int* cnt, const double* p, float* __restrict__ aux,
                                           int32_t* __restrict__ seg, int T, int E, int K, int C,
                                           int wave, int lane) {
  if (wave == 1) {
    const double inv_tk = 1.0 / ((double)T * K), inv_t = 1.0 / (double)T;
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) part += ((double)cnt[e] * inv_tk) * (p[e] * inv_t);
    }
    const double s = wave_sum_f64(part);
    if (lane == 0) *aux = (float)((double)E * s);
  }
  if (wave == 0) {
    int kept4[4], run = 0, drop = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      const int c = e < E ? cnt[e] : 0;
      kept4[i] = min(c, C);
      drop += c - kept4[i];
      run += kept4[i];
    }
    const int incl = wave_inclusive_scan(run);
    int off = incl - run;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        seg[e] = off;
        seg[E + 1 + e] = kept4[i];
      }
      off += kept4[i];
    }
    const int dropped = wave_sum(drop);
    if (lane == 63) seg[E] = incl;
    if (lane == 0) seg[2 * E + 1] = dropped;
  }
}

// Up to kAuxWaves experts: one workgroup, one wave per expert, then the aux
// loss and the segments from LDS.
constexpr int kAuxWaves = kAuxThreads / kWave;
__global__ __launch_bounds__(kAuxThreads) void k_aux(const int32_t* __restrict__ hist,
                                                     const float* __restrict__ psum,
                                                     float* __restrict__ aux,
                                                     int32_t* __restrict__ base,
                                                     int32_t* __restrict__ cnt_out,
                                                     int32_t* __restrict__ seg, int T, int E,
                                                     int K, int C, int nblk) {
  __shared__ double s_p[kAuxWaves];
  __shared__ int s_cnt[kAuxWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < E) {
    int c;
    double P;
    aux_expert(hist, psum, base, wave, nblk, lane, c, P);
    if (lane == 0) {
      cnt_out[wave] = c;
      s_cnt[wave] = c;
      s_p[wave] = P;
    }
  }
  __syncthreads();
  aux_finish(s_cnt, s_p, aux, seg, T, E, K, C, wave, lane);
}

// More experts: kAuxWaves per workgroup, one wave each, totals to global ...
__global__ __launch_bounds__(kAuxThreads) void k_aux_scan(const int32_t* __restrict__ hist,
                                                          const float* __restrict__ psum,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ cnt_out,
                                                          double* __restrict__ p_out, int E,
                                                          int nblk) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kAuxWaves + (threadIdx.x >> 6);
  if (e >= E) return;  // wave-uniform; no barrier in this kernel
  int c;
  double P;
  aux_expert(hist, psum, base, e, nblk, lane, c, P);
  if (lane == 0) {
    cnt_out[e] = c;
    p_out[e] = P;
  }
}

// ... and one small workgroup for the aux loss and the segments.
__global__ __launch_bounds__(128) void k_aux_finish(const int32_t* __restrict__ cnt,
                                                    const double* __restrict__ p,
                                                    float* __restrict__ aux,
                                                    int32_t* __restrict__ seg, int T, int E, int K,
                                                    int C) {
  aux_finish(cnt, p, aux, seg, T, E, K, C, threadIdx.x >> 6, threadIdx.x & 63);
}

hipError_t launch_aux(const int32_t* hist, const float* psum, float* aux, int32_t* base,
                      int32_t* cnt, double* p_scratch, int32_t* seg, int T, int E, int K, int C,
                      int nblk, hipStream_t st) {
  if (E <= kAuxWaves) {
    k_aux<<<1, kAuxThreads, 0, st>>>(hist, psum, aux, base, cnt, seg, T, E, K, C, nblk);
    return hipGetLastError();
  }
  k_aux_scan<<<(E + kAuxWaves - 1) / kAuxWaves, kAuxThreads, 0, st>>>(hist, psum, base, cnt,
                                                                       p_scratch, E, nblk);
  k_aux_finish<<<1, 128, 0, st>>>(cnt, p_scratch, aux, seg, T, E, K, C);
  return hipGetLastError();
}

}  // namespace moe
