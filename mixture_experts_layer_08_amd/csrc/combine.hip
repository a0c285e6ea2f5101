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
// each token row written once, in 16-byte vectors.
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
          if (c < nvec) v[j] = src[c];
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
        y[(size_t)t * nvec + c] = o;
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

// aux = E * sum_e (count_e / (T K)) (P_e) with P_e = (1/T) sum_t p[t,e].
// One workgroup of kAuxThreads threads.  Expert e's per-block partials are
// split over G = kAuxThreads / E_pad threads (E_pad = E rounded up to a power
// of two): thread (e, g) sums blocks g, g+G, g+2G, ... in order (fp64), then a
// fixed-shape tree over g combines them, and thread 0 adds the per-expert
// terms in expert order.  Deterministic: every sum has a fixed order.
constexpr int kAuxThreads = 1024;
__global__ __launch_bounds__(kAuxThreads) void k_aux(const int32_t* __restrict__ hist,
                                                     const float* __restrict__ psum,
                                                     float* __restrict__ aux, int T, int E, int K,
                                                     int nblk) {
  __shared__ double s_p[kAuxThreads];
  __shared__ long long s_c[kAuxThreads];
  int e_pad = 1;
  while (e_pad < E) e_pad <<= 1;
  const int G = kAuxThreads / e_pad;
  const int tid = threadIdx.x;
  const int e = tid / G, g = tid % G;
  double P = 0.0;
  long long cnt = 0;
  if (e < E) {
    for (int b = g; b < nblk; b += G) {
      cnt += hist[(size_t)e * nblk + b];
      P += (double)psum[(size_t)e * nblk + b];
    }
  }
  s_p[tid] = P;
  s_c[tid] = cnt;
  __syncthreads();
  for (int w = G >> 1; w > 0; w >>= 1) {
    if (g < w) {
      s_p[tid] += s_p[tid + w];
      s_c[tid] += s_c[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    double s = 0.0;
    for (int i = 0; i < E; ++i)
      s += ((double)s_c[i * G] / ((double)T * K)) * (s_p[i * G] / (double)T);
    *aux = (float)((double)E * s);
  }
}

hipError_t launch_aux(const int32_t* hist, const float* psum, float* aux, int T, int E, int K,
                      int nblk, hipStream_t st) {
  k_aux<<<1, kAuxThreads, 0, st>>>(hist, psum, aux, T, E, K, nblk);
  return hipGetLastError();
}

}  // namespace moe
