// Backward of the routed layer: the memory-bound pieces (combine adjoint,
// gate gradient, router weight gradient, un-permute).  The expert FFN's
// backward runs on the grouped GEMM (gemm.hip, NT and TN layouts).
//
// Method: the chain rule of the forward definition.  The gate receives
// gradients through the renormalised top-k weights (section 3.1 of the
// dpshk.com "MoE module infra notes": the gradient must reach the gate
// network) and through P_e of the aux loss with its coefficient alpha
// (section 3.2 of the cf-1.com page "Dissecting the MoE communication
// bottleneck"); dropped assignments pass no gradient (the same section's
// second pitfall: dropped tokens are absent in the backward pass).
//
// Every reduction runs in a fixed order (wave butterflies, slot order,
// token-chunk order), so results are deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}

// Elements of a 16-byte vector as fp32 (8 bf16 or 4 fp32) and back.
template <bool BF16>
__device__ __forceinline__ float vec_elem(const u32x4& v, int i) {
  if (BF16) return bf16_bits_to_f32(i & 1 ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xffffu));
  return __uint_as_float(v[i]);
}
template <bool BF16>
__device__ __forceinline__ u32x4 vec_pack(const float* f) {
  u32x4 o;
  if (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(f[q]);
  }
  return o;
}

}  // namespace

// One wave per token.  For each kept slot k: d_out[row] = w_k * dy[t]
// (rounded to the dtype) and d_w[t,k] = <dy[t], out[row]> (per-lane partial
// sums in vector order, then a wave butterfly).  Dropped slots: d_w = 0.
template <bool BF16, int VPL>
__global__ __launch_bounds__(256) void k_combine_bwd(
    const u32x4* __restrict__ dy, const u32x4* __restrict__ out,
    const int32_t* __restrict__ row_of, const float* __restrict__ topk_w,
    u32x4* __restrict__ d_out, float* __restrict__ d_topk_w, int T, int nvec, int K) {
  constexpr int EPV = BF16 ? 8 : 4;
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
  float ws[8], dot[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    rows[k] = __shfl(row, k, kWave);
    ws[k] = __shfl(wt, k, kWave);
    dot[k] = 0.0f;
  }
  for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
    u32x4 g[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c < nvec) g[j] = dy[(size_t)t * nvec + c];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K && rows[k] >= 0) {
        const u32x4* src = out + (size_t)rows[k] * nvec;
        u32x4* dst = d_out + (size_t)rows[k] * nvec;
        u32x4 o[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nvec) o[j] = src[c];
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nvec) {
            float f[EPV];
#pragma unroll
            for (int i = 0; i < EPV; ++i) {
              const float gv = vec_elem<BF16>(g[j], i);
              dot[k] = fmaf(gv, vec_elem<BF16>(o[j], i), dot[k]);
              f[i] = ws[k] * gv;
            }
            dst[c] = vec_pack<BF16>(f);
          }
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      const float s = wave_sum_f32(dot[k]);
      if (lane == 0) d_topk_w[(size_t)t * K + k] = rows[k] >= 0 ? s : 0.0f;
    }
  }
}

// Gate gradient, one wave per token; lane l holds experts l, l+64, l+128,
// l+192 (E <= 256).
//   d_l[e] = alpha (E/T) p_e (f_e - sum_e' f_e' p_e')       (aux term)
//          + [e = ids[k]] w_k (d_w_k - sum_j w_j d_w_j)    (weights term)
__global__ __launch_bounds__(256) void k_route_bwd_dl(
    const float* __restrict__ logits, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, const float* __restrict__ d_topk_w,
    const int32_t* __restrict__ counts, float alpha, float* __restrict__ d_logits, int T, int E,
    int K) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barrier in this kernel
  const int lane = threadIdx.x & 63;
  float dl[4] = {0.f, 0.f, 0.f, 0.f};
  if (alpha != 0.0f) {
    float l[4];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      l[i] = e < E ? logits[(size_t)t * E + e] : -INFINITY;
      m = fmaxf(m, l[i]);
    }
    m = wave_max_f32(m);
    float z[4], zs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = lane + 64 * i < E ? __expf(l[i] - m) : 0.0f;
      zs += z[i];
    }
    zs = wave_sum_f32(zs);
    const float inv_tk = 1.0f / ((float)T * (float)K);
    float p[4], f[4], sf = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      p[i] = z[i] / zs;
      f[i] = e < E ? (float)counts[e] * inv_tk : 0.0f;
      sf = fmaf(f[i], p[i], sf);
    }
    sf = wave_sum_f32(sf);
    const float scale = alpha * (float)E / (float)T;
#pragma unroll
    for (int i = 0; i < 4; ++i) dl[i] = scale * p[i] * (f[i] - sf);
  }
  int e_k = 0;
  float w_k = 0.0f, dw_k = 0.0f;
  if (lane < K) {
    e_k = ids[(size_t)t * K + lane];
    w_k = topk_w[(size_t)t * K + lane];
    dw_k = d_topk_w[(size_t)t * K + lane];
  }
  const float sw = wave_sum_f32(w_k * dw_k);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      const int e = __shfl(e_k, k, kWave);
      const float g = __shfl(w_k, k, kWave) * (__shfl(dw_k, k, kWave) - sw);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == e) dl[i] += g;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < E) d_logits[(size_t)t * E + e] = dl[i];
  }
}

// Router weight gradient, first pass: per token chunk c (kRouteBwdChunk
// tokens) and expert group g (32 experts), thread h of the workgroup's 256
// columns accumulates part[c][h][e] = sum_{t in c} x[t,h] d_l[t,e] in token
// order; the x-column-0 workgroup also sums d_l (db partials).  A 64-token
// slice of d_l[:, group] is staged in LDS and read as a broadcast.
template <bool BF16>
__global__ __launch_bounds__(256) void k_route_bwd_dw_part(
    const void* __restrict__ xv, const float* __restrict__ d_logits, float* __restrict__ part,
    float* __restrict__ dbpart, int T, int H, int E) {
  __shared__ float s_dl[64][33];
  const int tid = threadIdx.x;
  const int h = blockIdx.x * 256 + tid;
  const int c = blockIdx.y, g = blockIdx.z;
  const int e0 = g * 32;
  const int t_begin = c * kRouteBwdChunk, t_end = min(T, t_begin + kRouteBwdChunk);
  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = 0.0f;
  float db = 0.0f;
  for (int t0 = t_begin; t0 < t_end; t0 += 64) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = tid + 256 * q;
      const int tt = i >> 5, j = i & 31;
      const int t = t0 + tt, e = e0 + j;
      s_dl[tt][j] = (t < t_end && e < E) ? d_logits[(size_t)t * E + e] : 0.0f;
    }
    __syncthreads();
    const int nt = min(64, t_end - t0);
    for (int tt0 = 0; tt0 < nt; tt0 += 8) {
      float xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = t0 + tt0 + u;
        float v = 0.0f;
        if (h < H && tt0 + u < nt) {
          if (BF16) v = (float)((const bf16*)xv)[(size_t)t * H + h];
          else v = ((const float*)xv)[(size_t)t * H + h];
        }
        xs[u] = v;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[j] = fmaf(xs[u], s_dl[tt0 + u][j], acc[j]);
    }
    if (blockIdx.x == 0 && tid < 32)
      for (int tt = 0; tt < nt; ++tt) db += s_dl[tt][tid];
    __syncthreads();
  }
  if (h < H) {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (e0 + j < E) part[((size_t)c * H + h) * E + e0 + j] = acc[j];
  }
  if (blockIdx.x == 0 && tid < 32 && e0 + tid < E) dbpart[(size_t)c * E + e0 + tid] = db;
}

// Second pass: d_w_router[h][e] = sum_c part[c][h][e] in chunk order, and
// d_b_router[e] likewise from the db partials.
__global__ __launch_bounds__(256) void k_route_bwd_reduce(const float* __restrict__ part,
                                                          const float* __restrict__ dbpart,
                                                          float* __restrict__ d_w,
                                                          float* __restrict__ d_b, int nchunk,
                                                          int H, int E) {
  const size_t n = (size_t)H * E;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    float s = 0.0f;
    for (int c = 0; c < nchunk; ++c) s += part[(size_t)c * n + i];
    d_w[i] = s;
  } else if (d_b && i < n + E) {
    const int e = (int)(i - n);
    float s = 0.0f;
    for (int c = 0; c < nchunk; ++c) s += dbpart[(size_t)c * E + e];
    d_b[e] = s;
  }
}

// One wave per token: dx[t] = sum_{k kept} d_xp[row_of[t,k]] (+ d_x_shared[t])
// accumulated in fp32 in slot order, rounded once.
template <bool BF16, int VPL>
__global__ __launch_bounds__(256) void k_permute_bwd(
    const u32x4* __restrict__ d_xp, const int32_t* __restrict__ row_of,
    const u32x4* __restrict__ d_x_shared, u32x4* __restrict__ dx, int T, int nvec, int K) {
  constexpr int EPV = BF16 ? 8 : 4;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barrier in this kernel
  const int lane = threadIdx.x & 63;
  const int row = lane < K ? row_of[(size_t)t * K + lane] : -1;
  int rows[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rows[k] = __shfl(row, k, kWave);
  for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
    float acc[VPL][EPV];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
#pragma unroll
      for (int i = 0; i < EPV; ++i) acc[j][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K && rows[k] >= 0) {
        const u32x4* src = d_xp + (size_t)rows[k] * nvec;
        u32x4 v[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nvec) v[j] = src[c];
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j)
#pragma unroll
          for (int i = 0; i < EPV; ++i) acc[j][i] += vec_elem<BF16>(v[j], i);
      }
    }
    if (d_x_shared) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c < nvec) {
          const u32x4 v = d_x_shared[(size_t)t * nvec + c];
#pragma unroll
          for (int i = 0; i < EPV; ++i) acc[j][i] += vec_elem<BF16>(v, i);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c < nvec) dx[(size_t)t * nvec + c] = vec_pack<BF16>(acc[j]);
    }
  }
}

// dst [R][Ep] bf16 = src [R][E] (fp32 or bf16), zero in columns E..Ep-1.
template <bool SRC_F32>
__global__ __launch_bounds__(256) void k_pad_bf16(const void* __restrict__ src,
                                                  bf16* __restrict__ dst, int R, int E, int Ep) {
  const size_t n = (size_t)R * Ep;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / Ep), e = (int)(i % Ep);
    float v = 0.0f;
    if (e < E) v = SRC_F32 ? ((const float*)src)[(size_t)r * E + e]
                           : (float)((const bf16*)src)[(size_t)r * E + e];
    dst[i] = f32_to_bf16(v);
  }
}

hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t st) {
  const int nvec = a.H * (a.bf16 ? 2 : 4) / 16;
  const int grid = (a.T + 3) / 4;
  if (a.bf16)
    k_combine_bwd<true, 4><<<grid, 256, 0, st>>>((const u32x4*)a.dy, (const u32x4*)a.out,
                                                a.row_of, a.topk_w, (u32x4*)a.d_out,
                                                a.d_topk_w, a.T, nvec, a.K);
  else
    k_combine_bwd<false, 4><<<grid, 256, 0, st>>>((const u32x4*)a.dy, (const u32x4*)a.out,
                                                 a.row_of, a.topk_w, (u32x4*)a.d_out,
                                                 a.d_topk_w, a.T, nvec, a.K);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const RouteBwdArgs& a, hipStream_t st) {
  k_route_bwd_dl<<<(a.T + 3) / 4, 256, 0, st>>>(a.logits, a.topk_ids, a.topk_w, a.d_topk_w,
                                                  a.counts, a.alpha, a.d_logits, a.T, a.E, a.K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nchunk = route_bwd_chunks(a.T);
  const dim3 grid((a.H + 255) / 256, nchunk, (a.E + 31) / 32);
  if (a.bf16)
    k_route_bwd_dw_part<true><<<grid, 256, 0, st>>>(a.x, a.d_logits, a.part, a.dbpart, a.T, a.H,
                                                     a.E);
  else
    k_route_bwd_dw_part<false><<<grid, 256, 0, st>>>(a.x, a.d_logits, a.part, a.dbpart, a.T,
                                                      a.H, a.E);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t n = (size_t)a.H * a.E + a.E;
  k_route_bwd_reduce<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a.part, a.dbpart, a.d_w_router,
                                                                  a.d_b_router, nchunk, a.H, a.E);
  return hipGetLastError();
}

hipError_t launch_permute_bwd(const PermuteBwdArgs& a, hipStream_t st) {
  const int nvec = a.H * (a.bf16 ? 2 : 4) / 16;
  const int grid = (a.T + 3) / 4;
  if (a.bf16)
    k_permute_bwd<true, 8><<<grid, 256, 0, st>>>((const u32x4*)a.d_xp, a.row_of,
                                                (const u32x4*)a.d_x_shared, (u32x4*)a.dx, a.T,
                                                nvec, a.K);
  else
    k_permute_bwd<false, 4><<<grid, 256, 0, st>>>((const u32x4*)a.d_xp, a.row_of,
                                                 (const u32x4*)a.d_x_shared, (u32x4*)a.dx, a.T,
                                                 nvec, a.K);
  return hipGetLastError();
}

hipError_t launch_pad_bf16(const void* src, bool src_f32, bf16* dst, int R, int E, int Ep,
                           hipStream_t st) {
  const size_t n = (size_t)R * Ep;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  if (src_f32) k_pad_bf16<true><<<grid, 256, 0, st>>>(src, dst, R, E, Ep);
  else k_pad_bf16<false><<<grid, 256, 0, st>>>(src, dst, R, E, Ep);
  return hipGetLastError();
}

}  // namespace moe
