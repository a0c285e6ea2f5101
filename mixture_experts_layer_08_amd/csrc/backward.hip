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
#include <type_traits>

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

// c + a.lo * b.lo + a.hi * b.hi for bf16 pairs, accumulated in fp32
// (v_dot2c_f32_bf16: the products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
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
// l+192 (E <= 256).  With p the softmax of the selection scores z that the
// forward stored in `logits`:
//   d_z[e] = alpha (E/T) p_e (f_e - sum_e' f_e' p_e')       (aux term)
//          + [e = ids[k]] w_k (d_w_k - sum_j w_j d_w_j)    (weights term)
// and the output is d_l = d_z / tau, the gradient of the router GEMM output
// (z = (l + g) / tau; the noise g does not depend on any parameter).
__global__ __launch_bounds__(256) void k_route_bwd_dl(
    const float* __restrict__ logits, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, const float* __restrict__ d_topk_w,
    const int32_t* __restrict__ counts, float alpha, float inv_tau, float* __restrict__ d_logits,
    int T, int E, int K) {
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
  // dL/dz -> dL/dl for z = (l + g) / tau (inv_tau = 1 for the plain router)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < E) d_logits[(size_t)t * E + e] = dl[i] * inv_tau;
  }
}

// Router weight gradient, first pass: per token chunk c (route_bwd_chunk(E)
// tokens) and expert group g (EG experts), thread i of the workgroup owns
// columns h, h+1 (h = 2i + 512 blockIdx.x) and accumulates
// part[c][h][e] = sum_{t in c} x[t,h] d_l[t,e] in token order.  d_l for 256
// tokens at a time is staged in LDS (zero past the chunk and past E) and
// read as a broadcast.  x is read in double-buffered batches of U tokens
// from clamped addresses and kept raw until its batch is multiplied, so 2U
// loads per lane stay in flight; columns past H compute on column 0 and are
// never stored.
template <bool BF16, int EG>
__global__ __launch_bounds__(256) void k_route_bwd_dw_part(
    const void* __restrict__ xv, const float* __restrict__ d_logits, float* __restrict__ part,
    int T, int H, int E, int chunk) {
  constexpr int U = 16;
  constexpr int SUB = 256;  // tokens per staged slice of d_l
  static_assert(SUB % (2 * U) == 0, "whole double batches per slice");
  __shared__ __attribute__((aligned(16))) float s_dl[SUB][EG];
  using Raw = typename std::conditional<BF16, uint32_t, float2>::type;
  const int tid = threadIdx.x;
  const int h = blockIdx.x * 512 + 2 * tid;
  const bool h_ok = h < H;  // H is a multiple of 8: h < H implies h + 1 < H
  const int hc = h_ok ? h : 0;
  const int c = blockIdx.y;
  const int e0 = blockIdx.z * EG;
  const int t_begin = c * chunk, t_end = min(T, t_begin + chunk);
  float acc0[EG], acc1[EG];
#pragma unroll
  for (int j = 0; j < EG; ++j) acc0[j] = acc1[j] = 0.0f;
  auto load = [&](int t, Raw* r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t at = (size_t)min(t + u, T - 1) * H + hc;
      if constexpr (BF16) r[u] = *(const uint32_t*)((const bf16*)xv + at);
      else r[u] = *(const float2*)((const float*)xv + at);
    }
  };
  auto accumulate = [&](int tt, const Raw* r) {  // tt: token offset in the slice
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a, b;
      if constexpr (BF16) {
        a = bf16_bits_to_f32(r[u] & 0xffffu);
        b = bf16_bits_to_f32(r[u] >> 16);
      } else {
        a = r[u].x;
        b = r[u].y;
      }
#pragma unroll
      for (int j = 0; j < EG; j += 4) {
        const f32x4 g = *(const f32x4*)&s_dl[tt + u][j];  // broadcast read
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc0[j + q] = fmaf(a, g[q], acc0[j + q]);
          acc1[j + q] = fmaf(b, g[q], acc1[j + q]);
        }
      }
    }
  };
  for (int s0 = t_begin; s0 < t_end; s0 += SUB) {
    __syncthreads();  // the previous slice is no longer read
    for (int i = tid; i < SUB * EG; i += 256) {
      const int tt = i / EG, j = i % EG;
      const int t = s0 + tt, e = e0 + j;
      s_dl[tt][j] = (t < t_end && e < E) ? d_logits[(size_t)t * E + e] : 0.0f;
    }
    __syncthreads();
    const int n = min(SUB, t_end - s0);  // tokens of this slice; past them d_l is 0
    // Straight-line batches (a branch around a load would make the compiler
    // wait for every load in flight): loads past the slice read clamped rows
    // and multiply staged zeros; tt + U + u < SUB since tt <= SUB - 2U.
    // sched_barrier(0) keeps the scheduler from sinking a batch's loads below
    // the FMAs of the batch before it.
    Raw r0[U], r1[U];
    load(s0, r0);
    for (int tt = 0; tt < n; tt += 2 * U) {
      load(s0 + tt + U, r1);
      __builtin_amdgcn_sched_barrier(0);
      accumulate(tt, r0);
      __builtin_amdgcn_sched_barrier(0);
      load(s0 + tt + 2 * U, r0);
      __builtin_amdgcn_sched_barrier(0);
      accumulate(tt + U, r1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (h_ok) {
#pragma unroll
    for (int j = 0; j < EG; ++j) {
      if (e0 + j < E) {
        part[((size_t)c * H + h) * E + e0 + j] = acc0[j];
        part[((size_t)c * H + h + 1) * E + e0 + j] = acc1[j];
      }
    }
  }
}

// Router bias gradient, first pass: dbpart[b][e] = sum_{t in block b} d_l[t,e]
// over blocks of kDbBlock tokens.  G = 256 / E_pad threads per expert (E_pad =
// E rounded up to a power of two): thread (g, e) sums tokens g, g+G, ... of
// the block in order (a fixed trip count, so its loads are issued together),
// then a fixed-shape tree over g combines them.
constexpr int kDbBlock = 64;
__global__ __launch_bounds__(256) void k_route_bwd_db_part(const float* __restrict__ d_logits,
                                                           float* __restrict__ dbpart, int T,
                                                           int E) {
  __shared__ float s[256];
  int e_pad = 1;
  while (e_pad < E) e_pad <<= 1;
  const int G = 256 / e_pad;  // 1 .. 256, a power of two
  const int tid = threadIdx.x;
  const int g = tid / e_pad, e = tid % e_pad;
  const int t0 = blockIdx.x * kDbBlock;
  float v = 0.0f;
  if (e < E) {
    float x[kDbBlock];
#pragma unroll
    for (int i = 0; i < kDbBlock; ++i) {
      const int t = t0 + g + i * G;
      x[i] = (i * G < kDbBlock && t < T) ? d_logits[(size_t)t * E + e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kDbBlock; ++i) v += x[i];
  }
  s[tid] = v;
  __syncthreads();
  for (int w = G >> 1; w > 0; w >>= 1) {
    if (g < w) s[tid] += s[tid + w * e_pad];
    __syncthreads();
  }
  if (g == 0 && e < E) dbpart[(size_t)blockIdx.x * E + e] = s[tid];
}

// Token-chunk bounds [c * chunk, min(T, (c+1) * chunk)) as a segment table for
// the grouped GEMM (the MFMA form of the router weight gradient).
__global__ void k_chunk_offsets(int32_t* __restrict__ off, int nchunk, int chunk, int T) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i <= nchunk) off[i] = min(i * chunk, T);
}

// Second pass: d_w_router[h][e] = sum_c part[c][h][e] in chunk order (or,
// from the MFMA form, sum_c part[c][e][h] with rows of E_ld).
__global__ __launch_bounds__(256) void k_route_bwd_reduce(const float* __restrict__ part,
                                                          float* __restrict__ d_w, int nchunk,
                                                          int H, int E, int e_ld) {
  const size_t n = (size_t)H * E;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    float s = 0.0f;
    if (e_ld == 0) {
      for (int c = 0; c < nchunk; ++c) s += part[(size_t)c * n + i];
      d_w[i] = s;
    } else {
      // consecutive threads read consecutive h of one expert's row
      const int e = (int)(i / H), h = (int)(i % H);
      const size_t cs = (size_t)e_ld * H;
      for (int c = 0; c < nchunk; ++c) s += part[(size_t)c * cs + i];
      d_w[(size_t)h * E + e] = s;
    }
  }
}

// d_b_router[e] = sum_b dbpart[b][e]: one workgroup per expert; thread j
// sums blocks j, j+256, ... in order, then a fixed-shape tree.
__global__ __launch_bounds__(256) void k_route_bwd_db_reduce(const float* __restrict__ dbpart,
                                                             float* __restrict__ d_b, int ndb,
                                                             int E) {
  __shared__ float s[256];
  const int e = blockIdx.x, j = threadIdx.x;
  float v = 0.0f;
  for (int b = j; b < ndb; b += 256) v += dbpart[(size_t)b * E + e];
  s[j] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (j < w) s[j] += s[j + w];
    __syncthreads();
  }
  if (j == 0) d_b[e] = s[0];
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

// The same un-permute with the router's input gradient folded in (bf16, at
// most 16 experts):
//   dx[t] = sum_{k kept} d_xp[row_of[t,k]] (+ d_x_shared[t])
//           + sum_e bf16(d_logits[t,e]) W_r[:,e],
// summed in fp32 (the router term first, expert pairs in order on the bf16
// dot-product instruction, then the slots in order, then the shared term) and
// rounded once.  Each workgroup first stages W_r [H][E] in LDS as
// [h mod 8][e / 8][h / 8][8 experts] (zero past E): lane l of a wave then
// reads the 16-byte expert row of its column h = 8c + i at consecutive
// addresses, and the workgroup's tokens share one copy.  Wave w of workgroup
// b takes tokens b*8 + w, then steps of 8 * grid.
constexpr int kPermRouteThreads = 512, kPermRouteWaves = kPermRouteThreads / kWave;
template <int NQ, int VPL>
__global__ __launch_bounds__(kPermRouteThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_permute_bwd_route(
    const u32x4* __restrict__ d_xp, const int32_t* __restrict__ row_of,
    const u32x4* __restrict__ d_x_shared, const float* __restrict__ d_logits,
    const uint16_t* __restrict__ w_router, u32x4* __restrict__ dx, int T, int nvec, int K,
    int E, int w_vec16) {
  extern __shared__ u32x4 w_lds[];  // [8][NQ][nvec] rows of 8 bf16
  // Staging.  With 16-byte rows, kStage rows per thread are loaded before any
  // is stored (indexes clamped to the last row), so their L2 latencies
  // overlap; other widths gather the experts one by one.
  constexpr int kStage = 8;
  const int n_rows = 8 * NQ * nvec;
  if (w_vec16) {  // E a multiple of 8 and W_r 16-byte aligned
    for (int base = 0; base < n_rows; base += kStage * kPermRouteThreads) {
      u32x4 v[kStage];
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int idx = min(base + u * kPermRouteThreads + (int)threadIdx.x, n_rows - 1);
        const int c = idx % nvec, pq = idx / nvec;  // pq = i * NQ + q
        v[u] = *(const u32x4*)(w_router + (size_t)(8 * c + pq / NQ) * E + 8 * (pq % NQ));
      }
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int idx = base + u * kPermRouteThreads + (int)threadIdx.x;
        if (idx < n_rows) w_lds[idx] = v[u];
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < n_rows; idx += kPermRouteThreads) {
      const int c = idx % nvec, pq = idx / nvec;
      const int h = 8 * c + pq / NQ, e0 = 8 * (pq % NQ);
      uint32_t lo[8];
#pragma unroll
      for (int ee = 0; ee < 8; ++ee)
        lo[ee] = e0 + ee < E ? w_router[(size_t)h * E + e0 + ee] : 0u;
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = lo[2 * q] | (lo[2 * q + 1] << 16);
      w_lds[idx] = v;
    }
  }
  __syncthreads();  // the only barrier: every wave reaches it before its token loop

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Lane l < K holds the token's l-th row and lane e < E its logit gradient;
  // the next token's are requested before this one's rows.
  const int stride = gridDim.x * kPermRouteWaves;
  int t = blockIdx.x * kPermRouteWaves + wave;
  int row_n = -1;
  float dl_n = 0.0f;
  if (t < T) {
    if (lane < K) row_n = row_of[(size_t)t * K + lane];
    if (lane < E) dl_n = d_logits[(size_t)t * E + lane];
  }
  for (; t < T; t += stride) {
    const int row = row_n;
    const float dlv = dl_n;
    if (t + stride < T) {
      if (lane < K) row_n = row_of[(size_t)(t + stride) * K + lane];
      if (lane < E) dl_n = d_logits[(size_t)(t + stride) * E + lane];
    }
    int rows[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rows[k] = __builtin_amdgcn_readlane(row, k);
    uint32_t dl2[4 * NQ];  // bf16(d_logits[t]) in expert pairs, zero past E
#pragma unroll
    for (int p = 0; p < 4 * NQ; ++p)
      dl2[p] = pack_bf16x2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(dlv), 2 * p)),
                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dlv), 2 * p + 1)));
    for (int c0 = 0; c0 < nvec; c0 += 64 * VPL) {
      // The first two slots' rows are requested first (zero where dropped);
      // the router term, which needs only LDS, runs while they are in flight.
      u32x4 v01[2][VPL];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) v01[k][j] = u32x4{0u, 0u, 0u, 0u};
        if (k < K && rows[k] >= 0) {
          const u32x4* src = d_xp + (size_t)rows[k] * nvec;
#pragma unroll
          for (int j = 0; j < VPL; ++j) {
            const int c = c0 + lane + 64 * j;
            if (c < nvec) v01[k][j] = src[c];
          }
        }
      }
      float acc[VPL][8];
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int c = min(c0 + lane + 64 * j, nvec - 1);  // columns past H are not stored
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc[j][i] = 0.0f;
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const u32x4 w = w_lds[(i * NQ + q) * nvec + c];
#pragma unroll
            for (int p = 0; p < 4; ++p) acc[j][i] = dot2_bf16(w[p], dl2[4 * q + p], acc[j][i]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int j = 0; j < VPL; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j][i] += vec_elem<true>(v01[k][j], i);
#pragma unroll
      for (int k = 2; k < 8; ++k) {
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
            for (int i = 0; i < 8; ++i) acc[j][i] += vec_elem<true>(v[j], i);
        }
      }
      if (d_x_shared) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nvec) {
            const u32x4 v = d_x_shared[(size_t)t * nvec + c];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] += vec_elem<true>(v, i);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c < nvec) dx[(size_t)t * nvec + c] = vec_pack<true>(acc[j]);
      }
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
                                                  a.counts, a.alpha, a.inv_tau, a.d_logits, a.T,
                                                  a.E, a.K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int chunk = route_bwd_chunk(a.E);
  const int nchunk = route_bwd_chunks(a.T, a.E);
  int e_ld = 0;  // partials [c][H][E] (0) or [c][e_ld][H] (MFMA form)
  if (route_bwd_uses_mfma(a.bf16, a.E)) {
    // d_w_router^T, chunk by chunk: a TN grouped GEMM whose segments are the
    // token chunks, A = d_l in bf16 padded to E8 experts [T][E8], B = x [T][H]
    const int E8 = (a.E + 7) & ~7;
    k_chunk_offsets<<<(nchunk + 256) / 256, 256, 0, st>>>(a.chunk_off, nchunk, chunk, a.T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_pad_bf16(a.d_logits, true, a.dl16, a.T, a.E, E8, st)) != hipSuccess) return e;
    GemmArgs g;
    g.layout = kGemmTN;
    g.epi = kEpiStore;
    g.A = a.dl16;
    g.B = a.x;
    g.C = a.part;
    g.offsets = a.chunk_off;
    g.G = nchunk;
    g.M = E8;
    g.N = a.H;
    if ((e = launch_grouped_gemm_bf16(g, st)) != hipSuccess) return e;
    e_ld = E8;
  } else {
    // expert groups of 8, 16 or 32 (the widest that E fills)
    const int EG = a.E <= 8 ? 8 : (a.E <= 16 ? 16 : 32);
    const dim3 grid((a.H + 511) / 512, nchunk, (a.E + EG - 1) / EG);
#define MOE_DW_PART(BF, EGV) \
  k_route_bwd_dw_part<BF, EGV><<<grid, 256, 0, st>>>(a.x, a.d_logits, a.part, a.T, a.H, a.E, chunk)
    if (a.bf16) {
      if (EG == 8) MOE_DW_PART(true, 8);
      else if (EG == 16) MOE_DW_PART(true, 16);
      else MOE_DW_PART(true, 32);
    } else {
      if (EG == 8) MOE_DW_PART(false, 8);
      else if (EG == 16) MOE_DW_PART(false, 16);
      else MOE_DW_PART(false, 32);
    }
#undef MOE_DW_PART
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.d_b_router) {
    const int ndb = (a.T + kDbBlock - 1) / kDbBlock;
    k_route_bwd_db_part<<<ndb, 256, 0, st>>>(a.d_logits, a.dbpart, a.T, a.E);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_route_bwd_db_reduce<<<a.E, 256, 0, st>>>(a.dbpart, a.d_b_router, ndb, a.E);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const size_t n = (size_t)a.H * a.E;
  k_route_bwd_reduce<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a.part, a.d_w_router, nchunk,
                                                                  a.H, a.E, e_ld);
  return hipGetLastError();
}

bool permute_bwd_fuses_route(bool bf16, int H, int E) {
  const int e8 = (E + 7) / 8 * 8;
  return bf16 && e8 <= 16 && (long long)H * e8 * 2 <= kPermuteRouteLds;
}

hipError_t launch_permute_bwd(const PermuteBwdArgs& a, hipStream_t st) {
  const int nvec = a.H * (a.bf16 ? 2 : 4) / 16;
  if (a.d_logits) {
    if (!permute_bwd_fuses_route(a.bf16, a.H, a.E) || !a.w_router) return hipErrorInvalidValue;
    const int nq = (a.E + 7) / 8;
    const size_t lds = (size_t)a.H * nq * 16;
    // two workgroups of eight waves per CU at 64 KiB of LDS each
    const int grid = std::min((a.T + kPermRouteWaves - 1) / kPermRouteWaves, 2 * 256);
    const int vec16 = a.E % 8 == 0 && ((uintptr_t)a.w_router & 15) == 0;
    if (nq == 1)
      k_permute_bwd_route<1, 4><<<grid, kPermRouteThreads, lds, st>>>(
          (const u32x4*)a.d_xp, a.row_of, (const u32x4*)a.d_x_shared, a.d_logits,
          (const uint16_t*)a.w_router, (u32x4*)a.dx, a.T, nvec, a.K, a.E, vec16);
    else
      k_permute_bwd_route<2, 4><<<grid, kPermRouteThreads, lds, st>>>(
          (const u32x4*)a.d_xp, a.row_of, (const u32x4*)a.d_x_shared, a.d_logits,
          (const uint16_t*)a.w_router, (u32x4*)a.dx, a.T, nvec, a.K, a.E, vec16);
    return hipGetLastError();
  }
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
