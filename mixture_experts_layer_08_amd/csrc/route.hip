// Router: logits = x W_r (+ b), softmax over experts, top-k on the logits,
// renormalised weights, and per-block partial results for the aux loss and
// the permutation.
//
// Method: router of the dpshk.com "MoE module infra notes", section 3.1
// (softmax, top-k, renormalise) with the noise-free inference selection of
// section 5.2 tip 4 (top-k on logits); gate linear of the section 4.2 listing.
//
// One workgroup of 256 threads handles a route block of kRouteBlock = 64
// tokens.  bf16 mode runs the router GEMM on MFMA (v_mfma_f32_16x16x32_bf16):
// each wave owns 16 tokens and all experts, reading its x rows straight from
// HBM into the A operand (16 contiguous bytes per lane) and the transposed
// router weight (wT [E_pad][H], L2-resident) as the B operand.  fp32 mode
// uses plain FMA.  The epilogue puts the block's logits in LDS, then
//   - one thread per token selects the top-k, computes softmax and weights;
//   - one thread per expert sums the block's probabilities (fixed token
//     order) and ranks the block's assignments to it in token order.
#include "common.h"
#include "kernels.h"

namespace moe {

// wT[e][k] = W_r[k][e] for e < E, 0 for E <= e < E_pad.
__global__ __launch_bounds__(256) void k_transpose_router(const bf16* __restrict__ w_r,
                                                          bf16* __restrict__ wT, int H, int E,
                                                          int E_pad) {
  const size_t n = (size_t)E_pad * H;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / H), k = (int)(i % H);
    wT[i] = e < E ? w_r[(size_t)k * E + e] : f32_to_bf16(0.0f);
  }
}

// Shared epilogue.  s_logit holds the block's fp32 logits, row stride ES.
// Called by all 256 threads after a barrier that published s_logit.
__device__ void route_epilogue(float* s_logit, int ES, int32_t* s_ids, int t0, int nt,
                               int E, int K, int nblk, float* __restrict__ logits_out,
                               int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                               int32_t* __restrict__ hist, float* __restrict__ psum,
                               int32_t* __restrict__ lrank) {
  const int tid = threadIdx.x;
  if (logits_out) {
    for (int i = tid; i < nt * E; i += blockDim.x) {
      const int t = i / E, e = i - t * E;
      logits_out[(size_t)(t0 + t) * E + e] = s_logit[t * ES + e];
    }
  }
  __syncthreads();
  if (tid < nt) {
    float* L = s_logit + tid * ES;
    // Descending top-8 by insertion; equal values keep the earlier (lower)
    // expert index first because the comparison is strict.
    float bv[8];
    int bi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { bv[j] = -INFINITY; bi[j] = 0; }
    for (int e = 0; e < E; ++e) {
      const float v = L[e];
#pragma unroll
      for (int j = 7; j > 0; --j) {
        const bool shift = v > bv[j - 1];
        const bool place = !shift && v > bv[j];
        const float nv = shift ? bv[j - 1] : (place ? v : bv[j]);
        const int ni = shift ? bi[j - 1] : (place ? e : bi[j]);
        bv[j] = nv;
        bi[j] = ni;
      }
      if (v > bv[0]) { bv[0] = v; bi[0] = e; }
    }
    const float m = bv[0];
    float s = 0.0f;
    for (int e = 0; e < E; ++e) {
      const float z = __expf(L[e] - m);
      L[e] = z;
      s += z;
    }
    const float inv = 1.0f / s;
    for (int e = 0; e < E; ++e) L[e] *= inv;   // probabilities, for the aux partial sums
    float zsel[8];
    float zs = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      zsel[j] = j < K ? __expf(bv[j] - m) : 0.0f;
      zs += zsel[j];
    }
    const size_t t = (size_t)(t0 + tid);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K) {
        topk_ids[t * K + j] = bi[j];
        topk_w[t * K + j] = zsel[j] / zs;
        s_ids[tid * K + j] = bi[j];
      }
    }
  }
  __syncthreads();
  const int blk = blockIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    float ps = 0.0f;
    int cnt = 0;
    for (int t = 0; t < nt; ++t) {
      ps += s_logit[t * ES + e];
      for (int j = 0; j < K; ++j) {
        if (s_ids[t * K + j] == e) lrank[(size_t)(t0 + t) * K + j] = cnt++;
      }
    }
    psum[(size_t)e * nblk + blk] = ps;
    hist[(size_t)e * nblk + blk] = cnt;
  }
}

template <int CT>
__global__ __launch_bounds__(256) void k_route_bf16(
    const bf16* __restrict__ x, const bf16* __restrict__ wT, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, float* __restrict__ psum, int32_t* __restrict__ lrank, int T,
    int H, int E, int K, int nblk) {
  extern __shared__ float s_logit[];
  __shared__ int32_t s_ids[kRouteBlock * 8];
  const int ES = E | 1;
  const int t0 = blockIdx.x * kRouteBlock;
  const int nt = min(kRouteBlock, T - t0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = t0 + wave * 16 + (lane & 15);
  const bool row_ok = row < T;
  const int kg = (lane >> 4) * 8;
  const bf16* xr = x + (size_t)(row_ok ? row : 0) * H + kg;
  const bf16* wr = wT + (size_t)(lane & 15) * H + kg;
  f32x4 acc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero8 = {};
  int k = 0;
  // loads in flight per lane: enough bytes per wave to cover HBM latency
  constexpr int U = CT <= 2 ? 16 : (CT <= 4 ? 8 : (CT <= 8 ? 4 : 2));
  for (; k + 32 * U <= H; k += 32 * U) {
    bf16x8 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      a[u] = row_ok ? *(const bf16x8*)(xr + k + 32 * u) : zero8;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const bf16x8 b = *(const bf16x8*)(wr + (size_t)c * 16 * H + k + 32 * u);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b, acc[c], 0, 0, 0);
      }
    }
  }
  for (; k < H; k += 32) {
    const bool kin = k + kg < H;
    const bf16x8 a = (row_ok && kin) ? *(const bf16x8*)(xr + k) : zero8;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const bf16x8 b = kin ? *(const bf16x8*)(wr + (size_t)c * 16 * H + k) : zero8;
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  // D layout of the 16x16 tile: lane holds rows 4*(lane/16)+i, column lane%16.
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int e = c * 16 + (lane & 15);
    if (e < E) {
      const float b = bias ? bias[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = wave * 16 + (lane >> 4) * 4 + i;
        s_logit[tl * ES + e] = acc[c][i] + b;
      }
    }
  }
  __syncthreads();
  route_epilogue(s_logit, ES, s_ids, t0, nt, E, K, nblk, logits, topk_ids, topk_w, hist, psum,
                 lrank);
}

__global__ __launch_bounds__(256) void k_route_f32(
    const float* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, float* __restrict__ psum, int32_t* __restrict__ lrank, int T,
    int H, int E, int K, int nblk) {
  extern __shared__ float s_logit[];
  __shared__ int32_t s_ids[kRouteBlock * 8];
  const int ES = E | 1;
  const int t0 = blockIdx.x * kRouteBlock;
  const int nt = min(kRouteBlock, T - t0);
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x) {
    const int t = i / E, e = i - t * E;
    const float* xr = x + (size_t)(t0 + t) * H;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) acc = fmaf(xr[h], w_r[(size_t)h * E + e], acc);
    s_logit[t * ES + e] = acc + (bias ? bias[e] : 0.0f);
  }
  __syncthreads();
  route_epilogue(s_logit, ES, s_ids, t0, nt, E, K, nblk, logits, topk_ids, topk_w, hist, psum,
                 lrank);
}

// Routing from caller-given fp32 logits (no GEMM, logits not rewritten).
__global__ __launch_bounds__(256) void k_route_from_logits(
    const float* __restrict__ logits, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ psum,
    int32_t* __restrict__ lrank, int T, int E, int K, int nblk) {
  extern __shared__ float s_logit[];
  __shared__ int32_t s_ids[kRouteBlock * 8];
  const int ES = E | 1;
  const int t0 = blockIdx.x * kRouteBlock;
  const int nt = min(kRouteBlock, T - t0);
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x) {
    const int t = i / E, e = i - t * E;
    s_logit[t * ES + e] = logits[(size_t)(t0 + t) * E + e];
  }
  __syncthreads();
  route_epilogue(s_logit, ES, s_ids, t0, nt, E, K, nblk, nullptr, topk_ids, topk_w, hist, psum,
                 lrank);
}

size_t route_lds_bytes(int E) { return (size_t)kRouteBlock * (E | 1) * sizeof(float); }

// Column tiles of 16 experts for the bf16 router: a power of two from 1 to 16
// (rows of wT beyond E are zero and their logits are never stored).
int route_col_tiles(int E) {
  const int ct = (E + 15) / 16;
  return ct <= 1 ? 1 : ct <= 2 ? 2 : ct <= 4 ? 4 : ct <= 8 ? 8 : 16;
}

// Dynamic LDS above 64 KiB (E > 248) must be allowed explicitly; gfx950 has
// 160 KiB of LDS per workgroup.
template <typename F>
static hipError_t allow_lds(F* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const int nblk = (a.T + kRouteBlock - 1) / kRouteBlock;
  const size_t lds = route_lds_bytes(a.E);
  hipError_t err;
  if (a.logits_in) {
    if ((err = allow_lds(k_route_from_logits, lds)) != hipSuccess) return err;
    k_route_from_logits<<<nblk, 256, lds, st>>>(a.logits, a.topk_ids, a.topk_w, a.hist, a.psum,
                                                a.lrank, a.T, a.E, a.K, nblk);
    return hipGetLastError();
  }
  if (!a.bf16) {
    if ((err = allow_lds(k_route_f32, lds)) != hipSuccess) return err;
    k_route_f32<<<nblk, 256, lds, st>>>((const float*)a.x, (const float*)a.w_r, a.bias,
                                        a.logits, a.topk_ids, a.topk_w, a.hist, a.psum,
                                        a.lrank, a.T, a.H, a.E, a.K, nblk);
    return hipGetLastError();
  }
  const int CTp = route_col_tiles(a.E);
  {
    const size_t n = (size_t)CTp * 16 * a.H;
    const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
    k_transpose_router<<<grid, 256, 0, st>>>((const bf16*)a.w_r, (bf16*)a.wT, a.H, a.E,
                                             CTp * 16);
  }
#define MOE_ROUTE_CASE(ct)                                                                  \
  case ct:                                                                                  \
    if ((err = allow_lds(k_route_bf16<ct>, lds)) != hipSuccess) return err;                 \
    k_route_bf16<ct><<<nblk, 256, lds, st>>>((const bf16*)a.x, (const bf16*)a.wT, a.bias,   \
                                             a.logits, a.topk_ids, a.topk_w, a.hist, a.psum, \
                                             a.lrank, a.T, a.H, a.E, a.K, nblk);             \
    break;
  switch (CTp) {
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

}  // namespace moe
