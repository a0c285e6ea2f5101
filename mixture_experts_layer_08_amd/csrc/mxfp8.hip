// MXFP8 weight quantisation and the MXFP8 combine.
//
// The compression step of section 5.3 of the cf-1.com page "Dissecting the
// MoE communication bottleneck": combine reads the expert outputs in FP8
// (half the bytes of bf16) and returns bf16 token rows; section 4.2 of the
// same page quantises expert weights.  Formats and scale layouts: mx.h.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {

// w [G][Kd][N] (bf16 or fp32, row-major) -> q: E4M3 codes of the transposed
// [G][N][Kd] weights in 256 x 64-byte panels (mx.h), and
// s [G][ceil(Kd/128)][N][4] block scales (operand layout with R = N): the
// blocks run along Kd, the contraction dimension of the expert GEMM.  One
// workgroup per (expert, 128-row slab of Kd, 64 columns): the tile is staged
// through LDS as fp32; thread (block b, column n) then quantises the 32
// values of its block and writes them as 32 contiguous code bytes.
template <bool BF16>
__global__ __launch_bounds__(256) void k_quantize_weight_mx8(const void* __restrict__ w,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ s, int Kd,
                                                             int N) {
  __shared__ float tile[128][65];
  const int nslab = (Kd + 127) / 128;
  const int ntile = (N + 63) / 64;
  const int g = blockIdx.x / (nslab * ntile);
  const int rem = blockIdx.x - g * nslab * ntile;
  const int slab = rem / ntile, n0 = (rem - slab * ntile) * 64;
  const int k0 = slab * 128;
  const int tid = threadIdx.x;
  const size_t wbase = (size_t)g * Kd * N;
  for (int idx = tid; idx < 128 * 64; idx += 256) {
    const int kk = idx >> 6, nn = idx & 63;
    float v = 0.0f;
    if (k0 + kk < Kd && n0 + nn < N) {
      const size_t at = wbase + (size_t)(k0 + kk) * N + n0 + nn;
      v = BF16 ? (float)((const bf16*)w)[at] : ((const float*)w)[at];
    }
    tile[kk][nn] = v;
  }
  __syncthreads();
  const int nn = tid & 63, b = tid >> 6;  // block b of the slab, column nn
  const int n = n0 + nn, kb = k0 + 32 * b;
  if (n >= N || kb >= Kd) return;  // no barrier follows
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(tile[32 * b + i][nn]));
  const uint32_t code = mx_scale_code(amax);
  const float inv = mx_inv_scale(code);
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c[i] = mx_encode4(tile[32 * b + 4 * i][nn], tile[32 * b + 4 * i + 1][nn],
                      tile[32 * b + 4 * i + 2][nn], tile[32 * b + 4 * i + 3][nn], inv);
  u32x4* dst = (u32x4*)(q + mx_weight_code_offset(g, n, kb, Kd, N));  // 32 bytes in one panel row
  dst[0] = u32x4{c[0], c[1], c[2], c[3]};
  dst[1] = u32x4{c[4], c[5], c[6], c[7]};
  s[(((size_t)g * nslab + slab) * N + n) * 4 + b] = (uint8_t)code;
}

hipError_t launch_quantize_weight_mx8(const void* w, bool bf16_in, int G, int Kd, int N,
                                      uint8_t* q, uint8_t* s, hipStream_t st) {
  const long long grid = (long long)G * ((Kd + 127) / 128) * ((N + 63) / 64);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16_in)
    k_quantize_weight_mx8<true><<<(unsigned)grid, 256, 0, st>>>(w, q, s, Kd, N);
  else
    k_quantize_weight_mx8<false><<<(unsigned)grid, 256, 0, st>>>(w, q, s, Kd, N);
  return hipGetLastError();
}

// One wave per token: y[t] = sum_{k kept} w[t,k] * deq(out[row_of[t,k]])
// (+ deq(shared[t])), accumulated in fp32 in slot order (fused multiply-add;
// the dequantised values are exact in fp32), rounded to bf16.  A lane takes
// 16 code bytes (half a block) per vector and its block's scale byte (row
// layout); each token row is written once as bf16.  Code loads and y stores
// are non-temporal, as in the bf16 combine (T=32768, H=4096, E=8: 119 ->
// 115 us, and the next router call 81 -> 63 us).
template <int VPL>
__global__ __launch_bounds__(256) void k_combine_mx8(const u32x4* __restrict__ out_q,
                                                     const uint8_t* __restrict__ out_s,
                                                     const int32_t* __restrict__ row_of,
                                                     const float* __restrict__ topk_w,
                                                     const u32x4* __restrict__ sh_q,
                                                     const uint8_t* __restrict__ sh_s,
                                                     u32x4* __restrict__ y, int T, int nvec,
                                                     int K) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barrier in this kernel
  const int lane = threadIdx.x & 63;
  const int nblk = nvec / 2;  // 32-value blocks per row
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
    float acc[VPL][16];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    auto add_row = [&](const u32x4* src, const uint8_t* ssrc, float wk, bool fma) {
      u32x4 v[VPL];
      uint32_t sc[VPL];
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c < nvec) {
          v[j] = __builtin_nontemporal_load(src + c);
          sc[j] = ssrc[c >> 1];
        }
      }
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c < nvec) {
          const float sv = mx_scale_value(sc[j]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float f0, f1, f2, f3;
            mx_decode4(v[j][q], f0, f1, f2, f3);
            const float d[4] = {f0 * sv, f1 * sv, f2 * sv, f3 * sv};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[j][4 * q + i] = fma ? fmaf(wk, d[i], acc[j][4 * q + i]) : acc[j][4 * q + i] + d[i];
          }
        }
      }
    };
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < K && rows[k] >= 0)
        add_row(out_q + (size_t)rows[k] * nvec, out_s + (size_t)rows[k] * nblk, ws[k], true);
    if (sh_q) add_row(sh_q + (size_t)t * nvec, sh_s + (size_t)t * nblk, 1.0f, false);
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c < nvec) {
        u32x4 o0, o1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o0[q] = pack_bf16x2(acc[j][2 * q], acc[j][2 * q + 1]);
          o1[q] = pack_bf16x2(acc[j][8 + 2 * q], acc[j][8 + 2 * q + 1]);
        }
        __builtin_nontemporal_store(o0, y + (size_t)t * 2 * nvec + 2 * c);
        __builtin_nontemporal_store(o1, y + (size_t)t * 2 * nvec + 2 * c + 1);
      }
    }
  }
}

hipError_t launch_combine_mx8(const CombineMx8Args& a, hipStream_t st) {
  const int nvec = a.H / 16;  // 16-code vectors per row
  const int grid = (a.T + 3) / 4;
  k_combine_mx8<4><<<grid, 256, 0, st>>>((const u32x4*)a.out_q, a.out_s, a.row_of, a.topk_w,
                                         (const u32x4*)a.sh_q, a.sh_s, (u32x4*)a.y, a.T, nvec,
                                         a.K);
  return hipGetLastError();
}

}  // namespace moe
