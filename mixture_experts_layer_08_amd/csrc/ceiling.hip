// A measurement aid, not a step of the layer: the MFMA-only rate of the
// grouped GEMM's inner loop on this chip, the ceiling its roofline fraction
// is read against.
//
// Why: on MI355X a GEMM's MFMA rate is bounded below the nominal dense peak
// by the clock the chip holds under sustained MFMA load.  This kernel runs
// the four-wave GEMM kernel's MFMA pattern (one wave per SIMD, 8 x 8 tiles
// of v_mfma_f32_16x16x32_bf16, 256 fp32 accumulators per lane in AGPRs) with
// no memory traffic at all: consecutive MFMAs take different operand pairs
// from 8 A and 8 B fragments of random data held in registers, so the
// operand bits switch at every instruction, as they do on real data.
//
// Operands: 16 fragments of 64 lanes x 8 bf16 (fragments 0-7 A_0..A_7,
// 8-15 B_0..B_7); lane l of a fragment supplies row l % 16, k = 8 (l / 16)
// .. +7 of a 16 x 32 matrix.  Every wave of every workgroup loads the same
// fragments and then runs `iters` rounds t = 0 .. iters-1 of acc[i][j] +=
// B_j(t) A_i(t)^T (as the GEMM, with the B fragment as the MFMA's first
// operand).  Modes:
//   0  the given operands in every round;
//   1  two register sets alternate: the given operands in even rounds, those
//      with every bf16 sign and mantissa bit flipped (each 32-bit word XORed
//      with 0x807f807f) in odd rounds, so that every operand register
//      switches half its bits from one round to the next with no extra
//      instruction in the loop;
//   2  the given operands, XORed before every round with a zero word passed
//      in at run time: one VALU instruction per MFMA and no bit switch, the
//      cost of such instructions in the MFMA stream.
//   3  the eight-wave kernel's MFMA shape instead: 4 x 4 tiles of
//      v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane), fragments
//      0-3 as A_0..A_3 and 8-11 as B_0..B_3 of 32 x 16 matrices (lane l:
//      row l % 32, k = 8 (l / 32) .. +7), each round running the 16 MFMAs
//      twice on the same operands, so that a round does the FLOPs of the
//      other modes' rounds.
// Output (modes 0-2): each lane writes the four sums over i, j of its
// accumulator elements, which are rows 4 (l / 16) + r, column l % 16 of
// sum_t sum_{i,j} B_j(t) A_i(t)^T.  Mode 3: sixteen sums per lane, rows
// 8 (r / 4) + 4 (l / 32) + r % 4 (r = 0..15), column l % 32 of
// 2 sum_t sum_{i,j} B_j A_i^T.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// one round of the 8 x 8 tile: acc[i][j] += B_j A_i^T (FIRST: acc[i][j] =
// B_j A_i^T, the accumulators' first write)
template <bool FIRST = false>
__device__ __forceinline__ void mfma_round(f32x4 (&acc)[8][8], const u32x4 (&a)[8],
                                           const u32x4 (&b)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, b[j]), __builtin_bit_cast(bf16x8, a[i]),
          FIRST ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void k_mfma_ceiling(const bf16x8* __restrict__ operands,
                                                         float* __restrict__ out, int iters,
                                                         uint32_t zero) {
  const int lane = threadIdx.x & 63;
  // operands kept as 32-bit words, handed to the MFMA as bf16x8
  u32x4 a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    a[f] = __builtin_bit_cast(u32x4, operands[f * 64 + lane]);
    b[f] = __builtin_bit_cast(u32x4, operands[(8 + f) * 64 + lane]);
  }
  f32x4 acc[8][8];
  mfma_round<true>(acc, a, b);  // round 0: the given operands in every mode
  if (MODE == 1) {
    u32x4 af[8], bf[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      af[f] = a[f] ^ 0x807f807fu;
      bf[f] = b[f] ^ 0x807f807fu;
    }
    int t = 1;
    for (; t + 1 < iters; t += 2) {
      mfma_round(acc, af, bf);
      mfma_round(acc, a, b);
    }
    if (t < iters) mfma_round(acc, af, bf);
  } else {
    for (int t = 1; t < iters; ++t) {
      if (MODE == 2) {
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          a[f] ^= zero;
          b[f] ^= zero;
        }
      }
      mfma_round(acc, a, b);
    }
  }
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[i][j];
  *(f32x4*)(out + ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4) = s;
}

// Mode 3: the 32 x 32 x 16 shape, 4 x 4 tiles (see the header).
__global__ __launch_bounds__(256, 1) void k_mfma_ceiling32(const bf16x8* __restrict__ operands,
                                                           float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  u32x4 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    a[f] = __builtin_bit_cast(u32x4, operands[f * 64 + lane]);
    b[f] = __builtin_bit_cast(u32x4, operands[(8 + f) * 64 + lane]);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, b[j]), __builtin_bit_cast(bf16x8, a[i]), f32x16{}, 0, 0, 0);
  for (int t = 0; t < 2 * iters - 1; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, b[j]), __builtin_bit_cast(bf16x8, a[i]), acc[i][j], 0, 0,
            0);
  }
  f32x16 s = f32x16{};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j];
  float* o = out + ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 16;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(f32x4*)(o + 4 * q) = f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
}

}  // namespace

hipError_t launch_mfma_ceiling(const void* operands, float* out, int workgroups, int iters,
                               int mode, hipStream_t st) {
  const bf16x8* ops = (const bf16x8*)operands;
  if (mode == 3)
    k_mfma_ceiling32<<<workgroups, 256, 0, st>>>(ops, out, iters);
  else if (mode == 1)
    k_mfma_ceiling<1><<<workgroups, 256, 0, st>>>(ops, out, iters, 0u);
  else if (mode == 2)
    k_mfma_ceiling<2><<<workgroups, 256, 0, st>>>(ops, out, iters, 0u);
  else
    k_mfma_ceiling<0><<<workgroups, 256, 0, st>>>(ops, out, iters, 0u);
  return hipGetLastError();
}

}  // namespace moe
