// MXFP8 helpers: OCP E4M3 elements in blocks of 32 that share one E8M0
// (power-of-two) scale, the MXFP8 format of the OCP Microscaling (MX)
// specification 1.0.  The compression step of the cf-1.com page "Dissecting
// the MoE communication bottleneck" (section 5.3) carries the dispatched and
// combined hidden states in FP8; the page fixes neither the FP8 variant nor
// the scaling, and this is the form gfx950's scaled MFMA consumes.
//
// Quantising a block of float32 values v[0..31]:
//   X = floor(log2 max|v|) - 8, clamped to [-127, 127] (-127 for an all-zero
//       block); 8 is the exponent of E4M3's largest finite value 448;
//   scale code = X + 127; element code = E4M3(v / 2^X), round to nearest
//   even, magnitudes past 448 saturating to 448.
// For a float32 amax with exponent field f (f = 0 for zero and subnormals),
// floor(log2 amax) = f - 127 whenever f >= 1, so the scale code is
// max(f - 8, 0); a subnormal amax lies below 2^-126 and clamps the same way.
//
// Scale layouts (byte tensors):
//   operand layout (the A and B operands of the MXFP8 grouped GEMM): for R
//     rows of Kd columns, [ceil(Kd / 128)][R][4]: byte (q, r, j) is the scale
//     of block 4q + j of row r (one 4-byte word per row per 128 columns);
//     bytes of blocks past Kd / 32 are never read;
//   row layout (what combine reads): [R][cols / 32].
#pragma once

#include "common.h"

namespace moe {

constexpr int kMxBlock = 32;

// operand-layout scale bytes of an R x Kd operand
__host__ __device__ inline size_t mx_operand_scale_bytes(long long R, long long Kd) {
  return (size_t)((Kd + 127) / 128) * (size_t)R * 4;
}
__host__ __device__ inline size_t mx_operand_scale_index(long long ld, long long r, long long blk) {
  return ((size_t)(blk >> 2) * (size_t)ld + (size_t)r) * 4 + (size_t)(blk & 3);
}

// Weight codes in panels: for a [G][N][K] operand (K the contraction), the
// 256 x 64-byte block of rows 256 t .. 256 t + 255 and columns 64 j .. 64 j + 63
// of slice g is one contiguous 16 KiB panel, panels ordered (g, t, j):
//   code (g, n, k) at ((g * T + n / 256) * (K / 64) + k / 64) * 16384
//                     + (n % 256) * 64 + k % 64,   T = ceil(N / 256).
// One K-step of a GEMM tile's B operand is then one panel.  Rows n >= N of a
// slice's last panel are padding.
constexpr int kMxPanelRows = 256, kMxPanelK = 64;
__host__ __device__ inline size_t mx_weight_code_bytes(long long G, long long K, long long N) {
  return (size_t)G * (size_t)((N + kMxPanelRows - 1) / kMxPanelRows) * kMxPanelRows * (size_t)K;
}
__host__ __device__ inline size_t mx_weight_code_offset(long long g, long long n, long long k,
                                                        long long K, long long N) {
  const long long T = (N + kMxPanelRows - 1) / kMxPanelRows;
  return (size_t)(((g * T + n / kMxPanelRows) * (K / kMxPanelK) + k / kMxPanelK) *
                      (kMxPanelRows * kMxPanelK) +
                  (n % kMxPanelRows) * kMxPanelK + k % kMxPanelK);
}

// Scale code of a block from its float32 absolute maximum.
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  const int f = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return (uint32_t)max(f - 8, 0);
}

// 2^-X for scale code c = X + 127 (exponent field 254 - c, always normal).
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// 2^X for scale code c (c = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float mx_scale_value(uint32_t code) {
  return code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);
}

// Four float32 values times `inv`, clamped to +-448, as four E4M3 codes
// (value i in byte i).  The hardware conversion rounds to nearest even and
// keeps the sign of zero; it does not saturate, hence the clamp.
__device__ __forceinline__ uint32_t mx_encode4(float v0, float v1, float v2, float v3, float inv) {
  const float kMax = 448.0f;
  v0 = __builtin_amdgcn_fmed3f(v0 * inv, -kMax, kMax);
  v1 = __builtin_amdgcn_fmed3f(v1 * inv, -kMax, kMax);
  v2 = __builtin_amdgcn_fmed3f(v2 * inv, -kMax, kMax);
  v3 = __builtin_amdgcn_fmed3f(v3 * inv, -kMax, kMax);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
  return (uint32_t)w;
}

// The four E4M3 codes of `w` as float32 values (exact).
__device__ __forceinline__ void mx_decode4(uint32_t w, float& v0, float& v1, float& v2,
                                           float& v3) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  v0 = lo[0];
  v1 = lo[1];
  v2 = hi[0];
  v3 = hi[1];
}

}  // namespace moe
