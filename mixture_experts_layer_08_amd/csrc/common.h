// Shared device helpers of the gfx950 MoE kernels: vector types, bf16
// conversion, wave-level scans.  Wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace moe {

// Host side: a kernel that takes more than 64 KiB of dynamic LDS must be
// allowed to, per device (the attribute belongs to the device's copy of the
// kernel).  allow_dynamic_lds<kernel>() raises the kernel's cap to the
// device's LDS per workgroup (160 KiB on gfx950) less the kernel's static
// LDS, the first time it runs on each of the first 64 devices (every time on
// others).  Concurrent first calls both set the same value.  With kNoScratch
// it also refuses (hipErrorInvalidDeviceFunction) a kernel whose code object
// uses scratch memory: kernels that order their LDS ring with hand-counted
// vmcnt waits would count a spill's scratch loads and stores too.
template <auto kKernel, bool kNoScratch = false>
hipError_t allow_dynamic_lds() {
  static std::atomic<unsigned long long> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  int lds_per_block = 0;
  e = hipDeviceGetAttribute(&lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  hipFuncAttributes fa;
  e = hipFuncGetAttributes(&fa, (const void*)kKernel);
  if (e != hipSuccess) return e;
  if (kNoScratch && fa.localSizeBytes != 0) return hipErrorInvalidDeviceFunction;
  e = hipFuncSetAttribute((const void*)kKernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          lds_per_block - (int)fa.sharedSizeBytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16 f32_to_bf16(float f) { return static_cast<bf16>(f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16 a = f32_to_bf16(lo), b = f32_to_bf16(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// GELU, tanh form: 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3).
// Since 0.5 (1 + tanh(z)) = 1 / (1 + exp(-2z)), this is u / (1 + exp(-2z)),
// evaluated with the hardware base-2 exponential: exp(-2z) = 2^(-2z log2 e).
// For u -> -inf the exponential overflows to +inf and the quotient is -0,
// the limit; for u -> +inf it is u.
__device__ __forceinline__ float gelu_tanh_f32(float u) {
  const float kC = 0.7978845608028654f;           // sqrt(2/pi)
  const float kNeg2Log2e = -2.8853900817779268f;   // -2 / ln 2
  float z = kC * fmaf(0.044715f * u, u * u, u);
  float e = __builtin_amdgcn_exp2f(kNeg2Log2e * z);
  return u * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace moe
