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
// each wave owns 16 tokens and all experts.  Its x rows stream from HBM
// straight into the A operand through a ring of register slots, loads issued
// R-1 MFMA steps ahead so that every wave keeps ~16-32 KiB in flight.  The
// router weight W_r [H][E] is staged in LDS as it lies in memory, chunk by
// chunk ([k][E_pad + 16] rows; a chunk of k rows is one contiguous span of
// W_r), once per workgroup, double-buffered, and read from there as the B
// operand by all four waves with transposing LDS reads (ds_read_b64_tr_b16),
// which hand each lane 8 consecutive k of one expert.  fp32 mode uses plain
// FMA.
//
// The epilogue works on the block's fp32 logits in LDS:
//   - four lanes per token select the top-k (K rounds of a 4-lane argmax;
//     larger logit first, the lower expert index on equal logits), and
//     compute the softmax and the renormalised weights;
//   - each token ORs its bit into a 64-bit mask per chosen expert, so the
//     in-block rank of (t, e) is the popcount of e's mask below bit t and
//     the block histogram is the popcount of the whole mask (OR is
//     order-independent: the result is deterministic);
//   - one thread per expert sums the block's probabilities in token order.
#include "common.h"
#include "kernels.h"

namespace moe {

// Shared epilogue.  s_logit holds the block's fp32 logits, row stride ES.
// Called by all 256 threads after a barrier that published s_logit.  s_ids
// is [kRouteBlock][8], s_mask [E] (scratch).
// Philox4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): each round multiplies words 0 and 2
// by the Philox multipliers, mixes the halves with words 1, 3 and the key,
// then bumps the key by the two Weyl constants.
__device__ __forceinline__ void philox4x64_10(unsigned long long (&c)[4], unsigned long long k0,
                                              unsigned long long k1) {
  const unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const unsigned long long W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const unsigned long long hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const unsigned long long n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// The noisy router of section 3.1 of the dpshk.com "MoE module infra notes":
// selection scores z = (l + g) / tau with Gumbel noise g = -log(-log(U + 1e-9)
// + 1e-9).  U[t, e] is word e % 4 of the Philox block with counter
// (t, e / 4, offset, 0) and key (seed, 0), as (word >> 40) * 2^-24 (24 bits,
// on [0, 1)).  Applied in place to a block's logits tile in LDS (ES floats
// per token row), before selection.
__device__ void route_noise(float* s_logit, int ES, int t0, int nt, int E,
                            const RouterNoise& nz) {
  const int nq = (E + 3) >> 2;
  for (int i = threadIdx.x; i < nt * nq; i += blockDim.x) {
    const int t = i / nq, q = i - t * nq;
    float g[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (nz.gumbel) {
      unsigned long long c[4] = {(unsigned long long)(t0 + t), (unsigned long long)q, nz.offset,
                                 0ull};
      philox4x64_10(c, nz.seed, 0ull);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float u = (float)(uint32_t)(c[j] >> 40) * 0x1p-24f;
        g[j] = -logf(-logf(u + 1e-9f) + 1e-9f);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * q + j;
      if (e < E) {
        float* v = s_logit + t * ES + e;
        *v = (*v + g[j]) / nz.tau;
      }
    }
  }
  __syncthreads();
}

__device__ void route_epilogue(float* s_logit, int ES, int32_t* s_ids,
                               unsigned long long* s_mask, int t0, int nt, int E, int K,
                               int nblk, float* __restrict__ logits_out,
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
  for (int e = tid; e < E; e += blockDim.x) s_mask[e] = 0ull;
  __syncthreads();

  // ---- top-k, softmax, weights: lanes 4t .. 4t+3 handle token t ----
  const int tok = tid >> 2, sub = tid & 3;  // the 4 lanes of a token are adjacent
  float* L = s_logit + tok * ES;
  const bool tok_ok = tok < nt;  // uniform over the 4 lanes of a token
  float bv[8];
  int bi[8];
  unsigned long long taken = 0;  // bit i: expert sub + 4i already chosen
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bv[j] = -INFINITY;
    bi[j] = 0;
    if (j < K) {
      float v = -INFINITY;
      int ie = 0x7fffffff;
      if (tok_ok) {
        int i = 0;
        for (int e = sub; e < E; e += 4, ++i) {
          const float x = L[e];
          // strict compare in increasing e: the lower index wins a tie
          if (!((taken >> i) & 1ull) && (x > v || ie == 0x7fffffff)) {
            v = x;
            ie = e;
          }
        }
      }
#pragma unroll
      for (int d = 1; d <= 2; d <<= 1) {
        const float ov = __shfl_xor(v, d, kWave);
        const int oe = __shfl_xor(ie, d, kWave);
        if (ov > v || (ov == v && oe < ie)) {
          v = ov;
          ie = oe;
        }
      }
      bv[j] = v;
      bi[j] = ie;
      if (tok_ok && (ie & 3) == sub) taken |= 1ull << (ie >> 2);
    }
  }
  if (tok_ok) {
    const float m = bv[0];
    float s = 0.0f;
    for (int e = sub; e < E; e += 4) s += __expf(L[e] - m);
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    const float inv = 1.0f / s;
    for (int e = sub; e < E; e += 4) L[e] = __expf(L[e] - m) * inv;  // probabilities
    if (sub == 0) {
      float zsel[8];
      float zs = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        zsel[j] = j < K ? __expf(bv[j] - m) : 0.0f;
        zs += zsel[j];
      }
      const size_t t = (size_t)(t0 + tok);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          topk_ids[t * K + j] = bi[j];
          topk_w[t * K + j] = zsel[j] / zs;
          s_ids[tok * 8 + j] = bi[j];
          atomicOr(&s_mask[bi[j]], 1ull << tok);
        }
      }
    }
  }
  __syncthreads();

  // ---- per-block results for the aux loss and the permutation ----
  const int blk = blockIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    float ps = 0.0f;
    for (int t = 0; t < nt; ++t) ps += s_logit[t * ES + e];
    psum[(size_t)e * nblk + blk] = ps;
    hist[(size_t)e * nblk + blk] = __popcll(s_mask[e]);
  }
  for (int i = tid; i < nt * K; i += blockDim.x) {
    const int t = i / K, j = i - t * K;
    const unsigned long long below = (1ull << t) - 1ull;
    lrank[(size_t)(t0 + t) * K + j] = __popcll(s_mask[s_ids[t * 8 + j]] & below);
  }
}

// k per staged weight chunk (16 KiB of bf16 weights per chunk, at most 512)
// and the x ring depth in MFMA steps (a multiple of the steps per chunk).
template <int CT>
constexpr int route_kc() { return 8192 / (16 * CT) < 512 ? 8192 / (16 * CT) : 512; }
template <int CT>
constexpr int route_ring() { return CT <= 4 ? 32 : 16; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Two ds_read_b64_tr_b16 (LDS byte addresses addr and addr_hi) as one
// 8-value fragment.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(uint32_t addr, uint32_t addr_hi) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr_hi);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Buffer-descriptor word 3 for raw 32-bit-indexed loads, and an offset past
// any descriptor size used here (reads as zero).
constexpr int kBufferFormat = 0x00020000;
constexpr uint32_t kOffsetOob = 0x80000000u;

template <int CT>
__global__ __launch_bounds__(256) void k_route_bf16(
    const bf16* __restrict__ x, const bf16* __restrict__ w_r, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, float* __restrict__ psum, int32_t* __restrict__ lrank, int T,
    int H, int E, int K, int nblk, RouterNoise nz) {
  extern __shared__ __attribute__((aligned(16))) float s_logit[];
  __shared__ int32_t s_ids[kRouteBlock * 8];
  __shared__ unsigned long long s_mask[256];
  constexpr int EP = 16 * CT;            // padded experts (columns of a weight buffer)
  constexpr int KC = route_kc<CT>();     // k per weight chunk (rows of a buffer)
  constexpr int SPC = KC / 32;           // MFMA steps per chunk
  constexpr int EPS = EP + 16;           // LDS row stride (elements): 32-byte pad
  constexpr int WBUF = KC * EPS;         // elements per weight buffer
  constexpr int WVEC = EP * KC / 8;      // 16-byte vectors per chunk, at most
  constexpr int WPT = WVEC / 256;        // per thread
  constexpr int R = route_ring<CT>();    // x ring slots (MFMA steps in flight)
  static_assert(WVEC % 256 == 0 && R % SPC == 0, "route tiling");
  bf16* wbuf = (bf16*)s_logit;           // two weight buffers; later the logits tile

  const int ES = E | 1;
  const int t0 = blockIdx.x * kRouteBlock;
  const int nt = min(kRouteBlock, T - t0);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int kg = (lane >> 4) * 8;
  const int nsteps = (H + 31) / 32;
  const int nchunks = (H + KC - 1) / KC;
  const int ngroups = (nsteps + R - 1) / R;

  // All loads are buffer loads with no branch around them (a divergent
  // branch would make the compiler wait for every load in flight): the
  // descriptor's size bounds the rows (rows past T read as zero), and an
  // offset past the size zeroes k past H.
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * H), (short)0, nt * H * 2, kBufferFormat);
  const uint32_t xoff = (uint32_t)((wave * 16 + (lane & 15)) * H + kg) * 2;
  // Each workgroup walks the K range in its own rotated order: the chunks
  // start at chunk rc, and the steps inside every chunk at step ri.
  // Workgroups running side by side then read different column offsets of
  // their rows, rather than all hitting the same offsets of rows one route
  // block apart at once (measured: the route call after a combine at
  // T=32768, H=4096, E=8 went from 89 to 82 us).  The sum over k is taken
  // in a per-workgroup order, so logits differ from the plain order by
  // rounding only.
  const int rot = (int)((blockIdx.x * 37u) % (unsigned)(nchunks * SPC));
  const int rc = rot / SPC, ri = rot % SPC;
  auto kstep = [&](int s) {  // sequence step -> K-step (SPC is a power of two)
    const int c = s / SPC;
    return ((c + rc) % nchunks) * SPC + (((s % SPC) + ri) & (SPC - 1));
  };
  auto xload = [&](int s) -> bf16x8 {
    const int ks = kstep(s);
    const uint32_t off =
        s < nchunks * SPC && ks * 32 + kg < H ? xoff + (uint32_t)ks * 64 : kOffsetOob;
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
  };
  // Weight chunk c covers k rows [kc0, kc0 + kn) of W_r, kc0 the chunk's
  // first k in this workgroup's rotated order: elements kc0 E .. (kc0 + kn) E
  // of W_r, contiguous (kn E is a multiple of 8 and the span starts 16-byte
  // aligned).  Thread vectors v = tid + 256 q hold elements 8v .. 8v+7 of the
  // span, which wstore puts at row k - kc0, column e of the buffer: one
  // 16-byte write when E is a multiple of 8 (the 8 values are one row's),
  // else value by value.  Columns E .. EPS-1 only feed logits that are never
  // stored.  Rows past kn keep the weights of an earlier chunk, or the zeros
  // both buffers start with: finite values that multiply zero columns of x
  // (an offset past H reads as zero), so they add nothing.
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)w_r, (short)0, H * E * 2, kBufferFormat);
  u32x4 wreg[WPT];
  auto chunk_k0 = [&](int c) { return ((c + rc) % nchunks) * KC; };
  auto wload = [&](int c) {
    const int n = min(KC, H - chunk_k0(c)) * E;  // elements in the span
    const uint32_t span = (uint32_t)chunk_k0(c) * E * 2;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int v = tid + 256 * q;
      const uint32_t off = 8 * v < n ? span + (uint32_t)v * 16 : kOffsetOob;
      wreg[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
    }
  };
  const bool e_vec = (E & 7) == 0;
  auto wstore = [&](int buf, int c) {
    const int n = min(KC, H - chunk_k0(c)) * E;
    bf16* wb = wbuf + buf * WBUF;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int f = 8 * (tid + 256 * q);
      if (f < n) {
        int k = f / E, e = f - k * E;
        if (e_vec) {
          *(u32x4*)(wb + k * EPS + e) = wreg[q];
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t w = wreg[q][i >> 1];
            wb[k * EPS + e] = __builtin_bit_cast(bf16, (uint16_t)(i & 1 ? w >> 16 : w & 0xffffu));
            if (++e == E) {
              e = 0;
              ++k;
            }
          }
        }
      }
    }
  };
  // zero both buffers once: no stale LDS bits (possibly NaN) in rows past kn
  for (int i = tid; i < 2 * WBUF / 8; i += 256) *(u32x4*)(wbuf + 8 * i) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  f32x4 acc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 ring[R];
  wload(0);
  wstore(0, 0);
#pragma unroll
  for (int i = 0; i < R - 1; ++i) ring[i] = xload(i);
  if (nchunks > 1) wload(1);
  __syncthreads();
  // B fragment of tile ct at step s_in of a chunk: expert ct*16 + lane%16,
  // 8 k from s_in*32 + 8*(lane/16), by two transposing reads.  In each
  // 16-lane group, lane i gives the address of 4 consecutive experts
  // (columns ct*16 + 4 (i%4) ..) of row k0 + i/4 and receives column
  // ct*16 + i of that 4 x 16 block: 4 consecutive k; the second read takes
  // rows k0 + 4 ...  The 32-byte row pad puts the 4 rows of a read in
  // distinct banks.
  const int b_off = (kg + ((lane & 15) >> 2)) * EPS + 4 * (lane & 3);
  // Whole groups of R steps: steps past the last one multiply zero rows of x.
  for (int g = 0; g < ngroups; ++g) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int s = g * R + i;
      ring[(i + R - 1) % R] = xload(s + R - 1);
      const int c = s / SPC;
      // steps past the last chunk read the last chunk's buffer (finite
      // weights times zero rows of x): the other buffer may never have been
      // written, and stale LDS bits could be NaN
      const bf16* wb = wbuf + (min(c, nchunks - 1) & 1) * WBUF +
                       (((i % SPC) + ri) & (SPC - 1)) * 32 * EPS + b_off;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const uint32_t a0 = (uint32_t)(uintptr_t)(wb + ct * 16);
        const bf16x8 b = lds_read_tr_pair(a0, a0 + 4 * EPS * 2);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[i], b, acc[ct], 0, 0, 0);
      }
      if ((i + 1) % SPC == 0 && c + 1 < nchunks) {  // uniform over the workgroup
        // chunk c done: publish chunk c+1 into the other buffer, whose last
        // reads (chunk c-1) every wave finished before the previous barrier
        wstore((c + 1) & 1, c + 1);
        __syncthreads();
        if (c + 2 < nchunks) wload(c + 2);
      }
    }
  }
  __syncthreads();  // every wave is done with the weight buffers
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
  if (nz.active) route_noise(s_logit, ES, t0, nt, E, nz);
  route_epilogue(s_logit, ES, s_ids, s_mask, t0, nt, E, K, nblk, logits, topk_ids, topk_w,
                 hist, psum, lrank);
}

__global__ __launch_bounds__(256) void k_route_f32(
    const float* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, float* __restrict__ psum, int32_t* __restrict__ lrank, int T,
    int H, int E, int K, int nblk, RouterNoise nz) {
  extern __shared__ float s_logit[];
  __shared__ int32_t s_ids[kRouteBlock * 8];
  __shared__ unsigned long long s_mask[256];
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
  if (nz.active) route_noise(s_logit, ES, t0, nt, E, nz);
  route_epilogue(s_logit, ES, s_ids, s_mask, t0, nt, E, K, nblk, logits, topk_ids, topk_w,
                 hist, psum, lrank);
}

// Routing from caller-given fp32 logits (no GEMM, logits not rewritten).
__global__ __launch_bounds__(256) void k_route_from_logits(
    const float* __restrict__ logits, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ psum,
    int32_t* __restrict__ lrank, int T, int E, int K, int nblk) {
  extern __shared__ float s_logit[];
  __shared__ int32_t s_ids[kRouteBlock * 8];
  __shared__ unsigned long long s_mask[256];
  const int ES = E | 1;
  const int t0 = blockIdx.x * kRouteBlock;
  const int nt = min(kRouteBlock, T - t0);
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x) {
    const int t = i / E, e = i - t * E;
    s_logit[t * ES + e] = logits[(size_t)(t0 + t) * E + e];
  }
  __syncthreads();
  route_epilogue(s_logit, ES, s_ids, s_mask, t0, nt, E, K, nblk, nullptr, topk_ids, topk_w,
                 hist, psum, lrank);
}

// Number of non-finite values among n fp32 values, by one workgroup of 1024
// threads in a fixed order (64-bit counts, exact and deterministic).
__global__ __launch_bounds__(1024) void k_count_nonfinite(const float* __restrict__ v, size_t n,
                                                          long long* __restrict__ count) {
  __shared__ long long s_part[16];
  long long c = 0;
  for (size_t i = threadIdx.x; i < n; i += 1024) c += isfinite(v[i]) ? 0 : 1;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, kWave);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long t = 0;
    for (int w = 0; w < 16; ++w) t += s_part[w];
    *count = t;
  }
}

hipError_t launch_count_nonfinite(const float* v, size_t n, long long* count, hipStream_t st) {
  k_count_nonfinite<<<1, 1024, 0, st>>>(v, n, count);
  return hipGetLastError();
}

size_t route_lds_bytes(int E) { return (size_t)kRouteBlock * (E | 1) * sizeof(float); }

// bf16 router: the two weight buffers or the fp32 logits tile, whichever is
// larger (they share the space).
template <int CT>
static size_t route_bf16_lds_bytes(int E) {
  const size_t wbufs = 2 * (size_t)route_kc<CT>() * (16 * CT + 16) * 2;
  return std::max(wbufs, route_lds_bytes(E));
}

// Column tiles of 16 experts for the bf16 router: a power of two from 1 to 16
// (weight rows beyond E are zero and their logits are never stored).
int route_col_tiles(int E) {
  const int ct = (E + 15) / 16;
  return ct <= 1 ? 1 : ct <= 2 ? 2 : ct <= 4 ? 4 : ct <= 8 ? 8 : 16;
}

template <int CT>
static hipError_t launch_route_bf16(const RouteArgs& a, int nblk, hipStream_t st) {
  const size_t lds = route_bf16_lds_bytes<CT>(a.E);
  if (lds > 65536) {
    const hipError_t err = allow_dynamic_lds<k_route_bf16<CT>>();
    if (err != hipSuccess) return err;
  }
  k_route_bf16<CT><<<nblk, 256, lds, st>>>((const bf16*)a.x, (const bf16*)a.w_r, a.bias, a.logits,
                                           a.topk_ids, a.topk_w, a.hist, a.psum, a.lrank, a.T,
                                           a.H, a.E, a.K, nblk, a.noise);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const int nblk = (a.T + kRouteBlock - 1) / kRouteBlock;
  const size_t lds = route_lds_bytes(a.E);
  hipError_t err;
  if (a.logits_in) {
    if (lds > 65536 && (err = allow_dynamic_lds<k_route_from_logits>()) != hipSuccess) return err;
    k_route_from_logits<<<nblk, 256, lds, st>>>(a.logits, a.topk_ids, a.topk_w, a.hist, a.psum,
                                                a.lrank, a.T, a.E, a.K, nblk);
    return hipGetLastError();
  }
  if (!a.bf16) {
    if (lds > 65536 && (err = allow_dynamic_lds<k_route_f32>()) != hipSuccess) return err;
    k_route_f32<<<nblk, 256, lds, st>>>((const float*)a.x, (const float*)a.w_r, a.bias,
                                        a.logits, a.topk_ids, a.topk_w, a.hist, a.psum,
                                        a.lrank, a.T, a.H, a.E, a.K, nblk, a.noise);
    return hipGetLastError();
  }
  switch (route_col_tiles(a.E)) {
    case 1: return launch_route_bf16<1>(a, nblk, st);
    case 2: return launch_route_bf16<2>(a, nblk, st);
    case 4: return launch_route_bf16<4>(a, nblk, st);
    case 8: return launch_route_bf16<8>(a, nblk, st);
    case 16: return launch_route_bf16<16>(a, nblk, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
