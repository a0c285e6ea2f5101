// Grouped GEMM over variable-length expert segments:
//   C[r, :] = act(A[r, :] * B[g])   for every row r of segment g,
// with segment g the rows [offsets[g], offsets[g+1]) of the packed buffer.
//
// Method: the per-expert contractions of the MoELayer listing of the
// dpshk.com "MoE module infra notes" (section 4.2: x W1 -> GELU -> W2 over
// stacked expert weights), run as one grouped GEMM as section 5.1 of the
// cf-1.com page "Dissecting the MoE communication bottleneck" recommends
// (many thin per-expert GEMMs in one kernel).
//
// bf16 kernel (gfx950 MFMA):
//   - workgroup tile BM x BN x BK = 128 x 128 x 64, 256 threads = 4 waves in
//     a 2 x 2 grid, each wave a 64 x 64 tile of 2 x 2 v_mfma_f32_32x32x16_bf16;
//   - A (rows x K, K contiguous) is copied to LDS as [row][k];
//   - B (K x N, N contiguous, the ABI weight layout) is read in 8(k) x 4(n)
//     blocks, transposed in registers with v_perm_b32 and stored to LDS as
//     [n][k], so both MFMA operands are one 16-byte LDS read per lane;
//   - both LDS tiles swizzle their 16-byte chunks (chunk ^ (row & 7)) so a
//     wave's 32 row reads spread over all banks;
//   - two LDS buffers: the global loads of step k+1 are in flight while the
//     MFMAs of step k run, one barrier per step;
//   - epilogue: optional GELU(tanh) in fp32, round to bf16, staged through
//     LDS and written as 16-byte row vectors.
//   - tile order: blocks of 8 M-tiles sweep the N-tiles column by column so
//     concurrently running workgroups share A rows and B columns in L2.
//   - the segment of an M-tile is found on the device from offsets with a
//     wave-wide prefix sum of per-segment tile counts; the grid is sized for
//     the worst case and surplus workgroups exit at once (no host sync).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kGroupM = 8;

// Finds the segment of global M-tile `mt`.  Wave-uniform result (every wave
// of the workgroup computes the same), so an early exit is workgroup-uniform.
template <int TM>
__device__ __forceinline__ bool find_segment(const int32_t* __restrict__ offsets, int G,
                                             int fixed_rows, int mt, int& seg, int& row0,
                                             int& rows) {
  if (!offsets) {
    const int r0 = mt * TM;
    if (r0 >= fixed_rows) return false;
    seg = 0;
    row0 = r0;
    rows = min(TM, fixed_rows - r0);
    return true;
  }
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int st = 0, cnt = 0;
    if (g < G) {
      st = offsets[g];
      cnt = offsets[g + 1] - st;
    }
    const int tiles = (cnt + TM - 1) / TM;
    const int incl = wave_inclusive_scan(tiles);
    const int total = __shfl(incl, 63, kWave);
    if (mt < carry + total) {
      const unsigned long long m = __ballot(carry + incl > mt);
      const int first = __ffsll((long long)m) - 1;
      const int excl = carry + __shfl(incl - tiles, first, kWave);
      const int st_g = __shfl(st, first, kWave);
      const int cnt_g = __shfl(cnt, first, kWave);
      const int ml = mt - excl;
      seg = g0 + first;
      row0 = st_g + ml * TM;
      rows = min(TM, cnt_g - ml * TM);
      return true;
    }
    carry += total;
  }
  return false;
}

__device__ __forceinline__ void decode_tile(int tile, int mt_bound, int nt_count, int& mt,
                                            int& nt) {
  const int group = tile / (kGroupM * nt_count);
  const int first_mt = group * kGroupM;
  const int gsize = min(kGroupM, mt_bound - first_mt);
  const int in_g = tile - group * kGroupM * nt_count;
  mt = first_mt + in_g % gsize;
  nt = in_g / gsize;
}

__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row & 7)) << 3; }

}  // namespace

__global__ __launch_bounds__(256, 2) void k_grouped_gemm_bf16(
    const bf16* __restrict__ A, const bf16* __restrict__ B, bf16* __restrict__ C,
    const int32_t* __restrict__ offsets, int G, int fixed_rows, int mt_bound, int Kd, int N,
    int gelu) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM * BK + BN * BK)];
  const int nt_count = (N + BN - 1) / BN;
  int mt, nt;
  decode_tile(blockIdx.x, mt_bound, nt_count, mt, nt);
  int seg, row0, rows;
  if (!find_segment<BM>(offsets, G, fixed_rows, mt, seg, row0, rows)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int rr = lane & 31, kh = lane >> 5;
  const int n0 = nt * BN;
  const bf16* Bg = B + (size_t)seg * Kd * N;

  // A loader: 4 vectors of 8 bf16 per thread: row a_r[j], k-chunk a_c.
  const int a_c = tid & 7;
  int a_r[4];
  bool a_ok[4];
  const bf16* a_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a_r[j] = (tid >> 3) + 32 * j;
    a_ok[j] = a_r[j] < rows;
    a_src[j] = A + (size_t)(row0 + (a_ok[j] ? a_r[j] : 0)) * Kd + a_c * 8;
  }
  // B loader: an 8(k) x 4(n) block per thread.
  const int b_kb = tid >> 5, b_nb = tid & 31;
  const int b_n = n0 + b_nb * 4;
  const bool b_nok = b_n < N;
  const bf16* b_src = Bg + (size_t)(b_kb * 8) * N + (b_nok ? b_n : 0);

  u32x4 ra[4];
  u32x2 rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = a_ok[j] && (k0 + a_c * 8 < Kd);
      ra[j] = ok ? *(const u32x4*)(a_src[j] + k0) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = b_nok && (k0 + b_kb * 8 + i < Kd);
      rb[i] = ok ? *(const u32x2*)(b_src + (size_t)(k0 + i) * N) : u32x2{0, 0};
    }
  };
  auto lstore = [&](int buf) {
    bf16* sA = smem + buf * (BM * BK + BN * BK);
    bf16* sB = sA + BM * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4*)(sA + a_r[j] * BK + swz(a_r[j], a_c)) = ra[j];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const uint32_t sel = (jn & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        o[m] = __builtin_amdgcn_perm(rb[2 * m + 1][jn >> 1], rb[2 * m][jn >> 1], sel);
      const int n = b_nb * 4 + jn;
      *(u32x4*)(sB + n * BK + swz(n, b_kb)) = o;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = (Kd + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const bf16* sA = smem + buf * (BM * BK + BN * BK);
    const bf16* sB = sA + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ks * 2 + kh;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + rr;
        a[i] = *(const bf16x8*)(sA + r * BK + swz(r, chunk));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + j * 32 + rr;
        b[j] = *(const bf16x8*)(sB + n * BK + swz(n, chunk));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue through LDS: D layout of a 32x32 tile: lane holds column lane%32,
  // rows 8*(r/4) + 4*(lane/32) + r%4 for its 16 registers r.
  constexpr int CS = BN + 8;
  bf16* sC = smem;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        const int col = wn * 64 + j * 32 + rr;
        float v = acc[i][j][r];
        if (gelu) v = gelu_tanh_f32(v);
        sC[row * CS + col] = f32_to_bf16(v);
      }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < (BM * BN / 8) / 256; ++q) {
    const int v = tid + 256 * q;
    const int r = v / (BN / 8), c = v % (BN / 8);
    if (r < rows && n0 + c * 8 < N)
      *(u32x4*)(C + (size_t)(row0 + r) * N + n0 + c * 8) = *(const u32x4*)(sC + r * CS + c * 8);
  }
}

// fp32 grouped GEMM (plain FMA, 64 x 64 tiles, 4 x 4 outputs per thread).
__global__ __launch_bounds__(256) void k_grouped_gemm_f32(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C,
    const int32_t* __restrict__ offsets, int G, int fixed_rows, int mt_bound, int Kd, int N,
    int gelu) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float sA[TM][TK + 1];
  __shared__ float sB[TK][TN];
  const int nt_count = (N + TN - 1) / TN;
  const int mt = blockIdx.x / nt_count, nt = blockIdx.x % nt_count;
  int seg, row0, rows;
  if (!find_segment<TM>(offsets, G, fixed_rows, mt, seg, row0, rows)) return;
  const float* Bg = B + (size_t)seg * Kd * N;
  const int n0 = nt * TN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kd; k0 += TK) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + 256 * j;
      const int r = idx >> 4, c = idx & 15;
      sA[r][c] = (r < rows && k0 + c < Kd) ? A[(size_t)(row0 + r) * Kd + k0 + c] : 0.0f;
      const int kr = idx >> 6, nc = idx & 63;
      sB[kr][nc] = (k0 + kr < Kd && n0 + nc < N) ? Bg[(size_t)(k0 + kr) * N + n0 + nc] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[ty * 4 + i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = n0 + tx * 4 + j;
      if (c < N) {
        float v = acc[i][j];
        if (gelu) v = gelu_tanh_f32(v);
        C[(size_t)(row0 + r) * N + c] = v;
      }
    }
  }
}

static int mt_bound_for(const GemmArgs& a, int tm) {
  if (!a.offsets) return (a.fixed_rows + tm - 1) / tm;
  return (a.max_rows + tm - 1) / tm + a.G;
}

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  const int mtb = mt_bound_for(a, BM);
  const int ntc = (a.N + BN - 1) / BN;
  const long long grid = (long long)mtb * ntc;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  k_grouped_gemm_bf16<<<(unsigned)grid, 256, 0, st>>>((const bf16*)a.A, (const bf16*)a.B,
                                                      (bf16*)a.C, a.offsets, a.G, a.fixed_rows,
                                                      mtb, a.Kd, a.N, a.gelu);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_f32(const GemmArgs& a, hipStream_t st) {
  const int mtb = mt_bound_for(a, 64);
  const int ntc = (a.N + 63) / 64;
  const long long grid = (long long)mtb * ntc;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  k_grouped_gemm_f32<<<(unsigned)grid, 256, 0, st>>>((const float*)a.A, (const float*)a.B,
                                                     (float*)a.C, a.offsets, a.G, a.fixed_rows,
                                                     mtb, a.Kd, a.N, a.gelu);
  return hipGetLastError();
}

}  // namespace moe
