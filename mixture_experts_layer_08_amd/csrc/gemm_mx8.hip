// MXFP8 grouped GEMM over variable-length expert segments:
//   C[r, :] = quant(act(A[r, :] * B[g]^T))   for every row r of segment g,
// with A and B in MXFP8 (E4M3 codes, one E8M0 scale per 32 values along the
// contraction dimension, see mx.h), fp32 accumulation, and an epilogue that
// quantises the result to MXFP8 again, in blocks of 32 along its row.
//
// Method: the per-expert contractions of the MoELayer listing of the
// dpshk.com "MoE module infra notes" (section 4.2: x W1 -> GELU -> W2), run as
// one grouped GEMM (section 5.1 of the cf-1.com page "Dissecting the MoE
// communication bottleneck"), with the FP8 hidden states of section 5.3 of
// that page.  The quantisation of the GEMM output happens in the epilogue,
// from the accumulators, so no separate quantise pass reads it back (the
// cost warning of section 5.4).
//
// Design (gfx950): two kernels on the bf16 kernels' 256 x 256 tile.  The
// four-wave k_grouped_gemm_mx8w4 (below the eight-wave one) is the one the
// launcher runs; building with MOE_MX8_W4=0 selects the eight-wave form
// described here: eight waves (two per SIMD), each wave a 128 x 64 block of
// 4 x 2 v_mfma_scale_f32_32x32x64_f8f6f4 tiles; one K-step is 64 values = 64
// bytes per row, so a stage holds the same
// 32 KiB (A [256][64 B], B [256][64 B], 16-byte chunk c of row r stored at
// c ^ ((r >> 2) & 3)), filled by LDS-direct loads through a 4-stage ring.
// The key is the measured conflict-free one for this kernel's reads, in
// which the 32 lanes of each half-wave read 32 consecutive rows of one k
// chunk (SQ_LDS_BANK_CONFLICT on each read pattern alone: zero with this
// key, a 2-way conflict on every read with (r >> 1) & 3, the key the bf16
// four-wave kernel's reads of 16 rows per chunk need).
// The block scales ride in the same ring: every even step's stage also
// carries one 4-byte word per A row and per B row (the scales of that step
// and the next), loaded by one LDS-direct dword load per wave.
//
// Operand layout of the scaled MFMA (checked on the hardware): lane
// (r = lane % 32, h = lane / 32) supplies row r; its 32 bytes are the values
// k = 16h .. 16h+15 and k = 32+16h .. 32+16h+15 of the 64-value step, and its
// scale operand (byte 0) is the scale of block h (k = 32h .. 32h+31).  Both
// operands use the same mapping, so with 64-byte K rows lane h reads chunks
// h and h + 2.  The MFMA runs with the operands swapped (B^T fragment as
// "A"), so each lane accumulates C^T: per 32 x 32 tile it owns row
// m = lane % 32 and columns 8 (v / 4) + 4 (lane / 32) + v % 4, i.e. lanes m
// and m + 32 together hold the 32 columns of the tile, which is one MX block
// of the output row: the block maximum is one cross-lane max away.
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {

namespace {

constexpr int kMxBM = 256, kMxBN = 256, kMxBK = 64;  // BK in values (= bytes)
constexpr int kMxThreads = 512;
constexpr int kMxDma = 2;  // data LDS-direct loads per operand, per wave, per stage
constexpr int kMxStages = 4;
constexpr uint32_t kMxDataBytes = (kMxBM + kMxBN) * kMxBK;     // 32 KiB
constexpr uint32_t kMxScaleBytes = (kMxBM + kMxBN) * 4;        // 2 KiB
constexpr uint32_t kMxStageBytes = kMxDataBytes + kMxScaleBytes;
constexpr size_t kMxSmem = (size_t)kMxStages * kMxStageBytes;  // 136 KiB
static_assert(kMxSmem <= 160 * 1024, "LDS ring exceeds 160 KiB");
static_assert(kMxBN == kMxPanelRows && kMxBK == kMxPanelK, "a B K-step is one weight panel");
static_assert(kMxStages == 4, "the wait counts below assume four stages");

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) { return *(const lds_u32x4*)(uintptr_t)addr; }
__device__ __forceinline__ uint32_t lds_b32(uint32_t addr) { return *(const lds_u32*)(uintptr_t)addr; }
__device__ __forceinline__ int mx_swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

__device__ __forceinline__ i32x8 frag(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ f32x16 mfma_mx8(const i32x8& b, const i32x8& a, const f32x16& c,
                                           int sb, int sa) {
  // cbsz = blgp = 0: both operands E4M3; opsel 0: byte 0 of each scale word
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, sb, 0, sa);
}

}  // namespace

// Epilogues: kMxEpiQuantRows: C = quant(acc), scales in row layout
// [rows][N/32]; kMxEpiGeluQuantOperand: C = quant(GELU(acc)), scales in
// operand layout with leading dimension c_ld (the next GEMM's A operand).
//
// A: [a_rows][Kd] codes, As operand layout (leading dimension a_ld);
// B: [G][N][Kd] codes in 256 x 64-byte panels (mx.h), so that one K-step of a
// tile's B operand is 16 contiguous KiB; Bs [G][ceil(Kd/128)][N][4].  Kd is a
// multiple of 64 and N of 32.  Rows of a tile past its segment are computed from whatever the
// buffers hold there (even NaN) and never stored; each output row depends on
// its own A row only.
template <int EPI>
__global__ __launch_bounds__(kMxThreads, 1) void k_grouped_gemm_mx8(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, uint8_t* __restrict__ C,
    uint8_t* __restrict__ Cs, const int32_t* __restrict__ offsets, int G, int fixed_rows,
    int a_rows, int a_ld, int c_ld, int mt_bound, int Kd, int N, int xcd_chunk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_mx[];
  const int nt_count = (N + kMxBN - 1) / kMxBN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x, xcd_chunk);
  if (tile >= mt_bound * nt_count) return;
  int mt, nt, seg, row0, rows;
  decode_tile(tile, mt_bound, nt_count, mt, nt);
  if (!find_segment<kMxBM>(offsets, G, fixed_rows, mt, seg, row0, rows)) return;
  seg = __builtin_amdgcn_readfirstlane(seg);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int rr = lane & 31, kh = lane >> 5;
  const int n0 = nt * kMxBN;
  const int nslab = (Kd + 127) / 128;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem_mx;

  // ---- global -> LDS loaders ----
  // data: instruction d of this wave covers stage rows 16 (8d + wave) .. +15,
  // four lanes per 64-byte row; rows past the buffer read as zero.
  const int r_row_l = lane >> 2;
  const int r_chunk = mx_swz(r_row_l, lane & 3);
  const u32x4 ra = make_rsrc_words(A + (size_t)row0 * Kd, (long long)(a_rows - row0) * Kd);
  // B: this tile's panels, one per K-step (rows past N are panel padding)
  const u32x4 rb = make_rsrc_words(B + ((size_t)seg * nt_count + nt) * kMxBN * (size_t)Kd,
                                   (long long)kMxBN * Kd);
  const uint32_t b_off = (uint32_t)((r_row_l + 16 * wave) * kMxBK + r_chunk * 16);
  const uint32_t d_off = (uint32_t)((r_row_l + 16 * wave) * Kd + r_chunk * 16);
  const uint32_t d_stride = (uint32_t)(8 * 16 * Kd);
  // scales: waves 0-3 load A rows 64 w .. +63, waves 4-7 B rows 64 (w-4) ..
  // +63; lane l fetches the word of row (.. + l) of slab s / 2.
  const bool s_is_a = wave < 4;
  const int s_row = 64 * (wave & 3) + lane;
  const u32x4 rs = s_is_a
      ? make_rsrc_words(As, (long long)nslab * a_ld * 4)
      : make_rsrc_words(Bs + (size_t)seg * nslab * N * 4, (long long)nslab * N * 4);
  const uint32_t s_base = s_is_a ? (uint32_t)(row0 + s_row) * 4 : (uint32_t)(n0 + s_row) * 4;
  const uint32_t s_slab = s_is_a ? (uint32_t)a_ld * 4 : (uint32_t)N * 4;
  const uint32_t s_lds = kMxDataBytes + (s_is_a ? 0u : 1024u) + (uint32_t)(wave & 3) * 256;

  auto stage_addr = [&](int kt) {
    return __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(kt & (kMxStages - 1)) * kMxStageBytes);
  };
  // load d (0, 1: A; 2, 3: B; 4: the scale word, even steps only) of step kt
  auto dma = [&](uint32_t st, int d, int kt) {
    const bool in_k = kt * kMxBK < Kd;
    if (d < kMxDma) {
      dma_load16(st + (8 * d + wave) * 1024,
                 in_k ? d_off + d * d_stride + (uint32_t)kt * kMxBK : kOob, ra);
    } else if (d < 2 * kMxDma) {
      dma_load16(st + kMxBM * kMxBK + (8 * (d - kMxDma) + wave) * 1024,
                 in_k ? b_off + (d - kMxDma) * (8 * 16 * kMxBK) + (uint32_t)kt * (kMxBN * kMxBK)
                      : kOob,
                 rb);
    } else {
      dma_load4(st + s_lds, in_k ? s_base + (uint32_t)(kt >> 1) * s_slab : kOob, rs);
    }
  };
  auto issue_step = [&](int kt) {
    const uint32_t st = stage_addr(kt);
#pragma unroll
    for (int d = 0; d < 2 * kMxDma; ++d) dma(st, d, kt);
    if ((kt & 1) == 0) dma(st, 2 * kMxDma, kt);
  };

  // ---- LDS -> register fragment addresses (relative to a stage) ----
  uint32_t a_rd[4][2], b_rd[2][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wm * 128 + i * 32 + rr;
#pragma unroll
    for (int c = 0; c < 2; ++c) a_rd[i][c] = (uint32_t)r * kMxBK + (uint32_t)mx_swz(r, kh + 2 * c) * 16;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wn * 64 + j * 32 + rr;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      b_rd[j][c] = kMxBM * kMxBK + (uint32_t)r * kMxBK + (uint32_t)mx_swz(r, kh + 2 * c) * 16;
  }
  uint32_t sa_rd[4], sb_rd[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) sa_rd[i] = kMxDataBytes + (uint32_t)(wm * 128 + i * 32 + rr) * 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) sb_rd[j] = kMxDataBytes + 1024 + (uint32_t)(wn * 64 + j * 32 + rr) * 4;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto read_a = [&](uint32_t st, int i) { return frag(lds_b128(st + a_rd[i][0]), lds_b128(st + a_rd[i][1])); };
  auto read_b = [&](uint32_t st, int j) { return frag(lds_b128(st + b_rd[j][0]), lds_b128(st + b_rd[j][1])); };

  // Software pipeline, one barrier per K-step, the step's eight MFMAs in two
  // halves (tiles i = 0, 1, then i = 2, 3):
  //   read a2, a3 of step kt                | half 0 of step kt
  //   wait: step kt+1 landed; barrier
  //   read a0, a1, b of step kt+1 (+ scale  | half 1 of step kt, refill of
  //   words when kt+1 is even)              | step kt+3
  // b of consecutive steps alternates between two register sets.  Scale words
  // (4 A + 2 B per lane) cover a pair of steps; each step's bytes are
  // extracted at its start.  Ring: step kt lives in slot kt % 4; iteration kt
  // refills slot (kt-1) % 4, whose reads every wave finished before this
  // iteration's barrier.  Loads younger than step kt+1 at the wait: step
  // kt+2's four data loads, plus its scale word when kt+2 is even.
  // The counts assume these LDS-direct loads are the only vector-memory
  // instructions in the loop: the build refuses a spill (its scratch loads
  // and stores would count too), and so does the launcher.
  const int KT = Kd / kMxBK;
  issue_step(0);
  issue_step(1);
  issue_step(2);
  wait_vmcnt<9>();  // step 0 landed: younger are step 1 (4) and step 2 (4 + 1)
  block_barrier();
  i32x8 a01[2], a23[2], bs[2][2];
  uint32_t wa[4], wb[2];
  {
    const uint32_t st = lds0;
    a01[0] = read_a(st, 0);
    a01[1] = read_a(st, 1);
    bs[0][0] = read_b(st, 0);
    bs[0][1] = read_b(st, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) wa[i] = lds_b32(st + sa_rd[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) wb[j] = lds_b32(st + sb_rd[j]);
  }

  auto step = [&](int kt, auto par) {
    constexpr int P = decltype(par)::value;  // kt & 1
    const uint32_t st = lds0 + (uint32_t)(kt & 3) * kMxStageBytes;
    const uint32_t st1 = lds0 + (uint32_t)((kt + 1) & 3) * kMxStageBytes;
    // this step's scale bytes: byte 2 (kt & 1) + kh of each word
    int sa[4], sb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = (int)((wa[i] >> (8 * (2 * P + kh))) & 0xffu);
#pragma unroll
    for (int j = 0; j < 2; ++j) sb[j] = (int)((wb[j] >> (8 * (2 * P + kh))) & 0xffu);
    a23[0] = read_a(st, 2);
    a23[1] = read_a(st, 3);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_mx8(bs[P][j], a01[i], acc[i][j], sb[j], sa[i]);
    if (P == 0)
      wait_vmcnt<5>();
    else
      wait_vmcnt<4>();
    wait_lgkm0();
    block_barrier();
    // operands of step kt+1 (past the last step: harmless reads of a landed stage)
    a01[0] = read_a(st1, 0);
    a01[1] = read_a(st1, 1);
    bs[P ^ 1][0] = read_b(st1, 0);
    bs[P ^ 1][1] = read_b(st1, 1);
    if (P == 1) {  // step kt+1 is even: the next pair's scale words
#pragma unroll
      for (int i = 0; i < 4; ++i) wa[i] = lds_b32(st1 + sa_rd[i]);
#pragma unroll
      for (int j = 0; j < 2; ++j) wb[j] = lds_b32(st1 + sb_rd[j]);
    }
    // half 1 with the refill of step kt+3 (past K: zeros into a slot never read)
    const int kf = kt + 3;
    const uint32_t stf = stage_addr(kf);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 2 + (t >> 1), j = t & 1;
      acc[i][j] = mfma_mx8(bs[P][j], a23[i - 2], acc[i][j], sb[j], sa[i]);
      dma(stf, t, kf);
    }
    if (P == 1) dma(stf, 2 * kMxDma, kf);  // kt + 3 even
  };
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < KT) step(kt + 1, std::integral_constant<int, 1>{});
  }
  wait_vmcnt<0>();  // drain the loads issued past the end before the grid exits

  // ---- epilogue: (GELU,) MX block maxima over lane pairs, E4M3 codes ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = wm * 128 + i * 32 + rr;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nb = n0 + wn * 64 + j * 32;  // first column of this tile's block
      float v[16];
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        v[r] = EPI == kMxEpiGeluQuantOperand ? gelu_tanh_f32(acc[i][j][r]) : acc[i][j][r];
        amax = fmaxf(amax, fabsf(v[r]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      const uint32_t code = mx_scale_code(amax);
      const float inv = mx_inv_scale(code);
      uint32_t d[4];  // columns 8g + 4kh .. +3 of the block
#pragma unroll
      for (int g = 0; g < 4; ++g) d[g] = mx_encode4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], inv);
      // lane pair exchange: lane kh = 0 stores columns 0-15, kh = 1 columns 16-31
      const uint32_t x0 = __shfl_xor(kh ? d[0] : d[2], 32, kWave);
      const uint32_t x1 = __shfl_xor(kh ? d[1] : d[3], 32, kWave);
      const u32x4 o = kh ? u32x4{x0, d[2], x1, d[3]} : u32x4{d[0], x0, d[1], x1};
      if (m < rows && nb < N) {
        *(u32x4*)(C + (size_t)(row0 + m) * N + nb + 16 * kh) = o;
        if (kh == 0) {
          if (EPI == kMxEpiQuantRows)
            Cs[(size_t)(row0 + m) * (N / kMxBlock) + nb / kMxBlock] = (uint8_t)code;
          else
            Cs[mx_operand_scale_index(c_ld, row0 + m, nb / kMxBlock)] = (uint8_t)code;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Four-wave form: the same tile, stage layout, ring and epilogue, with one
// wave per SIMD owning a 128 x 128 block as 4 x 4 scaled 32x32x64 tiles (256
// fp32 accumulators per lane, in AGPRs).  A K-step then reads 64 KiB of
// fragments from LDS per CU instead of the eight-wave layout's 96 KiB (with
// the 32 KiB the LDS-direct loads write, the eight-wave kernel keeps the LDS
// busy for about as long as its MFMAs run), and the four waves hide their
// own latencies.  Per K-step: wait until step kt+1 has landed for every wave
// (own loads by vmcnt, own LDS reads by lgkmcnt, then the barrier), then the
// 16 MFMAs on fragments read during the previous step, in 4 groups; group i
// runs two MFMAs, reads the A fragment i of step kt+1, issues A refill load
// i, runs two more, reads B fragment i and issues B refill load i.  The
// refills are for step kt+4 into slot kt % 4 itself, whose fragments every
// wave read during step kt-1: three steps of latency cover for each load.
// The scale words of a step pair are read early in the step before the pair
// and their bytes extracted at the start of each step.  The two row-waves
// take the tile's 32-row groups in turn, and a wave whose groups hold no
// valid rows (a segment's last tile) skips their MFMAs, A fragment reads
// and A loads: the loop is instantiated for 0 to 4 active groups.  (With
// contiguous rows per wave, one SIMD of a short last tile would keep all of
// its work, as the bf16 four-wave kernel showed.)
//
// Measured against the eight-wave kernel (mixtral-sized MXFP8 forward, A/B
// on one box, before the row-group skipping, which took another 1.2%):
// 6.41 vs 6.47 ms for both GEMMs, at a higher clock (1.9 vs
// 1.7-1.8 GHz: less LDS traffic) but fewer MFMA-busy cycles (57-63% vs
// 60-70%).  Counter runs of the earlier forms: two loads back to back per
// group of four MFMAs, 6.74 ms; spread as above, 6.58 ms; the refill
// distance of two steps left the waves waiting 21% of their cycles, three
// steps 17%.
//
// As in the bf16 four-wave kernel, the loop keeps vector ALU work off the
// MFMA stream: the data loads' per-lane offsets are fixed for the tile with
// the K-step advance in the scalar offset, and the fragment and scale-word
// reads of each pair of steps share per-lane bases made once per pair.  Per
// two K-steps 25 VALU instructions instead of 95 (-0.4% for both GEMMs of
// the MXFP8 forward, A/B on one box, outputs bitwise equal: the 64-cycle
// MFMAs leave more room for them than the bf16 kernel's 16-cycle ones).
constexpr int kMxW4Threads = 256;
constexpr int kMxW4Dma = 4;  // data LDS-direct loads per operand, per wave, per stage

// Stage: data, then the A and the B scale words (2 KiB each: a tile's 256
// rows start up to 3 words into the block).
constexpr uint32_t kMx4AScale = kMxDataBytes, kMx4BScale = kMxDataBytes + 2048;
constexpr uint32_t kMx4StageBytes = kMxDataBytes + 4096;
constexpr size_t kMx4Smem = (size_t)kMxStages * kMx4StageBytes;  // 144 KiB
static_assert(kMx4Smem <= 160 * 1024, "LDS ring exceeds 160 KiB");

template <int EPI>
__global__ __launch_bounds__(kMxW4Threads, 1) void k_grouped_gemm_mx8w4(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, uint8_t* __restrict__ C,
    uint8_t* __restrict__ Cs, const int32_t* __restrict__ offsets, int G, int fixed_rows,
    int a_rows, int a_ld, int c_ld, int mt_bound, int Kd, int N, int xcd_chunk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_mx4[];
  const int nt_count = (N + kMxBN - 1) / kMxBN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x, xcd_chunk);
  if (tile >= mt_bound * nt_count) return;
  int mt, nt, seg, row0, rows;
  decode_tile(tile, mt_bound, nt_count, mt, nt);
  if (!find_segment<kMxBM>(offsets, G, fixed_rows, mt, seg, row0, rows)) return;
  seg = __builtin_amdgcn_readfirstlane(seg);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int rr = lane & 31, kh = lane >> 5;
  const int n0 = nt * kMxBN;
  const int nslab = (Kd + 127) / 128;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem_mx4;

  // ---- global -> LDS loaders ----
  // data: load d of this wave covers stage rows 16 (4d + wave) .. +15, four
  // lanes per 64-byte row; rows past the buffer read as zero.  Scales, 16
  // bytes per lane from 16-byte aligned addresses (the dword form of the
  // LDS-direct load costs about as much per instruction and needs four
  // times as many): counting words from the scale pointer rounded down to
  // 16 bytes, the words of tile rows 0.. of slab q start at word w(q); the
  // stage receives the 512 words from w(q) & ~3 on (waves 0 and 1: A; 2 and
  // 3: B), so tile row m sits at word m + (w(q) & 3) of its block.  For B,
  // w(q) & 3 is the same for every q (N and n0 are multiples of 32 and 256).
  const int r_row_l = lane >> 2;
  const int r_chunk = mx_swz(r_row_l, lane & 3);
  const u32x4 ra = make_rsrc_words(A + (size_t)row0 * Kd, (long long)(a_rows - row0) * Kd);
  const u32x4 rb = make_rsrc_words(B + ((size_t)seg * nt_count + nt) * kMxBN * (size_t)Kd,
                                   (long long)kMxBN * Kd);
  const uint32_t b_off = (uint32_t)((r_row_l + 16 * wave) * kMxBK + r_chunk * 16);
  const uint32_t d_off = (uint32_t)((r_row_l + 16 * wave) * Kd + r_chunk * 16);
  const uint32_t d_stride = (uint32_t)(4 * 16 * Kd);
  const int a_mis = (int)(((uintptr_t)As & 15) >> 2);
  const uint8_t* bs_seg = Bs + (size_t)seg * nslab * N * 4;
  const int b_mis = (int)(((uintptr_t)bs_seg & 15) >> 2);
  const u32x4 rsa = make_rsrc_words(As - 4 * a_mis, ((long long)nslab * a_ld + a_mis) * 4);
  const u32x4 rsb = make_rsrc_words(bs_seg - 4 * b_mis, ((long long)nslab * N + b_mis) * 4);
  auto a_word0 = [&](int q) { return a_mis + q * a_ld + row0; };  // w(q) of A
  auto b_word0 = [&](int q) { return b_mis + q * N + n0; };       // w(q) of B

  auto stage_addr = [&](int kt) {
    return __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(kt & (kMxStages - 1)) * kMx4StageBytes);
  };
  // load d of step kt: 0-3 A, 4-7 B, 8 this wave's scale words (even steps,
  // waves 0-2)
  // Data loads: a lane's offsets are fixed for the tile (rows past the
  // tile's valid rows already past num_records) and the K-step advance is
  // the scalar offset, clamped to the last step for the refills issued past
  // the end (never read), so that every load stays inside its operand.
  const int kt_last = Kd / kMxBK - 1;  // the launcher requires Kd a positive multiple of kMxBK
  uint32_t av[kMxW4Dma], bv[kMxW4Dma];
#pragma unroll
  for (int d = 0; d < kMxW4Dma; ++d) {
    av[d] = 16 * (4 * d + wave) + r_row_l < rows ? d_off + d * d_stride : kOob;
    bv[d] = b_off + d * (4 * 16 * kMxBK);
  }
  auto dma = [&](uint32_t st, int d, int kt) {
    const bool in_k = kt * kMxBK < Kd;
    const uint32_t kc = (uint32_t)min(kt, kt_last);
    if (d < kMxW4Dma) {
      dma_load16_s(st + (4 * d + wave) * 1024, av[d], kc * kMxBK, ra);
    } else if (d < 2 * kMxW4Dma) {
      const int e = d - kMxW4Dma;
      dma_load16_s(st + kMxBM * kMxBK + (4 * e + wave) * 1024, bv[e], kc * (kMxBN * kMxBK), rb);
    } else {
      const int w = wave < 2 ? a_word0(kt >> 1) : b_word0(kt >> 1);
      const uint32_t off = ((uint32_t)(w & ~3) + 256u * (wave & 1) + 4u * lane) * 4;
      dma_load16(st + kMx4AScale + wave * 1024, in_k ? off : kOob, wave < 2 ? rsa : rsb);
    }
  };
  auto issue_step = [&](int kt) {
    const uint32_t st = stage_addr(kt);
#pragma unroll
    for (int d = 0; d < 2 * kMxW4Dma; ++d) dma(st, d, kt);
    if ((kt & 1) == 0) dma(st, 2 * kMxW4Dma, kt);
  };

  // ---- LDS -> register fragments: row tile i of the wave is rows
  // (2 i + wm) 32 + rr (+ 4 KiB per i; the two row-waves take the tile's 32-row
  // groups in turn, so that a segment's last tile, whose valid rows are a
  // prefix, leaves both about the same number of groups), chunks kh and
  // kh + 2; column tile j is columns wn 128 + 32 j + rr ----
  const int ra_row = wm * 32 + rr, rb_row = wn * 128 + rr;
  const uint32_t a_rd0 = (uint32_t)ra_row * kMxBK + (uint32_t)mx_swz(ra_row, kh) * 16;
  const uint32_t a_rd1 = (uint32_t)ra_row * kMxBK + (uint32_t)mx_swz(ra_row, kh + 2) * 16;
  const uint32_t b_rd0 = kMxBM * kMxBK + (uint32_t)rb_row * kMxBK + (uint32_t)mx_swz(rb_row, kh) * 16;
  const uint32_t b_rd1 = kMxBM * kMxBK + (uint32_t)rb_row * kMxBK + (uint32_t)mx_swz(rb_row, kh + 2) * 16;
  const uint32_t sa_rd = kMx4AScale + (uint32_t)ra_row * 4;  // + 4 sh(q)
  const uint32_t sb_rd = kMx4BScale + (uint32_t)(rb_row + (b_mis + n0) % 4) * 4;
  auto read_a = [&](uint32_t st, int i) {
    return frag(lds_b128(st + a_rd0 + i * 64 * kMxBK), lds_b128(st + a_rd1 + i * 64 * kMxBK));
  };
  auto read_b = [&](uint32_t st, int j) {
    return frag(lds_b128(st + b_rd0 + j * 32 * kMxBK), lds_b128(st + b_rd1 + j * 32 * kMxBK));
  };

  f32x16 acc[4][4];  // set by the first step's MFMAs (zero C operand)
  uint32_t wa[4], wb[4];
  // Per-lane read addresses with the stage slot included, made once per pair
  // of steps by an opaque add (a pair reads slots 2q and 2q + 1, the second
  // at +kMx4StageBytes), so that the reads differ by immediate offsets only.
  auto obase = [&](uint32_t st, uint32_t rd) {
    uint32_t r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(st), "v"(rd));
    return r;
  };
  struct Bases {
    uint32_t a0, a1, b0, b1, sa, sb;
  };
  auto bases = [&](int kt_read) {  // kt_read: the first step of the pair whose slots are read
    const uint32_t st = stage_addr(kt_read);
    const uint32_t sh = (uint32_t)(a_word0(kt_read >> 1) & 3) * 4;
    return Bases{obase(st, a_rd0), obase(st, a_rd1), obase(st, b_rd0),
                 obase(st, b_rd1), obase(st, sa_rd + sh), obase(st, sb_rd)};
  };
  // One K-step with the MFMAs of the first NT row tiles (the rest hold no
  // valid rows of this tile).  bs: the bases of the slot this step reads
  // (slot kt + 1), boff: 0 or kMx4StageBytes.
  auto step = [&](auto nt_c, auto par, auto first_c, int kt, const i32x8* ca, const i32x8* cb,
                  i32x8* na, i32x8* nb, const Bases& bs, uint32_t boff) {
    constexpr int NT = decltype(nt_c)::value;
    constexpr int P = decltype(par)::value;  // kt & 1
    // younger than step kt+1: steps kt+2 and kt+3 (one of them even)
    wait_vmcnt<4 * kMxW4Dma + 1>();
    wait_lgkm0();  // this wave's reads of slot kt % 4 (refilled below) are done
    block_barrier();

    int sa[4], sb[4];  // this step's scale bytes: byte 2 P + kh of each word
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = (int)((wa[i] >> (8 * (2 * P + kh))) & 0xffu);
      sb[i] = (int)((wb[i] >> (8 * (2 * P + kh))) & 0xffu);
    }
    const uint32_t stf = stage_addr(kt + kMxStages);
    if (P == 1) {  // step kt+1 starts a pair: its scale words, early
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wa[i] = lds_b32(bs.sa + boff + i * 256);
        wb[i] = lds_b32(bs.sb + boff + i * 128);
      }
    }
    auto mm = [&](int i, int j) {
      if (i >= NT) {
        // defined on every path (the epilogue skips these tiles)
        if (decltype(first_c)::value) acc[i][j] = f32x16{};
      } else if (decltype(first_c)::value) {
        acc[i][j] = mfma_mx8(cb[j], ca[i], f32x16{}, sb[j], sa[i]);
      } else {
        acc[i][j] = mfma_mx8(cb[j], ca[i], acc[i][j], sb[j], sa[i]);
      }
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mm(i, 0);
      mm(i, 1);
      if (i < NT)
        na[i] = frag(lds_b128(bs.a0 + boff + i * 64 * kMxBK), lds_b128(bs.a1 + boff + i * 64 * kMxBK));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      dma(stf, i, kt + kMxStages);
      mm(i, 2);
      mm(i, 3);
      nb[i] = frag(lds_b128(bs.b0 + boff + i * 32 * kMxBK), lds_b128(bs.b1 + boff + i * 32 * kMxBK));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      dma(stf, kMxW4Dma + i, kt + kMxStages);
    }
    if (P == 0) dma(stf, 2 * kMxW4Dma, kt + kMxStages);  // step kt+4 is even
  };
  using kTrue = std::integral_constant<bool, true>;
  using kFalse = std::integral_constant<bool, false>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // The counts assume these LDS-direct loads are the only vector-memory
  // instructions in the loop: the build refuses a spill, and so does the
  // launcher.
  const int KT = Kd / kMxBK;
  issue_step(0);
  issue_step(1);
  issue_step(2);
  issue_step(3);
  wait_vmcnt<6 * kMxW4Dma + 1>();  // step 0 landed: younger are steps 1-3 (+1 scale load)
  block_barrier();
  auto k_loop = [&](auto nt_c) {
    constexpr int NT = decltype(nt_c)::value;
    i32x8 pa[4], pb[4], qa[4], qb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < NT) pa[i] = read_a(lds0, i);
      pb[i] = read_b(lds0, i);
      wa[i] = lds_b32(lds0 + sa_rd + (uint32_t)(a_word0(0) & 3) * 4 + i * 256);
      wb[i] = lds_b32(lds0 + sb_rd + i * 128);
    }
    {
      const Bases b1 = bases(1);  // step 0 reads slot 1 (its scale words are not read: P = 0)
      step(nt_c, P0{}, kTrue{}, 0, pa, pb, qa, qb, b1, 0u);
    }
    int kt = 1;
    for (; kt + 1 < KT; kt += 2) {
      const Bases b = bases(kt + 1);  // slots 2q and 2q + 1
      step(nt_c, P1{}, kFalse{}, kt, qa, qb, pa, pb, b, 0u);
      step(nt_c, P0{}, kFalse{}, kt + 1, pa, pb, qa, qb, b, kMx4StageBytes);
    }
    if (kt < KT) {
      const Bases b = bases(kt + 1);
      step(nt_c, P1{}, kFalse{}, kt, qa, qb, pa, pb, b, 0u);
    }
  };
  // row tiles of this wave that hold valid rows: tile i starts at row (2 i + wm) 32
  const int nt_rows = __builtin_amdgcn_readfirstlane(min(max((rows - 32 * wm + 63) >> 6, 0), 4));
  if (nt_rows == 4) k_loop(std::integral_constant<int, 4>{});
  else if (nt_rows == 3) k_loop(std::integral_constant<int, 3>{});
  else if (nt_rows == 2) k_loop(std::integral_constant<int, 2>{});
  else if (nt_rows == 1) k_loop(std::integral_constant<int, 1>{});
  else k_loop(std::integral_constant<int, 0>{});
  wait_vmcnt<0>();  // drain the loads issued past the end before the grid exits

  // ---- epilogue, per 32 x 32 tile as in the eight-wave kernel ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= nt_rows) continue;  // no valid rows (uniform)
    const int m = (2 * i + wm) * 32 + rr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nb = n0 + wn * 128 + j * 32;  // first column of this tile's block
      float v[16];
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        v[r] = EPI == kMxEpiGeluQuantOperand ? gelu_tanh_f32(acc[i][j][r]) : acc[i][j][r];
        amax = fmaxf(amax, fabsf(v[r]));
      }
      // The exchanges between lanes l and l ^ 32 use v_permlane32_swap, which
      // trades the upper half-wave of its first operand for the lower
      // half-wave of its second, in the VALU: swapping a value with itself
      // leaves each lane its own value and its partner's, in some order.
      {
        const auto am = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax),
                                                         __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(am[0]), __uint_as_float(am[1]));
      }
      const uint32_t code = mx_scale_code(amax);
      const float inv = mx_inv_scale(code);
      uint32_t d[4];  // columns 8g + 4kh .. +3 of the block
#pragma unroll
      for (int g = 0; g < 4; ++g) d[g] = mx_encode4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], inv);
      // lower half: its own d[0] and its partner's, its own d[1] and its
      // partner's; upper half: its partner's d[2] and its own, likewise d[3]
      const auto s0 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
      const u32x4 o = u32x4{s0[0], s0[1], s1[0], s1[1]};
      if (m < rows && nb < N) {
        *(u32x4*)(C + (size_t)(row0 + m) * N + nb + 16 * kh) = o;
        if (kh == 0) {
          if (EPI == kMxEpiQuantRows)
            Cs[(size_t)(row0 + m) * (N / kMxBlock) + nb / kMxBlock] = (uint8_t)code;
          else
            Cs[mx_operand_scale_index(c_ld, row0 + m, nb / kMxBlock)] = (uint8_t)code;
        }
      }
    }
  }
}

#ifndef MOE_MX8_W4
#define MOE_MX8_W4 1
#endif

template <int EPI>
static hipError_t launch_mx8(const MxGemmArgs& a, hipStream_t st) {
  const hipError_t e = MOE_MX8_W4 ? allow_dynamic_lds<k_grouped_gemm_mx8w4<EPI>, true>()
                                  : allow_dynamic_lds<k_grouped_gemm_mx8<EPI>, true>();
  if (e != hipSuccess) return e;
  if (a.Kd <= 0 || a.Kd % kMxBK != 0 || a.N <= 0 || a.N % kMxBlock != 0) return hipErrorInvalidValue;
  const int ntc = (a.N + kMxBN - 1) / kMxBN;
  const int mtb = a.offsets ? (a.max_rows + kMxBM - 1) / kMxBM + a.G
                            : (a.fixed_rows + kMxBM - 1) / kMxBM;
  const long long grid = (long long)mtb * ntc;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (MOE_MX8_W4)
    k_grouped_gemm_mx8w4<EPI><<<(unsigned)grid, kMxW4Threads, kMx4Smem, st>>>(
        a.A, a.As, a.B, a.Bs, a.C, a.Cs, a.offsets, a.G, a.fixed_rows,
        a.offsets ? a.max_rows : a.fixed_rows, a.a_ld, a.c_ld, mtb, a.Kd, a.N, xcd_chunk_for(ntc));
  else
    k_grouped_gemm_mx8<EPI><<<(unsigned)grid, kMxThreads, kMxSmem, st>>>(
        a.A, a.As, a.B, a.Bs, a.C, a.Cs, a.offsets, a.G, a.fixed_rows,
        a.offsets ? a.max_rows : a.fixed_rows, a.a_ld, a.c_ld, mtb, a.Kd, a.N, xcd_chunk_for(ntc));
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_mx8(const MxGemmArgs& a, hipStream_t st) {
  switch (a.epi) {
    case kMxEpiQuantRows: return launch_mx8<kMxEpiQuantRows>(a, st);
    case kMxEpiGeluQuantOperand: return launch_mx8<kMxEpiGeluQuantOperand>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
