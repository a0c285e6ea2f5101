// Grouped GEMM over variable-length expert segments.  Forward form (NN):
//   C[r, :] = act(A[r, :] * B[g])   for every row r of segment g,
// with segment g the rows [offsets[g], offsets[g+1]) of the packed buffer.
// The backward pass adds NT (A[r, :] * B[g]^T, the transposed weights) and
// TN (C[g] = A_g^T B_g over the rows of segment g: per-expert weight
// gradients); see GemmLayout.
//
// Method: the per-expert contractions of the MoELayer listing of the
// dpshk.com "MoE module infra notes" (section 4.2: x W1 -> GELU -> W2 over
// stacked expert weights), run as one grouped GEMM as section 5.1 of the
// cf-1.com page "Dissecting the MoE communication bottleneck" recommends
// (many thin per-expert GEMMs in one kernel).
//
// Two bf16 kernels share the tile (256 x 256 x 32), the 4-stage LDS ring
// filled by direct HBM->LDS loads, the N-contiguous weight operand read
// through LDS transpose reads, and an epilogue with the optional GELU(tanh)
// straight from the accumulators: k_grouped_gemm_w4 (four waves, 16 x 16
// MFMAs) runs the row-major forward form, k_grouped_gemm_bf16 (eight waves,
// 32 x 32 MFMAs) the transposed forms of the backward.  Each is described
// above its definition.  Segment lookup happens on the device from
// `offsets` (a wave-wide prefix sum of per-segment tile counts); the grid is
// sized for the worst case and surplus workgroups exit at once, so there is
// no host sync.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

#include <type_traits>

namespace moe {


// 256 x 256 x 32 tile on 8 waves in 2 (M) x 4 (N); each wave owns a 128 x 64
// block = 4 x 2 MFMA 32x32x16 tiles (128 fp32 accumulators per lane).  Two
// waves share each SIMD, so one wave's MFMAs run while the other is held at
// a load issue, an LDS read or the barrier.
//
// Both operands go from HBM/L2 straight into LDS (buffer_load_dwordx4 ...
// lds, no register staging) through a ring of kStages stages; step kt's loads
// are issued while step kt-kStages+1 is multiplied, so an L2 miss is hidden
// behind several steps of MFMA work.  One s_barrier per K-step; the wait for
// a stage's loads is an explicit vmcnt.
//
// LDS stage (32 KiB): A [256 m][32 k] (64-byte rows, 16-byte chunk c stored
// at c ^ ((m >> 2) & 3)) then B [32 k][256 n] (512-byte rows, 16-byte chunk c
// stored at c ^ (4 * (k & 3))).  Each LDS-direct instruction of a wave fills
// 1 KiB in lane order; a lane fetches the global chunk that the swizzle maps
// to its slot.  Both swizzles make the fragment reads below conflict-free
// (measured with SQ_LDS_BANK_CONFLICT on the read pattern alone: the 32
// lanes of a half-wave read 32 consecutive rows of one k chunk).
//
// The MFMA runs with the operands swapped (B^T fragment as "A"), so each lane
// accumulates C^T: per 32x32 tile it owns row m = lane%32 and columns
// 8*(r/4) + 4*(lane/32) + r%4.  The B^T fragment (8 consecutive k of one n per
// lane) comes from two ds_read_b64_tr_b16 on the row-major B stage: within
// each 16-lane group, lane i supplies the address of 4 consecutive n of row
// (i / 4) and receives column i of that 4 x 16 block.
constexpr int BM2 = 256, BN2 = 256, BK2 = 32;
constexpr int kGemmThreads = 512;
constexpr int kSub = BK2 / 16;  // MFMA k-substeps per K-step
constexpr int kDma = 2;         // LDS-direct loads per operand, per wave, per stage
__device__ __forceinline__ int a_swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 4
#endif
constexpr int kStages = MOE_GEMM_STAGES;
static_assert(kStages >= 3, "the refill of a stage is issued after the barrier of the step before");
constexpr uint32_t kStageBytes = (BM2 + BN2) * BK2 * 2;
constexpr size_t kSmem2 = (size_t)kStages * kStageBytes;
static_assert(kSmem2 <= 160 * 1024, "LDS ring exceeds 160 KiB");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  return *(const lds_bf16x8*)(uintptr_t)addr;
}
__device__ __forceinline__ bf16x8 lds_read_tr_pair(uint32_t addr, uint32_t addr_hi) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr_hi);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// GELU'(u) of the tanh form: with s = 1 / (1 + exp(-2z)) = 0.5 (1 + tanh z)
// and 1 - tanh^2 z = 4 s (1 - s):  s + 2 u s (1 - s) z'(u),
// z'(u) = sqrt(2/pi) (1 + 3 * 0.044715 u^2).
__device__ __forceinline__ float gelu_tanh_grad_f32(float u) {
  const float kC = 0.7978845608028654f;           // sqrt(2/pi)
  const float kNeg2Log2e = -2.8853900817779268f;   // -2 / ln 2
  const float z = kC * fmaf(0.044715f * u, u * u, u);
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(kNeg2Log2e * z));
  const float dz = kC * fmaf(3.0f * 0.044715f * u, u, 1.0f);
  return fmaf(2.0f * u * s * (1.0f - s), dz, s);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Operand staging.  Each operand of a K-step lands in its 16 KiB half of
// the stage in one of two forms:
//   K-contiguous rows ("rows": A of NN/NT, B of NT): [256 rows][32 k], 64-byte
//     rows, 16-byte chunk c at c ^ ((row >> 2) & 3); fragments by ds_read_b128;
//   row-contiguous k-rows ("cols": B of NN/TN, A of TN): [32 k][256], 512-byte
//     rows, chunk c at c ^ (4 * (k & 3)); fragments by ds_read_b64_tr_b16 pairs.
// A fragment is 8 consecutive k of one row/column per lane (row lane % 32,
// k half lane / 32) whichever form it came from.  Cv and Ep may be the same
// buffer (the GELU-derivative epilogue in place): each element is read, then
// written, by one lane.
template <int LAYOUT, int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void k_grouped_gemm_bf16(
    const bf16* __restrict__ A, const bf16* __restrict__ B, void* Cv,
    bf16* Ep, const int32_t* __restrict__ offsets, int G, int fixed_rows,
    int a_rows, int mt_bound, int M, int Kd, int N, int xcd_chunk) {
  constexpr bool kTN = LAYOUT == kGemmTN;
  constexpr bool kARows = !kTN;               // A in "rows" form
  constexpr bool kBRows = LAYOUT == kGemmNT;  // B in "rows" form
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  const int nt_count = (N + BN2 - 1) / BN2;
  int mt, nt, seg, row0, rows;
  int k_begin = 0, k_end = Kd;  // contraction range; TN: the segment's packed rows
  if (kTN) {
    const int mt_count = (M + BM2 - 1) / BM2;
    const int per_seg = mt_count * nt_count;
    const int tile = xcd_tile(blockIdx.x, gridDim.x, xcd_chunk);
    if (tile >= G * per_seg) return;
    seg = tile / per_seg;
    decode_tile(tile - seg * per_seg, mt_count, nt_count, mt, nt);
    k_begin = offsets ? offsets[seg] : 0;
    k_end = offsets ? offsets[seg + 1] : fixed_rows;
    row0 = mt * BM2;  // rows of C = columns of A
    rows = min(BM2, M - row0);
  } else {
    const int tile = xcd_tile(blockIdx.x, gridDim.x, xcd_chunk);
    if (tile >= mt_bound * nt_count) return;
    decode_tile(tile, mt_bound, nt_count, mt, nt);
    if (!find_segment<BM2>(offsets, G, fixed_rows, mt, seg, row0, rows)) return;
  }
  // The tile is wave-uniform; keep it in scalar registers so the buffer
  // descriptors below are scalar too.
  seg = __builtin_amdgcn_readfirstlane(seg);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  k_begin = __builtin_amdgcn_readfirstlane(k_begin);
  k_end = __builtin_amdgcn_readfirstlane(k_end);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rr = lane & 31, kh = lane >> 5;
  const int n0 = nt * BN2;
  // Wave layout.  Normally 2 (M) x 4 (N): the wave owns rows rbase ..
  // rbase + 127 and columns cbase .. cbase + 63 of the tile.  A tile with at
  // most 128 valid columns (the last N-tile of an output whose width is not
  // a multiple of 256) uses 4 (M) x 2 (N) instead, 64 x 64 per wave: the
  // waves of the empty half would otherwise multiply zeros, and with waves
  // dealt to SIMDs in turn (SIMD = wave % 4) all four SIMDs keep work.
  const bool narrow = !kTN && N - n0 <= BN2 / 2;
  const int rbase = narrow ? (wave & 3) * 64 : (wave >> 2) * 128;
  const int cbase = narrow ? (wave >> 2) * 64 : (wave & 3) * 64;
  const int na_max = narrow ? 2 : 4;  // 32-row blocks the wave owns
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- global -> LDS loaders (2 + 2 instructions per wave per stage) ----
  // "rows" form: instruction d of this wave covers stage rows 16*(8d + wave)
  // .. +15, four lanes per 64-byte row; a k chunk past Kd reads as zero.
  const int r_row_l = lane >> 2;
  const int r_chunk = a_swz(r_row_l, lane & 3);  // (row >> 2) & 3 is d- and wave-invariant
  // "cols" form: instruction d covers k rows 2*(8d + wave) .. +1, 32 lanes per
  // 512-byte row; k rows past the contraction range lie beyond num_records.
  const int c_row0 = (lane >> 5) + 2 * wave;     // (row & 3) is d-invariant
  const int c_chunk = (lane & 31) ^ (4 * (c_row0 & 3));
  // A rows past the tile's valid rows are not fetched (they read as zero and
  // their outputs are never stored): a segment's last tile moves only its
  // own rows.  Likewise the weight columns past N in the row-major form
  // (which would otherwise read the next k row's first columns).
  bool a_live[kDma];
#pragma unroll
  for (int d = 0; d < kDma; ++d) a_live[d] = kTN || 16 * (8 * d + wave) + r_row_l < rows;
  const bool b_live = kBRows || kTN || n0 + c_chunk * 8 < N;
  // A
  u32x4 ra_src;
  uint32_t a_off, a_dstride, a_kstride;
  if (kARows) {
    // rows [row0, a_rows) of A are addressable; rows past the segment are
    // read but their outputs never stored
    ra_src = make_rsrc_words(A + (size_t)row0 * Kd, (long long)(a_rows - row0) * Kd * 2);
    a_off = (uint32_t)((r_row_l + 16 * wave) * Kd + r_chunk * 8) * 2;
    a_dstride = (uint32_t)(8 * 16 * Kd) * 2;
    a_kstride = BK2 * 2;
  } else {
    // TN: A_g^T; k rows are the segment's packed rows, columns row0.. of A
    ra_src = make_rsrc_words(A + (size_t)k_begin * M + row0,
                             ((long long)(k_end - k_begin) * M - row0) * 2);
    a_off = (uint32_t)(c_row0 * M + c_chunk * 8) * 2;
    a_dstride = (uint32_t)(16 * M) * 2;
    a_kstride = (uint32_t)(BK2 * M) * 2;
  }
  // B
  u32x4 rb_src;
  uint32_t b_off, b_dstride, b_kstride;
  if (kBRows) {
    // NT: B_g^T rows n0.. (rows past N lie beyond num_records)
    rb_src = make_rsrc_words(B + ((size_t)seg * N + n0) * Kd, (long long)(N - n0) * Kd * 2);
    b_off = (uint32_t)((r_row_l + 16 * wave) * Kd + r_chunk * 8) * 2;
    b_dstride = (uint32_t)(8 * 16 * Kd) * 2;
    b_kstride = BK2 * 2;
  } else if (kTN) {
    rb_src = make_rsrc_words(B + (size_t)k_begin * N + n0,
                             ((long long)(k_end - k_begin) * N - n0) * 2);
    b_off = (uint32_t)(c_row0 * N + c_chunk * 8) * 2;
    b_dstride = (uint32_t)(16 * N) * 2;
    b_kstride = (uint32_t)(BK2 * N) * 2;
  } else {
    // NN: this expert's slice from column n0 on
    rb_src = make_rsrc_words(B + (size_t)seg * Kd * N + n0, ((long long)Kd * N - n0) * 2);
    b_off = (uint32_t)(c_row0 * N + c_chunk * 8) * 2;
    b_dstride = (uint32_t)(16 * N) * 2;
    b_kstride = (uint32_t)(BK2 * N) * 2;
  }

  // load d (0, 1: A; 2, 3: B) of step kt into the stage at LDS address st
  auto dma = [&](uint32_t st, int d, int kt) {
    const int k0 = kt * BK2;
    if (d < kDma) {
      const uint32_t off = a_off + d * a_dstride + (uint32_t)kt * a_kstride;
      dma_load16(st + (8 * d + wave) * 1024,
                 kARows ? (k0 + r_chunk * 8 < Kd && a_live[d] ? off : kOob) : off, ra_src);
    } else {
      const uint32_t off = b_off + (d - kDma) * b_dstride + (uint32_t)kt * b_kstride;
      dma_load16(st + BM2 * BK2 * 2 + (8 * (d - kDma) + wave) * 1024,
                 kBRows ? (k0 + r_chunk * 8 < Kd ? off : kOob) : (b_live ? off : kOob), rb_src);
    }
  };
  auto stage_addr = [&](int kt) {
    return __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(kt % kStages) * kStageBytes);
  };

  // ---- LDS -> register operand addresses (relative to a stage) ----
  // "rows" fragment of row r, substep ks: row r, chunk 2ks + kh (b128).
  // "cols" fragment of column c: lane group g = lane/16, i = lane%16 reads k
  // row (g>>1)*8 + i/4 (+4 for the high half, +16 per substep) at column
  // c + (g&1)*16 + 4*(i%4) of its 32-column block.
  const int bg = lane >> 4, bi = lane & 15;
  const int c_krow = (bg >> 1) * 8 + (bi >> 2);
  auto cols_addr = [&](int col) {
    const int c = col + (bg & 1) * 16 + 4 * (bi & 3);
    const int chunk = (c >> 3) ^ (4 * (c_krow & 3));
    return (uint32_t)c_krow * 512 + (uint32_t)chunk * 16 + (uint32_t)(c & 7) * 2;
  };
  uint32_t a_rd[4];  // rows form: [ks] (2 used); cols form: [i]
  if (kARows) {
#pragma unroll
    for (int ks = 0; ks < kSub; ++ks)
      a_rd[ks] = (uint32_t)(rbase + rr) * (BK2 * 2) + (uint32_t)(a_swz(rr, 2 * ks + kh) * 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) a_rd[i] = cols_addr(rbase + i * 32);
  }
  uint32_t b_rd[2];
  if (kBRows) {
#pragma unroll
    for (int ks = 0; ks < kSub; ++ks)
      b_rd[ks] = BM2 * BK2 * 2 + (uint32_t)(cbase + rr) * (BK2 * 2) +
                 (uint32_t)(a_swz(rr, 2 * ks + kh) * 16);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) b_rd[j] = BM2 * BK2 * 2 + cols_addr(cbase + j * 32);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // The loop below is instantiated for NA = 0..4 active 32-row blocks of
  // the wave's 128 rows: in a segment's last tile the waves skip the MFMAs
  // and A-fragment reads of rows past the segment (rows form only; TN tiles
  // always run NA = 4).  Each SIMD holds one wave of each row half, so the
  // skipped work shortens the tile.  Every instantiation issues the same
  // LDS-direct loads and barriers.
  // Operand fragments of one k-substep (16 k): NA of A, 2 of B (none if
  // NA = 0).
  auto read_ops = [&](auto na_c, uint32_t st, int ks, bf16x8* a, bf16x8* b) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      a[i] = kARows ? lds_read_b128(st + a_rd[ks] + i * 32 * BK2 * 2)
                    : lds_read_tr_pair(st + a_rd[i] + ks * 8192, st + a_rd[i] + ks * 8192 + 2048);
    if (NA > 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = kBRows ? lds_read_b128(st + b_rd[ks] + j * 32 * BK2 * 2)
                      : lds_read_tr_pair(st + b_rd[j] + ks * 8192, st + b_rd[j] + ks * 8192 + 2048);
    }
  };
  // 8 LDS reads (12 with A in cols form) spread between 8 MFMAs (mask 0x008
  // MFMA, 0x100 DS read).
  auto mma_reads = [&](auto na_c, const bf16x8* a, const bf16x8* b) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 2 * NA; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kARows ? 1 : (kBRows ? 1 : 2), 0);
    }
  };
  // The last substep's MFMAs with the refill loads of step kt_fill between
  // them (one after every second MFMA slot).
  auto mma_refill = [&](auto na_c, const bf16x8* a, const bf16x8* b, int kt_fill) {
    constexpr int NA = decltype(na_c)::value;
    const uint32_t st = stage_addr(kt_fill);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = t >> 1, j = t & 1;
      if (i < NA)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
      if (t & 1) dma(st, t >> 1, kt_fill);
    }
  };

  // Software pipeline, one barrier per K-step (BK = 32 = two substeps):
  //   read substep-1 operands (Q) of step kt  | MFMAs of substep 0 (P)
  //   wait: step kt+1's loads landed (own), own LDS reads done; barrier
  //   read substep-0 operands (P) of step kt+1 | MFMAs of substep 1 (Q),
  //                                              refill step kt+kStages-1
  // Ring: step kt lives in slot kt % kStages.  Iteration kt refills slot
  // (kt-1) % kStages, whose last reads every wave completed before this
  // iteration's barrier.  At the wait of iteration kt this wave has issued
  // steps up to kt+kStages-2, so allowing kStages-3 steps in flight means
  // step kt+1 has landed; after the barrier it has landed for every wave.
  // These counts hold only while the LDS-direct loads are the kernel's only
  // vector-memory instructions in the loop: the build refuses a spill
  // (scratch loads and stores would count too), and so does the launcher.
  const int KT = (k_end - k_begin + BK2 - 1) / BK2;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    const uint32_t st = stage_addr(s);
#pragma unroll
    for (int d = 0; d < 2 * kDma; ++d) dma(st, d, s);
  }
  wait_vmcnt<(kStages - 2) * 2 * kDma>();  // step 0 landed (own loads)
  block_barrier();                          // ... and every wave's
  auto k_loop = [&](auto na_c) {
    bf16x8 pa[4], pb[2], qa[4], qb[2];
    read_ops(na_c, lds0, 0, pa, pb);
    for (int kt = 0; kt < KT; ++kt) {
      const uint32_t st = lds0 + (uint32_t)(kt % kStages) * kStageBytes;
      const uint32_t st1 = lds0 + (uint32_t)((kt + 1) % kStages) * kStageBytes;
      read_ops(na_c, st, 1, qa, qb);
      mma_reads(na_c, pa, pb);
      wait_vmcnt<(kStages - 3) * 2 * kDma>();
      wait_lgkm0();
      block_barrier();
      read_ops(na_c, st1, 0, pa, pb);  // past the last step: harmless reads of a landed stage
      mma_refill(na_c, qa, qb, kt + kStages - 1);  // past K: zeros into a slot never read
    }
  };
  using NA4 = std::integral_constant<int, 4>;
  if (kTN) {
    k_loop(NA4{});
  } else {
    // active 32-row blocks of this wave (wave-uniform)
    const int na = __builtin_amdgcn_readfirstlane(min(max((rows - rbase + 31) >> 5, 0), na_max));
    if (na == 4) k_loop(NA4{});
    else if (na == 3) k_loop(std::integral_constant<int, 3>{});
    else if (na == 2) k_loop(std::integral_constant<int, 2>{});
    else if (na == 1) k_loop(std::integral_constant<int, 1>{});
    else k_loop(std::integral_constant<int, 0>{});
  }
  wait_vmcnt<0>();  // drain the loads issued past the end before the grid exits

  // Epilogue straight from registers: lane owns row m of each 32x32 tile and
  // four runs of 4 consecutive columns, 8 g + 4 kh .. +3 (g = 0..3).  Lanes m
  // and m + 32 hold the two halves of every 8-column group, so one exchange
  // of a 4-value half per pair of groups gives each lane 8 consecutive
  // columns: lane kh = 0 stores columns 16 p .. 16 p + 7, kh = 1 columns
  // 16 p + 8 .. 16 p + 15, one 16-byte store each (the weight-gradient form
  // stores its fp32 groups of 4 directly).
  // GELU' and accumulate read a bf16 tensor that may be C itself: every
  // value this lane needs is loaded before the first store (one memory
  // latency per tile, not one per store the loads could not pass).
  constexpr bool kReads = EPI == kEpiGeluGrad || EPI == kEpiAccum;
  u32x2 rd[kReads ? 4 : 1][kReads ? 2 : 1][kReads ? 4 : 1];
  if (kReads) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = rbase + i * 32 + rr;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = n0 + cbase + j * 32 + 8 * g + 4 * kh;
          const bf16* src = EPI == kEpiGeluGrad ? Ep : (const bf16*)Cv;
          rd[kReads ? i : 0][kReads ? j : 0][kReads ? g : 0] =
              i < na_max && m < rows && c < N ? *(const u32x2*)(src + (size_t)(row0 + m) * N + c)
                                              : u32x2{0u, 0u};
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = rbase + i * 32 + rr;
    if (i >= na_max || m >= rows) continue;  // uniform over the lane pair (m, m + 32)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (kTN) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + cbase + j * 32 + 8 * g + 4 * kh;
          if (n < N) {
            float* crow = (float*)Cv + ((size_t)seg * M + row0 + m) * N;
            *(f32x4*)(crow + n) = f32x4{acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                                        acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          }
        }
        continue;
      }
      bf16* crow = (bf16*)Cv;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int nb = n0 + cbase + j * 32 + 16 * p;  // first column of the pair
        u32x2 d[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int g = 2 * p + h;
          const bool ok = nb + 8 * h < N;  // whole 8-column group in or out (N % 8 == 0)
          const size_t at = (size_t)(row0 + m) * N + nb + 8 * h + 4 * kh;
          float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
          float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if (EPI == kEpiGeluSave && ok)
            *(u32x2*)(Ep + at) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          if (EPI == kEpiGelu || EPI == kEpiGeluSave) {
            v0 = gelu_tanh_f32(v0);
            v1 = gelu_tanh_f32(v1);
            v2 = gelu_tanh_f32(v2);
            v3 = gelu_tanh_f32(v3);
          } else if (EPI == kEpiGeluGrad) {
            const u32x2 u = rd[kReads ? i : 0][kReads ? j : 0][kReads ? g : 0];
            v0 *= gelu_tanh_grad_f32(bf16_lo(u[0]));
            v1 *= gelu_tanh_grad_f32(bf16_hi(u[0]));
            v2 *= gelu_tanh_grad_f32(bf16_lo(u[1]));
            v3 *= gelu_tanh_grad_f32(bf16_hi(u[1]));
          } else if (EPI == kEpiAccum) {
            const u32x2 c = rd[kReads ? i : 0][kReads ? j : 0][kReads ? g : 0];
            v0 += bf16_lo(c[0]);
            v1 += bf16_hi(c[0]);
            v2 += bf16_lo(c[1]);
            v3 += bf16_hi(c[1]);
          }
          d[h] = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
        // kh = 0 needs its partner's first group, kh = 1 its partner's second
        const u32x2 send = kh ? d[0] : d[1];
        const uint32_t x0 = (uint32_t)__shfl_xor((int)send[0], 32, kWave);
        const uint32_t x1 = (uint32_t)__shfl_xor((int)send[1], 32, kWave);
        const u32x4 o = kh ? u32x4{x0, x1, d[1][0], d[1][1]} : u32x4{d[0][0], d[0][1], x0, x1};
        const int c0 = nb + 8 * kh;
        if (c0 < N) *(u32x4*)(crow + (size_t)(row0 + m) * N + c0) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Four-wave form: 256 x 256 x 32 tiles, one wave per SIMD owning a 128 x 128
// block as 8 x 8 v_mfma_f32_16x16x32_bf16 tiles (256 fp32 accumulators per
// lane, in AGPRs).  Same layouts and epilogues as the eight-wave kernel.
//
// Why a second kernel: the eight-wave kernel runs its MFMAs ~75% of its
// cycles at only ~1.5 GHz.  With one wave per SIMD and 128 x 128 per wave, a
// K-step reads 64 KiB of fragments from LDS per CU instead of 96, and the
// clock holds ~1.7-1.8 GHz (an MFMA-only loop of this shape holds ~2.0); the
// four waves must then hide their own latencies, which the schedule below
// does.
//
// Stage layout and LDS-direct loads as in the eight-wave kernel (4-stage
// ring, 32 KiB stages), except the chunk swizzles.  "cols" form: chunk c of k
// row k is stored at c ^ (4 (k & 3) + 2 ((k >> 3) & 1)); the fragment of k
// rows 8g .. 8g+7 that lane group g reads by transposing reads would
// otherwise put the rows k and k + 8 of one read on the same banks.  "rows"
// form: chunk c of row m at c ^ ((m >> 1) & 3).  Here the 16 lanes of a
// quarter-wave read 16 consecutive rows of one k chunk, and the eight-wave
// kernel's key (m >> 2) & 3 gave every such read a 2-way conflict (a third of
// the LDS's busy cycles, SQ_LDS_BANK_CONFLICT); this key gives none.  Each
// key was chosen by measuring the read pattern alone: the eight-wave and
// MXFP8 reads (32 rows per chunk) conflict with this key and not with theirs.
//
// Per K-step: wait until step kt+1 has landed for every wave (s_waitcnt on
// the own loads, then the barrier), then 64 MFMAs on fragments read during
// the previous step, in 8 groups of 8; group i also reads fragment i of both
// operands for step kt+1 and issues refill load i of step kt + D + 1, D the
// prefetch distance.  D = 2 (row-major form) refills slot kt - 1, which every
// wave finished reading during step kt - 2.  D = 3 (transposed forms of the
// backward, whose loads arrive later) refills slot kt itself, read during
// step kt - 1: each wave first waits for its own LDS reads (lgkmcnt 0), then
// the barrier.  Measured: D = 3 takes the expert backward from 25.3 to
// 24.7 ms, and costs the forward 1% (the exposed wait for the last
// fragment reads).  A fragment is 8 consecutive k (k chunk l / 16) of one row
// or column (l % 16) per lane.  With the operands swapped, lane l holds row
// l % 16 and columns 4 (l / 16) .. +3 of each 16 x 16 output tile.
//
// A segment's last tile runs the loop instantiated for fewer 16-row groups
// (their A rows are not fetched either).  A tile with at most 128 valid
// columns (row-major forms) uses 4 x 1 waves of 64 x 128 instead of 2 x 2 of
// 128 x 128, so no wave multiplies only zeros.
//
// Address arithmetic in the loop.  With one wave per SIMD, every instruction
// besides the MFMAs takes an issue slot of the wave that the MFMA stream
// competes for (an MFMA-only loop of this shape loses 11-12% of its rate to
// one independent VALU instruction per MFMA, issued in a group per round).
// When the contraction is a multiple of BK2 and A is in "rows" form
// (row-major and transposed-weight forms), no load crosses the contraction's
// end: each lane's load offsets are then fixed for the tile (those of invalid
// rows or columns already past num_records) and the K-step advance rides in
// the buffer instruction's scalar offset, and the "rows" fragment reads of a
// pair of steps share one per-lane base (slots 2q and 2q + 1, the second at
// an immediate +kStageBytes) made by an opaque add, so that the reads differ
// by immediate offsets only.  Per two K-steps that leaves 17 VALU
// instructions beside the 128 MFMAs instead of 76 (the transposing reads'
// XOR-swizzled addresses still take one add each; giving them per-pair bases
// as well was 1.8% slower).  Measured A/B on one box: expert FFN 12.13 ->
// 11.67 ms at T=32768 H=4096 E=8 top-2 h=14336, its backward 25.2 -> 24.9 ms,
// outputs bitwise equal.
// The epilogue's exchange between the lanes l and l ^ 16 (rows 2q and 2q + 1
// of 16 lanes), which hold the 4-column groups g0 and g1 of one row: the lane
// of the even row gets its own g0 and then its partner's, the lane of the odd
// row its partner's g1 and then its own, i.e. 8 consecutive columns each.
// v_permlane16_swap trades the odd rows of its first operand for the even
// rows of its second, all in the VALU (no LDS round trip per exchange).
__device__ __forceinline__ u32x4 pair_rows16(u32x2 g0, u32x2 g1) {
  const auto s0 = __builtin_amdgcn_permlane16_swap(g0[0], g1[0], false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(g0[1], g1[1], false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}
constexpr int kW4Threads = 256;
constexpr int kW4Dma = 4;  // LDS-direct loads per operand, per wave, per stage
__device__ __forceinline__ int w4_swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }
template <int LAYOUT, int EPI>
__global__ __launch_bounds__(kW4Threads, 1) void k_grouped_gemm_w4(
    const bf16* __restrict__ A, const bf16* __restrict__ B, void* Cv, bf16* Ep,
    const int32_t* __restrict__ offsets, int G, int fixed_rows, int a_rows, int mt_bound, int M,
    int Kd, int N, int xcd_chunk) {
  constexpr bool kTN = LAYOUT == kGemmTN;
  constexpr bool kARows = !kTN;               // A in "rows" form
  constexpr bool kBRows = LAYOUT == kGemmNT;  // B in "rows" form
  // Prefetch distance in K-steps (see the schedule below).
  constexpr int kDist = LAYOUT == kGemmNN ? 2 : 3;
  static_assert(kDist + 1 <= kStages, "a refill needs a free slot");
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  const int nt_count = (N + BN2 - 1) / BN2;
  int mt, nt, seg, row0, rows;
  int k_begin = 0, k_end = Kd;  // contraction range; TN: the segment's packed rows
  {
    const int tile = xcd_tile(blockIdx.x, gridDim.x, xcd_chunk);
    if (kTN) {
      const int mt_count = (M + BM2 - 1) / BM2;
      const int per_seg = mt_count * nt_count;
      if (tile >= G * per_seg) return;
      seg = tile / per_seg;
      decode_tile(tile - seg * per_seg, mt_count, nt_count, mt, nt);
      k_begin = offsets ? offsets[seg] : 0;
      k_end = offsets ? offsets[seg + 1] : fixed_rows;
      row0 = mt * BM2;  // rows of C = columns of A
      rows = min(BM2, M - row0);
    } else {
      if (tile >= mt_bound * nt_count) return;
      decode_tile(tile, mt_bound, nt_count, mt, nt);
      if (!find_segment<BM2>(offsets, G, fixed_rows, mt, seg, row0, rows)) return;
    }
  }
  seg = __builtin_amdgcn_readfirstlane(seg);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  k_begin = __builtin_amdgcn_readfirstlane(k_begin);
  k_end = __builtin_amdgcn_readfirstlane(k_end);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n0 = nt * BN2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- global -> LDS: 4 + 4 loads per wave per stage ----
  // "rows" form: load d covers stage rows 16 (4d + wave) .. +15, four lanes
  // per 64-byte row; k past Kd reads as zero, and so do A rows past the
  // tile's valid rows (not fetched).  "cols" form: load d covers k rows
  // 8d + c_row0 (c_row0 = 2 wave + lane / 32), 32 lanes per 512-byte row, so
  // (k >> 3) & 1 = d & 1; k rows past the contraction range lie beyond
  // num_records, and columns past the operand's width are not fetched.
  const int r_row_l = lane >> 2;
  const int r_chunk = w4_swz(r_row_l, lane & 3);  // (row >> 1) & 3 is d- and wave-invariant
  const int c_row0 = (lane >> 5) + 2 * wave;
  const int c_chunk0 = (lane & 31) ^ (4 * (c_row0 & 3)), c_chunk1 = c_chunk0 ^ 2;
  // A
  u32x4 ra_src;
  uint32_t a_off0, a_off1, a_dstride, a_kstride;
  bool a_live[kW4Dma];
  if (kARows) {
    ra_src = make_rsrc_words(A + (size_t)row0 * Kd, (long long)(a_rows - row0) * Kd * 2);
    a_off0 = a_off1 = (uint32_t)((r_row_l + 16 * wave) * Kd + r_chunk * 8) * 2;
    a_dstride = (uint32_t)(4 * 16 * Kd) * 2;
    a_kstride = BK2 * 2;
#pragma unroll
    for (int d = 0; d < kW4Dma; ++d) a_live[d] = 16 * (4 * d + wave) + r_row_l < rows;
  } else {
    // TN: A_g^T; k rows are the segment's packed rows, columns row0.. of A
    ra_src = make_rsrc_words(A + (size_t)k_begin * M + row0,
                             ((long long)(k_end - k_begin) * M - row0) * 2);
    a_off0 = (uint32_t)(c_row0 * M + c_chunk0 * 8) * 2;
    a_off1 = (uint32_t)(c_row0 * M + c_chunk1 * 8) * 2;
    a_dstride = (uint32_t)(8 * M) * 2;
    a_kstride = (uint32_t)(BK2 * M) * 2;
#pragma unroll
    for (int d = 0; d < kW4Dma; ++d) a_live[d] = row0 + ((d & 1) ? c_chunk1 : c_chunk0) * 8 < M;
  }
  // B
  u32x4 rb_src;
  uint32_t b_off0, b_off1, b_dstride, b_kstride;
  bool b_live0 = true, b_live1 = true;
  if (kBRows) {
    // NT: B_g^T rows n0.. (rows past N lie beyond num_records)
    rb_src = make_rsrc_words(B + ((size_t)seg * N + n0) * Kd, (long long)(N - n0) * Kd * 2);
    b_off0 = b_off1 = (uint32_t)((r_row_l + 16 * wave) * Kd + r_chunk * 8) * 2;
    b_dstride = (uint32_t)(4 * 16 * Kd) * 2;
    b_kstride = BK2 * 2;
  } else {
    rb_src = kTN ? make_rsrc_words(B + (size_t)k_begin * N + n0,
                                   ((long long)(k_end - k_begin) * N - n0) * 2)
                 : make_rsrc_words(B + (size_t)seg * Kd * N + n0, ((long long)Kd * N - n0) * 2);
    b_off0 = (uint32_t)(c_row0 * N + c_chunk0 * 8) * 2;
    b_off1 = (uint32_t)(c_row0 * N + c_chunk1 * 8) * 2;
    b_dstride = (uint32_t)(8 * N) * 2;
    b_kstride = (uint32_t)(BK2 * N) * 2;
    b_live0 = n0 + c_chunk0 * 8 < N;
    b_live1 = n0 + c_chunk1 * 8 < N;
  }
  // Fixed-offset loads (contraction a multiple of BK2, not the TN form): a
  // lane's offsets, invalid ones already past num_records, and the K-step
  // advance as the scalar offset.  Whether or not the range check counts the
  // scalar offset, the result is the same: a valid offset plus the advance
  // stays inside the operand.
  // The loop also issues the refills of up to kDist + 1 steps past the last
  // one (never read): their advance is clamped to the last step's, so that
  // every load stays inside its operand whichever reading holds, with no
  // per-lane instruction.
  const bool kfast = !kTN && Kd > 0 && Kd % BK2 == 0;
  const int kt_last = Kd / BK2 - 1;
  uint32_t av[kW4Dma], bv[kW4Dma];
#pragma unroll
  for (int d = 0; d < kW4Dma; ++d) {
    av[d] = a_live[d] ? ((d & 1) ? a_off1 : a_off0) + d * a_dstride : kOob;
    bv[d] = (kBRows || ((d & 1) ? b_live1 : b_live0)) ? ((d & 1) ? b_off1 : b_off0) + d * b_dstride
                                                      : kOob;
  }
  auto dma_fast = [&](uint32_t st, int d, int kt) {
    const uint32_t kc = (uint32_t)min(kt, kt_last);
    if (d < kW4Dma)
      dma_load16_s(st + (4 * d + wave) * 1024, av[d], kc * a_kstride, ra_src);
    else
      dma_load16_s(st + BM2 * BK2 * 2 + (4 * (d - kW4Dma) + wave) * 1024, bv[d - kW4Dma],
                   kc * b_kstride, rb_src);
  };
  auto dma = [&](uint32_t st, int d, int kt) {
    if (d < kW4Dma) {
      const uint32_t off = ((d & 1) ? a_off1 : a_off0) + d * a_dstride + (uint32_t)kt * a_kstride;
      const bool ok = kARows ? kt * BK2 + r_chunk * 8 < Kd && a_live[d] : a_live[d];
      dma_load16(st + (4 * d + wave) * 1024, ok ? off : kOob, ra_src);
    } else {
      const int e = d - kW4Dma;
      const uint32_t off = ((e & 1) ? b_off1 : b_off0) + e * b_dstride + (uint32_t)kt * b_kstride;
      const bool ok = kBRows ? kt * BK2 + r_chunk * 8 < Kd : ((e & 1) ? b_live1 : b_live0);
      dma_load16(st + BM2 * BK2 * 2 + (4 * e + wave) * 1024, ok ? off : kOob, rb_src);
    }
  };
  auto stage_addr = [&](int kt) {
    return __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(kt % kStages) * kStageBytes);
  };

  // ---- wave block and fragment addresses ----
  // Row-major forms: the 16 row groups of the tile are dealt to the two waves
  // of a column half in turn (group g to row-wave g % 2), so that a segment's
  // last tile, whose valid rows are a prefix, gives every SIMD (one wave
  // each) about the same number of groups to multiply.  The narrow layout
  // (four waves of 64 contiguous rows) and the weight-gradient form (A in
  // "cols" form, contiguous 128-row blocks) keep contiguous groups.
  const bool narrow = !kTN && N - n0 <= BN2 / 2;
  const bool inter = !kTN && !narrow;
  const int r0 = kTN ? (wave >> 1) * 128 : (narrow ? wave * 64 : 16 * (wave >> 1));
  const int rstep = inter ? 32 : 16;  // rows between a wave's groups
  const int cbase = narrow ? 0 : (wave & 1) * 128;
  const int li = lane & 15, lg = lane >> 4;
  // "rows" fragment f: row r + f * step + li of the rows r, r + step, ...
  // (step 16 for the weight operand, rstep for A), k chunk lg (one b128 read
  // at + 64 step f).  "cols" fragment f of a block
  // starting at column c0 (a multiple of 128): columns c0 + 16 f + 4 (li %
  // 4) .. +3 of k rows 8 lg + li / 4 and, +2048 bytes, 4 rows further (two
  // transposing reads give lane column li, k 8 lg .. +7); with the swizzle,
  // the 32-byte column step f becomes an XOR with 32 (f ^ (2 (li / 4) +
  // lg % 2)).
  auto rows_rd = [&](int r0) { return (uint32_t)(r0 + li) * 64 + 16 * w4_swz(li, lg); };
  auto cols_rd = [&](int c0) {
    return (uint32_t)(8 * lg + (li >> 2)) * 512 + 16 * (c0 / 8 + ((li >> 1) & 1)) + 8 * (li & 1) +
           32 * (2 * (li >> 2) + (lg & 1));
  };
  const uint32_t a_rd = kARows ? rows_rd(r0) : cols_rd(r0);
  const uint32_t b_rd = BM2 * BK2 * 2 + (kBRows ? rows_rd(cbase) : cols_rd(cbase));
  auto frag = [&](bool rows_form, uint32_t st, uint32_t rd, uint32_t fstride, int f) {
    if (rows_form) return lds_read_b128(st + rd + f * fstride);
    const uint32_t ad = st + (rd ^ (32u * f));
    return lds_read_tr_pair(ad, ad + 2048);
  };
  // this wave's row groups that hold rows (8 = all, the common case), rounded
  // up to a pair: the loop is instantiated for 0, 2, 4, 6, 8
  const int ng = __builtin_amdgcn_readfirstlane(
      min(max((((rows - r0 + rstep - 1) >> (inter ? 5 : 4)) + 1) & ~1, 0), narrow ? 4 : 8));

  f32x4 acc[8][8];  // set by the first step's MFMAs (zero C operand)
  auto mma = [&](auto first_c, int i, int j, const bf16x8* a, const bf16x8* b) {
    if (decltype(first_c)::value)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], f32x4{0.f, 0.f, 0.f, 0.f},
                                                          0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  };
  // One K-step with the MFMAs of the first NG groups.  The first step's
  // accumulators start from a zero C operand, so that the compiler never
  // materialises 256 zeros in ordinary registers.
  // The per-lane address of a "rows" fragment read, stage slot included,
  // made once per pair of steps by an opaque add (a pair reads slots 2q and
  // 2q + 1, the second at +kStageBytes): the reads then differ only by
  // immediate offsets, where the compiler would otherwise keep 8 hoisted
  // per-fragment addresses and add the stage base to each.
  auto rows_base = [&](uint32_t st, uint32_t rd) {
    uint32_t r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(st), "v"(rd));
    return r;
  };
  auto step = [&](auto ng_c, auto first_c, auto afs_c, auto fast_c, int kt, const bf16x8* ca,
                  const bf16x8* cb, bf16x8* na, bf16x8* nb, uint32_t ra, uint32_t rb) {
    constexpr int NG = decltype(ng_c)::value;
    constexpr uint32_t AFS = decltype(afs_c)::value;  // A fragment stride (rows form)
    wait_vmcnt<(kDist - 1) * 2 * kW4Dma>();  // younger than step kt+1: kDist - 1 steps
    if (kDist == 3) wait_lgkm0();  // this wave's reads of slot kt (refilled below) are done
    block_barrier();
    const uint32_t st1 = stage_addr(kt + 1);
    const uint32_t stf = stage_addr(kt + kDist + 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < NG) {
#pragma unroll
        for (int j = 0; j < 8; ++j) mma(first_c, i, j, ca, cb);
      } else if (decltype(first_c)::value) {
        // defined on every path (the epilogue skips these groups)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (decltype(fast_c)::value) {
        na[i] = lds_read_b128(ra + i * AFS);  // A is in "rows" form here
        nb[i] = kBRows ? lds_read_b128(rb + i * 1024) : frag(false, st1, b_rd, 1024, i);
      } else {
        na[i] = frag(kARows, st1, a_rd, AFS, i);
        nb[i] = frag(kBRows, st1, b_rd, 1024, i);
      }
      if (decltype(fast_c)::value)
        dma_fast(stf, i, kt + kDist + 1);
      else
        dma(stf, i, kt + kDist + 1);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };
  using kTrue = std::integral_constant<bool, true>;
  using kFalse = std::integral_constant<bool, false>;
  const int KT = (k_end - k_begin + BK2 - 1) / BK2;
  // These vmcnt counts hold only while the LDS-direct loads are the loop's
  // only vector-memory instructions: the build refuses a spill.
  auto k_loop = [&](auto ng_c, auto afs_c, auto fast_c) {
    constexpr uint32_t AFS = decltype(afs_c)::value;
#pragma unroll
    for (int s = 0; s <= kDist; ++s) {
      const uint32_t st = stage_addr(s);
#pragma unroll
      for (int d = 0; d < 2 * kW4Dma; ++d) {
        if (decltype(fast_c)::value)
          dma_fast(st, d, s);
        else
          dma(st, d, s);
      }
    }
    wait_vmcnt<kDist * 2 * kW4Dma>();  // step 0 landed (own loads)
    block_barrier();                   // ... and every wave's
    bf16x8 pa[8], pb[8], qa[8], qb[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      pa[f] = frag(kARows, lds0, a_rd, AFS, f);
      pb[f] = frag(kBRows, lds0, b_rd, 1024, f);
    }
    constexpr bool F = decltype(fast_c)::value;
    {
      const uint32_t st = stage_addr(1);
      const uint32_t ra = F ? rows_base(st, a_rd) : 0u, rb = F && kBRows ? rows_base(st, b_rd) : 0u;
      step(ng_c, kTrue{}, afs_c, fast_c, 0, pa, pb, qa, qb, ra, rb);
    }
    int kt = 1;
    for (; kt + 1 < KT; kt += 2) {
      const uint32_t st = stage_addr(kt + 1);  // slot 2 or 0; the pair's second step reads the next
      const uint32_t ra = F ? rows_base(st, a_rd) : 0u, rb = F && kBRows ? rows_base(st, b_rd) : 0u;
      step(ng_c, kFalse{}, afs_c, fast_c, kt, qa, qb, pa, pb, ra, rb);
      step(ng_c, kFalse{}, afs_c, fast_c, kt + 1, pa, pb, qa, qb, ra + kStageBytes,
           rb + kStageBytes);
    }
    if (kt < KT) {
      const uint32_t st = stage_addr(kt + 1);
      const uint32_t ra = F ? rows_base(st, a_rd) : 0u, rb = F && kBRows ? rows_base(st, b_rd) : 0u;
      step(ng_c, kFalse{}, afs_c, fast_c, kt, qa, qb, pa, pb, ra, rb);
    }
  };
  // a segment's last tile, and the narrow layout, run fewer groups
  using Inter = std::integral_constant<uint32_t, 32 * 64>;
  using Contig = std::integral_constant<uint32_t, 16 * 64>;
  auto by_ng = [&](auto afs_c, auto fast_c) {
    if (ng == 8) k_loop(std::integral_constant<int, 8>{}, afs_c, fast_c);
    else if (ng == 6) k_loop(std::integral_constant<int, 6>{}, afs_c, fast_c);
    else if (ng == 4) k_loop(std::integral_constant<int, 4>{}, afs_c, fast_c);
    else if (ng == 2) k_loop(std::integral_constant<int, 2>{}, afs_c, fast_c);
    else k_loop(std::integral_constant<int, 0>{}, afs_c, fast_c);
  };
  if (kfast) {
    if (inter) by_ng(Inter{}, kTrue{});
    else by_ng(Contig{}, kTrue{});
  } else {
    if (inter) by_ng(Inter{}, kFalse{});
    else by_ng(Contig{}, kFalse{});
  }
  wait_vmcnt<0>();  // drain the loads issued past the end before the grid exits

  // ---- epilogue: lane holds row r0 + rstep i + li, columns cbase + 16 j +
  // 4 lg .. +3.  The weight-gradient form stores its fp32 groups of 4
  // directly.  The bf16 forms pair tiles (2p, 2p + 1): even lg stores
  // columns 16 (2p) + 4 lg .. +7 (its own 4 and its partner's, lane l ^ 16),
  // odd lg columns 16 (2p + 1) + 4 (lg - 1) .. +7.  Each lane reads what it
  // needs of Ep / C (GELU', accumulate) for its own 4 columns before the
  // exchange, so an in-place epilogue reads every element before it is
  // written.
  // The lane's coordinates are recomputed here from a fresh lane id (an
  // instruction the compiler cannot hoist): kept live across the K loop they
  // would not fit beside its fragments and spill, and a spill's scratch
  // accesses would upset the loop's counted vmcnt waits.
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int li_e = lane_e & 15, lg_e = lane_e >> 4;
  const bool odd = lg_e & 1;
  const int r0_e = kTN ? (wave >> 1) * 128 : (narrow ? wave * 64 : 16 * (wave >> 1));
  const int rstep_e = inter ? 32 : 16;
  const int cbase_e = narrow ? 0 : (wave & 1) * 128;
  // GELU' and accumulate read a bf16 tensor that may be C itself: every
  // value this lane needs is loaded before the first store (one memory
  // latency per tile, not one per store the loads could not pass).
  constexpr bool kReads = EPI == kEpiGeluGrad || EPI == kEpiAccum;
  u32x2 rd[kReads ? 8 : 1][kReads ? 8 : 1];
  if (kReads) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = r0_e + rstep_e * i + li_e;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = n0 + cbase_e + 16 * j + 4 * lg_e;
        const bf16* src = EPI == kEpiGeluGrad ? Ep : (const bf16*)Cv;
        rd[kReads ? i : 0][kReads ? j : 0] =
            i < ng && m < rows && c < N ? *(const u32x2*)(src + (size_t)(row0 + m) * N + c)
                                        : u32x2{0u, 0u};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = r0_e + rstep_e * i + li_e;
    if (i >= ng || m >= rows) continue;  // uniform over the lane pair (l, l ^ 16)
    if (kTN) {
      float* crow = (float*)Cv + ((size_t)seg * M + row0 + m) * N;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = n0 + cbase_e + 16 * j + 4 * lg_e;
        if (c < N) *(f32x4*)(crow + c) = acc[i][j];
      }
      continue;
    }
    bf16* crow = (bf16*)Cv + (size_t)(row0 + m) * N;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      u32x2 d[2], us[2];  // output and (train-mode GELU) pre-activation groups
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * p + h;
        float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
        if (EPI == kEpiGeluSave) us[h] = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        if (EPI == kEpiGelu || EPI == kEpiGeluSave) {
          v0 = gelu_tanh_f32(v0);
          v1 = gelu_tanh_f32(v1);
          v2 = gelu_tanh_f32(v2);
          v3 = gelu_tanh_f32(v3);
        } else if (EPI == kEpiGeluGrad) {
          const u32x2 u = rd[kReads ? i : 0][kReads ? j : 0];
          v0 *= gelu_tanh_grad_f32(bf16_lo(u[0]));
          v1 *= gelu_tanh_grad_f32(bf16_hi(u[0]));
          v2 *= gelu_tanh_grad_f32(bf16_lo(u[1]));
          v3 *= gelu_tanh_grad_f32(bf16_hi(u[1]));
        } else if (EPI == kEpiAccum) {
          const u32x2 cc = rd[kReads ? i : 0][kReads ? j : 0];
          v0 += bf16_lo(cc[0]);
          v1 += bf16_hi(cc[0]);
          v2 += bf16_lo(cc[1]);
          v3 += bf16_hi(cc[1]);
        }
        d[h] = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      }
      const u32x4 o = pair_rows16(d[0], d[1]);
      const int c0 = n0 + cbase_e + 16 * (2 * p + (odd ? 1 : 0)) + 4 * (lg_e & ~1);
      if (c0 < N) *(u32x4*)(crow + c0) = o;
      if (EPI == kEpiGeluSave) {  // the pre-activations, paired the same way
        const u32x4 ou = pair_rows16(us[0], us[1]);
        if (c0 < N) *(u32x4*)(Ep + (size_t)(row0 + m) * N + c0) = ou;
      }
    }
  }
}

// fp32 grouped GEMM (plain FMA, 64 x 64 tiles, 4 x 4 outputs per thread), in
// the same layouts and epilogues; operands are gathered with strided loads.
// C and Ep may be the same buffer (the GELU-derivative epilogue in place):
// each element is read, then written, by one thread.
template <int LAYOUT, int EPI>
__global__ __launch_bounds__(256) void k_grouped_gemm_f32(
    const float* __restrict__ A, const float* __restrict__ B, float* C,
    float* Ep, const int32_t* __restrict__ offsets, int G, int fixed_rows,
    int mt_bound, int M, int Kd, int N) {
  constexpr int TM = 64, TN = 64, TK = 16;
  constexpr bool kTN = LAYOUT == kGemmTN;
  __shared__ float sA[TM][TK + 1];
  __shared__ float sB[TK][TN];
  const int nt_count = (N + TN - 1) / TN;
  int mt, nt, seg, row0, rows, k_begin = 0, k_end = Kd;
  if (kTN) {
    const int mt_count = (M + TM - 1) / TM;
    const int per_seg = mt_count * nt_count;
    seg = blockIdx.x / per_seg;
    const int t = blockIdx.x - seg * per_seg;
    mt = t / nt_count;
    nt = t % nt_count;
    k_begin = offsets ? offsets[seg] : 0;
    k_end = offsets ? offsets[seg + 1] : fixed_rows;
    row0 = mt * TM;
    rows = min(TM, M - row0);
  } else {
    mt = blockIdx.x / nt_count;
    nt = blockIdx.x % nt_count;
    if (!find_segment<TM>(offsets, G, fixed_rows, mt, seg, row0, rows)) return;
  }
  const int n0 = nt * TN;
  const int klen = k_end - k_begin;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < klen; k0 += TK) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + 256 * j;
      const int r = idx >> 4, c = idx & 15;  // A element (row0 + r, k0 + c)
      float av = 0.0f;
      if (r < rows && k0 + c < klen)
        av = kTN ? A[(size_t)(k_begin + k0 + c) * M + row0 + r] : A[(size_t)(row0 + r) * Kd + k0 + c];
      sA[r][c] = av;
      const int kr = idx >> 6, nc = idx & 63;  // B element (k0 + kr, n0 + nc)
      float bv = 0.0f;
      if (k0 + kr < klen && n0 + nc < N) {
        if (LAYOUT == kGemmNN) bv = B[((size_t)seg * Kd + k0 + kr) * N + n0 + nc];
        else if (LAYOUT == kGemmNT) bv = B[((size_t)seg * N + n0 + nc) * Kd + k0 + kr];
        else bv = B[(size_t)(k_begin + k0 + kr) * N + n0 + nc];
      }
      sB[kr][nc] = bv;
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
      if (c >= N) continue;
      float v = acc[i][j];
      if (kTN) {
        C[((size_t)seg * M + row0 + r) * N + c] = v;
        continue;
      }
      const size_t at = (size_t)(row0 + r) * N + c;
      if (EPI == kEpiGeluSave) Ep[at] = v;
      if (EPI == kEpiGelu || EPI == kEpiGeluSave) v = gelu_tanh_f32(v);
      else if (EPI == kEpiGeluGrad) v *= gelu_tanh_grad_f32(Ep[at]);
      else if (EPI == kEpiAccum) v += C[at];
      C[at] = v;
    }
  }
}

static int mt_bound_for(const GemmArgs& a, int tm) {
  if (!a.offsets) return (a.fixed_rows + tm - 1) / tm;
  return (a.max_rows + tm - 1) / tm + a.G;
}

// Layouts that run on the four-wave kernel (the others, and contractions of
// at most two K-steps, on the eight-wave one).
#ifndef MOE_W4_LAYOUTS
#define MOE_W4_LAYOUTS 7  // bit per layout: NN 1, NT 2, TN 4
#endif
template <int LAYOUT>
constexpr bool kUseW4 = ((MOE_W4_LAYOUTS >> LAYOUT) & 1) != 0;

template <int LAYOUT, int EPI>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t st) {
  const hipError_t e = allow_dynamic_lds<k_grouped_gemm_bf16<LAYOUT, EPI>, true>();
  if (e != hipSuccess) return e;
  const int ntc = (a.N + BN2 - 1) / BN2;
  int mtb = 0;
  long long grid;
  if (LAYOUT == kGemmTN) {
    grid = (long long)a.G * ((a.M + BM2 - 1) / BM2) * ntc;
  } else {
    mtb = mt_bound_for(a, BM2);
    grid = (long long)mtb * ntc;
  }
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // A contraction of one or two K-steps (the d_logits W_r^T accumulate: E
  // rounded up to 8) is all epilogue, which eight waves share better.
  if (kUseW4<LAYOUT> && (LAYOUT == kGemmTN || a.Kd > 2 * BK2)) {
    const hipError_t e4 = allow_dynamic_lds<k_grouped_gemm_w4<LAYOUT, EPI>, true>();
    if (e4 != hipSuccess) return e4;
    k_grouped_gemm_w4<LAYOUT, EPI><<<(unsigned)grid, kW4Threads, kSmem2, st>>>(
        (const bf16*)a.A, (const bf16*)a.B, a.C, (bf16*)a.E, a.offsets, a.G, a.fixed_rows,
        a.offsets ? a.max_rows : a.fixed_rows, mtb, a.M, a.Kd, a.N, xcd_chunk_for(ntc));
    return hipGetLastError();
  }
  k_grouped_gemm_bf16<LAYOUT, EPI><<<(unsigned)grid, kGemmThreads, kSmem2, st>>>(
      (const bf16*)a.A, (const bf16*)a.B, a.C, (bf16*)a.E, a.offsets, a.G, a.fixed_rows,
      a.offsets ? a.max_rows : a.fixed_rows, mtb, a.M, a.Kd, a.N, xcd_chunk_for(ntc));
  return hipGetLastError();
}

template <int LAYOUT, int EPI>
static hipError_t launch_f32(const GemmArgs& a, hipStream_t st) {
  const int ntc = (a.N + 63) / 64;
  int mtb = 0;
  long long grid;
  if (LAYOUT == kGemmTN) {
    grid = (long long)a.G * ((a.M + 63) / 64) * ntc;
  } else {
    mtb = mt_bound_for(a, 64);
    grid = (long long)mtb * ntc;
  }
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  k_grouped_gemm_f32<LAYOUT, EPI><<<(unsigned)grid, 256, 0, st>>>(
      (const float*)a.A, (const float*)a.B, (float*)a.C, (float*)a.E, a.offsets, a.G,
      a.fixed_rows, mtb, a.M, a.Kd, a.N);
  return hipGetLastError();
}

// The (layout, epilogue) pairs the layer uses.
#define MOE_GEMM_DISPATCH(LAUNCH)                                               \
  switch (a.layout * 8 + a.epi) {                                               \
    case kGemmNN * 8 + kEpiStore: return LAUNCH<kGemmNN, kEpiStore>(a, st);     \
    case kGemmNN * 8 + kEpiGelu: return LAUNCH<kGemmNN, kEpiGelu>(a, st);       \
    case kGemmNN * 8 + kEpiGeluSave: return LAUNCH<kGemmNN, kEpiGeluSave>(a, st); \
    case kGemmNT * 8 + kEpiStore: return LAUNCH<kGemmNT, kEpiStore>(a, st);     \
    case kGemmNT * 8 + kEpiGeluGrad: return LAUNCH<kGemmNT, kEpiGeluGrad>(a, st); \
    case kGemmNT * 8 + kEpiAccum: return LAUNCH<kGemmNT, kEpiAccum>(a, st);     \
    case kGemmTN * 8 + kEpiStore: return LAUNCH<kGemmTN, kEpiStore>(a, st);     \
    default: return hipErrorInvalidValue;                                       \
  }

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  MOE_GEMM_DISPATCH(launch_bf16)
}

hipError_t launch_grouped_gemm_f32(const GemmArgs& a, hipStream_t st) {
  MOE_GEMM_DISPATCH(launch_f32)
}
#undef MOE_GEMM_DISPATCH

}  // namespace moe
