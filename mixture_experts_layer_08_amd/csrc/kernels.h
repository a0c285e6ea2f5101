// Internal launch interface between the C-ABI layer (api.hip) and the
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

namespace moe {

// Tokens per route block: the unit of the router's workgroups and of the
// per-block histograms / in-block ranks the permutation builds on.
constexpr int kRouteBlock = 64;

// Router variant of section 3.1 of the dpshk.com "MoE module infra notes":
// selection scores (logits + Gumbel noise) / tau.  active = gumbel || tau != 1.
struct RouterNoise {
  int active;
  int gumbel;
  float tau;
  unsigned long long seed;
  unsigned long long offset;
};

struct RouteArgs {
  bool bf16;
  bool logits_in;
  const void* x;
  const void* w_r;
  const float* bias;
  float* logits;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* hist;       // [E][nblk]
  float* psum;         // [E][nblk]
  int32_t* lrank;      // [T][K]
  int T, H, E, K;
  RouterNoise noise;
};

size_t route_lds_bytes(int E);
int route_col_tiles(int E);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
hipError_t launch_count_nonfinite(const float* v, size_t n, long long* count, hipStream_t st);

struct PermuteArgs {
  bool bf16;
  const void* x;
  const int32_t* topk_ids;
  const int32_t* lrank;
  const int32_t* base;  // [E][nblk] from moe_aux_loss's block scan
  const int32_t* cnt;   // [E] per-expert assignment counts, from the same scan
  const int32_t* seg;   // [2E + 2] offsets, kept, n_dropped, from the same scan
  int32_t* counts;
  int32_t* kept;
  int32_t* offsets;
  int32_t* row_of;
  int32_t* token_of;
  int32_t* n_dropped;
  void* xp;
  int T, H, E, K;
  int C;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);

// The dispatch copy in MXFP8: bf16 token rows quantised on the way (mx.h),
// codes [max_rows][H] and operand-layout scales (leading dimension xp_ld);
// optionally also every token's own row (x_q [T][H], scales with ld T).
struct PermuteMx8Args {
  const void* x;       // bf16 [T][H]
  const int32_t* topk_ids;
  const int32_t* lrank;
  const int32_t* base;
  const int32_t* cnt;
  const int32_t* seg;
  int32_t* counts;
  int32_t* kept;
  int32_t* offsets;
  int32_t* row_of;
  int32_t* token_of;
  int32_t* n_dropped;
  uint8_t* xp_q;
  uint8_t* xp_s;
  int xp_ld;
  uint8_t* x_q;        // nullable
  uint8_t* x_s;
  int T, H, E, K;
  int C;
};
hipError_t launch_permute_mx8(const PermuteMx8Args& a, hipStream_t st);

// Operand layouts of the grouped GEMM (the contraction runs over K):
//   kGemmNN: A [rows][Kd], B [G][Kd][N] -> C [rows][N]; rows segmented by offsets
//   kGemmNT: A [rows][Kd], B [G][N][Kd] -> C [rows][N]; rows segmented by offsets
//   kGemmTN: A [rows][M],  B [rows][N]  -> C [G][M][N] (fp32); K = the rows of
//            segment g, so C[g] = A_g^T B_g (a per-expert weight gradient)
enum GemmLayout { kGemmNN = 0, kGemmNT = 1, kGemmTN = 2 };
// Epilogues of NN / NT (TN always stores the fp32 accumulators):
//   kEpiStore C = acc;  kEpiGelu C = GELU(acc);  kEpiGeluSave C = GELU(acc), E = acc;
//   kEpiGeluGrad C = acc * GELU'(E);  kEpiAccum C = C + acc.
enum GemmEpi { kEpiStore = 0, kEpiGelu = 1, kEpiGeluSave = 2, kEpiGeluGrad = 3, kEpiAccum = 4 };

struct GemmArgs {
  int layout = kGemmNN;
  int epi = kEpiStore;
  const void* A = nullptr;
  const void* B = nullptr;
  void* C = nullptr;
  void* E = nullptr;               // epilogue tensor [rows][N] (written or read, see GemmEpi)
  const int32_t* offsets = nullptr;  // [G+1] device, or nullptr: one segment of fixed_rows rows
  int G = 1;
  int fixed_rows = 0;
  int max_rows = 0;                // upper bound on offsets[G] (sizes the NN / NT grid)
  int M = 0;                       // TN: rows of each C block (columns of A)
  int Kd = 0;                      // NN / NT: contraction length
  int N = 0;                       // columns of B and C
};
hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, hipStream_t st);
hipError_t launch_grouped_gemm_f32(const GemmArgs& a, hipStream_t st);

// MXFP8 grouped GEMM (mx.h for the formats):
//   A [a_rows][Kd] codes + As (operand layout, leading dimension a_ld),
//   B [G][N][Kd] codes + Bs [G][ceil(Kd/128)][N][4],
//   C [rows][N] codes + Cs: row layout [rows][N/32] (kMxEpiQuantRows) or
//   operand layout with leading dimension c_ld (kMxEpiGeluQuantOperand).
// Kd is a multiple of 64, N of 32.
enum MxEpi { kMxEpiQuantRows = 0, kMxEpiGeluQuantOperand = 1 };
struct MxGemmArgs {
  int epi = kMxEpiQuantRows;
  const uint8_t* A = nullptr;
  const uint8_t* As = nullptr;
  int a_ld = 0;
  const uint8_t* B = nullptr;
  const uint8_t* Bs = nullptr;
  uint8_t* C = nullptr;
  uint8_t* Cs = nullptr;
  int c_ld = 0;
  const int32_t* offsets = nullptr;  // [G+1] device, or nullptr: one segment of fixed_rows rows
  int G = 1;
  int fixed_rows = 0;
  int max_rows = 0;
  int Kd = 0;
  int N = 0;
};
hipError_t launch_grouped_gemm_mx8(const MxGemmArgs& a, hipStream_t st);

struct CombineArgs {
  bool bf16;
  const void* out;
  const int32_t* row_of;
  const float* topk_w;
  const void* shared_out;
  void* y;
  int T, H, K;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// MXFP8 combine: out_q [rows][H] codes with row-layout scales [rows][H/32];
// sh_q / sh_s the same for the shared expert's [T][H] output (nullable);
// y bf16 [T][H].
struct CombineMx8Args {
  const uint8_t* out_q;
  const uint8_t* out_s;
  const int32_t* row_of;
  const float* topk_w;
  const uint8_t* sh_q;
  const uint8_t* sh_s;
  void* y;
  int T, H, K;
};
hipError_t launch_combine_mx8(const CombineMx8Args& a, hipStream_t st);

// w [G][Kd][N] (bf16 or fp32) -> codes [G][N][Kd] + operand-layout scales
// [G][ceil(Kd/128)][N][4] (blocks along Kd).
hipError_t launch_quantize_weight_mx8(const void* w, bool bf16_in, int G, int Kd, int N,
                                      uint8_t* q, uint8_t* s, hipStream_t st);

// The aux loss from the router's per-block partials, and with it the
// permutation's block scan: base [E][nblk] = per-expert exclusive prefix over
// route blocks of the block histograms, cnt [E] = the per-expert totals, seg
// [2E + 2] = segment offsets (E + 1), kept (E) and the number of dropped
// assignments at capacity C.  Up to 16 experts one workgroup does it all;
// more experts are scanned by one wave each over several workgroups, which
// leave their probability totals in p_scratch [E] (doubles) for a second,
// one-workgroup kernel.
hipError_t launch_aux(const int32_t* hist, const float* psum, float* aux, int32_t* base,
                      int32_t* cnt, double* p_scratch, int32_t* seg, int T, int E, int K, int C,
                      int nblk, hipStream_t st);

// ---- backward ----
struct CombineBwdArgs {
  bool bf16;
  const void* dy;
  const void* out;
  const int32_t* row_of;
  const float* topk_w;
  void* d_out;
  float* d_topk_w;
  int T, H, K;
};
hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t st);

// Tokens per chunk of the router weight gradient's first pass (wider for
// many experts, so that its fp32 partials [chunks][H][E] stay small).
inline int route_bwd_chunk(int E) { return E <= 32 ? 512 : (E <= 64 ? 1024 : 2048); }
inline int route_bwd_chunks(int T, int E) { return (T + route_bwd_chunk(E) - 1) / route_bwd_chunk(E); }
// bf16 mode with more than 32 experts computes the router weight gradient on
// MFMA (a TN grouped GEMM over token chunks), else on the vector ALUs.
inline bool route_bwd_uses_mfma(bool bf16, int E) { return bf16 && E > 32; }

struct RouteBwdArgs {
  bool bf16;
  float inv_tau;       // d_logits = (dL/dz) / tau: the gradient of the router GEMM output
  const void* x;
  const float* logits;
  const int32_t* topk_ids;
  const float* topk_w;
  const float* d_topk_w;
  const int32_t* counts;
  float alpha;
  float* d_logits;
  float* d_w_router;
  float* d_b_router;   // nullable
  float* part;         // [chunks][H][E] (or [chunks][E8][H], MFMA form) scratch
  float* dbpart;       // [ceil(T / 64)][E] scratch
  ::moe::bf16* dl16;   // [T][E8] scratch (MFMA form)
  int32_t* chunk_off;  // [chunks + 1] scratch (MFMA form)
  int T, H, E, K;
};
hipError_t launch_route_bwd(const RouteBwdArgs& a, hipStream_t st);

// dx = the kept slots' d_xp rows (+ d_x_shared); with d_logits set, also
// + bf16(d_logits) W_r^T in the same pass (only where
// permute_bwd_fuses_route holds: bf16, at most 16 experts, W_r within
// kPermuteRouteLds bytes of LDS once padded to a multiple of 8 experts).
constexpr long long kPermuteRouteLds = 64 * 1024;
bool permute_bwd_fuses_route(bool bf16, int H, int E);
struct PermuteBwdArgs {
  bool bf16;
  const void* d_xp;
  const int32_t* row_of;
  const void* d_x_shared;  // nullable
  const float* d_logits;   // nullable: no router term
  const void* w_router;    // [H][E] in the layer dtype, with d_logits
  void* dx;
  int T, H, K, E;
};
hipError_t launch_permute_bwd(const PermuteBwdArgs& a, hipStream_t st);

// dst [R][Ep] bf16 = src [R][E] (fp32 or bf16), zero-padded to Ep columns.
hipError_t launch_pad_bf16(const void* src, bool src_f32, bf16* dst, int R, int E, int Ep,
                           hipStream_t st);

// MFMA-only measurement kernel (ceiling.hip): `workgroups` workgroups of four
// waves run `iters` rounds of 64 v_mfma_f32_16x16x32_bf16 on register
// operands (mode 1: two register sets alternating; 2: a zero-word XOR of
// every operand before each round; 3: 4 x 4 tiles of 32x32x16 MFMAs); out
// gets 4 floats per lane (16 in mode 3).
hipError_t launch_mfma_ceiling(const void* operands, float* out, int workgroups, int iters,
                               int mode, hipStream_t st);

}  // namespace moe
