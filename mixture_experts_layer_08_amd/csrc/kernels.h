// Internal launch interface between the C-ABI layer (api.hip) and the
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

// Tokens per route block: the unit of the router's workgroups and of the
// per-block histograms / in-block ranks the permutation builds on.
constexpr int kRouteBlock = 64;

struct RouteArgs {
  bool bf16;
  bool logits_in;
  const void* x;
  const void* w_r;
  const float* bias;
  void* wT;            // bf16 [E_pad][H] scratch (bf16 mode)
  float* logits;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* hist;       // [E][nblk]
  float* psum;         // [E][nblk]
  int32_t* lrank;      // [T][K]
  int T, H, E, K;
};

size_t route_lds_bytes(int E);
int route_col_tiles(int E);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

struct PermuteArgs {
  bool bf16;
  const void* x;
  const int32_t* topk_ids;
  const int32_t* hist;
  const int32_t* lrank;
  int32_t* base;       // [E][nblk] scratch
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

struct GemmArgs {
  const void* A;        // [rows][Kd]
  const void* B;        // [G][Kd][N]
  void* C;              // [rows][N]
  const int32_t* offsets;  // [G+1] device, or nullptr: one group of fixed_rows rows
  int G;
  int fixed_rows;
  int max_rows;         // upper bound on offsets[G] (sizes the grid)
  int Kd, N;
  int gelu;             // 1: C = GELU_tanh(A B), 0: C = A B
};
hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, hipStream_t st);
hipError_t launch_grouped_gemm_f32(const GemmArgs& a, hipStream_t st);

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

hipError_t launch_aux(const int32_t* hist, const float* psum, float* aux, int T, int E, int K,
                      int nblk, hipStream_t st);

}  // namespace moe
