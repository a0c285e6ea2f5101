// C ABI of the MoE-layer forward (declared in include/moe.h): argument
// validation, workspace layout and kernel launches.  Every check runs on the
// host before any HIP call, so invalid arguments never reach a kernel.
#include <math.h>
#include <string.h>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct WsLayout {
  size_t wT, hist, psum, base, lrank, total;
};

int n_route_blocks(const moe_shape* s) { return (s->T + kRouteBlock - 1) / kRouteBlock; }

WsLayout ws_layout(const moe_shape* s) {
  WsLayout L{};
  const size_t nblk = (size_t)n_route_blocks(s);
  size_t off = 0;
  L.wT = off;
  if (s->dtype == MOE_BF16) off += align_up((size_t)route_col_tiles(s->E) * 16 * s->H * 2);
  L.hist = off;
  off += align_up((size_t)s->E * nblk * 4);
  L.psum = off;
  off += align_up((size_t)s->E * nblk * 4);
  L.base = off;
  off += align_up((size_t)s->E * nblk * 4);
  L.lrank = off;
  off += align_up((size_t)s->T * s->K * 4);
  L.total = off;
  return L;
}

moe_status check_ws(const moe_shape* s, const void* ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & (kAlign - 1))) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(s).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer, bad size or misaligned pointer";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside what the kernels support";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_size()";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch or runtime call failed";
    default: return "unknown moe_status";
  }
}

moe_status moe_check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 1 || s->H < 1 || s->E < 1 || s->K < 1 || s->h_exp < 1 || s->h_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->K > s->E) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->flags & ~MOE_FLAG_LOGITS_IN) return MOE_ERR_INVALID_ARG;
  if (!isfinite(s->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (s->K > 8 || s->E > 256) return MOE_ERR_UNSUPPORTED;
  if (s->H % 8 || s->h_exp % 8 || s->h_shared % 8) return MOE_ERR_UNSUPPORTED;
  // int32 row indices and element offsets inside one row-block stay in range
  const long long TK = (long long)s->T * s->K;
  if (TK >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (s->H > (1 << 20) || s->h_exp > (1 << 20) || s->h_shared > (1 << 20))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t moe_capacity(const moe_shape* s) {
  if (moe_check_shape(s) != MOE_OK) return -1;
  const double cf = (double)s->capacity_factor;
  if (cf <= 0.0) return s->T;
  const double c = ceil(cf * (double)((long long)s->T * s->K) / (double)s->E);
  if (c >= (double)s->T) return s->T;  // no expert can receive more than T
  return (int64_t)c;
}

int64_t moe_max_rows(const moe_shape* s) {
  const int64_t C = moe_capacity(s);
  if (C < 0) return -1;
  const int64_t TK = (int64_t)s->T * s->K, EC = (int64_t)s->E * C;
  return TK < EC ? TK : EC;
}

size_t moe_workspace_size(const moe_shape* s) {
  if (moe_check_shape(s) != MOE_OK) return 0;
  return ws_layout(s).total;
}

moe_status moe_route(const moe_shape* s, const void* x, const void* w_router,
                     const float* b_router, float* logits, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  const bool lin = (s->flags & MOE_FLAG_LOGITS_IN) != 0;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!lin && (!x || !w_router || !aligned16(x) || !aligned16(w_router)))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  RouteArgs a{};
  a.bf16 = s->dtype == MOE_BF16;
  a.logits_in = lin;
  a.x = x;
  a.w_r = w_router;
  a.bias = b_router;
  a.wT = at<void>(ws, L.wT);
  a.logits = logits;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.hist = at<int32_t>(ws, L.hist);
  a.psum = at<float>(ws, L.psum);
  a.lrank = at<int32_t>(ws, L.lrank);
  a.T = s->T;
  a.H = s->H;
  a.E = s->E;
  a.K = s->K;
  return hip_status(launch_route(a, (hipStream_t)stream));
}

moe_status moe_aux_loss(const moe_shape* s, const void* ws, size_t ws_bytes, float* aux,
                        void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!aux) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  void* w = const_cast<void*>(ws);
  return hip_status(launch_aux(at<int32_t>(w, L.hist), at<float>(w, L.psum), aux, s->T, s->E,
                               s->K, n_route_blocks(s), (hipStream_t)stream));
}

moe_status moe_permute(const moe_shape* s, const void* x, const int32_t* topk_ids, void* ws,
                       size_t ws_bytes, int32_t* counts, int32_t* kept, int32_t* offsets,
                       int32_t* row_of, int32_t* token_of, int32_t* n_dropped, void* xp,
                       void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!x || !topk_ids || !counts || !kept || !offsets || !row_of || !token_of || !n_dropped ||
      !xp)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(xp)) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  PermuteArgs a{};
  a.bf16 = s->dtype == MOE_BF16;
  a.x = x;
  a.topk_ids = topk_ids;
  a.hist = at<int32_t>(ws, L.hist);
  a.lrank = at<int32_t>(ws, L.lrank);
  a.base = at<int32_t>(ws, L.base);
  a.counts = counts;
  a.kept = kept;
  a.offsets = offsets;
  a.row_of = row_of;
  a.token_of = token_of;
  a.n_dropped = n_dropped;
  a.xp = xp;
  a.T = s->T;
  a.H = s->H;
  a.E = s->E;
  a.K = s->K;
  a.C = (int)moe_capacity(s);
  return hip_status(launch_permute(a, (hipStream_t)stream));
}

moe_status moe_expert_ffn(const moe_shape* s, const void* xp, const int32_t* offsets,
                          const void* w1, const void* w2, void* hbuf, void* out, const void* x,
                          const void* ws1, const void* ws2, void* hshared, void* shared_out,
                          void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!xp || !offsets || !w1 || !w2 || !hbuf || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(xp) || !aligned16(w1) || !aligned16(w2) || !aligned16(hbuf) ||
      !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  const bool shared = s->h_shared > 0;
  if (shared) {
    if (!x || !ws1 || !ws2 || !hshared || !shared_out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(ws1) || !aligned16(ws2) || !aligned16(hshared) ||
        !aligned16(shared_out))
      return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const bool bf = s->dtype == MOE_BF16;
  auto gemm = [&](const GemmArgs& g) {
    return bf ? launch_grouped_gemm_bf16(g, (hipStream_t)stream)
              : launch_grouped_gemm_f32(g, (hipStream_t)stream);
  };
  const int max_rows = (int)moe_max_rows(s);
  GemmArgs g1{xp, w1, hbuf, offsets, s->E, 0, max_rows, s->H, s->h_exp, 1};
  GemmArgs g2{hbuf, w2, out, offsets, s->E, 0, max_rows, s->h_exp, s->H, 0};
  hipError_t e = gemm(g1);
  if (e == hipSuccess) e = gemm(g2);
  if (e == hipSuccess && shared) {
    GemmArgs s1{x, ws1, hshared, nullptr, 1, s->T, s->T, s->H, s->h_shared, 1};
    GemmArgs s2{hshared, ws2, shared_out, nullptr, 1, s->T, s->T, s->h_shared, s->H, 0};
    e = gemm(s1);
    if (e == hipSuccess) e = gemm(s2);
  }
  return hip_status(e);
}

moe_status moe_combine(const moe_shape* s, const void* out, const int32_t* row_of,
                       const float* topk_w, const void* shared_out, void* y, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!out || !row_of || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(y) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  CombineArgs a{};
  a.bf16 = s->dtype == MOE_BF16;
  a.out = out;
  a.row_of = row_of;
  a.topk_w = topk_w;
  a.shared_out = s->h_shared > 0 ? shared_out : nullptr;
  a.y = y;
  a.T = s->T;
  a.H = s->H;
  a.K = s->K;
  if (s->h_shared > 0 && !shared_out) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(a, (hipStream_t)stream));
}

}  // extern "C"
