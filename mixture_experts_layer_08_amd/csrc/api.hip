// C ABI of the MoE layer, forward and backward (declared in include/moe.h):
// argument validation, workspace layout and kernel launches.  Every check
// runs on the host before any HIP call, so invalid arguments never reach a
// kernel.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"
#include "mx.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest byte range the kernels address through one buffer descriptor
// (offsets are unsigned 32-bit and must stay below 2^31).
constexpr long long kBufferBytes = 0x7ffffff0LL;

// Expert capacity C of a shape whose fields have been validated.
int64_t capacity_of(const moe_shape* s) {
  const double cf = (double)s->capacity_factor;
  if (cf <= 0.0) return s->T;
  const double c = ceil(cf * (double)((long long)s->T * s->K) / (double)s->E);
  if (c >= (double)s->T) return s->T;  // no expert can receive more than T
  return (int64_t)c;
}

struct WsLayout {
  size_t hist, psum, base, lrank, cnt, seg, pe;
  // MOE_FLAG_TRAIN only: GELU pre-activations (routed, shared), the router
  // weight gradient's partials, and bf16 copies of d_logits / W_r padded to
  // a multiple of 8 experts for the d_logits * W_r^T GEMM
  size_t preact, preact_sh, part, dbpart, dl8, wr8, chunk_off;
  size_t total;
};

int64_t max_rows_of(const moe_shape* s);
int pad8(int v) { return (v + 7) & ~7; }

int n_route_blocks(const moe_shape* s) { return (s->T + kRouteBlock - 1) / kRouteBlock; }

WsLayout ws_layout(const moe_shape* s) {
  WsLayout L{};
  const size_t nblk = (size_t)n_route_blocks(s);
  size_t off = 0;
  L.hist = off;
  off += align_up((size_t)s->E * nblk * 4);
  L.psum = off;
  off += align_up((size_t)s->E * nblk * 4);
  L.base = off;
  off += align_up((size_t)s->E * nblk * 4);
  L.lrank = off;
  off += align_up((size_t)s->T * s->K * 4);
  L.cnt = off;
  off += align_up((size_t)s->E * 4);
  L.seg = off;
  off += align_up((size_t)(2 * s->E + 2) * 4);
  L.pe = off;  // per-expert probability totals (doubles) between the aux kernels
  off += align_up((size_t)s->E * 8);
  if (s->flags & MOE_FLAG_TRAIN) {
    const size_t elem = s->dtype == MOE_BF16 ? 2 : 4;
    const size_t nch = (size_t)route_bwd_chunks(s->T, s->E);
    L.preact = off;
    off += align_up((size_t)max_rows_of(s) * s->h_exp * elem);
    L.preact_sh = off;
    off += align_up((size_t)s->T * s->h_shared * elem);
    L.part = off;
    off += align_up(nch * s->H * pad8(s->E) * 4);
    L.dbpart = off;
    off += align_up((size_t)((s->T + 63) / 64) * s->E * 4);  // 64-token blocks
    L.dl8 = off;
    if (s->dtype == MOE_BF16) off += align_up((size_t)s->T * pad8(s->E) * 2);
    L.wr8 = off;
    if (s->dtype == MOE_BF16) off += align_up((size_t)s->H * pad8(s->E) * 2);
    L.chunk_off = off;
    off += align_up((nch + 1) * 4);
  }
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

// The router temperature (0 in the shape means 1).
float router_tau_of(const moe_shape* s) { return s->router_tau > 0.0f ? s->router_tau : 1.0f; }

// GEMM over rows (NN / NT): C [rows][N] = A [rows][Kd] * B_g (or B_g^T).
GemmArgs rows_gemm(int layout, int epi, const void* A, const void* B, void* C, void* E,
                   const int32_t* offsets, int G, int fixed_rows, int max_rows, int Kd, int N) {
  GemmArgs g;
  g.layout = layout;
  g.epi = epi;
  g.A = A;
  g.B = B;
  g.C = C;
  g.E = E;
  g.offsets = offsets;
  g.G = G;
  g.fixed_rows = fixed_rows;
  g.max_rows = max_rows;
  g.Kd = Kd;
  g.N = N;
  return g;
}

// Weight-gradient GEMM (TN): C [G][M][N] fp32 = A_g^T [M][rows_g] * B_g [rows_g][N].
GemmArgs tn_gemm(const void* A, const void* B, float* C, const int32_t* offsets, int G,
                 int fixed_rows, int M, int N) {
  GemmArgs g;
  g.layout = kGemmTN;
  g.epi = kEpiStore;
  g.A = A;
  g.B = B;
  g.C = C;
  g.offsets = offsets;
  g.G = G;
  g.fixed_rows = fixed_rows;
  g.M = M;
  g.N = N;
  return g;
}

// The MXFP8 forward: bf16 tokens, hidden sizes that are whole 64-value
// K-steps of the FP8 GEMM, no training mode (the FP8 path is forward only),
// and byte offsets of every FP8 tensor inside the 2 GiB a buffer descriptor
// addresses.
moe_status check_mx_shape(const moe_shape* s);

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

MxGemmArgs mx_gemm(int epi, const uint8_t* A, const uint8_t* As, int a_ld, const uint8_t* B,
                   const uint8_t* Bs, uint8_t* C, uint8_t* Cs, int c_ld,
                   const int32_t* offsets, int G, int fixed_rows, int max_rows, int Kd, int N) {
  MxGemmArgs g;
  g.epi = epi;
  g.A = A;
  g.As = As;
  g.a_ld = a_ld;
  g.B = B;
  g.Bs = Bs;
  g.C = C;
  g.Cs = Cs;
  g.c_ld = c_ld;
  g.offsets = offsets;
  g.G = G;
  g.fixed_rows = fixed_rows;
  g.max_rows = max_rows;
  g.Kd = Kd;
  g.N = N;
  return g;
}

}  // namespace

extern "C" int64_t moe_capacity(const moe_shape* s);

namespace {
int64_t max_rows_of(const moe_shape* s) {
  const int64_t C = moe_capacity(s);
  if (C < 0) return -1;
  const int64_t TK = (int64_t)s->T * s->K, EC = (int64_t)s->E * C;
  return TK < EC ? TK : EC;
}
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
  if (s->flags & ~(MOE_FLAG_LOGITS_IN | MOE_FLAG_TRAIN | MOE_FLAG_GUMBEL))
    return MOE_ERR_INVALID_ARG;
  if (!isfinite(s->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (!isfinite(s->router_tau) || s->router_tau < 0.0f) return MOE_ERR_INVALID_ARG;
  if (s->K > 8 || s->E > 256) return MOE_ERR_UNSUPPORTED;
  if (s->H % 8 || s->h_exp % 8 || s->h_shared % 8) return MOE_ERR_UNSUPPORTED;
  // int32 row indices and element offsets inside one row-block stay in range
  const long long TK = (long long)s->T * s->K;
  if (TK >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (s->H > (1 << 20) || s->h_exp > (1 << 20) || s->h_shared > (1 << 20))
    return MOE_ERR_UNSUPPORTED;
  if (s->dtype == MOE_BF16) {
    // The bf16 grouped GEMM reads a whole weight matrix (one expert's, or
    // the shared expert's) through one buffer descriptor, whose range stays
    // below 2 GiB; so do the weight-gradient GEMMs of training mode with one
    // segment's rows (an expert's at most min(C, T), the shared expert's
    // and the router's T) times an operand width.
    const long long lim = kBufferBytes / 2;  // bf16 elements
    const long long H = s->H, h = s->h_exp, hs = s->h_shared;
    if (H * h > lim || H * hs > lim) return MOE_ERR_UNSUPPORTED;
    if (s->flags & MOE_FLAG_TRAIN) {
      const long long seg = capacity_of(s);
      const long long wide = H > h ? H : h;
      long long wide_t = H > hs ? H : hs;
      if (s->E > wide_t) wide_t = s->E;
      if (seg * wide > lim || (long long)s->T * wide_t > lim) return MOE_ERR_UNSUPPORTED;
    }
  }
  return MOE_OK;
}

int64_t moe_capacity(const moe_shape* s) {
  if (moe_check_shape(s) != MOE_OK) return -1;
  return capacity_of(s);
}

int64_t moe_max_rows(const moe_shape* s) { return max_rows_of(s); }

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
  a.noise.gumbel = (s->flags & MOE_FLAG_GUMBEL) != 0;
  a.noise.tau = router_tau_of(s);
  a.noise.active = a.noise.gumbel || a.noise.tau != 1.0f;
  a.noise.seed = s->noise_seed;
  a.noise.offset = s->noise_offset;
  return hip_status(launch_route(a, (hipStream_t)stream));
}

moe_status moe_count_nonfinite(const moe_shape* s, const float* logits, int64_t* count,
                               void* stream) {
  const moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!logits || !count) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_count_nonfinite(logits, (size_t)s->T * (size_t)s->E,
                                           (long long*)count, (hipStream_t)stream));
}

moe_status moe_mfma_ceiling(const void* operands, float* out, int32_t workgroups, int32_t iters,
                            int32_t mode, void* stream) {
  if (!operands || !out || !aligned16(operands) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (workgroups < 1 || workgroups > (1 << 16) || iters < 1 || iters > (1 << 24) ||
      mode < 0 || mode > 3)
    return MOE_ERR_INVALID_ARG;
  return hip_status(
      launch_mfma_ceiling(operands, out, workgroups, iters, mode, (hipStream_t)stream));
}

moe_status moe_aux_loss(const moe_shape* s, const void* ws, size_t ws_bytes, float* aux,
                        void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!aux) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  void* w = const_cast<void*>(ws);
  return hip_status(launch_aux(at<int32_t>(w, L.hist), at<float>(w, L.psum), aux,
                               at<int32_t>(w, L.base), at<int32_t>(w, L.cnt),
                               at<double>(w, L.pe), at<int32_t>(w, L.seg), s->T, s->E, s->K,
                               (int)capacity_of(s), n_route_blocks(s), (hipStream_t)stream));
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
  a.lrank = at<int32_t>(ws, L.lrank);
  a.base = at<int32_t>(ws, L.base);
  a.cnt = at<int32_t>(ws, L.cnt);
  a.seg = at<int32_t>(ws, L.seg);
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
  const bool train = (s->flags & MOE_FLAG_TRAIN) != 0;
  const WsLayout L = ws_layout(s);
  // GEMM1 (+GELU; with MOE_FLAG_TRAIN the pre-activations are kept), GEMM2
  const GemmArgs g1 = rows_gemm(kGemmNN, train ? kEpiGeluSave : kEpiGelu, xp, w1, hbuf,
                                train ? at<void>(ws, L.preact) : nullptr, offsets, s->E, 0,
                                max_rows, s->H, s->h_exp);
  const GemmArgs g2 = rows_gemm(kGemmNN, kEpiStore, hbuf, w2, out, nullptr, offsets, s->E, 0,
                                max_rows, s->h_exp, s->H);
  hipError_t e = gemm(g1);
  if (e == hipSuccess) e = gemm(g2);
  if (e == hipSuccess && shared) {
    const GemmArgs s1 = rows_gemm(kGemmNN, train ? kEpiGeluSave : kEpiGelu, x, ws1, hshared,
                                  train ? at<void>(ws, L.preact_sh) : nullptr, nullptr, 1, s->T,
                                  s->T, s->H, s->h_shared);
    const GemmArgs s2 = rows_gemm(kGemmNN, kEpiStore, hshared, ws2, shared_out, nullptr, nullptr,
                                  1, s->T, s->T, s->h_shared, s->H);
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


moe_status moe_combine_backward(const moe_shape* s, const void* dy, const void* out,
                                const int32_t* row_of, const float* topk_w, void* d_out,
                                float* d_topk_w, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!dy || !out || !row_of || !topk_w || !d_out || !d_topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(out) || !aligned16(d_out)) return MOE_ERR_INVALID_ARG;
  CombineBwdArgs a{};
  a.bf16 = s->dtype == MOE_BF16;
  a.dy = dy;
  a.out = out;
  a.row_of = row_of;
  a.topk_w = topk_w;
  a.d_out = d_out;
  a.d_topk_w = d_topk_w;
  a.T = s->T;
  a.H = s->H;
  a.K = s->K;
  return hip_status(launch_combine_bwd(a, (hipStream_t)stream));
}

moe_status moe_route_backward(const moe_shape* s, const void* x, const float* logits,
                              const int32_t* topk_ids, const float* topk_w,
                              const float* d_topk_w, const int32_t* counts, float alpha,
                              float* d_logits, float* d_w_router, float* d_b_router,
                              void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!(s->flags & MOE_FLAG_TRAIN)) return MOE_ERR_INVALID_ARG;
  if (!x || !logits || !topk_ids || !topk_w || !d_topk_w || !counts || !d_logits ||
      !d_w_router)
    return MOE_ERR_INVALID_ARG;
  if (!isfinite(alpha)) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  RouteBwdArgs a{};
  a.bf16 = s->dtype == MOE_BF16;
  a.inv_tau = (s->flags & MOE_FLAG_LOGITS_IN) ? 1.0f : 1.0f / router_tau_of(s);
  a.x = x;
  a.logits = logits;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.d_topk_w = d_topk_w;
  a.counts = counts;
  a.alpha = alpha;
  a.d_logits = d_logits;
  a.d_w_router = d_w_router;
  a.d_b_router = d_b_router;
  a.part = at<float>(ws, L.part);
  a.dbpart = at<float>(ws, L.dbpart);
  a.dl16 = at<bf16>(ws, L.dl8);  // the padded bf16 d_logits (also used by moe_permute_backward)
  a.chunk_off = at<int32_t>(ws, L.chunk_off);
  a.T = s->T;
  a.H = s->H;
  a.E = s->E;
  a.K = s->K;
  return hip_status(launch_route_bwd(a, (hipStream_t)stream));
}

moe_status moe_expert_ffn_backward(const moe_shape* s, const void* xp, const int32_t* offsets,
                                   const void* w1, const void* w2, const void* hbuf,
                                   const void* d_out, void* d_xp, float* d_w1, float* d_w2,
                                   const void* x, const void* ws1, const void* ws2,
                                   const void* hshared, const void* dy, void* d_x_shared,
                                   float* d_ws1, float* d_ws2, void* ws, size_t ws_bytes,
                                   void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!(s->flags & MOE_FLAG_TRAIN)) return MOE_ERR_INVALID_ARG;
  if (!xp || !offsets || !w1 || !w2 || !hbuf || !d_out || !d_xp || !d_w1 || !d_w2)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(xp) || !aligned16(w1) || !aligned16(w2) || !aligned16(hbuf) ||
      !aligned16(d_out) || !aligned16(d_xp) || !aligned16(d_w1) || !aligned16(d_w2))
    return MOE_ERR_INVALID_ARG;
  const bool shared = s->h_shared > 0;
  if (shared) {
    if (!x || !ws1 || !ws2 || !hshared || !dy || !d_x_shared || !d_ws1 || !d_ws2)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(ws1) || !aligned16(ws2) || !aligned16(hshared) ||
        !aligned16(dy) || !aligned16(d_x_shared) || !aligned16(d_ws1) || !aligned16(d_ws2))
      return MOE_ERR_INVALID_ARG;
  }
  // (moe_check_shape has already refused bf16 training shapes whose
  // weight-gradient GEMMs would address more than one buffer range.)
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  const bool bf = s->dtype == MOE_BF16;
  auto gemm = [&](const GemmArgs& g) {
    return bf ? launch_grouped_gemm_bf16(g, (hipStream_t)stream)
              : launch_grouped_gemm_f32(g, (hipStream_t)stream);
  };
  const int max_rows = (int)moe_max_rows(s);
  void* u = at<void>(ws, L.preact);  // pre-activations in, d u out (in place)
  // d u = (d_out W2^T) .* GELU'(u);  d W2 = hbuf^T d_out;  d W1 = xp^T d u;  d xp = d u W1^T
  hipError_t e = gemm(rows_gemm(kGemmNT, kEpiGeluGrad, d_out, w2, u, u, offsets, s->E, 0,
                                max_rows, s->H, s->h_exp));
  if (e == hipSuccess) e = gemm(tn_gemm(hbuf, d_out, d_w2, offsets, s->E, 0, s->h_exp, s->H));
  if (e == hipSuccess) e = gemm(tn_gemm(xp, u, d_w1, offsets, s->E, 0, s->H, s->h_exp));
  if (e == hipSuccess)
    e = gemm(rows_gemm(kGemmNT, kEpiStore, u, w1, d_xp, nullptr, offsets, s->E, 0, max_rows,
                       s->h_exp, s->H));
  if (e == hipSuccess && shared) {
    void* us = at<void>(ws, L.preact_sh);
    const int T = s->T, hs = s->h_shared;
    e = gemm(rows_gemm(kGemmNT, kEpiGeluGrad, dy, ws2, us, us, nullptr, 1, T, T, s->H, hs));
    if (e == hipSuccess) e = gemm(tn_gemm(hshared, dy, d_ws2, nullptr, 1, T, hs, s->H));
    if (e == hipSuccess) e = gemm(tn_gemm(x, us, d_ws1, nullptr, 1, T, s->H, hs));
    if (e == hipSuccess)
      e = gemm(rows_gemm(kGemmNT, kEpiStore, us, ws1, d_x_shared, nullptr, nullptr, 1, T, T, hs,
                         s->H));
  }
  return hip_status(e);
}

moe_status moe_permute_backward(const moe_shape* s, const void* d_xp, const int32_t* row_of,
                                const void* d_x_shared, const float* d_logits,
                                const void* w_router, void* dx, void* ws, size_t ws_bytes,
                                void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!(s->flags & MOE_FLAG_TRAIN)) return MOE_ERR_INVALID_ARG;
  if (!d_xp || !row_of || !d_logits || !w_router || !dx) return MOE_ERR_INVALID_ARG;
  if (s->h_shared > 0 && !d_x_shared) return MOE_ERR_INVALID_ARG;
  if (!aligned16(d_xp) || !aligned16(dx) || (d_x_shared && !aligned16(d_x_shared)))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  const bool bf = s->dtype == MOE_BF16;
  hipStream_t hs = (hipStream_t)stream;
  PermuteBwdArgs a{};
  a.bf16 = bf;
  a.d_xp = d_xp;
  a.row_of = row_of;
  a.d_x_shared = s->h_shared > 0 ? d_x_shared : nullptr;
  a.dx = dx;
  a.T = s->T;
  a.H = s->H;
  a.K = s->K;
  a.E = s->E;
  const bool fused = permute_bwd_fuses_route(bf, s->H, s->E);
  if (fused) {
    a.d_logits = d_logits;
    a.w_router = w_router;
  }
  hipError_t e = launch_permute_bwd(a, hs);
  // Otherwise dx += d_logits W_r^T: an NT GEMM with K = E accumulating into
  // dx; in bf16 mode over copies padded to a multiple of 8 experts (16-byte
  // rows)
  if (e == hipSuccess && !fused) {
    if (bf) {
      const int E8 = pad8(s->E);
      bf16* dl8 = at<bf16>(ws, L.dl8);
      bf16* wr8 = at<bf16>(ws, L.wr8);
      e = launch_pad_bf16(d_logits, true, dl8, s->T, s->E, E8, hs);
      if (e == hipSuccess) e = launch_pad_bf16(w_router, false, wr8, s->H, s->E, E8, hs);
      if (e == hipSuccess)
        e = launch_grouped_gemm_bf16(rows_gemm(kGemmNT, kEpiAccum, dl8, wr8, dx, nullptr,
                                               nullptr, 1, s->T, s->T, E8, s->H),
                                     hs);
    } else {
      e = launch_grouped_gemm_f32(rows_gemm(kGemmNT, kEpiAccum, d_logits, w_router, dx, nullptr,
                                            nullptr, 1, s->T, s->T, s->E, s->H),
                                  hs);
    }
  }
  return hip_status(e);
}

// ---------------------------------------------------------------------------
// MXFP8 forward
// ---------------------------------------------------------------------------

size_t moe_mx_operand_scale_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  size_t n;
  if (__builtin_mul_overflow((uint64_t)((cols + 127) / 128), (uint64_t)rows, &n) ||
      __builtin_mul_overflow(n, (size_t)4, &n))
    return 0;
  return n;
}

size_t moe_mx_weight_code_bytes(int32_t batch, int32_t K, int32_t N) {
  if (batch < 1 || K < 1 || N < 1) return 0;
  const uint64_t rows = ((uint64_t)N + kMxPanelRows - 1) / kMxPanelRows * kMxPanelRows;
  size_t n;
  if (__builtin_mul_overflow(rows, (uint64_t)K, &n) ||
      __builtin_mul_overflow(n, (uint64_t)batch, &n))
    return 0;
  return n;
}

moe_status moe_quantize_weights_mxfp8(const void* w, int32_t dtype, int32_t batch, int32_t K,
                                      int32_t N, uint8_t* q, uint8_t* scales, void* stream) {
  if (!w || !q || !scales) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (batch < 1 || K < 1 || N < 1) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(q) || !aligned4(scales)) return MOE_ERR_INVALID_ARG;
  if (K % 64 || N % 32) return MOE_ERR_UNSUPPORTED;
  if ((long long)N * K > 0x7ffffff0LL) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_weight_mx8(w, dtype == MOE_BF16, batch, K, N, q, scales,
                                               (hipStream_t)stream));
}

moe_status moe_permute_mxfp8(const moe_shape* s, const void* x, const int32_t* topk_ids,
                             void* ws, size_t ws_bytes, int32_t* counts, int32_t* kept,
                             int32_t* offsets, int32_t* row_of, int32_t* token_of,
                             int32_t* n_dropped, uint8_t* xp_q, uint8_t* xp_s, uint8_t* x_q,
                             uint8_t* x_s, void* stream) {
  moe_status st = check_mx_shape(s);
  if (st != MOE_OK) return st;
  if (!x || !topk_ids || !counts || !kept || !offsets || !row_of || !token_of || !n_dropped ||
      !xp_q || !xp_s)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(xp_q) || !aligned4(xp_s)) return MOE_ERR_INVALID_ARG;
  const bool shared = s->h_shared > 0;
  if (shared && (!x_q || !x_s || !aligned16(x_q) || !aligned4(x_s))) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  PermuteMx8Args a{};
  a.x = x;
  a.topk_ids = topk_ids;
  a.lrank = at<int32_t>(ws, L.lrank);
  a.base = at<int32_t>(ws, L.base);
  a.cnt = at<int32_t>(ws, L.cnt);
  a.seg = at<int32_t>(ws, L.seg);
  a.counts = counts;
  a.kept = kept;
  a.offsets = offsets;
  a.row_of = row_of;
  a.token_of = token_of;
  a.n_dropped = n_dropped;
  a.xp_q = xp_q;
  a.xp_s = xp_s;
  a.xp_ld = (int)moe_max_rows(s);
  a.x_q = shared ? x_q : nullptr;
  a.x_s = shared ? x_s : nullptr;
  a.T = s->T;
  a.H = s->H;
  a.E = s->E;
  a.K = s->K;
  a.C = (int)moe_capacity(s);
  return hip_status(launch_permute_mx8(a, (hipStream_t)stream));
}

moe_status moe_expert_ffn_mxfp8(const moe_shape* s, const uint8_t* xp_q, const uint8_t* xp_s,
                                const int32_t* offsets, const uint8_t* w1_q,
                                const uint8_t* w1_s, const uint8_t* w2_q, const uint8_t* w2_s,
                                uint8_t* h_q, uint8_t* h_s, uint8_t* out_q, uint8_t* out_s,
                                const uint8_t* x_q, const uint8_t* x_s, const uint8_t* ws1_q,
                                const uint8_t* ws1_s, const uint8_t* ws2_q,
                                const uint8_t* ws2_s, uint8_t* hsh_q, uint8_t* hsh_s,
                                uint8_t* sh_q, uint8_t* sh_s, void* stream) {
  moe_status st = check_mx_shape(s);
  if (st != MOE_OK) return st;
  const void* need[] = {xp_q, xp_s, offsets, w1_q, w1_s, w2_q, w2_s, h_q, h_s, out_q, out_s};
  for (const void* p : need)
    if (!p || !aligned4(p)) return MOE_ERR_INVALID_ARG;
  const void* codes[] = {xp_q, w1_q, w2_q, h_q, out_q};
  for (const void* p : codes)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  const bool shared = s->h_shared > 0;
  if (shared) {
    const void* need_sh[] = {x_q, x_s, ws1_q, ws1_s, ws2_q, ws2_s, hsh_q, hsh_s, sh_q, sh_s};
    for (const void* p : need_sh)
      if (!p || !aligned4(p)) return MOE_ERR_INVALID_ARG;
    const void* codes_sh[] = {x_q, ws1_q, ws2_q, hsh_q, sh_q};
    for (const void* p : codes_sh)
      if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  }
  const hipStream_t hs = (hipStream_t)stream;
  const int max_rows = (int)moe_max_rows(s);
  // GEMM1 + GELU -> h (operand-layout scales for GEMM2), GEMM2 -> out (row layout for combine)
  hipError_t e = launch_grouped_gemm_mx8(
      mx_gemm(kMxEpiGeluQuantOperand, xp_q, xp_s, max_rows, w1_q, w1_s, h_q, h_s, max_rows,
              offsets, s->E, 0, max_rows, s->H, s->h_exp),
      hs);
  if (e == hipSuccess)
    e = launch_grouped_gemm_mx8(mx_gemm(kMxEpiQuantRows, h_q, h_s, max_rows, w2_q, w2_s, out_q,
                                        out_s, 0, offsets, s->E, 0, max_rows, s->h_exp, s->H),
                                hs);
  if (e == hipSuccess && shared) {
    e = launch_grouped_gemm_mx8(mx_gemm(kMxEpiGeluQuantOperand, x_q, x_s, s->T, ws1_q, ws1_s,
                                        hsh_q, hsh_s, s->T, nullptr, 1, s->T, s->T, s->H,
                                        s->h_shared),
                                hs);
    if (e == hipSuccess)
      e = launch_grouped_gemm_mx8(mx_gemm(kMxEpiQuantRows, hsh_q, hsh_s, s->T, ws2_q, ws2_s,
                                          sh_q, sh_s, 0, nullptr, 1, s->T, s->T, s->h_shared,
                                          s->H),
                                  hs);
  }
  return hip_status(e);
}

moe_status moe_combine_mxfp8(const moe_shape* s, const uint8_t* out_q, const uint8_t* out_s,
                             const int32_t* row_of, const float* topk_w, const uint8_t* sh_q,
                             const uint8_t* sh_s, void* y, void* stream) {
  moe_status st = check_mx_shape(s);
  if (st != MOE_OK) return st;
  if (!out_q || !out_s || !row_of || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out_q) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  const bool shared = s->h_shared > 0;
  if (shared && (!sh_q || !sh_s || !aligned16(sh_q))) return MOE_ERR_INVALID_ARG;
  CombineMx8Args a{};
  a.out_q = out_q;
  a.out_s = out_s;
  a.row_of = row_of;
  a.topk_w = topk_w;
  a.sh_q = shared ? sh_q : nullptr;
  a.sh_s = shared ? sh_s : nullptr;
  a.y = y;
  a.T = s->T;
  a.H = s->H;
  a.K = s->K;
  return hip_status(launch_combine_mx8(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {
moe_status check_mx_shape(const moe_shape* s) {
  const moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->flags & MOE_FLAG_TRAIN) return MOE_ERR_UNSUPPORTED;
  if (s->H % 64 || s->h_exp % 64 || s->h_shared % 64) return MOE_ERR_UNSUPPORTED;
  const long long rows = moe_max_rows(s);
  const long long wide = s->H > s->h_exp ? s->H : s->h_exp;
  const long long wide_sh = s->H > s->h_shared ? s->H : s->h_shared;
  if (rows * wide > kBufferBytes || (long long)s->T * wide_sh > kBufferBytes ||
      (long long)s->H * s->h_exp > kBufferBytes || (long long)s->H * s->h_shared > kBufferBytes)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free forward: the five calls with the workspace in a static
// device array (for callers that cannot allocate).
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kStaticWsBytes = (size_t)16 << 20;

// The workspace of moe_forward_noalloc.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code this name is only a
// stand-in: its device address on the current device comes from
// hipGetSymbolAddress (static_ws_ptr), and only that address is ever given to
// a kernel.  Nothing in it needs to start at zero: every region a call reads
// (block histograms, softmax partials and ranks from moe_route; block bases,
// counts and segments from moe_aux_loss) is written earlier in the same call.
static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];

std::mutex g_static_ws_mu;
void* g_static_ws[64];

// scratch's address on the current device, looked up once per device with
// that device current.
hipError_t static_ws_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_static_ws_mu);
  if (!g_static_ws[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_static_ws[dev] = p;
  }
  *out = g_static_ws[dev];
  return hipSuccess;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(
    const moe_shape* s, const void* x, const void* w_router, const float* b_router,
    const void* w1, const void* w2, const void* ws1, const void* ws2, float* logits,
    int32_t* topk_ids, float* topk_w, float* aux, int32_t* counts, int32_t* kept,
    int32_t* offsets, int32_t* row_of, int32_t* token_of, int32_t* n_dropped, void* xp,
    void* hbuf, void* out, void* hshared, void* shared_out, void* y, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (s->flags & MOE_FLAG_TRAIN) return MOE_ERR_UNSUPPORTED;
  // every argument the five calls check, checked before the first launch
  const bool lin = (s->flags & MOE_FLAG_LOGITS_IN) != 0;
  const bool shared = s->h_shared > 0;
  const void* need_ptr[] = {x, w1, w2, logits, topk_ids, topk_w, aux, counts, kept, offsets,
                            row_of, token_of, n_dropped, xp, hbuf, out, y};
  for (const void* p : need_ptr)
    if (!p) return MOE_ERR_INVALID_ARG;
  const void* need16[] = {x, w1, w2, xp, hbuf, out, y};
  for (const void* p : need16)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (!lin && (!w_router || !aligned16(w_router))) return MOE_ERR_INVALID_ARG;
  if (shared) {
    const void* sh[] = {ws1, ws2, hshared, shared_out};
    for (const void* p : sh)
      if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  }
  if (ws_layout(s).total > kStaticWsBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (static_ws_ptr(&ws) != hipSuccess) return MOE_ERR_HIP;
  if ((st = moe_route(s, x, w_router, b_router, logits, topk_ids, topk_w, ws, kStaticWsBytes,
                      stream)) != MOE_OK)
    return st;
  if ((st = moe_aux_loss(s, ws, kStaticWsBytes, aux, stream)) != MOE_OK) return st;
  if ((st = moe_permute(s, x, topk_ids, ws, kStaticWsBytes, counts, kept, offsets, row_of,
                        token_of, n_dropped, xp, stream)) != MOE_OK)
    return st;
  if ((st = moe_expert_ffn(s, xp, offsets, w1, w2, hbuf, out, x, ws1, ws2, hshared, shared_out,
                           ws, kStaticWsBytes, stream)) != MOE_OK)
    return st;
  return moe_combine(s, out, row_of, topk_w, shared_out, y, stream);
}
