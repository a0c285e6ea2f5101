/*
 * moe.h - C ABI of the MI355X (gfx950) top-k-routed Mixture-of-Experts layer
 * forward.
 *
 * One forward pass is five calls, issued in this order on one HIP stream:
 *
 *   moe_route      router GEMM, softmax, top-k, renormalised weights
 *   moe_aux_loss   E * sum_e f_e * P_e load-balancing loss
 *   moe_permute    capacity drop in token order, packed expert-major rows,
 *                  dispatch copy of the token rows
 *   moe_expert_ffn grouped GEMM1 + GELU(tanh), grouped GEMM2 (and the
 *                  optional shared expert)
 *   moe_combine    weighted un-permute back to token order
 *
 * The method is the one of three web pages on MoE layers:
 *   [infra] "MoE module infra notes" (dpshk.com/news/5154311): the router of
 *           section 3.1, the expert module of 3.3 and the MoELayer listing of
 *           4.2 (stacked expert weights, capacity, per-expert contractions).
 *   [comm]  "Dissecting the MoE communication bottleneck" (cf-1.com/news/
 *           4950847): dispatch / FFN / combine of section 1.1, capacity and
 *           token drop of 3.1, the aux-loss formula of 3.2, fine-grained plus
 *           shared experts of 2.3, grouped GEMM of 5.1.
 *
 * Conventions for every call
 * --------------------------
 * - All tensors are caller-owned, dense, row-major, device memory.  Pointers
 *   to the bf16/fp32 activation and weight tensors must be 16-byte aligned.
 *   "bf16 mode" (dtype MOE_BF16): x, w_router, w1, w2, ws1, ws2, xp, hbuf,
 *   out, hshared, shared_out and y are bfloat16; accumulation is fp32.
 *   "fp32 mode" (MOE_F32): all of them are float.  Router bias, logits,
 *   top-k weights and aux are always float; ids, counts and row maps int32.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream), never allocate, never synchronise the host, and keep row counts
 *   on the device.  Errors from invalid arguments are returned before any
 *   launch; device faults surface at the caller's next synchronisation.
 * - `ws` is a caller-provided device workspace of at least
 *   moe_workspace_size(shape) bytes (256-byte aligned).  moe_route fills it
 *   with per-block partial results that moe_aux_loss and moe_permute read, so
 *   one forward must use one workspace, and calls that share a workspace must
 *   not overlap.
 * - Results are deterministic: no floating-point atomics, fixed reduction
 *   orders.
 * - The per-block partial results of routing (expert histograms per block of
 *   64 tokens, softmax column sums per block, in-block ranks) are an internal
 *   format of the library, so they travel inside `ws` rather than as
 *   arguments: moe_route writes them, moe_aux_loss and moe_permute read them.
 *   moe_aux_loss runs before moe_permute and derives the per-expert counts
 *   from those histograms itself.  One workspace serves every call of a
 *   forward (and, with MOE_FLAG_TRAIN, of its backward), so
 *   moe_workspace_size takes only the shape.
 * - `stream` is a hipStream_t passed as void*, so that this header needs no
 *   HIP include and a plain C caller can use it.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned pointer  */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels support  */
  MOE_ERR_WORKSPACE = -3,    /* ws_bytes below moe_workspace_size()         */
  MOE_ERR_HIP = -4           /* a HIP launch or runtime call failed          */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* moe_shape.flags */
#define MOE_FLAG_LOGITS_IN 1u  /* moe_route reads `logits` instead of running the router GEMM */
#define MOE_FLAG_TRAIN 2u      /* moe_expert_ffn keeps the GELU pre-activations in the
                                  workspace for moe_expert_ffn_backward, and the
                                  workspace also holds the backward's scratch */
#define MOE_FLAG_GUMBEL 4u     /* moe_route adds Gumbel noise drawn from
                                  (noise_seed, noise_offset) to the logits */

typedef struct {
  int32_t T;        /* tokens in the batch                                   */
  int32_t H;        /* hidden size (multiple of 8)                           */
  int32_t E;        /* routed experts, 1..256                                */
  int32_t K;        /* experts per token (top-k), 1..min(E, 8)               */
  int32_t h_exp;    /* expert FFN width (multiple of 8)                      */
  int32_t h_shared; /* shared-expert FFN width (multiple of 8), 0 = none     */
  float capacity_factor; /* > 0: C = ceil(cf*T*K/E); <= 0: no limit (C = T)  */
  int32_t dtype;    /* moe_dtype                                             */
  uint32_t flags;   /* MOE_FLAG_*                                            */
  float router_tau; /* router softmax temperature tau > 0; 0 means 1          */
  uint64_t noise_seed;   /* MOE_FLAG_GUMBEL: Philox key word 0               */
  uint64_t noise_offset; /* MOE_FLAG_GUMBEL: Philox counter word 2 (advance it
                            every step for fresh noise)                       */
} moe_shape;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* Validates `s` alone (sizes, dtype, flags); MOE_OK when the shape is usable.
 * MOE_ERR_INVALID_ARG for values outside the field ranges above, T < 1,
 * K > E, unknown flags, a non-finite capacity factor or a negative or
 * non-finite router_tau.  MOE_ERR_UNSUPPORTED for shapes the kernels do not
 * cover: E > 256, K > 8, H / h_exp / h_shared not multiples of 8 or above
 * 2^20, T*K >= 2^31, and in bf16 mode (whose GEMM reads each operand through
 * a buffer range below 2 GiB) H*h_exp or H*h_shared above 2^30 - 8 elements,
 * and with MOE_FLAG_TRAIN min(C, T)*max(H, h_exp) or T*max(H, h_shared, E)
 * above that same count (the weight-gradient GEMMs read one segment's rows
 * through one range). */
moe_status moe_check_shape(const moe_shape* s);

/* Expert capacity C: ceil(cf*T*K/E) computed in double for cf > 0, else T
 * ([comm] 3.1, read with T*K assignments), capped at T since no expert can
 * receive more than T assignments (the cap never changes which rows are
 * kept).  -1 for an invalid shape. */
int64_t moe_capacity(const moe_shape* s);

/* Upper bound on kept rows N = sum_e min(count_e, C): min(T*K, E*C).  xp and
 * out need this many rows, hbuf this many rows of h_exp.  -1 if invalid. */
int64_t moe_max_rows(const moe_shape* s);

/* Bytes of device workspace every call of one forward (and, with
 * MOE_FLAG_TRAIN, of its backward) needs (0 if invalid). */
size_t moe_workspace_size(const moe_shape* s);

/*
 * moe_route - router logits, softmax, top-k and renormalised weights
 * ([infra] 3.1 and 4.2; [comm] 1.1 step 1; inference top-k on logits,
 * [infra] 5.2 tip 4).
 *
 * Selection scores z = (l + g) / tau with l = x*W_r + b (fp32 accumulation),
 * tau = router_tau, and g = 0 unless MOE_FLAG_GUMBEL, when g is the Gumbel
 * noise of [infra] 3.1: g = -log(-log(U + 1e-9) + 1e-9), U[t, e] word e % 4
 * of the Philox4x64-10 block with counter (t, e / 4, noise_offset, 0) and key
 * (noise_seed, 0), as (word >> 40) * 2^-24.  Top-k, the softmax, the weights
 * and the aux loss's probabilities all act on z.
 *
 *   x        [T,H]   token rows (dtype)
 *   w_router [H,E]   router weight (dtype)
 *   b_router [E]     fp32 router bias, or NULL for none
 *   logits   [T,E]   fp32 out: z (= x*W_r + b with no noise and tau 1).  With
 *                    MOE_FLAG_LOGITS_IN it is an input, taken as z (no noise
 *                    or temperature applied), and x / w_router / b_router are
 *                    ignored (may be NULL).
 *   topk_ids [T,K]   int32 out: the K experts with the largest z, slot 0 the
 *                    largest; equal scores go to the lower expert index.
 *   topk_w   [T,K]   fp32 out: p[t,e]/sum_{chosen} p[t,e'] with p the softmax
 *                    of the z row.
 *   ws               workspace; receives per-block expert histograms, in-block
 *                    ranks and per-block softmax column sums.
 * Logits must be finite (not checked here; moe_count_nonfinite checks them).
 */
moe_status moe_route(const moe_shape* s, const void* x, const void* w_router,
                     const float* b_router, float* logits, int32_t* topk_ids,
                     float* topk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_count_nonfinite - a debugging aid for moe_route's precondition: writes
 * to *count the number of non-finite values (NaN, +inf, -inf) among the T*E
 * fp32 logits.  One workgroup counts in a fixed order, so the result is exact
 * and deterministic; call it between moe_route and moe_permute, on the same
 * stream, when inputs may hold NaN or infinities.
 *
 *   logits   [T,E]   fp32: what moe_route wrote (or the caller's logits with
 *                    MOE_FLAG_LOGITS_IN)
 *   count    [1]     int64 out (device)
 * Errors: the shape checks of moe_check_shape; MOE_ERR_INVALID_ARG for a NULL
 * pointer.
 */
moe_status moe_count_nonfinite(const moe_shape* s, const float* logits, int64_t* count,
                               void* stream);

/*
 * moe_aux_loss - aux = E * sum_e f_e * P_e ([comm] 3.2), f_e = count_e/(T*K)
 * from the pre-drop top-k choices, P_e = mean over all T tokens of the full
 * softmax probability of e.  No coefficient is applied.  Reads the workspace
 * filled by the preceding moe_route.
 *
 *   aux      [1]     fp32 out (device)
 */
moe_status moe_aux_loss(const moe_shape* s, const void* ws, size_t ws_bytes,
                        float* aux, void* stream);

/*
 * moe_permute - capacity drop, packed row map and dispatch copy
 * ([comm] 1.1 step 2 and 3.1; [infra] 4.2 expert counts and capacity).
 *
 * Assignment (t,k) to e = topk_ids[t,k] has rank r = #{t' < t : e chosen by
 * t'}; it is kept iff r < C.  Kept rows of expert e form the contiguous
 * segment [offsets[e], offsets[e+1]) in token order.
 *
 *   x         [T,H]      token rows (dtype)
 *   topk_ids  [T,K]      from moe_route (same workspace)
 *   counts    [E]        int32 out: pre-drop assignments per expert
 *   kept      [E]        int32 out: min(counts, C)
 *   offsets   [E+1]      int32 out: exclusive prefix sum of kept; N = offsets[E]
 *   row_of    [T,K]      int32 out: packed row of (t,k), -1 when dropped
 *   token_of  [max_rows] int32 out: token of each packed row (rows >= N untouched)
 *   n_dropped [1]        int32 out: sum_e (counts - kept)
 *   xp        [max_rows,H] out (dtype): xp[row_of[t,k]] = x[t]; rows >= N untouched
 */
moe_status moe_permute(const moe_shape* s, const void* x, const int32_t* topk_ids,
                       void* ws, size_t ws_bytes, int32_t* counts, int32_t* kept,
                       int32_t* offsets, int32_t* row_of, int32_t* token_of,
                       int32_t* n_dropped, void* xp, void* stream);

/*
 * moe_expert_ffn - grouped expert FFN over the packed segments
 * ([infra] 3.3 and the per-expert contractions of 4.2; [comm] 2.2 FLOP count,
 * 5.1 grouped GEMM; shared expert [comm] 2.3).
 *
 *   hbuf[r] = GELU_tanh(xp[r] * W1[e])   (fp32 accumulate, GELU in fp32,
 *                                         stored in dtype)
 *   out[r]  = hbuf[r] * W2[e]            (fp32 accumulate, stored in dtype)
 * for every row r of segment e.  With h_shared > 0 also
 *   hshared = GELU_tanh(x * Ws1), shared_out = hshared * Ws2 over all T rows.
 *
 *   xp       [max_rows,H]     packed rows from moe_permute
 *   offsets  [E+1]            int32 device segment bounds from moe_permute
 *   w1       [E,H,h_exp], w2 [E,h_exp,H]   expert weights (dtype)
 *   hbuf     [max_rows,h_exp] scratch out (dtype)
 *   out      [max_rows,H]     out (dtype); rows >= N untouched
 *   x, ws1 [H,h_shared], ws2 [h_shared,H], hshared [T,h_shared],
 *   shared_out [T,H]          used only when h_shared > 0 (else may be NULL)
 * With MOE_FLAG_TRAIN the pre-activations xp*W1[e] (and x*Ws1) are also
 * stored, in dtype, in the workspace for moe_expert_ffn_backward.
 */
moe_status moe_expert_ffn(const moe_shape* s, const void* xp, const int32_t* offsets,
                          const void* w1, const void* w2, void* hbuf, void* out,
                          const void* x, const void* ws1, const void* ws2,
                          void* hshared, void* shared_out,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine - y[t] = sum_{k : row_of[t,k] >= 0} topk_w[t,k] * out[row_of[t,k]]
 * (+ shared_out[t]), accumulated in fp32 in slot order, then rounded to dtype
 * ([comm] 1.1 step 4).  Dropped slots contribute zero and the kept weights
 * are not renormalised; a token with every slot dropped gets 0 (plus its
 * shared-expert row).
 *
 *   out        [max_rows,H] expert outputs (dtype)
 *   row_of     [T,K], topk_w [T,K]
 *   shared_out [T,H] or NULL
 *   y          [T,H] out (dtype)
 */
moe_status moe_combine(const moe_shape* s, const void* out, const int32_t* row_of,
                       const float* topk_w, const void* shared_out, void* y,
                       void* stream);


/*
 * MXFP8 forward ([comm] 5.3: dispatch and combine carry the hidden states in
 * FP8 instead of bf16, halving their bytes; [comm] 5.4: the quantise /
 * dequantise work must stay cheap; [comm] 4.2: FP8 expert weights).  The
 * page fixes no FP8 variant or scaling; this library uses MXFP8 from the OCP
 * Microscaling (MX) specification 1.0: OCP E4M3 elements (largest finite
 * value 448) in blocks of 32 consecutive values that share one E8M0 scale
 * 2^X, X = floor(log2 max|v|) - 8 clamped to [-127, 127] (-127 for an
 * all-zero block), stored as the byte X + 127; element = E4M3(v / 2^X),
 * round to nearest even, magnitudes past 448 saturating to 448.  Blocks run
 * along the contraction dimension of the GEMM that reads the tensor.
 *
 * Routing (moe_route, moe_aux_loss) is unchanged and runs on the bf16 x; the
 * FP8 calls replace moe_permute, moe_expert_ffn and moe_combine.  Shapes:
 * dtype MOE_BF16, H, h_exp and h_shared multiples of 64, no MOE_FLAG_TRAIN
 * (forward only), else MOE_ERR_UNSUPPORTED; each FP8 tensor under 2 GiB.
 *
 * Scale layouts (byte tensors):
 *   operand layout, for an R x Kd tensor that a GEMM reads as its A or B
 *     operand: [ceil(Kd/128)][R][4]; byte (q, r, j) is the scale of block
 *     4q + j of row r.  Size: moe_mx_operand_scale_bytes(R, Kd).  Bytes of
 *     blocks past Kd/32 are neither written nor read.
 *   row layout, for a tensor that combine reads: [R][cols/32].
 * Codes are row-major [R][cols] bytes.  Code pointers must be 16-byte
 * aligned, scale pointers 4-byte aligned.
 */

/* Bytes of an operand-layout scale tensor for `rows` x `cols` values (0 for
 * negative arguments or a size that does not fit in size_t). */
size_t moe_mx_operand_scale_bytes(int64_t rows, int64_t cols);

/*
 * Bytes of the weight codes moe_quantize_weights_mxfp8 writes for `batch`
 * [K,N] weights: batch * ceil(N/256) * 256 * K (0 if an argument is < 1 or
 * the size does not fit in size_t).
 */
size_t moe_mx_weight_code_bytes(int32_t batch, int32_t K, int32_t N);

/*
 * moe_quantize_weights_mxfp8 - expert weights to MXFP8, once, outside the
 * forward ([comm] 4.2).
 *
 *   w       [batch,K,N]  weights (dtype MOE_BF16 or MOE_F32), K the
 *                        contraction dimension (H for W1, h for W2)
 *   q       out: E4M3 codes of the transposed [batch,N,K] weights in panels
 *           of 256 rows x 64 codes, moe_mx_weight_code_bytes(batch, K, N)
 *           bytes: code (b, n, k) lies at byte
 *             ((b*P + n/256) * (K/64) + k/64) * 16384 + (n%256) * 64 + k%64,
 *           P = ceil(N/256), so one 64-value K-step of a 256-row GEMM tile
 *           is 16 contiguous KiB.  Rows n >= N of each slice's last panel
 *           are padding: never written, and read only into GEMM output
 *           columns that are never stored.
 *   scales  [batch,ceil(K/128),N,4]  out: operand layout of each [N,K] slice
 * K must be a multiple of 64 and N of 32 (MOE_ERR_UNSUPPORTED), N*K < 2^31.
 */
moe_status moe_quantize_weights_mxfp8(const void* w, int32_t dtype, int32_t batch, int32_t K,
                                      int32_t N, uint8_t* q, uint8_t* scales, void* stream);

/*
 * moe_permute_mxfp8 - moe_permute with the dispatch copy in MXFP8: every
 * bf16 token row is quantised once and its codes copied to each kept row.
 * Outputs counts, kept, offsets, row_of, token_of, n_dropped exactly as
 * moe_permute, plus
 *   xp_q  [max_rows,H]  E4M3 codes of the packed rows (rows >= N untouched)
 *   xp_s  operand layout, R = max_rows, Kd = H
 *   x_q   [T,H], x_s operand layout (R = T): every token's own quantised row,
 *         for the shared expert; written only when h_shared > 0 (else NULL
 *         is allowed).
 */
moe_status moe_permute_mxfp8(const moe_shape* s, const void* x, const int32_t* topk_ids,
                             void* ws, size_t ws_bytes, int32_t* counts, int32_t* kept,
                             int32_t* offsets, int32_t* row_of, int32_t* token_of,
                             int32_t* n_dropped, uint8_t* xp_q, uint8_t* xp_s, uint8_t* x_q,
                             uint8_t* x_s, void* stream);

/*
 * moe_expert_ffn_mxfp8 - the grouped expert FFN on MXFP8 operands ([infra]
 * 3.3 and 4.2; [comm] 5.1 grouped GEMM, 5.3 FP8): for every row r of
 * segment e (fp32 accumulation of the block-scaled products),
 *   h[r]   = MXFP8(GELU_tanh(xp[r] * W1[e]))   -> h_q [max_rows,h_exp] codes,
 *            h_s operand layout (R = max_rows, Kd = h_exp)
 *   out[r] = MXFP8(h[r] * W2[e])               -> out_q [max_rows,H] codes,
 *            out_s row layout [max_rows, H/32]
 * (each result quantised from its fp32 value in blocks of 32 along the row).
 *   w1_q, w1_s   moe_quantize_weights_mxfp8 of W1 [E,H,h_exp] (K = H)
 *   w2_q, w2_s   moe_quantize_weights_mxfp8 of W2 [E,h_exp,H] (K = h_exp)
 * With h_shared > 0 the same over all T rows of x_q / x_s: hsh_q [T,h_shared]
 * (operand layout, R = T) and sh_q [T,H] (row layout), from the quantised
 * Ws1 [1,H,h_shared] and Ws2 [1,h_shared,H]; else those may be NULL.
 * Rows >= N of h_q / out_q are untouched.
 */
moe_status moe_expert_ffn_mxfp8(const moe_shape* s, const uint8_t* xp_q, const uint8_t* xp_s,
                                const int32_t* offsets, const uint8_t* w1_q,
                                const uint8_t* w1_s, const uint8_t* w2_q, const uint8_t* w2_s,
                                uint8_t* h_q, uint8_t* h_s, uint8_t* out_q, uint8_t* out_s,
                                const uint8_t* x_q, const uint8_t* x_s, const uint8_t* ws1_q,
                                const uint8_t* ws1_s, const uint8_t* ws2_q,
                                const uint8_t* ws2_s, uint8_t* hsh_q, uint8_t* hsh_s,
                                uint8_t* sh_q, uint8_t* sh_s, void* stream);

/*
 * moe_combine_mxfp8 - y[t] = sum_{k kept} topk_w[t,k] * deq(out[row_of[t,k]])
 * (+ deq(shared[t])), accumulated in fp32 in slot order, rounded to bf16
 * ([comm] 1.1 step 4 with [comm] 5.3's FP8 payload).  deq(code) =
 * E4M3(code) * 2^(scale - 127), exact in fp32.
 *   out_q, out_s   from moe_expert_ffn_mxfp8 (row layout)
 *   sh_q, sh_s     shared-expert output (row layout) or NULL
 *   y [T,H]        bf16 out
 */
moe_status moe_combine_mxfp8(const moe_shape* s, const uint8_t* out_q, const uint8_t* out_s,
                             const int32_t* row_of, const float* topk_w, const uint8_t* sh_q,
                             const uint8_t* sh_s, void* y, void* stream);

/*
 * Backward pass.  The gradient of L = <dy, y> + alpha * aux by the chain rule
 * of the forward above, for a forward run with MOE_FLAG_TRAIN.  The routing
 * decisions (top-k sets, capacity drops, counts) are held fixed: they are
 * piecewise constant in the logits.  The gradient reaches the gate through
 * the renormalised top-k weights ([infra] 3.1: the gate network must receive
 * gradients) and through P_e of the aux loss (alpha is the coefficient of
 * [comm] 3.2's aux_loss = alpha * N * sum f_i P_i).  A dropped assignment
 * passes no gradient ([comm] 3.2, second pitfall: dropped tokens are absent
 * in the backward pass).  Call order on one stream, one workspace:
 *   moe_combine_backward, moe_route_backward, moe_expert_ffn_backward,
 *   moe_permute_backward.
 * Weight gradients are fp32 and overwritten (not accumulated); activation
 * gradients are in dtype.  Every result is deterministic.
 */

/*
 * moe_combine_backward - adjoint of moe_combine's routed part.
 *   d_out[row_of[t,k]] = topk_w[t,k] * dy[t]            (dtype)
 *   d_topk_w[t,k]      = <dy[t], out[row_of[t,k]]>      (fp32, 0 when dropped)
 *
 *   dy        [T,H]        gradient of y (dtype)
 *   out, row_of, topk_w    as given to moe_combine
 *   d_out     [max_rows,H] out (dtype); rows >= N untouched
 *   d_topk_w  [T,K]        out (fp32)
 */
moe_status moe_combine_backward(const moe_shape* s, const void* dy, const void* out,
                                const int32_t* row_of, const float* topk_w, void* d_out,
                                float* d_topk_w, void* stream);

/*
 * moe_route_backward - gradient of the router.  With z the selection scores
 * moe_route stored in `logits` (p their softmax, w = topk_w, f_e =
 * counts[e]/(T*K)):
 *   d_z[t, e] = [e chosen as slot k] w_k (d_w_k - sum_j w_j d_w_j)
 *               + alpha * (E/T) p[t,e] (f_e - sum_e' f_e' p[t,e'])
 * and, since z = (l + g) / tau and the noise depends on no parameter,
 *   d_logits = d_z / tau        (the gradient of l = x*W_r + b; tau = 1 with
 *                                MOE_FLAG_LOGITS_IN)
 * then d_w_router = x^T d_logits and d_b_router = sum_t d_logits[t] (fp32,
 * fixed summation order).
 *
 *   x [T,H]                      as given to moe_route (dtype)
 *   logits, topk_ids, topk_w     from moe_route; counts from moe_permute
 *   d_topk_w  [T,K]              from moe_combine_backward
 *   alpha                        aux-loss coefficient (0: no aux term)
 *   d_logits  [T,E]              out (fp32)
 *   d_w_router [H,E]             out (fp32)
 *   d_b_router [E]               out (fp32), or NULL
 */
moe_status moe_route_backward(const moe_shape* s, const void* x, const float* logits,
                              const int32_t* topk_ids, const float* topk_w,
                              const float* d_topk_w, const int32_t* counts, float alpha,
                              float* d_logits, float* d_w_router, float* d_b_router,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_backward - gradient of the grouped expert FFN (and of the
 * shared expert when h_shared > 0), from the pre-activations u = xp*W1[e]
 * that the MOE_FLAG_TRAIN forward left in the workspace (this call
 * overwrites them with d u).  For every row r of segment e:
 *   d_u[r]  = (d_out[r] * W2[e]^T) .* GELU'(u[r])
 *   d_w2[e] = hbuf_e^T d_out_e,  d_w1[e] = xp_e^T d_u_e   (fp32)
 *   d_xp[r] = d_u[r] * W1[e]^T                            (dtype)
 * and for the shared expert the same with x, Ws1, Ws2, hshared and dy:
 *   d_ws1, d_ws2 (fp32), d_x_shared = d_us * Ws1^T (dtype).
 *
 *   xp, offsets, w1, w2, hbuf     as in the forward
 *   d_out     [max_rows,H]        from moe_combine_backward
 *   d_xp      [max_rows,H]        out (dtype); rows >= N untouched
 *   d_w1 [E,H,h_exp], d_w2 [E,h_exp,H]   out (fp32; zero for an empty expert)
 *   x, ws1, ws2, hshared, dy [T,H], d_x_shared [T,H], d_ws1 [H,h_shared],
 *   d_ws2 [h_shared,H]            used only when h_shared > 0
 */
moe_status moe_expert_ffn_backward(const moe_shape* s, const void* xp, const int32_t* offsets,
                                   const void* w1, const void* w2, const void* hbuf,
                                   const void* d_out, void* d_xp, float* d_w1, float* d_w2,
                                   const void* x, const void* ws1, const void* ws2,
                                   const void* hshared, const void* dy, void* d_x_shared,
                                   float* d_ws1, float* d_ws2, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * moe_permute_backward - gradient of x: the adjoint of the dispatch copy
 * plus the router's and the shared expert's input gradients,
 *   dx[t] = sum_{k kept} d_xp[row_of[t,k]] (+ d_x_shared[t])
 *           + d_logits[t] * W_r^T
 * summed in fp32; in bf16 mode the last term uses d_logits rounded to bf16.
 * In bf16 mode with at most 16 experts and H * pad8(E) * 2 <= 64 KiB, one
 * kernel sums all three terms (router term, slots in order, shared term) and
 * rounds once; otherwise the slots (in order) and the shared term are summed
 * and rounded, and the router term is then accumulated by a GEMM.
 *
 *   d_xp      [max_rows,H]   from moe_expert_ffn_backward
 *   row_of    [T,K]
 *   d_x_shared [T,H] or NULL (required when h_shared > 0)
 *   d_logits  [T,E]          from moe_route_backward
 *   w_router  [H,E]          (dtype)
 *   dx        [T,H]          out (dtype)
 */
moe_status moe_permute_backward(const moe_shape* s, const void* d_xp, const int32_t* row_of,
                                const void* d_x_shared, const float* d_logits,
                                const void* w_router, void* dx, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * moe_mfma_ceiling - a measurement aid, not a step of the layer: the
 * MFMA-only rate of the grouped GEMM's inner loop, the ceiling its roofline
 * fraction is read against.  `workgroups` workgroups of four waves (one wave
 * per SIMD when there is one workgroup per CU) each run `iters` rounds
 * t = 0 .. iters-1 of 64 v_mfma_f32_16x16x32_bf16 (8 x 8 tiles, 256 fp32
 * accumulators per lane) on operands held in registers, with no memory
 * traffic in the loop: 2 * 16 * 16 * 32 * 64 * iters FLOP per wave.
 *   mode 0    the given operands in every round
 *   mode 1    two register sets alternate: the given operands in even
 *             rounds, in odd rounds those with every bf16 sign and mantissa
 *             bit flipped (each 32-bit word XORed with 0x807f807f)
 *   mode 2    the given operands, each XORed before every round with a zero
 *             word passed in at run time (one VALU instruction per MFMA,
 *             results as mode 0)
 *   mode 3    the eight-wave kernel's shape instead: 4 x 4 tiles of
 *             v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane) on
 *             fragments 0-3 (A_0..A_3) and 8-11 (B_0..B_3) read as 32 x 16
 *             matrices (lane l: row l % 32, k = 8 (l / 32) .. +7), each
 *             round running its 16 MFMAs twice: the same FLOPs per round
 *   operands  16 x 64 x 8 bf16, 16-byte aligned: fragments 0-7 are A_0..A_7,
 *             8-15 are B_0..B_7; lane l of a fragment holds row l % 16,
 *             k = 8 (l / 16) .. +7 of a 16 x 32 matrix
 *   out       workgroups * 256 * 4 floats (mode 3: * 16), 16-byte aligned:
 *             lane l of a wave writes rows 4 (l / 16) + r (r = 0..3), column
 *             l % 16 of sum over the rounds t of sum_{i,j} B_j(t) A_i(t)^T;
 *             mode 3: rows 8 (r / 4) + 4 (l / 32) + r % 4 (r = 0..15),
 *             column l % 32 of 2 * iters * sum_{i,j} B_j A_i^T
 * MOE_ERR_INVALID_ARG for null or misaligned pointers, workgroups outside
 * [1, 65536], iters outside [1, 2^24] or mode other than 0, 1, 2 or 3.
 */
moe_status moe_mfma_ceiling(const void* operands, float* out, int32_t workgroups, int32_t iters,
                            int32_t mode, void* stream);

/*
 * moe_forward_noalloc - the whole forward (moe_route, moe_aux_loss,
 * moe_permute, moe_expert_ffn, moe_combine, in that order, on `stream`) in
 * one call that allocates nothing, for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The arguments are those of the five calls (same meaning,
 * layout and ownership); the workspace is instead a static device array of
 * 16 MiB inside the library, one per GPU, held until the process ends.
 * Nothing in it needs clearing.  Calls that overlap on one GPU (other
 * streams, other host threads) share that array and race: serialise them.
 * Returns MOE_ERR_WORKSPACE when moe_workspace_size(s) exceeds 16 MiB,
 * MOE_ERR_UNSUPPORTED with MOE_FLAG_TRAIN (training keeps pre-activations in
 * the workspace), and the five calls' argument errors, all before any launch;
 * MOE_ERR_HIP if a launch or the array's address lookup fails.
 */
moe_status moe_forward_noalloc(const moe_shape* s, const void* x, const void* w_router,
                               const float* b_router, const void* w1, const void* w2,
                               const void* ws1, const void* ws2, float* logits,
                               int32_t* topk_ids, float* topk_w, float* aux, int32_t* counts,
                               int32_t* kept, int32_t* offsets, int32_t* row_of,
                               int32_t* token_of, int32_t* n_dropped, void* xp, void* hbuf,
                               void* out, void* hshared, void* shared_out, void* y,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
