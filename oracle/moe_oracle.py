"""CPU oracle of the top-k-routed MoE layer, forward and backward (test infrastructure).

This module is test infrastructure, not product code.  Only the tests, the
smoke check of ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it; the HIP path never does, and this module imports nothing from
the HIP path.

It is the plain definition of the layer, written out step by step in float64
with numpy (a matmul, a stable sort and ``tanh`` are the only library
primitives used).  There is no blocking, fusion or reordering beyond what the
definition states.  Inputs are the exact float values of the bf16 / fp32
tensors, widened to float64.

Pages cited (their addresses; the first two carry no title of their own):

* [infra]  "MoE module infra notes", dpshk.com/news/5154311
* [comm]   "Dissecting the MoE communication bottleneck" (拆解MoE的通信瓶颈),
           cf-1.com/news/4950847

Readings taken where the pages are silent or disagree (each also listed in
the design notes of the repository):

* Selection is on the fp32 router logits, ties going to the lower expert
  index, slots in descending order ([infra] 5.2 tip 4 selects on logits at
  inference; [comm] 3.2 listing selects on logits; softmax is monotone so
  this equals top-k of the probabilities).
* No Gumbel noise, temperature 1 (inference router, [infra] 5.2 tip 4).
* Weights are the full-softmax probabilities of the chosen experts divided by
  their sum ([infra] 3.1 step 3); equal, in exact arithmetic, to a softmax over
  the chosen logits ([comm] 3.2 listing).
* Capacity C = ceil(cf * T * K / E) with cf > 0, else no limit (C = T).  The
  [comm] 3.1 formula omits K and [infra] 4.2 floors; ceil with K is the
  reading adopted.  Later tokens are dropped ([comm] 3.1).
* A dropped assignment contributes zero; kept weights are not renormalised.
* Aux loss = E * sum_e f_e * P_e with f_e = (pre-drop count of e) / (T*K) and
  P_e the mean over all T tokens of the full softmax ([comm] 3.2 text).  No
  coefficient alpha is applied.  It is 1 for uniform routing.
* Expert FFN is Linear -> GELU(tanh form) -> Linear with no biases
  ([infra] 3.3 expert module and 4.2 listing; tanh form of Hendrycks and
  Gimpel's GELU).
* Optional shared expert: the same FFN applied to every token with weight 1
  ([comm] 2.3, fine-grained plus shared experts).

Backward (the gradient of a scalar L = <dy, y> + alpha * aux, by the chain
rule of the forward definition above):

* The routing decisions (top-k sets, capacity drops, the counts f_e) are
  piecewise constant in the logits and get no gradient; the gradient reaches
  the gate through the renormalised top-k weights ([infra] 3.1: the gate must
  receive gradients) and through P_e of the aux loss.
* A dropped assignment contributes nothing to y, so it passes no gradient to
  the expert FFN or to its routing weight ([comm] 3.2, second pitfall:
  dropped tokens are absent in the backward pass, their gradient masked).
* alpha is the aux-loss coefficient of [comm] 3.2 (aux_loss = alpha * N *
  sum f_i P_i); the forward reports aux without it.
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


# ---------------------------------------------------------------------------
# a1: router logits
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_r: np.ndarray, b_r: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[h, e] (+ b_r[e]), in float64.

    [infra] 4.2 listing: the gate is a linear map from hidden_dim to
    num_experts; [comm] 1.1 step 1: the router scores each token.
    """
    l = np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64)
    if b_r is not None:
        l = l + np.asarray(b_r, dtype=np.float64)[None, :]
    return l


# ---------------------------------------------------------------------------
# a2: softmax, top-k, renormalisation
# ---------------------------------------------------------------------------

def select_topk(logits: np.ndarray, K: int) -> np.ndarray:
    """Expert ids [T, K] (int32) chosen per token.

    Order experts by (logit descending, index ascending) and keep the first
    K; slot 0 holds the largest.  [infra] 3.1 and 5.2 tip 4 (top-k, sorted);
    ties go to the lower index.  A stable sort of the negated logits gives
    exactly that order (negation of a float is exact; -0.0 and +0.0 compare
    equal, so they tie).
    """
    l = np.asarray(logits)
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def softmax(logits: np.ndarray) -> np.ndarray:
    """p[t, e] = exp(l[t,e] - m_t) / sum_j exp(l[t,j] - m_t), float64.

    [infra] 3.1 listing, softmax over the expert axis.
    """
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m)
    return z / z.sum(axis=1, keepdims=True)


def topk_weights(probs: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, k] = p[t, S_t[k]] / sum_j p[t, S_t[j]]  ([infra] 3.1 step 3)."""
    sel = np.take_along_axis(probs, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def topk_weights_from_chosen_logits(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """The other form on the pages: softmax over the K chosen logits only.

    [comm] 3.2 listing.  Equal to :func:`topk_weights` in exact arithmetic.
    """
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# a3: load-balancing aux loss
# ---------------------------------------------------------------------------

def expert_counts(ids: np.ndarray, E: int) -> np.ndarray:
    """counts[e] = number of tokens whose chosen set holds e (pre-drop)."""
    return np.bincount(ids.reshape(-1).astype(np.int64), minlength=E).astype(np.int64)


def aux_loss(ids: np.ndarray, probs: np.ndarray, E: int, K: int) -> float:
    """aux = E * sum_e f_e * P_e ([comm] 3.2, the N * sum_i f_i * P_i formula).

    f_e = counts_e / (T*K) is the fraction of assignments routed to e, and
    P_e = (1/T) sum_t p[t, e] is the mean router probability of e.  No alpha.
    """
    T = ids.shape[0]
    f = expert_counts(ids, E).astype(np.float64) / float(T * K)
    P = probs.sum(axis=0) / float(T)
    return float(E * np.sum(f * P))


# ---------------------------------------------------------------------------
# a4: capacity, drop, stable rank, rows
# ---------------------------------------------------------------------------

def capacity(cf: float, T: int, K: int, E: int) -> int:
    """C = ceil(cf * T * K / E) for cf > 0 (computed in double), else T.

    [comm] 3.1: capacity = ceil(capacity_factor * tokens / num_experts), read
    with tokens = T*K assignments; cf <= 0 means no limit, and T is the most
    any expert can receive.
    """
    cf = float(np.float32(cf))
    if cf <= 0.0:
        return T
    return int(math.ceil(cf * float(T * K) / float(E)))


def assign_rows(ids: np.ndarray, E: int, C: int) -> Dict[str, np.ndarray]:
    """Capacity drop in token order and the packed expert-major row map.

    Visit tokens t = 0..T-1 in order (and slots k in order within a token);
    the assignment (t, k) to e = ids[t,k] keeps rank fill[e] if fill[e] < C,
    else it is dropped ([comm] 3.1: overflow tokens are dropped, later ones
    first).  Segment e of the packed buffer starts at offsets[e], the
    exclusive prefix sum of kept counts, and row_of[t,k] = offsets[e] + rank
    (or -1 when dropped); token_of is the inverse map.
    """
    T, K = ids.shape
    counts = expert_counts(ids, E)
    kept = np.minimum(counts, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    N = int(offsets[E])
    row_of = np.full((T, K), -1, dtype=np.int64)
    token_of = np.full(N, -1, dtype=np.int64)
    fill = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            if fill[e] < C:
                r = int(offsets[e] + fill[e])
                row_of[t, k] = r
                token_of[r] = t
                fill[e] += 1
    return dict(counts=counts, kept=kept, offsets=offsets, row_of=row_of,
                token_of=token_of, n_dropped=int(counts.sum() - kept.sum()))


# ---------------------------------------------------------------------------
# a5: dispatch
# ---------------------------------------------------------------------------

def permute(x: np.ndarray, token_of: np.ndarray) -> np.ndarray:
    """xp[row] = x[token_of[row]]  ([comm] 1.1 step 2, dispatch)."""
    return np.asarray(x)[token_of]


# ---------------------------------------------------------------------------
# a6-a8: expert FFN
# ---------------------------------------------------------------------------

def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))), the tanh form of GELU."""
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u * u * u)))


def ffn(rows: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """GELU_tanh(rows @ W1) @ W2 in float64 ([infra] 3.3: Linear -> GELU -> Linear)."""
    u = np.asarray(rows, dtype=np.float64) @ np.asarray(w1, dtype=np.float64)
    return gelu_tanh(u) @ np.asarray(w2, dtype=np.float64)


def expert_ffn(xp: np.ndarray, offsets: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """out[rows of e] = FFN_e(xp[rows of e]) for each expert segment.

    [infra] 4.2 listing: the two per-expert contractions over stacked
    weights W1 [E,H,h] and W2 [E,h,H] with GELU between.
    """
    E = w1.shape[0]
    out = np.zeros((xp.shape[0], w2.shape[2]), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            out[a:b] = ffn(xp[a:b], w1[e], w2[e])
    return out


# ---------------------------------------------------------------------------
# a9: combine
# ---------------------------------------------------------------------------

def combine(out: np.ndarray, row_of: np.ndarray, w: np.ndarray,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t] = sum_{k kept} w[t,k] * out[row_of[t,k]] (+ shared[t]).

    [comm] 1.1 step 4: expert outputs are weighted by the routing weights and
    returned to the token's position.  Dropped slots add nothing.
    """
    T, K = row_of.shape
    y = np.zeros((T, out.shape[1]), dtype=np.float64)
    for k in range(K):
        r = row_of[:, k]
        m = r >= 0
        y[m] += w[m, k][:, None] * out[r[m]]
    if shared is not None:
        y += shared
    return y


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def route(logits: np.ndarray, E: int, K: int, cf: float) -> Dict[str, np.ndarray]:
    """Steps a2-a4 from given router logits (float32 values, widened exactly)."""
    T = logits.shape[0]
    ids = select_topk(logits, K)
    p = softmax(logits)
    w = topk_weights(p, ids)
    C = capacity(cf, T, K, E)
    r = assign_rows(ids, E, C)
    r.update(ids=ids, probs=p, w=w, C=C, aux=aux_loss(ids, p, E, K))
    return r


def forward(x, w_r, b_r, w1, w2, ws1=None, ws2=None, *, K: int, cf: float,
            logits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The whole layer, every intermediate returned.

    When ``logits`` is given (float32 values) routing starts from them instead
    of the oracle's own router GEMM; the GEMM result is still returned as
    ``logits_oracle``.  The oracle's own logits are rounded to float32 before
    selection, because selection compares float32 logits.
    """
    E = w1.shape[0]
    l_own = router_logits(x, w_r, b_r)
    l_sel = np.asarray(logits, dtype=np.float64) if logits is not None \
        else l_own.astype(np.float32).astype(np.float64)
    r = route(l_sel, E, K, cf)
    xp = permute(x, r["token_of"])
    out = expert_ffn(xp, r["offsets"], w1, w2)
    shared = ffn(x, ws1, ws2) if ws1 is not None else None
    y = combine(out, r["row_of"], r["w"], shared)
    r.update(logits_oracle=l_own, xp=xp, out=out, shared=shared, y=y)
    return r


def forward_tokens(x, w1, w2, ws1, ws2, routing: Dict[str, np.ndarray],
                   tokens: np.ndarray) -> np.ndarray:
    """y for a subset of tokens, given the full routing (ids, w, row_of).

    Once routing is fixed each token's output depends only on its own row:
    y[t] = sum_{k kept} w[t,k] * FFN_{ids[t,k]}(x[t]) (+ FFN_shared(x[t])).
    The FFN rows are grouped per expert only to call the matmul once per
    expert; every row is still the plain definition.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    ids, w, row_of = routing["ids"], routing["w"], routing["row_of"]
    E = w1.shape[0]
    K = ids.shape[1]
    xs = np.asarray(x[tokens], dtype=np.float64)
    y = np.zeros((len(tokens), w2.shape[2]), dtype=np.float64)
    for e in range(E):
        for k in range(K):
            sel = np.nonzero((ids[tokens, k] == e) & (row_of[tokens, k] >= 0))[0]
            if len(sel):
                y[sel] += w[tokens[sel], k][:, None] * ffn(xs[sel], w1[e], w2[e])
    if ws1 is not None:
        y += ffn(xs, ws1, ws2)
    return y


def dense_all_experts(x, w1, w2, routing: Dict[str, np.ndarray], ws1=None, ws2=None) -> np.ndarray:
    """Brute force without any permutation: y_t = sum_e g[t,e] * FFN_e(x_t).

    g[t,e] is the routing weight of e for token t when (t, e) is a kept
    assignment, else 0.  This is the all-experts form of [infra] 3.3 (every
    expert applied to every token, then the chosen ones gathered), usable
    only on tiny inputs; it shares no permutation code with :func:`forward`.
    """
    ids, w, row_of = routing["ids"], routing["w"], routing["row_of"]
    T, K = ids.shape
    E = w1.shape[0]
    g = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            if row_of[t, k] >= 0:
                g[t, ids[t, k]] += w[t, k]
    y = np.zeros((T, w2.shape[2]), dtype=np.float64)
    for e in range(E):
        y += g[:, e:e + 1] * ffn(x, w1[e], w2[e])
    if ws1 is not None:
        y += ffn(x, ws1, ws2)
    return y


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def gelu_tanh_grad(u: np.ndarray) -> np.ndarray:
    """d/du of 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3):

    0.5 (1 + tanh z) + 0.5 u (1 - tanh^2 z) sqrt(2/pi) (1 + 3 * 0.044715 u^2).
    """
    u = np.asarray(u, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    th = np.tanh(c * (u + 0.044715 * u * u * u))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * c * (1.0 + 3.0 * 0.044715 * u * u)


def ffn_backward(rows, w1, w2, dout):
    """Gradients of out = GELU(rows W1) W2 for a given d(out).

    Returns (d rows, dW1, dW2), all float64.
    """
    a = np.asarray(rows, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    u = a @ w1
    g = gelu_tanh(u)
    dg = dout @ w2.T
    du = dg * gelu_tanh_grad(u)
    return du @ w1.T, a.T @ du, g.T @ dout


def combine_backward(dy, out, row_of, w):
    """Adjoint of :func:`combine` for the routed part.

    d out[row_of[t,k]] = w[t,k] dy[t] and d w[t,k] = <dy[t], out[row_of[t,k]]>
    for kept (t, k); a dropped slot gets d w = 0 and touches no row.
    """
    dy = np.asarray(dy, dtype=np.float64)
    T, K = row_of.shape
    dout = np.zeros_like(np.asarray(out, dtype=np.float64))
    dw = np.zeros((T, K), dtype=np.float64)
    for k in range(K):
        r = row_of[:, k]
        m = r >= 0
        dout[r[m]] += w[m, k][:, None] * dy[m]
        dw[m, k] = np.sum(dy[m] * out[r[m]], axis=1)
    return dout, dw


def permute_backward(dxp, row_of, d_logits_raw, w_r, dxs=None):
    """dx, the input gradient: the adjoint of :func:`permute` (each kept row's
    gradient returns to its token), plus the router's term d_logits W_r^T
    (the logits are x W_r + b), plus the shared expert's input gradient when
    there is one.
    """
    dxp = np.asarray(dxp, dtype=np.float64)
    T, K = row_of.shape
    dx = np.zeros((T, dxp.shape[1]), dtype=np.float64)
    for k in range(K):
        r = row_of[:, k]
        m = r >= 0
        dx[m] += dxp[r[m]]
    dx += np.asarray(d_logits_raw, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T
    if dxs is not None:
        dx += np.asarray(dxs, dtype=np.float64)
    return dx


def route_backward(logits, ids, w, dw, E: int, K: int, alpha: float):
    """d L / d logits from the routing weights and from alpha * aux.

    Weights: w = softmax over the chosen logits ([comm] 3.2 form, equal to
    [infra] 3.1's p_sel / sum p_sel), so for chosen expert s_k
    dl[t, s_k] = w_k (dw_k - sum_j w_j dw_j); unchosen experts get nothing
    from this path.  Aux: P_e = (1/T) sum_t p[t,e] with p the full softmax,
    f_e fixed, so d aux / d l[t,e] = (E/T) p[t,e] (f_e - sum_e' f_e' p[t,e']).
    """
    l = np.asarray(logits, dtype=np.float64)
    T = l.shape[0]
    ids64 = ids.astype(np.int64)
    dl = np.zeros((T, E), dtype=np.float64)
    s = np.sum(w * dw, axis=1, keepdims=True)
    np.put_along_axis(dl, ids64, w * (dw - s), axis=1)
    if alpha != 0.0:
        p = softmax(l)
        f = expert_counts(ids, E).astype(np.float64) / float(T * K)
        dl += alpha * (E / float(T)) * p * (f[None, :] - (p @ f)[:, None])
    return dl


def backward(x, w_r, b_r, w1, w2, ws1=None, ws2=None, *, dy, K: int, cf: float,
             alpha: float = 0.0, logits: Optional[np.ndarray] = None,
             tau: float = 1.0) -> Dict[str, np.ndarray]:
    """Every gradient of L = <dy, y> + alpha * aux for one layer forward.

    Routing is that of :func:`forward` with the same arguments (from the given
    logits when passed).  Returns dx, dw_r, db_r, dw1, dw2, dws1, dws2 and the
    intermediates d_out (rows of the packed expert outputs), d_w (routing
    weights), d_xp (rows of the packed inputs) and d_logits.

    With a temperature (or noise) the given ``logits`` are the selection
    scores z = (x W_r + b + g) / tau the forward routed on: d_logits is dL/dz,
    and the router's own gradients use dL/d(x W_r + b) = dL/dz / tau (the noise
    g does not depend on any parameter; the noisy router of [infra] 3.1).
    """
    fw = forward(x, w_r, b_r, w1, w2, ws1, ws2, K=K, cf=cf, logits=logits)
    E = w1.shape[0]
    x64 = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    row_of, offsets = fw["row_of"], fw["offsets"]
    dout, dw = combine_backward(dy, fw["out"], row_of, fw["w"])
    dxp = np.zeros_like(fw["xp"], dtype=np.float64)
    dw1 = np.zeros(w1.shape, dtype=np.float64)
    dw2 = np.zeros(w2.shape, dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            dxp[a:b], dw1[e], dw2[e] = ffn_backward(fw["xp"][a:b], w1[e], w2[e], dout[a:b])
    l_sel = np.asarray(logits, dtype=np.float64) if logits is not None \
        else fw["logits_oracle"].astype(np.float32).astype(np.float64)
    dl = route_backward(l_sel, fw["ids"], fw["w"], dw, E, K, alpha)
    dl_raw = dl / float(tau)
    dw_r = x64.T @ dl_raw
    db_r = dl_raw.sum(axis=0)
    dxs = dws1 = dws2 = None
    if ws1 is not None:
        dxs, dws1, dws2 = ffn_backward(x64, ws1, ws2, dy)
    dx = permute_backward(dxp, row_of, dl_raw, w_r, dxs)
    return dict(dx=dx, dw_r=dw_r, db_r=db_r, dw1=dw1, dw2=dw2, dws1=dws1, dws2=dws2,
                d_out=dout, d_w=dw, d_xp=dxp, d_logits=dl, forward=fw)
