"""Pins of the CPU oracle's backward pass (all on the CPU).

Each test checks ``moe_oracle.backward`` against something other than itself:
central finite differences of the oracle's forward (with the routing
decisions held where they are, which the test asserts), torch's autograd on
cases that reduce to textbook routines (a dense GELU-tanh FFN, a softmax),
and closed forms of the aux-loss gradient.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _case(seed, T=7, H=5, E=4, K=2, h=3, hs=0, bias=True):
    r = np.random.default_rng(seed)
    p = dict(
        x=r.standard_normal((T, H)),
        w_r=r.standard_normal((H, E)) * 0.7,
        b_r=r.standard_normal(E) * 0.3 if bias else None,
        w1=r.standard_normal((E, H, h)) * 0.6,
        w2=r.standard_normal((E, h, H)) * 0.6,
        ws1=r.standard_normal((H, hs)) * 0.6 if hs else None,
        ws2=r.standard_normal((hs, H)) * 0.6 if hs else None,
    )
    dy = r.standard_normal((T, H))
    return p, dy


def _loss(p, dy, K, cf, alpha):
    """L = <dy, y> + alpha * aux, routing from the float64 logits, and the
    routing decisions (to check that a perturbation kept them)."""
    l = O.router_logits(p["x"], p["w_r"], p["b_r"])
    fw = O.forward(p["x"], p["w_r"], p["b_r"], p["w1"], p["w2"], p["ws1"], p["ws2"], K=K, cf=cf,
                   logits=l)
    return float(np.sum(dy * fw["y"]) + alpha * fw["aux"]), (fw["ids"].copy(), fw["row_of"].copy())


def _grads(p, dy, K, cf, alpha):
    l = O.router_logits(p["x"], p["w_r"], p["b_r"])
    return O.backward(p["x"], p["w_r"], p["b_r"], p["w1"], p["w2"], p["ws1"], p["ws2"], dy=dy,
                      K=K, cf=cf, alpha=alpha, logits=l)


GRAD_OF = {"x": "dx", "w_r": "dw_r", "b_r": "db_r", "w1": "dw1", "w2": "dw2", "ws1": "dws1",
           "ws2": "dws2"}


@pytest.mark.parametrize("seed,K,cf,alpha,hs", [
    (0, 2, 0.0, 0.0, 0),      # no capacity limit, no aux term
    (1, 2, 0.0, 0.7, 0),      # aux-loss gradient through P_e
    (2, 2, 0.6, 0.3, 0),      # capacity 3 of 14 assignments' experts: drops
    (3, 1, 0.0, 0.5, 3),      # top-1 plus a shared expert
    (4, 4, 0.0, 0.2, 0),      # K = E: weights are the full softmax
])
def test_backward_matches_central_differences(seed, K, cf, alpha, hs):
    """Every parameter entry perturbed by +-eps; (L+ - L-)/(2 eps) must match
    the analytic gradient.  The routing (top-k sets and row map) is asserted
    unchanged by each perturbation, so L is smooth there."""
    p, dy = _case(seed, K=K, hs=hs)
    g = _grads(p, dy, K, cf, alpha)
    _, route0 = _loss(p, dy, K, cf, alpha)
    if cf > 0:
        assert (route0[1] < 0).any(), "the case must drop some assignments"
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if p[name] is None:
            continue
        a = p[name]
        num = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + eps
            lp, rp = _loss(p, dy, K, cf, alpha)
            a[idx] = old - eps
            lm, rm = _loss(p, dy, K, cf, alpha)
            a[idx] = old
            for u, v in zip(rp + rm, route0 + route0):
                assert np.array_equal(u, v), f"perturbing {name}{idx} changed the routing"
            num[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - g[gname])) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, f"{gname}: relative error {err:.3g}"


def test_dense_single_expert_matches_torch_autograd():
    """E = K = 1, no limit: y = GELU_tanh(x W1) W2 with weight 1 exactly, so
    the layer's gradients are those of a dense FFN (torch autograd, float64),
    and the router gets none (w is identically 1; with one expert the aux
    loss is the constant 1)."""
    p, dy = _case(5, T=9, H=6, E=1, K=1, h=4)
    g = _grads(p, dy, 1, 0.0, 0.5)
    x = torch.tensor(p["x"], requires_grad=True)
    w1 = torch.tensor(p["w1"][0], requires_grad=True)
    w2 = torch.tensor(p["w2"][0], requires_grad=True)
    y = torch.nn.functional.gelu(x @ w1, approximate="tanh") @ w2
    (y * torch.tensor(dy)).sum().backward()
    assert np.allclose(g["dx"], x.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(g["dw1"][0], w1.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(g["dw2"][0], w2.grad.numpy(), rtol=0, atol=1e-12)
    assert np.all(g["dw_r"] == 0) and np.all(g["db_r"] == 0)


def test_gelu_grad_matches_torch_autograd():
    u = torch.linspace(-9, 9, 2001, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(u, approximate="tanh").sum().backward()
    assert np.allclose(O.gelu_tanh_grad(u.detach().numpy()), u.grad.numpy(), rtol=0, atol=1e-14)


def test_route_backward_k_equals_e_is_softmax_vjp():
    """With K = E every expert is chosen and w is the full softmax (in the
    order of the chosen ids), so the weight path of d logits is the softmax
    vector-Jacobian product (torch autograd)."""
    r = np.random.default_rng(6)
    T, E = 11, 5
    l = r.standard_normal((T, E))
    ids = O.select_topk(l, E)
    w = O.topk_weights(O.softmax(l), ids)
    dw = r.standard_normal((T, E))
    dl = O.route_backward(l, ids, w, dw, E, E, 0.0)
    lt = torch.tensor(l, requires_grad=True)
    sm = torch.softmax(lt, dim=1)
    # dw is given per slot; slot k holds expert ids[t, k]
    g = torch.zeros((T, E), dtype=torch.float64)
    g.scatter_(1, torch.tensor(ids, dtype=torch.int64), torch.tensor(dw))
    (sm * g).sum().backward()
    assert np.allclose(dl, lt.grad.numpy(), rtol=0, atol=1e-13)


def test_aux_gradient_vanishes_for_uniform_assignment():
    """f_e = 1/E makes d aux / d l[t,e] = (E/T) p (1/E - (1/E) sum p) = 0."""
    T, E, K = 16, 4, 2
    r = np.random.default_rng(7)
    l = r.standard_normal((T, E)) * 0.1
    for t in range(T):  # token t prefers experts t mod E and t+1 mod E
        l[t, t % E] += 5.0
        l[t, (t + 1) % E] += 4.0
    ids = O.select_topk(l, K)
    assert np.all(O.expert_counts(ids, E) == T * K // E)
    w = O.topk_weights(O.softmax(l), ids)
    dl = O.route_backward(l, ids, w, np.zeros((T, K)), E, K, 1.0)
    assert np.max(np.abs(dl)) < 1e-15


def test_aux_gradient_closed_form_two_experts():
    """E = 2, K = 1: aux = 2 (f_0 P_0 + f_1 P_1), P_e = mean_t p[t,e], so
    d aux / d l[t,0] = (2/T) p0 p1 (f_0 - f_1) and d/d l[t,1] is its negative."""
    l = np.array([[1.0, 0.0], [0.3, -0.2], [-1.0, 0.5]])
    T, E, K = 3, 2, 1
    ids = O.select_topk(l, K)
    f = O.expert_counts(ids, E) / float(T * K)
    p = O.softmax(l)
    dl = O.route_backward(l, ids, np.ones((T, 1)), np.zeros((T, 1)), E, K, 1.0)
    want0 = (2.0 / T) * p[:, 0] * p[:, 1] * (f[0] - f[1])
    assert np.allclose(dl[:, 0], want0, rtol=0, atol=1e-15)
    assert np.allclose(dl[:, 1], -want0, rtol=0, atol=1e-15)


def test_dropped_assignments_pass_no_gradient():
    """C = 1: only the first token of each expert is kept.  A token whose
    slots are all dropped gets no expert-path gradient: its dx is the router
    part alone (d logits W_r^T) and its routing weights get d w = 0."""
    p, dy = _case(8, T=10, E=2, K=1)
    cf = 0.1  # C = ceil(0.1 * 10 / 2) = 1
    g = _grads(p, dy, 1, cf, 0.4)
    fw = g["forward"]
    assert fw["C"] == 1
    dropped = np.nonzero((fw["row_of"] < 0).all(axis=1))[0]
    assert len(dropped) >= 5
    router_part = g["d_logits"] @ p["w_r"].T
    assert np.allclose(g["dx"][dropped], router_part[dropped], rtol=0, atol=1e-15)
    assert np.all(g["d_w"][dropped] == 0)
    # and the kept rows' d_out is exactly w * dy
    for t in range(10):
        r = fw["row_of"][t, 0]
        if r >= 0:
            assert np.array_equal(g["d_out"][r], fw["w"][t, 0] * dy[t])
