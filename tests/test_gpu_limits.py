"""GPU parity at the largest shapes moe_check_shape accepts in bf16 mode, through the C ABI.

The bf16 grouped GEMM reads a whole weight matrix through one buffer range
below 2 GiB, and in training mode the weight-gradient GEMMs read one
segment's rows the same way, so the header caps H*h_exp, H*h_shared and
(training) min(C, T)*max(H, h_exp) and T*max(H, h_shared, E) at 2^30 - 8
elements.  These tests run just inside those caps:

  * forward with two experts of 8192 x 131064 weights (2 GiB - 128 KiB each,
    the second expert's matrices starting 2 GiB past the first's) and a
    shared expert of the same size: 4096 N-tiles of GEMM1 with a ragged last
    one, a 131064-deep GEMM2 contraction with a ragged last K-step; routing
    bit-exact, y on sampled tokens against the float64 oracle;
  * a training step with one segment of 65528 rows of width 16384 (the
    pre-activations, d_u and h each 2 GiB - 256 KiB) and a shared expert of
    the same width: routing bit-exact, y, d_topk_w and dx on sampled tokens,
    and sampled entries of every weight gradient from column slices computed
    over all rows (matrix-vector products in float64).

Tolerances are the bf16 ones of the other parity tests (max |g - ref| /
max |ref| <= 2e-2).
"""

import sys

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import binding as B
from mixture_experts_layer_08_amd import layer
from mixture_experts_layer_08_amd.inputs import (Workload, make_grad_output, make_inputs,
                                                 sample_tokens)
from oracle import moe_oracle as O
from tests.test_gpu_parity import check_routing, f32np, sample_for

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


class HostExperts:
    """Stacked expert weights on the device, copied to the host one expert at
    a time when the oracle indexes them (the whole stack would not fit the
    host comfortably in float64)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return f32np(self.t[e])


def test_forward_at_the_weight_range_limit():
    w = Workload("weight_limit", T=512, H=8192, E=2, K=1, h=131064, hs=131064, cf=0.0)
    s = layer.shape_of(w)
    assert B.moe_check_shape(s) == B.MOE_OK
    assert w.H * w.h * 2 > 0x7ffffff0 - (1 << 18)  # within 256 KiB of the range
    say(f"[limit forward] {w}")
    p = make_inputs(w, seed=21, device="cuda")
    buf = layer.MoeBuffers.allocate(w)
    layer.forward(buf, p)
    torch.cuda.synchronize()
    r = check_routing(w, buf)
    toks = sample_for(w, r, n=24)
    say(f"  counts {r['counts'].tolist()}, checking y on {len(toks)} tokens")
    x = f32np(p["x"])
    ref = O.forward_tokens(x, HostExperts(p["w1"]), HostExperts(p["w2"]), f32np(p["ws1"]),
                           f32np(p["ws2"]), r, toks)
    got = buf.y.cpu().to(torch.float64).numpy()[toks]
    err = relerr(got, ref)
    say(f"  y max rel err {err:.2e}")
    assert err <= TOL


def test_training_at_the_segment_range_limit():
    w = Workload("segment_limit", T=65528, H=64, E=1, K=1, h=16384, hs=16384, cf=0.0)
    alpha = 0.01
    s = layer.shape_of(w, train=True)
    assert B.moe_check_shape(s) == B.MOE_OK
    assert w.T * w.h * 2 > 0x7ffffff0 - (1 << 19)  # within 512 KiB of the range
    say(f"[limit training step] {w}")
    p = make_inputs(w, seed=22, device="cuda")
    dy = make_grad_output(w, seed=22, device="cuda")
    buf = layer.MoeBuffers.allocate(w, train=True)
    g = layer.GradBuffers.allocate(w)
    layer.forward(buf, p)
    layer.backward(buf, g, p, dy, alpha)
    torch.cuda.synchronize()
    r = check_routing(w, buf)
    assert int(r["offsets"][-1]) == w.T  # one segment of every token

    f64 = lambda t: f32np(t).astype(np.float64)
    x, dyh = f64(p["x"]), f64(dy)
    W1, W2 = f64(p["w1"][0]), f64(p["w2"][0])
    S1, S2 = f64(p["ws1"]), f64(p["ws2"])
    wr = f64(p["w_r"])
    l = buf.logits.cpu().numpy().astype(np.float64)
    d_tw = g.d_topk_w.cpu().numpy().astype(np.float64)
    errs = {}

    # gate gradient from the GPU's d_topk_w (zero for a single expert: the
    # renormalised weight is 1 whatever the logit)
    dl = O.route_backward(l, r["ids"], r["w"], d_tw, w.E, w.K, alpha)
    scale = np.abs(d_tw).max()
    assert np.abs(g.d_logits.cpu().numpy() - dl).max() <= 1e-6 * scale

    # sampled tokens: y, d_topk_w, dx
    toks = sample_tokens(w.T, 64, seed=4).numpy()
    ref_y = O.forward_tokens(f32np(p["x"]), HostExperts(p["w1"]), HostExperts(p["w2"]),
                             f32np(p["ws1"]), f32np(p["ws2"]), r, toks)
    errs["y (sampled)"] = relerr(buf.y.cpu().to(torch.float64).numpy()[toks], ref_y)
    xt, dyt = x[toks], dyh[toks]
    wt = r["w"][toks, 0][:, None]
    u = xt @ W1
    us = xt @ S1
    errs["d_topk_w (sampled)"] = relerr(d_tw[toks, 0], np.sum(dyt * (O.gelu_tanh(u) @ W2), 1))
    du = ((wt * dyt) @ W2.T) * O.gelu_tanh_grad(u)
    dus = (dyt @ S2.T) * O.gelu_tanh_grad(us)
    dx_ref = du @ W1.T + dus @ S1.T + dl[toks] @ wr.T
    errs["dx (sampled)"] = relerr(f64(g.dx)[toks], dx_ref)

    # sampled weight-gradient entries, each a sum over all 65528 rows
    rng = np.random.default_rng(6)
    rows = np.arange(r["offsets"][0], r["offsets"][1])
    tok = r["token_of"][rows]
    xe, d_out = x[tok], r["w"][tok, 0][:, None] * dyh[tok]
    js = rng.choice(w.h, 8, replace=False)
    is_ = rng.choice(w.H, 8, replace=False)
    ue = xe @ W1[:, js]
    due = (d_out @ W2[js, :].T) * O.gelu_tanh_grad(ue)
    errs["d_w1 (sampled)"] = relerr(g.d_w1[0][is_][:, js].cpu().numpy(), xe[:, is_].T @ due)
    errs["d_w2 (sampled)"] = relerr(g.d_w2[0][js][:, is_].cpu().numpy(),
                                    O.gelu_tanh(ue).T @ d_out[:, is_])
    us_all = x @ S1[:, js]
    dus_all = (dyh @ S2[js, :].T) * O.gelu_tanh_grad(us_all)
    errs["d_ws1 (sampled)"] = relerr(g.d_ws1[is_][:, js].cpu().numpy(), x[:, is_].T @ dus_all)
    errs["d_ws2 (sampled)"] = relerr(g.d_ws2[js][:, is_].cpu().numpy(),
                                     O.gelu_tanh(us_all).T @ dyh[:, is_])
    say("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, f"relative errors above {TOL}: {bad}"
