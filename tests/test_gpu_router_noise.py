"""GPU parity of the noisy router (Gumbel noise and temperature), through the C ABI.

Protocol:
  1. the GPU routes with MOE_FLAG_GUMBEL (seed, offset) and a temperature tau;
     its `logits` output is the selection scores z = (l + g) / tau;
  2. the same inputs routed without noise at tau = 1 give l (the router is
     deterministic, so l is the l of step 1); the noise the GPU added,
     z * tau - l, is checked against the oracle's Philox + Gumbel noise for
     the same (t, e, seed, offset): within 2e-5 (1 + |g|) of the transform
     evaluated in float32 like the kernel, and within 1e-4 (1 + |g|) of the
     float64 transform except in the far tail u > 1 - 2^-14, where float32
     cannot hold u + 1e-9 (there within 0.05);
  3. routing is then bit-exact against the oracle routing from the GPU's z
     (top-k, counts, row map, drops), weights to 1e-6 and aux to 1e-5, as for
     the plain router;
  4. y and, in training mode, every gradient against the float64 oracle at
     the plain router's tolerances; the router gradients use d l = d z / tau.
"""

import sys

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import binding as B
from mixture_experts_layer_08_amd import layer
from mixture_experts_layer_08_amd.inputs import (WORKLOADS, Workload, make_grad_output,
                                                 make_inputs, sample_tokens)
from oracle import gumbel_oracle as G
from oracle import moe_oracle as O
from tests.test_gpu_backward import relerr
from tests.test_gpu_parity import check_routing, check_y, f64, sample_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def route(w, p, tau=0.0, noise=None):
    buf = layer.MoeBuffers.allocate(w, router_tau=tau, noise=noise)
    layer.route(buf, p)
    layer.aux_loss(buf)
    layer.permute(buf, p)
    torch.cuda.synchronize()
    return buf


def gumbel_f32(u):
    """The page's transform in float32 arithmetic (the kernel's precision)."""
    u = np.asarray(u, dtype=np.float32)
    e = np.float32(1e-9)
    return -np.log(-np.log(u + e) + e)


def check_noise(w, p, z_buf, tau, seed, offset, tokens=None):
    plain = route(w, p)
    l = plain.logits.cpu().numpy().astype(np.float64)
    z = z_buf.logits.cpu().numpy().astype(np.float64)
    if tokens is None:
        tokens = np.arange(w.T)
    u = G.uniforms(w.T, w.E, seed, offset)[tokens]
    g64 = G.gumbel(u)
    g32 = gumbel_f32(u).astype(np.float64)
    teff = tau if tau > 0 else 1.0
    got = z[tokens] * teff - l[tokens]
    # rounding of the fp32 sum l + g and of the division by tau
    slack = 2.0 ** -22 * (np.abs(l[tokens]) + np.abs(g64) + 1.0)
    e32 = np.abs(got - g32) / (1.0 + np.abs(g32))
    tail = u > 1.0 - 2.0 ** -14
    e64 = np.abs(got - g64)
    say(f"  noise: {got.size} values, max err vs float32 transform {e32.max():.2e}, "
        f"vs float64 {np.max(e64[~tail] / (1 + np.abs(g64[~tail]))):.2e} (tail {tail.sum()})")
    assert np.all(np.abs(got - g32) <= 2e-5 * (1.0 + np.abs(g32)) + slack)
    assert np.all(e64[~tail] <= 1e-4 * (1.0 + np.abs(g64[~tail])) + slack[~tail])
    assert np.all(e64[tail] <= 0.05)
    return l, z


CASES = [
    ("E8_tau08", dict(T=1000, H=256, E=8, K=2, h=64, cf=1.25), 0.8),
    ("E6_tau1", dict(T=777, H=128, E=6, K=2, h=64, cf=0.0), 0.0),
    ("E64_tau12", dict(T=640, H=128, E=64, K=4, h=64, cf=1.0, bias="normal"), 1.2),
    ("E256_K8", dict(T=130, H=64, E=256, K=8, h=32, cf=1.25), 0.5),
    ("shared_tau07", dict(T=500, H=128, E=16, K=4, h=64, hs=96, cf=1.25), 0.7),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,kw,tau", CASES, ids=[c[0] for c in CASES])
def test_noisy_router_forward(name, kw, tau, dtype):
    w = Workload(name, dtype=dtype, **kw)
    seed, offset = 0x0123456789ABCDEF, 17
    say(f"[noise {name} {dtype}] tau {tau}")
    p = make_inputs(w, seed=3, device="cuda")
    buf = layer.MoeBuffers.allocate(w, router_tau=tau, noise=(seed, offset))
    layer.forward(buf, p)
    torch.cuda.synchronize()
    check_noise(w, p, buf, tau, seed, offset)
    r = check_routing(w, buf)
    check_y(w, p, buf, r)


def test_temperature_without_noise_is_a_division():
    """tau alone: z = fl32(l / tau) bitwise, and the top-k set equals the
    plain router's (a positive scale is monotone)."""
    w = Workload("tau", T=900, H=128, E=8, K=2, h=64, cf=1.25)
    p = make_inputs(w, seed=4, device="cuda")
    plain = route(w, p)
    hot = route(w, p, tau=0.5)
    l = plain.logits.cpu().numpy()
    z = hot.logits.cpu().numpy()
    assert np.array_equal(z, (l / np.float32(0.5)).astype(np.float32))
    assert torch.equal(plain.topk_ids, hot.topk_ids)
    check_routing(w, hot)


def test_noise_streams():
    """The same (seed, offset) gives bitwise the same scores; another offset
    or seed gives different noise; offset 0 and seed 0 are valid."""
    w = Workload("streams", T=300, H=64, E=8, K=2, h=64, cf=0.0)
    p = make_inputs(w, seed=5, device="cuda")
    a = route(w, p, noise=(0, 0))
    b = route(w, p, noise=(0, 0))
    c = route(w, p, noise=(0, 1))
    d = route(w, p, noise=(1, 0))
    assert torch.equal(a.logits, b.logits) and torch.equal(a.topk_ids, b.topk_ids)
    assert not torch.equal(a.logits, c.logits) and not torch.equal(a.logits, d.logits)
    check_noise(w, p, c, 0.0, 0, 1)


@pytest.mark.parametrize("dtype,tau,alpha", [("f32", 0.7, 0.3), ("bf16", 1.3, 0.01)])
def test_noisy_router_backward(dtype, tau, alpha):
    """Training step with noise and temperature: every gradient against the
    oracle backward on the GPU's scores, with d l = d z / tau."""
    w = Workload("bwd_noise", T=600, H=128, E=8, K=2, h=64, cf=1.0, dtype=dtype)
    seed, offset = 99, 3
    p = make_inputs(w, seed=6, device="cuda")
    dy = make_grad_output(w, seed=6, device="cuda")
    buf = layer.MoeBuffers.allocate(w, train=True, router_tau=tau, noise=(seed, offset))
    g = layer.GradBuffers.allocate(w)
    layer.forward(buf, p)
    layer.backward(buf, g, p, dy, alpha)
    torch.cuda.synchronize()
    check_routing(w, buf)
    z = buf.logits.cpu().numpy().astype(np.float64)
    ref = O.backward(f64(p["x"]), f64(p["w_r"]), None, f64(p["w1"]), f64(p["w2"]), dy=f64(dy),
                     K=w.K, cf=w.cf, alpha=alpha, logits=z, tau=tau)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    pairs = [("d_topk_w", g.d_topk_w, ref["d_w"]), ("d_logits", g.d_logits, ref["d_logits"] / tau),
             ("d_w_router", g.d_w_router, ref["dw_r"]), ("d_b_router", g.d_b_router, ref["db_r"]),
             ("d_w1", g.d_w1, ref["dw1"]), ("d_w2", g.d_w2, ref["dw2"]), ("dx", g.dx, ref["dx"])]
    errs = {n: relerr(f64(a), b) for n, a, b in pairs}
    say("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= tol for v in errs.values()), errs


def test_mixtral_full_size_with_noise():
    """T=32768, H=4096, E=8, top-2 in the bench's launch configuration with
    noise and tau = 1.2: routing complete and bit-exact, the noise on a token
    sample, y on sampled tokens."""
    w = WORKLOADS["mixtral_bf16"]
    seed, offset, tau = 2024, 5, 1.2
    say(f"[noise mixtral full size] tau {tau}")
    p = make_inputs(w, seed=0, device="cuda")
    buf = layer.MoeBuffers.allocate(w, router_tau=tau, noise=(seed, offset))
    layer.forward(buf, p)
    torch.cuda.synchronize()
    toks = sample_tokens(w.T, 4096, seed=8).numpy()
    check_noise(w, p, buf, tau, seed, offset, tokens=toks)
    r = check_routing(w, buf)
    counts = r["counts"]
    say(f"  counts {counts.min()}..{counts.max()}, dropped {r['n_dropped']}, aux {r['aux']:.4f}")
    check_y(w, p, buf, r, sample_for(w, r, n=512))
