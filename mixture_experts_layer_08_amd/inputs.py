"""Seeded synthetic workloads for the MoE-layer forward.

This module only draws random numbers and names the workload sizes; it holds
none of the layer's arithmetic (no routing, capacity, GEMM or activation), so
that the HIP path and the CPU oracle can both be fed from it without sharing
any of the method's code.

Workloads (the token mixes of the pages they stand in for):

* ``tiny_fp32``  T=256, H=64, E=4, top-2, h=128, fp32, no capacity limit.
* ``small_bf16`` T=4096, H=1024, E=8, top-2, h=2816, bf16, capacity factor 1.25
  (the default layer settings of the MoE-layer listing in the dpshk.com
  "MoE module infra notes", section 4.2).
* ``mixtral_bf16`` T=32768 (seq 4096 x micro-batch 8), H=4096, E=8, top-2,
  h=14336, bf16, capacity factor 1.25 (the worked example of the cf-1.com
  page "Dissecting the MoE communication bottleneck", section 2.2).
* ``finegrained_bf16`` T=16384, H=4096, E=64, top-4, h=2048 plus one shared
  expert of width 2048, per-expert router bias ~N(0,1), capacity factor 1.25
  (fine-grained plus shared experts, same page, section 2.3).
* ``skewed_bf16`` T=32768, H=4096, E=128, top-2, h=1408, router bias +4 on
  experts 0 and 1, no capacity limit (the skewed routing of the same page,
  section 3.1).

Recipe: one ``torch.Generator`` seeded with ``seed`` draws, in this order,
x [T,H] ~ N(0,1); W_r [H,E] ~ N(0,0.02); the router bias when it is random;
W1 [E,H,h] (expert by expert); W2 [E,h,H] (expert by expert); Ws1 [H,hs];
Ws2 [hs,H], all weights ~ N(0, 0.02) with 0.02 the standard deviation.  The
fp32 draws are then rounded to the workload dtype (round to nearest even for
bf16).  The router bias stays fp32.  The generator lives on the device the
tensors are made on, so a CPU draw and a GPU draw of one workload differ; a
test feeds both sides from one draw.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    K: int
    h: int
    hs: int = 0                 # shared-expert width, 0 = no shared expert
    cf: float = 0.0             # capacity factor, <= 0 = no capacity limit
    dtype: str = "bf16"         # "bf16" or "f32"
    bias: str = "none"          # "none" | "normal" | "hot01"

    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=256, H=64, E=4, K=2, h=128, cf=0.0, dtype="f32"),
    "small_bf16": Workload("small_bf16", T=4096, H=1024, E=8, K=2, h=2816, cf=1.25),
    "mixtral_bf16": Workload("mixtral_bf16", T=32768, H=4096, E=8, K=2, h=14336, cf=1.25),
    "finegrained_bf16": Workload("finegrained_bf16", T=16384, H=4096, E=64, K=4, h=2048,
                                 hs=2048, cf=1.25, bias="normal"),
    "skewed_bf16": Workload("skewed_bf16", T=32768, H=4096, E=128, K=2, h=1408,
                            cf=0.0, bias="hot01"),
}


def _randn(gen: torch.Generator, shape, std: float, dtype: torch.dtype, device) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> dict:
    """Draw every tensor of workload ``w``; returns a dict of tensors on ``device``.

    Keys: x [T,H], w_r [H,E], b_r [E] fp32 or None, w1 [E,H,h], w2 [E,h,H],
    ws1 [H,hs] / ws2 [hs,H] or None.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = w.torch_dtype()
    x = _randn(gen, (w.T, w.H), 1.0, dt, device)
    w_r = _randn(gen, (w.H, w.E), WEIGHT_STD, dt, device)
    b_r: Optional[torch.Tensor]
    if w.bias == "normal":
        b_r = torch.randn((w.E,), generator=gen, dtype=torch.float32, device=device)
    elif w.bias == "hot01":
        b_r = torch.zeros((w.E,), dtype=torch.float32, device=device)
        b_r[:2] = 4.0
    else:
        b_r = None
    w1 = torch.empty((w.E, w.H, w.h), dtype=dt, device=device)
    for e in range(w.E):
        w1[e] = _randn(gen, (w.H, w.h), WEIGHT_STD, dt, device)
    w2 = torch.empty((w.E, w.h, w.H), dtype=dt, device=device)
    for e in range(w.E):
        w2[e] = _randn(gen, (w.h, w.H), WEIGHT_STD, dt, device)
    ws1 = ws2 = None
    if w.hs > 0:
        ws1 = _randn(gen, (w.H, w.hs), WEIGHT_STD, dt, device)
        ws2 = _randn(gen, (w.hs, w.H), WEIGHT_STD, dt, device)
    return dict(x=x, w_r=w_r, b_r=b_r, w1=w1, w2=w2, ws1=ws1, ws2=ws2)


def make_grad_output(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """The upstream gradient dy [T,H] of a backward test: N(0,1) drawn from its
    own generator seeded with ``seed + 7919`` (independent of the forward
    inputs), rounded to the workload dtype."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 7919)
    return _randn(gen, (w.T, w.H), 1.0, w.torch_dtype(), device)


def to_numpy_f64(t: Optional[torch.Tensor]):
    """Widen a tensor exactly to a float64 numpy array (bf16 and fp32 both fit)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def sample_tokens(T: int, n: int, seed: int = 1) -> torch.Tensor:
    """A sorted seeded sample of ``n`` distinct token indices out of ``T``."""
    g = torch.Generator().manual_seed(seed)
    n = min(n, T)
    return torch.randperm(T, generator=g)[:n].sort().values
