"""Per-call parity: moe_expert_ffn, moe_combine and moe_permute_backward
alone, on inputs the test builds itself, against the oracle's function for
the same step.

  * moe_expert_ffn on a packed buffer whose segment sizes are chosen directly
    (empty segments, 1 row, 255 / 256 / 257 rows around the 256-row tile,
    several tiles with a ragged tail), with and without a shared expert,
    against oracle.expert_ffn and oracle.ffn;
  * moe_combine on random expert outputs and an arbitrary row map with
    dropped slots (-1) and repeated rows, with and without a shared output,
    against oracle.combine;
  * moe_permute_backward on random row gradients, a row map with dropped
    slots, router gradients and weights, with and without a shared expert's
    input gradient, against oracle.permute_backward.

Tolerances are those of the layer (max |got - ref| / max |ref|: 2e-2 in bf16
mode, 1e-4 in fp32 mode).
"""

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import binding as B
from mixture_experts_layer_08_amd import layer
from mixture_experts_layer_08_amd.inputs import Workload, make_inputs
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def relerr(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hs", [0, 72, 192])
def test_expert_ffn_alone(dtype, hs):
    """The shared expert narrower than, and (hs = 192) as wide as the routed
    ones; T = 800 gives its launches a 32-row last tile."""
    sizes = [0, 1, 255, 256, 257, 700, 0]
    E = len(sizes)
    w = Workload("ffn_alone", T=800, H=256, E=E, K=2, h=192, hs=hs, cf=0.0, dtype=dtype)
    p = make_inputs(w, seed=31, device="cuda")
    buf = layer.MoeBuffers.allocate(w)
    N = sum(sizes)
    assert N <= buf.xp.shape[0]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    g = torch.Generator(device="cuda").manual_seed(32)
    xp = torch.randn((buf.xp.shape[0], w.H), generator=g, device="cuda").to(buf.xp.dtype)
    buf.xp.copy_(xp)
    buf.offsets.copy_(torch.from_numpy(offsets))
    layer.expert_ffn(buf, p)
    torch.cuda.synchronize()
    ref = O.expert_ffn(f64(buf.xp[:N]), offsets, f64(p["w1"]), f64(p["w2"]))
    err = relerr(f64(buf.out[:N]), ref)
    errs = {"out": err}
    if hs:
        ref_sh = O.ffn(f64(p["x"]), f64(p["ws1"]), f64(p["ws2"]))
        errs["shared_out"] = relerr(f64(buf.shared_out), ref_sh)
    print(f"[ffn alone {dtype} hs={hs}] segments {sizes}: {errs}", flush=True)
    assert all(v <= TOL[dtype] for v in errs.values()), errs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,h", [(256, 192), (328, 136), (200, 120)])
def test_expert_ffn_short_segments(dtype, H, h):
    """Segments shorter than one 256-row tile, and tails of every length class
    around the 32-row MFMA blocks and the 128-row halves of a tile: 1, 31, 32,
    33, 63, 64, 65, 96, 127, 128, 129, 160, 192, 224, 255, 257 and 300 rows.
    In a segment's last tile the kernel skips the MFMA blocks and A loads of
    rows past the segment, so every row of every segment is compared, segment
    by segment, and the rows past the last segment must stay untouched.  Widths
    of 120, 200 and 328 give output tiles with at most 128 valid columns, which
    the kernel runs in its narrow wave layout."""
    sizes = [1, 31, 32, 33, 63, 64, 65, 96, 0, 127, 128, 129, 160, 192, 224, 255, 257, 300]
    E = len(sizes)
    N = sum(sizes)
    # T > N, so the packed buffers have rows past the last segment
    w = Workload("ffn_short", T=N + 100, H=H, E=E, K=1, h=h, hs=0, cf=0.0, dtype=dtype)
    p = make_inputs(w, seed=37, device="cuda")
    buf = layer.MoeBuffers.allocate(w)
    assert buf.xp.shape[0] == N + 100
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    g = torch.Generator(device="cuda").manual_seed(38)
    buf.xp.copy_(torch.randn((buf.xp.shape[0], w.H), generator=g, device="cuda").to(buf.xp.dtype))
    buf.offsets.copy_(torch.from_numpy(offsets))
    sentinel = torch.full_like(buf.out, 7.0)
    buf.out.copy_(sentinel)
    layer.expert_ffn(buf, p)
    torch.cuda.synchronize()
    got = f64(buf.out[:N])
    ref = O.expert_ffn(f64(buf.xp[:N]), offsets, f64(p["w1"]), f64(p["w2"]))
    scale = max(np.abs(ref).max(), 1e-30)
    per_seg = {}
    for e, n in enumerate(sizes):
        if n == 0:
            continue
        a, b = offsets[e], offsets[e + 1]
        per_seg[n] = float(np.abs(got[a:b] - ref[a:b]).max() / scale)
    print(f"[ffn short segments {dtype} H={H} h={h}] worst {max(per_seg.values()):.2e}", flush=True)
    bad = {n: v for n, v in per_seg.items() if not v <= TOL[dtype]}
    assert not bad, bad
    assert torch.equal(buf.out[N:], sentinel[N:]), "rows past the last segment were written"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shared", [False, True])
def test_combine_alone(dtype, shared):
    T, K, H, N = 500, 3, 264, 900
    w = Workload("combine_alone", T=T, H=H, E=4, K=K, h=64, hs=64 if shared else 0, cf=0.0,
                 dtype=dtype)
    s = layer.shape_of(w)
    dt = w.torch_dtype()
    r = np.random.default_rng(33)
    row_of = r.integers(0, N, size=(T, K)).astype(np.int32)
    row_of[r.random((T, K)) < 0.2] = -1
    row_of[7] = -1  # a token with every slot dropped
    wts = r.random((T, K)).astype(np.float32)
    g = torch.Generator(device="cuda").manual_seed(34)
    out = torch.randn((N, H), generator=g, device="cuda").to(dt)
    sh = torch.randn((T, H), generator=g, device="cuda").to(dt) if shared else None
    y = torch.empty((T, H), dtype=dt, device="cuda")
    B.moe_combine(s, out, torch.from_numpy(row_of).cuda(), torch.from_numpy(wts).cuda(), sh, y)
    torch.cuda.synchronize()
    ref = O.combine(f64(out), row_of.astype(np.int64), wts.astype(np.float64),
                    f64(sh) if shared else None)
    err = relerr(f64(y), ref)
    print(f"[combine alone {dtype} shared={shared}] max rel err {err:.2e}", flush=True)
    assert err <= TOL[dtype]
    assert not torch.any(y[7] != (sh[7] if shared else 0))


# (dtype, T, H, E, K, shared): bf16 with at most 16 experts folds d_logits W_r^T
# into the un-permute kernel (router weights staged in LDS, at most 64 KiB
# once padded to 8 experts); wider routers, fp32 mode and larger H run it as
# a separate accumulating GEMM.
PERMUTE_BWD = [
    ("bf16", 5000, 4096, 8, 2, False),   # 64 KiB of weights, more tokens than one sweep
    ("bf16", 700, 2048, 16, 4, True),    # two 8-expert planes, 64 KiB
    ("bf16", 333, 1336, 12, 3, False),   # E not a multiple of 8: scalar staging
    ("bf16", 129, 264, 1, 1, True),      # one expert
    ("bf16", 300, 4160, 8, 2, False),    # above the LDS limit: GEMM form
    ("bf16", 250, 256, 32, 4, True),     # more than 16 experts: GEMM form
    ("f32", 300, 264, 8, 2, True),
]


@pytest.mark.parametrize("dtype,T,H,E,K,shared", PERMUTE_BWD,
                         ids=lambda v: str(v))
def test_permute_backward_alone(dtype, T, H, E, K, shared):
    """dx = sum of the kept slots' d_xp rows (+ the shared expert's dx)
    + d_logits W_r^T, against oracle.permute_backward."""
    w = Workload("permute_bwd_alone", T=T, H=H, E=E, K=K, h=64, hs=64 if shared else 0,
                 cf=0.0, dtype=dtype)
    buf = layer.MoeBuffers.allocate(w, train=True)
    dt = w.torch_dtype()
    N = T * K
    r = np.random.default_rng(T + H + E)
    row_of = r.permutation(N).reshape(T, K).astype(np.int32)
    row_of[r.random((T, K)) < 0.15] = -1
    row_of[T // 2] = -1  # a token with every slot dropped
    g = torch.Generator(device="cuda").manual_seed(H)
    d_xp = torch.randn((N, H), generator=g, device="cuda").to(dt)
    dxs = torch.randn((T, H), generator=g, device="cuda").to(dt) if shared else None
    d_logits = torch.randn((T, E), generator=g, device="cuda") * 0.5
    w_r = (torch.randn((H, E), generator=g, device="cuda") * 0.05).to(dt)
    dx = torch.full((T, H), float("nan"), dtype=dt, device="cuda")
    print(f"[permute backward alone {dtype} T={T} H={H} E={E} K={K} shared={shared}]",
          flush=True)
    B.moe_permute_backward(buf.shape, d_xp, torch.from_numpy(row_of).cuda(), dxs, d_logits,
                           w_r, dx, buf.ws)
    torch.cuda.synchronize()
    ref = O.permute_backward(f64(d_xp), row_of.astype(np.int64), f64(d_logits), f64(w_r),
                             f64(dxs) if shared else None)
    got = f64(dx)
    assert np.all(np.isfinite(got)), "rows of dx left unwritten"
    err = relerr(got, ref)
    print(f"  max rel err {err:.2e}", flush=True)
    assert err <= TOL[dtype]
