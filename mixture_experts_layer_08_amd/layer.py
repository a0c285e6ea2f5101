"""One MoE-layer forward (and backward) through the C ABI, with torch
supplying device memory.

:class:`MoeBuffers` allocates every output and scratch buffer of a shape once
(callers reuse it across steps); :func:`forward` issues the five library calls
in order on one stream, :func:`backward` the four backward calls after a
forward run with ``train=True``.  No arithmetic of the layer happens here.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import binding as B
from .inputs import Workload


def shape_of(w: Workload, logits_in: bool = False, train: bool = False,
             router_tau: float = 0.0, noise: Optional[tuple] = None) -> B.moe_shape:
    """The C shape of workload w.  router_tau: softmax temperature (0 = 1);
    noise: (seed, offset) turns on the router's Gumbel noise."""
    flags = (B.MOE_FLAG_LOGITS_IN if logits_in else 0) | (B.MOE_FLAG_TRAIN if train else 0)
    seed = offset = 0
    if noise is not None:
        flags |= B.MOE_FLAG_GUMBEL
        seed, offset = noise
    return B.make_shape(w.T, w.H, w.E, w.K, w.h, w.hs, w.cf,
                        B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32, flags, router_tau,
                        seed, offset)


@dataclasses.dataclass
class MoeBuffers:
    shape: B.moe_shape
    logits: torch.Tensor
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    aux: torch.Tensor
    counts: torch.Tensor
    kept: torch.Tensor
    offsets: torch.Tensor
    row_of: torch.Tensor
    token_of: torch.Tensor
    n_dropped: torch.Tensor
    xp: torch.Tensor
    hbuf: torch.Tensor
    out: torch.Tensor
    hshared: Optional[torch.Tensor]
    shared_out: Optional[torch.Tensor]
    y: torch.Tensor
    ws: torch.Tensor

    @staticmethod
    def allocate(w: Workload, device="cuda", logits_in: bool = False,
                 train: bool = False, router_tau: float = 0.0,
                 noise: Optional[tuple] = None) -> "MoeBuffers":
        s = shape_of(w, logits_in, train, router_tau, noise)
        st = B.moe_check_shape(s)
        if st != B.MOE_OK:
            raise B.MoeError("moe_check_shape", st, B.moe_status_string(st))
        dt = w.torch_dtype()
        n = B.moe_max_rows(s)
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        act = dict(dtype=dt, device=device)
        return MoeBuffers(
            shape=s,
            logits=torch.empty((w.T, w.E), **f32),
            topk_ids=torch.empty((w.T, w.K), **i32),
            topk_w=torch.empty((w.T, w.K), **f32),
            aux=torch.empty((1,), **f32),
            counts=torch.empty((w.E,), **i32),
            kept=torch.empty((w.E,), **i32),
            offsets=torch.empty((w.E + 1,), **i32),
            row_of=torch.empty((w.T, w.K), **i32),
            token_of=torch.empty((max(n, 1),), **i32),
            n_dropped=torch.empty((1,), **i32),
            xp=torch.empty((max(n, 1), w.H), **act),
            hbuf=torch.empty((max(n, 1), w.h), **act),
            out=torch.empty((max(n, 1), w.H), **act),
            hshared=torch.empty((w.T, w.hs), **act) if w.hs else None,
            shared_out=torch.empty((w.T, w.H), **act) if w.hs else None,
            y=torch.empty((w.T, w.H), **act),
            ws=torch.empty((B.moe_workspace_size(s),), dtype=torch.uint8, device=device),
        )


def route(buf: MoeBuffers, p: dict, stream=None):
    B.moe_route(buf.shape, p["x"], p["w_r"], p.get("b_r"), buf.logits, buf.topk_ids,
                buf.topk_w, buf.ws, stream)


def aux_loss(buf: MoeBuffers, stream=None):
    B.moe_aux_loss(buf.shape, buf.ws, buf.aux, stream)


def permute(buf: MoeBuffers, p: dict, stream=None):
    B.moe_permute(buf.shape, p["x"], buf.topk_ids, buf.ws, buf.counts, buf.kept, buf.offsets,
                  buf.row_of, buf.token_of, buf.n_dropped, buf.xp, stream)


def expert_ffn(buf: MoeBuffers, p: dict, stream=None):
    B.moe_expert_ffn(buf.shape, buf.xp, buf.offsets, p["w1"], p["w2"], buf.hbuf, buf.out,
                     p["x"], p.get("ws1"), p.get("ws2"), buf.hshared, buf.shared_out, buf.ws,
                     stream)


def combine(buf: MoeBuffers, stream=None):
    B.moe_combine(buf.shape, buf.out, buf.row_of, buf.topk_w, buf.shared_out, buf.y, stream)


def forward(buf: MoeBuffers, p: dict, stream=None) -> MoeBuffers:
    """route -> aux_loss -> permute -> expert_ffn -> combine, asynchronously."""
    route(buf, p, stream)
    aux_loss(buf, stream)
    permute(buf, p, stream)
    expert_ffn(buf, p, stream)
    combine(buf, stream)
    return buf


@dataclasses.dataclass
class GradBuffers:
    """Outputs of the backward calls (weight gradients fp32, the rest in the
    activation dtype or fp32 as the C ABI states)."""
    d_out: torch.Tensor
    d_topk_w: torch.Tensor
    d_logits: torch.Tensor
    d_w_router: torch.Tensor
    d_b_router: torch.Tensor
    d_xp: torch.Tensor
    d_w1: torch.Tensor
    d_w2: torch.Tensor
    d_x_shared: Optional[torch.Tensor]
    d_ws1: Optional[torch.Tensor]
    d_ws2: Optional[torch.Tensor]
    dx: torch.Tensor

    @staticmethod
    def allocate(w: Workload, device="cuda") -> "GradBuffers":
        dt = w.torch_dtype()
        n = max(B.moe_max_rows(shape_of(w)), 1)
        f32 = dict(dtype=torch.float32, device=device)
        act = dict(dtype=dt, device=device)
        return GradBuffers(
            d_out=torch.empty((n, w.H), **act),
            d_topk_w=torch.empty((w.T, w.K), **f32),
            d_logits=torch.empty((w.T, w.E), **f32),
            d_w_router=torch.empty((w.H, w.E), **f32),
            d_b_router=torch.empty((w.E,), **f32),
            d_xp=torch.empty((n, w.H), **act),
            d_w1=torch.empty((w.E, w.H, w.h), **f32),
            d_w2=torch.empty((w.E, w.h, w.H), **f32),
            d_x_shared=torch.empty((w.T, w.H), **act) if w.hs else None,
            d_ws1=torch.empty((w.H, w.hs), **f32) if w.hs else None,
            d_ws2=torch.empty((w.hs, w.H), **f32) if w.hs else None,
            dx=torch.empty((w.T, w.H), **act),
        )


def combine_backward(buf: MoeBuffers, g: GradBuffers, dy, stream=None):
    B.moe_combine_backward(buf.shape, dy, buf.out, buf.row_of, buf.topk_w, g.d_out, g.d_topk_w,
                           stream)


def route_backward(buf: MoeBuffers, g: GradBuffers, p: dict, alpha: float, stream=None):
    B.moe_route_backward(buf.shape, p["x"], buf.logits, buf.topk_ids, buf.topk_w, g.d_topk_w,
                         buf.counts, alpha, g.d_logits, g.d_w_router, g.d_b_router, buf.ws,
                         stream)


def expert_ffn_backward(buf: MoeBuffers, g: GradBuffers, p: dict, dy, stream=None):
    B.moe_expert_ffn_backward(buf.shape, buf.xp, buf.offsets, p["w1"], p["w2"], buf.hbuf,
                              g.d_out, g.d_xp, g.d_w1, g.d_w2, p["x"], p.get("ws1"),
                              p.get("ws2"), buf.hshared, dy, g.d_x_shared, g.d_ws1, g.d_ws2,
                              buf.ws, stream)


def permute_backward(buf: MoeBuffers, g: GradBuffers, p: dict, stream=None):
    B.moe_permute_backward(buf.shape, g.d_xp, buf.row_of, g.d_x_shared, g.d_logits, p["w_r"],
                           g.dx, buf.ws, stream)


def backward(buf: MoeBuffers, g: GradBuffers, p: dict, dy, alpha: float = 0.0,
             stream=None) -> GradBuffers:
    """combine -> route -> expert FFN -> permute backward, asynchronously,
    for the gradient of <dy, y> + alpha * aux after a train-mode forward."""
    combine_backward(buf, g, dy, stream)
    route_backward(buf, g, p, alpha, stream)
    expert_ffn_backward(buf, g, p, dy, stream)
    permute_backward(buf, g, p, stream)
    return g


# ---------------------------------------------------------------------------
# MXFP8 forward (moe_*_mxfp8): FP8 dispatch, expert GEMMs and combine
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class MxWeights:
    """Expert weights in MXFP8 (moe_quantize_weights_mxfp8): codes of the
    [E,N,K] transposed weights (K the contraction dimension) in 256 x 64
    panels, flat uint8 of moe_mx_weight_code_bytes; operand-layout scales."""
    w1_q: torch.Tensor
    w1_s: torch.Tensor
    w2_q: torch.Tensor
    w2_s: torch.Tensor
    ws1_q: Optional[torch.Tensor]
    ws1_s: Optional[torch.Tensor]
    ws2_q: Optional[torch.Tensor]
    ws2_s: Optional[torch.Tensor]

    @staticmethod
    def quantize(w: Workload, p: dict, stream=None) -> "MxWeights":
        dev = p["w1"].device
        dt = B.MOE_BF16 if p["w1"].dtype == torch.bfloat16 else B.MOE_F32

        def q(t, G, K, N):
            codes = torch.empty((B.moe_mx_weight_code_bytes(G, K, N),), dtype=torch.uint8,
                                device=dev)
            sc = torch.empty((G * B.moe_mx_operand_scale_bytes(N, K),), dtype=torch.uint8,
                             device=dev)
            B.moe_quantize_weights_mxfp8(t, dt, G, K, N, codes, sc, stream)
            return codes, sc

        w1_q, w1_s = q(p["w1"], w.E, w.H, w.h)
        w2_q, w2_s = q(p["w2"], w.E, w.h, w.H)
        ws1_q = ws1_s = ws2_q = ws2_s = None
        if w.hs:
            ws1_q, ws1_s = q(p["ws1"], 1, w.H, w.hs)
            ws2_q, ws2_s = q(p["ws2"], 1, w.hs, w.H)
        return MxWeights(w1_q, w1_s, w2_q, w2_s, ws1_q, ws1_s, ws2_q, ws2_s)


@dataclasses.dataclass
class MxBuffers:
    """Buffers of one MXFP8 forward: the routing outputs of :class:`MoeBuffers`
    and FP8 codes + scales in place of the bf16 intermediates."""
    shape: B.moe_shape
    logits: torch.Tensor
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    aux: torch.Tensor
    counts: torch.Tensor
    kept: torch.Tensor
    offsets: torch.Tensor
    row_of: torch.Tensor
    token_of: torch.Tensor
    n_dropped: torch.Tensor
    xp_q: torch.Tensor
    xp_s: torch.Tensor
    x_q: Optional[torch.Tensor]
    x_s: Optional[torch.Tensor]
    h_q: torch.Tensor
    h_s: torch.Tensor
    out_q: torch.Tensor
    out_s: torch.Tensor
    hsh_q: Optional[torch.Tensor]
    hsh_s: Optional[torch.Tensor]
    sh_q: Optional[torch.Tensor]
    sh_s: Optional[torch.Tensor]
    y: torch.Tensor
    ws: torch.Tensor

    @staticmethod
    def allocate(w: Workload, device="cuda") -> "MxBuffers":
        s = shape_of(w)
        st = B.moe_check_shape(s)
        if st != B.MOE_OK:
            raise B.MoeError("moe_check_shape", st, B.moe_status_string(st))
        n = max(B.moe_max_rows(s), 1)
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        u8 = dict(dtype=torch.uint8, device=device)
        opsc = lambda R, K: torch.empty((B.moe_mx_operand_scale_bytes(R, K),), **u8)
        return MxBuffers(
            shape=s,
            logits=torch.empty((w.T, w.E), **f32),
            topk_ids=torch.empty((w.T, w.K), **i32),
            topk_w=torch.empty((w.T, w.K), **f32),
            aux=torch.empty((1,), **f32),
            counts=torch.empty((w.E,), **i32),
            kept=torch.empty((w.E,), **i32),
            offsets=torch.empty((w.E + 1,), **i32),
            row_of=torch.empty((w.T, w.K), **i32),
            token_of=torch.empty((n,), **i32),
            n_dropped=torch.empty((1,), **i32),
            xp_q=torch.empty((n, w.H), **u8),
            xp_s=opsc(n, w.H),
            x_q=torch.empty((w.T, w.H), **u8) if w.hs else None,
            x_s=opsc(w.T, w.H) if w.hs else None,
            h_q=torch.empty((n, w.h), **u8),
            h_s=opsc(n, w.h),
            out_q=torch.empty((n, w.H), **u8),
            out_s=torch.empty((n, w.H // 32), **u8),
            hsh_q=torch.empty((w.T, w.hs), **u8) if w.hs else None,
            hsh_s=opsc(w.T, w.hs) if w.hs else None,
            sh_q=torch.empty((w.T, w.H), **u8) if w.hs else None,
            sh_s=torch.empty((w.T, w.H // 32), **u8) if w.hs else None,
            y=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=device),
            ws=torch.empty((B.moe_workspace_size(s),), **u8),
        )


def permute_mxfp8(buf: MxBuffers, p: dict, stream=None):
    B.moe_permute_mxfp8(buf.shape, p["x"], buf.topk_ids, buf.ws, buf.counts, buf.kept,
                        buf.offsets, buf.row_of, buf.token_of, buf.n_dropped, buf.xp_q,
                        buf.xp_s, buf.x_q, buf.x_s, stream)


def expert_ffn_mxfp8(buf: MxBuffers, mw: MxWeights, stream=None):
    B.moe_expert_ffn_mxfp8(buf.shape, buf.xp_q, buf.xp_s, buf.offsets, mw.w1_q, mw.w1_s,
                           mw.w2_q, mw.w2_s, buf.h_q, buf.h_s, buf.out_q, buf.out_s, buf.x_q,
                           buf.x_s, mw.ws1_q, mw.ws1_s, mw.ws2_q, mw.ws2_s, buf.hsh_q,
                           buf.hsh_s, buf.sh_q, buf.sh_s, stream)


def combine_mxfp8(buf: MxBuffers, stream=None):
    B.moe_combine_mxfp8(buf.shape, buf.out_q, buf.out_s, buf.row_of, buf.topk_w, buf.sh_q,
                        buf.sh_s, buf.y, stream)


def forward_mxfp8(buf: MxBuffers, p: dict, mw: MxWeights, stream=None) -> MxBuffers:
    """route -> aux_loss -> permute_mxfp8 -> expert_ffn_mxfp8 -> combine_mxfp8."""
    route(buf, p, stream)
    aux_loss(buf, stream)
    permute_mxfp8(buf, p, stream)
    expert_ffn_mxfp8(buf, mw, stream)
    combine_mxfp8(buf, stream)
    return buf
