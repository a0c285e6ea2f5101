"""One MoE-layer forward through the C ABI, with torch supplying device memory.

:class:`MoeBuffers` allocates every output and scratch buffer of a shape once
(callers reuse it across steps); :func:`forward` issues the five library calls
in order on one stream.  No arithmetic of the layer happens here.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import binding as B
from .inputs import Workload


def shape_of(w: Workload, logits_in: bool = False) -> B.moe_shape:
    return B.make_shape(w.T, w.H, w.E, w.K, w.h, w.hs, w.cf,
                        B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32,
                        B.MOE_FLAG_LOGITS_IN if logits_in else 0)


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
    def allocate(w: Workload, device="cuda", logits_in: bool = False) -> "MoeBuffers":
        s = shape_of(w, logits_in)
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
