"""Algorithmic byte and FLOP counts of the MoE-layer forward.

These are the counted work of each step (what the method must move or
multiply), not what a kernel happens to read.  They follow the traffic and
compute formulas of the cf-1.com page "Dissecting the MoE communication
bottleneck": section 2.1 (dispatch bytes = tokens x top_k x hidden x dtype
bytes, combine the same) and section 2.2 (expert FFN = 2 x 2 x H x h_exp
FLOP per token-expert pair).
"""

from __future__ import annotations


def dispatch_bytes(tokens: int, top_k: int, hidden: int, dtype_bytes: int) -> int:
    """Bytes one layer's dispatch moves: B * K * H * dtype (section 2.1)."""
    return tokens * top_k * hidden * dtype_bytes


def combine_bytes(tokens: int, top_k: int, hidden: int, dtype_bytes: int) -> int:
    """Combine moves the same payload back (section 2.1)."""
    return tokens * top_k * hidden * dtype_bytes


def ffn_flop_per_assignment(hidden: int, h_exp: int) -> int:
    """2 x 2 x H x h_exp: two matmuls of 2*H*h FLOP each (section 2.2)."""
    return 4 * hidden * h_exp


def comm_compute_ratio(dtype_bytes: int, h_exp: int) -> float:
    """Bytes per FLOP of one token-expert pair: 2*H*dtype / (4*H*h) (section 2.3)."""
    return dtype_bytes / (2.0 * h_exp)


# -- per-launch algorithmic work of this library's kernels -------------------

def grouped_gemm_flop_per_launch(n_rows: int, H: int, h: int) -> int:
    """One grouped-GEMM launch (GEMM1 or GEMM2) over n_rows kept rows: 2*n*H*h."""
    return 2 * n_rows * H * h


def segment_roofline_s(rows, H: int, h: int, b: int, peak_flops: float, peak_bytes: float,
                       shared_rows: int = 0, hs: int = 0):
    """Roofline times of the expert FFN (GEMM1 + GEMM2) over segments of
    `rows` kept rows (plus a shared expert over shared_rows tokens).

    Per segment with n > 0 rows: 4*n*H*h FLOP and the bytes it must move at
    least once, its two weight matrices (2*H*h*b) plus its activations (x
    rows read, hidden rows written and read, output rows written:
    2*n*(H + h)*b).  Returns (flop-bound s, byte-bound s, per-segment bound s)
    where the first two total the whole launch pair and the last sums
    max(flop time, byte time) over the segments, the bound of a segment that
    is too small to reach the MFMA rate (a few hundred rows against its
    weights) being its weight traffic.
    """
    segs = [(int(n), h) for n in rows if int(n) > 0]
    if shared_rows > 0 and hs > 0:
        segs.append((shared_rows, hs))
    flop = byte = seg = 0.0
    for n, width in segs:
        f = 4.0 * n * H * width
        m = (2.0 * H * width + 2.0 * n * (H + width)) * b
        flop += f
        byte += m
        seg += max(f / peak_flops, m / peak_bytes)
    return flop / peak_flops, byte / peak_bytes, seg


def permute_bytes(T: int, n_kept: int, H: int, b: int, K: int) -> int:
    """Dispatch kernel: each token row read once, each kept row written once,
    plus the int32 routing ids read and row_of written (T*K each) and token_of
    written (n_kept)."""
    return T * H * b + n_kept * H * b + 4 * (2 * T * K + n_kept)


def combine_kernel_bytes(T: int, n_kept: int, H: int, b: int, K: int, shared: bool) -> int:
    """Combine kernel: each kept expert-output row read once, each token row
    written once (plus the shared-expert row read when present), plus row_of
    and the fp32 weights read (T*K each)."""
    return n_kept * H * b + T * H * b * (2 if shared else 1) + 8 * T * K


def router_bytes(T: int, H: int, E: int, K: int, b: int) -> int:
    """Router kernel: x read once, router weight read once, fp32 logits and
    the top-k ids/weights written."""
    return T * H * b + H * E * b + 4 * T * E + 8 * T * K


# -- the MXFP8 forward (one E8M0 scale byte per 32 E4M3 code bytes) ----------

def mx_bytes(values: int) -> int:
    """Bytes of `values` MXFP8 values: one code byte each plus one scale byte
    per block of 32."""
    return values + values // 32


def permute_mx8_bytes(T: int, n_kept: int, H: int, K: int, shared: bool) -> int:
    """Quantising dispatch: each bf16 token row read once, each kept row
    written once in MXFP8 (and every token's own row when a shared expert
    reads it), plus the int32 routing traffic of the bf16 dispatch."""
    rows_out = n_kept + (T if shared else 0)
    return T * H * 2 + mx_bytes(rows_out * H) + 4 * (2 * T * K + n_kept)


def combine_mx8_bytes(T: int, n_kept: int, H: int, K: int, shared: bool) -> int:
    """FP8 combine: each kept output row read once in MXFP8 (and the shared
    expert's row), each bf16 token row written once, plus row_of and the fp32
    weights."""
    rows_in = n_kept + (T if shared else 0)
    return mx_bytes(rows_in * H) + T * H * 2 + 8 * T * K
