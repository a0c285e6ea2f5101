"""CPU oracle of the MXFP8 forward of the MoE layer (test infrastructure).

This module is test infrastructure, not product code.  Only the tests, the
smoke check of ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it; the HIP path never does, and this module imports nothing from
the HIP path.

What it computes.  The compression step of the page "Dissecting the MoE
communication bottleneck" (cf-1.com, section 5.3): the hidden states that
dispatch sends to the experts and that combine brings back are carried in
FP8 instead of bf16, halving their bytes, and section 5.4 adds that the
quantise / dequantise work must stay cheap.  Section 4.2 of the same page
applies FP8 to the expert weights too.  The page names no FP8 variant and no
scaling rule; the readings taken here (also listed in the design notes):

* Element format: OCP 8-bit floating point E4M3 (bias 7, three mantissa
  bits, subnormals, no infinities, largest finite value 448, the codes with
  all exponent and mantissa bits set are NaN), from the OCP "8-bit Floating
  Point Specification (OFP8)" 1.0.  Hidden states need range less than
  precision, so the format with more mantissa bits is taken.
* Scaling: the OCP "Microscaling (MX) Formats Specification" 1.0, format
  MXFP8 (E4M3): blocks of 32 consecutive elements along the contraction
  dimension share one power-of-two scale stored as an E8M0 exponent (code
  X + 127).  The shared exponent of a block is X = floor(log2(max |v|)) - 8,
  8 being the exponent of E4M3's largest normal; each element is v / 2^X
  rounded to the nearest E4M3 value, ties to the even code, magnitudes past
  448 saturating to 448.  An all-zero block takes the smallest exponent
  (X = -127); X is clamped to [-127, 127].
* Which tensors are FP8: the token rows that dispatch copies (x), the expert
  weights (quantised once, along their contraction dimension), the GELU
  output h that the second expert GEMM reads, and the expert outputs that
  combine reads.  Routing (logits, softmax, top-k, weights), the aux loss,
  combine's weighted sum and the layer output y stay in float (the router is
  untouched: it sees the unquantised x).  A shared expert, when present, runs
  in the same FP8 form on the quantised x.
* Each rounding decision is taken on the float32 value, as the kernels take
  it: a block is quantised from its float32 values (x is bf16 and exact in
  float32; h and the expert outputs are rounded from float64 to float32
  first).

Everything else (products, GELU, the weighted sum) is float64 on the exact
dequantised values, as in the float oracle.  Formulas are the plain
definitions; the only library primitives are a matmul, ``tanh`` (through the
float oracle's GELU), ``frexp``/``ldexp`` and a sorted search.
"""

from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from oracle import moe_oracle as O

BLOCK = 32            # elements per MX block (MX specification, MXFP8)
E4M3_MAX = 448.0      # largest finite E4M3 magnitude (OFP8 specification)
E4M3_EMAX = 8         # exponent of that value: 448 = 1.75 * 2^8
E8M0_BIAS = 127


# ---------------------------------------------------------------------------
# E4M3 element codes (OFP8 specification)
# ---------------------------------------------------------------------------

def e4m3_value(code) -> np.ndarray:
    """Value of each E4M3 code, float64 (NaN for 0x7f and 0xff).

    sign = bit 7, exponent field e = bits 6..3 (bias 7), mantissa m = bits 2..0:
    e = 0 gives the subnormal (m/8) 2^-6, otherwise (1 + m/8) 2^(e-7); e = 15
    with m = 7 is NaN (the format has no infinities).
    """
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    v = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


# the 127 finite non-negative values, code 0 .. 126 (increasing with the code)
_POS = e4m3_value(np.arange(0x7F))
assert np.all(np.diff(_POS) > 0)


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even code, saturating.

    |v| is first clamped to 448; then the nearest of the 127 finite
    non-negative values is taken by search, a tie going to the value whose
    code is even (its last mantissa bit is 0).  The sign bit is the sign of v
    (so -0.0 and negative values that round to zero give 0x80).  Inputs must
    not be NaN.
    """
    v = np.asarray(v, dtype=np.float64)
    assert not np.isnan(v).any(), "NaN has no E4M3 code here"
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)  # first >= a
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - a
    d_lo = a - _POS[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(take_lo, lo, hi).astype(np.int64)
    code = np.where(np.signbit(v), code | 0x80, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# MX blocks (MX specification, MXFP8)
# ---------------------------------------------------------------------------

def shared_exponent(amax) -> np.ndarray:
    """X = floor(log2(amax)) - 8 clamped to [-127, 127]; -127 when amax = 0.

    floor(log2 a) is read exactly from frexp: a = f 2^e with f in [0.5, 1).
    """
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)
    X = (e.astype(np.int64) - 1) - E4M3_EMAX
    X = np.where(a > 0, X, -E8M0_BIAS)
    return np.clip(X, -E8M0_BIAS, E8M0_BIAS)


def mx_quantize(a, axis: int = -1) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP8 codes and E8M0 scale codes of ``a`` in blocks of 32 along ``axis``.

    The values are taken as float32 (rounded from ``a`` if it is wider), as
    the kernels hold them when they quantise.  Returns (codes, scales): codes
    has the shape of ``a``; scales has ``axis`` shortened to n / 32, and holds
    X + 127 per block.
    """
    a = np.asarray(a).astype(np.float32).astype(np.float64)
    a = np.moveaxis(a, axis, -1)
    n = a.shape[-1]
    assert n % BLOCK == 0, f"length {n} along the blocked axis is not a multiple of {BLOCK}"
    blk = a.reshape(a.shape[:-1] + (n // BLOCK, BLOCK))
    X = shared_exponent(np.max(np.abs(blk), axis=-1))
    scaled = np.ldexp(blk, -X[..., None])  # exact: a power-of-two scaling
    codes = e4m3_encode(scaled).reshape(a.shape)
    scales = (X + E8M0_BIAS).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def mx_dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    """value = E4M3(code) * 2^(scale - 127), float64 (exact)."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1).astype(np.int64)
    v = e4m3_value(c)
    n = v.shape[-1]
    v = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    v = np.ldexp(v, (s - E8M0_BIAS)[..., None]).reshape(c.shape)
    return np.moveaxis(v, -1, axis)


def mx_roundtrip(a, axis: int = -1) -> np.ndarray:
    """Dequantised MXFP8 form of ``a`` (the value an FP8 consumer sees)."""
    return mx_dequantize(*mx_quantize(a, axis), axis=axis)


# ---------------------------------------------------------------------------
# the layer with FP8 dispatch, expert GEMMs and combine
# ---------------------------------------------------------------------------

def ffn_mxfp8(rows_d: np.ndarray, w1_d: np.ndarray, w2_d: np.ndarray) -> Dict[str, np.ndarray]:
    """One expert on dequantised FP8 rows with dequantised FP8 weights.

    u = rows W1 (float64), h = GELU_tanh(u), h quantised along its row (the
    contraction dimension of the second product), out = h_fp8 W2, out
    quantised along its row (the payload combine reads).
    """
    u = rows_d @ w1_d
    h = O.gelu_tanh(u)
    h_codes, h_scales = mx_quantize(h, axis=1)
    o = mx_dequantize(h_codes, h_scales, axis=1) @ w2_d
    o_codes, o_scales = mx_quantize(o, axis=1)
    return dict(u=u, h=h, h_codes=h_codes, h_scales=h_scales, o=o, o_codes=o_codes,
                o_scales=o_scales, out=mx_dequantize(o_codes, o_scales, axis=1))


def quantize_weights(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Expert weights [B, K, N] in blocks of 32 along K (their contraction
    dimension): codes [B, K, N], scales [B, K/32, N]."""
    return mx_quantize(w, axis=1)


def forward_mxfp8(x, w_r, b_r, w1, w2, ws1=None, ws2=None, *, K: int, cf: float,
                  logits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The layer with FP8 dispatch, FP8 expert FFN and FP8 combine.

    Routing is the float oracle's, from the unquantised x (or from the given
    float32 ``logits``).  Dispatch carries mx_quantize(x) rows; every expert
    runs :func:`ffn_mxfp8` with its quantised weights; combine weights the
    dequantised FP8 outputs by the routing weights in float64.  Besides the
    codes and scales, ``h`` (and ``sh_h``) hold the GELU outputs before
    quantisation, float64, packed rows.
    """
    E = w1.shape[0]
    l_own = O.router_logits(x, w_r, b_r)
    l_sel = np.asarray(logits, dtype=np.float64) if logits is not None \
        else l_own.astype(np.float32).astype(np.float64)
    r = O.route(l_sel, E, K, cf)
    x_codes, x_scales = mx_quantize(x, axis=1)
    x_d = mx_dequantize(x_codes, x_scales, axis=1)
    w1c, w1s = quantize_weights(w1)
    w2c, w2s = quantize_weights(w2)
    w1d = mx_dequantize(w1c, w1s, axis=1)
    w2d = mx_dequantize(w2c, w2s, axis=1)
    token_of = r["token_of"]
    offsets = r["offsets"]
    N = int(offsets[-1])
    H, h = x.shape[1], w1.shape[2]
    h_val = np.zeros((N, h), np.float64)
    h_codes = np.zeros((N, h), np.uint8)
    h_scales = np.zeros((N, h // BLOCK), np.uint8)
    o_codes = np.zeros((N, H), np.uint8)
    o_scales = np.zeros((N, H // BLOCK), np.uint8)
    out = np.zeros((N, H), np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            f = ffn_mxfp8(x_d[token_of[a:b]], w1d[e], w2d[e])
            h_val[a:b] = f["h"]
            h_codes[a:b], h_scales[a:b] = f["h_codes"], f["h_scales"]
            o_codes[a:b], o_scales[a:b] = f["o_codes"], f["o_scales"]
            out[a:b] = f["out"]
    shared = None
    if ws1 is not None:
        s1c, s1s = mx_quantize(ws1, axis=0)
        s2c, s2s = mx_quantize(ws2, axis=0)
        fs = ffn_mxfp8(x_d, mx_dequantize(s1c, s1s, axis=0), mx_dequantize(s2c, s2s, axis=0))
        shared = fs["out"]
        r.update(sh_h=fs["h"], sh_h_codes=fs["h_codes"], sh_h_scales=fs["h_scales"],
                 sh_codes=fs["o_codes"], sh_scales=fs["o_scales"])
    y = O.combine(out, r["row_of"], r["w"], shared)
    r.update(x_codes=x_codes, x_scales=x_scales, w1_codes=w1c, w1_scales=w1s,
             w2_codes=w2c, w2_scales=w2s, h=h_val, h_codes=h_codes, h_scales=h_scales,
             o_codes=o_codes, o_scales=o_scales, out=out, shared=shared, y=y)
    return r
