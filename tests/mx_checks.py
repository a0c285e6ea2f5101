"""Checks of MXFP8 GEMM results (the GELU output h and the expert outputs)
against float64 references, shared by the GPU parity tests and their CPU pins.

Both sides quantise values that differ in their last bits: the GPU rounds
its own float32 accumulators (the scaled MFMA's internal precision, fp32
accumulation over 64-value K-steps, GELU in fp32), the reference rounds a
float64 value.  A neighbouring code is therefore legitimate exactly where the
reference value lies within the GPU's error bound delta of the midpoint
between two codes, and nowhere else.  check_mx_rounding requires every GPU
code to be the round-to-nearest, at the GPU's own block scale, of some value
within delta of the reference, and every block scale to be the shared
exponent of a block maximum within delta of the reference's.  It therefore
rejects rounding toward zero, the farther neighbour and a wrong scale on any
lane, however few values they touch.

check_mx_close is the weaker closeness check (a share of equal codes, every
value within one code step plus a multiple of 2^X); it is kept as a reported
figure and as the baseline the CPU pins show to be too weak.
"""

from __future__ import annotations

import sys

import numpy as np

from oracle import mxfp8_oracle as M

# A 64-value step of v_mfma_scale_f32_32x32x64_f8f6f4 is exact to within 2^-11
# of its largest product (measured on adversarial codes).
MFMA_STEP_REL = 2.0 ** -11
GELU_SLOPE_MAX = 1.13  # max |d GELU_tanh / du| is 1.1289 (at u = 1.48)
STEP = 64              # values per scaled-MFMA K-step


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def step_of(codes, scales_rows):
    """E4M3 spacing at each element times its block's 2^X (the step to the
    next larger magnitude; 32 * 2^X at 448), and 2^X itself."""
    c = codes.astype(np.int64) & 0x7F
    pos = M.e4m3_value(np.arange(0x7F))
    nxt = np.where(c < 0x7E, pos[np.minimum(c + 1, 0x7E)] - pos[np.minimum(c, 0x7E)], 32.0)
    X = np.repeat(scales_rows.astype(np.int64) - 127, 32, axis=1)
    return nxt * np.exp2(X), np.exp2(X)


def check_mx_close(name, gc, gs, rc, rs, min_exact=0.99, units=1.0):
    """Dequantised GPU vs reference MXFP8 tensors (codes [R][C], row-layout
    scales): at least ``min_exact`` of the values equal and each within one
    step plus ``units`` * 2^X of its block.  Returns the per-value bound."""
    a = M.mx_dequantize(gc, gs, axis=1)
    b = M.mx_dequantize(rc, rs, axis=1)
    sa, ua = step_of(gc, gs)
    sb, ub = step_of(rc, rs)
    tol = np.maximum(sa, sb) + units * np.maximum(ua, ub)
    d = np.abs(a - b)
    exact = float(np.mean(d == 0)) if d.size else 1.0
    worst = float(np.max(d / tol)) if d.size else 0.0
    say(f"  {name}: {d.size} values, {exact:.5%} equal, scales equal {np.mean(gs == rs):.5%}, "
        f"worst |diff| / tol {worst:.3f}")
    assert exact >= min_exact, f"{name}: only {exact:.4%} equal"
    assert worst <= 1.0, f"{name}: a value off by more than the bound"
    return tol


def accum_bounds(xd, wd):
    """For every (row, column) of xd @ wd: the sum over 64-value K-steps of
    the step's largest |x_k w_kn|, and the sum of all |x_k w_kn| (float64)."""
    R, Kd = xd.shape
    n = wd.shape[1]
    tmax = np.zeros((R, n))
    tsum = np.abs(xd) @ np.abs(wd)
    chunk = max(1, (8 << 20) // max(STEP * n, 1))
    for r0 in range(0, R, chunk):
        xa = np.abs(xd[r0:r0 + chunk])
        for k0 in range(0, Kd, STEP):
            prod = xa[:, k0:k0 + STEP, None] * np.abs(wd[None, k0:k0 + STEP, :])
            tmax[r0:r0 + chunk] += prod.max(axis=1)
    return tmax, tsum


def accum_bounds_fast(xd, wd):
    """Upper bounds of accum_bounds' step maxima from two matmuls: the
    largest product of a step is at most the step's largest |x| times its
    largest |w|, so sum_s max|x|_s max|w|_s bounds the sum of step maxima.
    Returns (that bound, the exact sum of all |x_k w_kn|)."""
    R, Kd = xd.shape
    n = wd.shape[1]
    s = (Kd + STEP - 1) // STEP
    xa = np.zeros((R, s * STEP))
    xa[:, :Kd] = np.abs(xd)
    wa = np.zeros((s * STEP, n))
    wa[:Kd] = np.abs(wd)
    xmax = xa.reshape(R, s, STEP).max(axis=2)
    wmax = wa.reshape(s, STEP, n).max(axis=1)
    return xmax @ wmax, np.abs(xd) @ np.abs(wd)


def gemm_delta(tmax, tsum, Kd):
    """Bound on |GPU float32 accumulator - exact product| of an MXFP8 GEMM
    over Kd values: the scaled MFMA's per-step error plus the fp32
    accumulation over Kd / 64 steps, twice over for margin."""
    return 2.0 * (MFMA_STEP_REL * tmax + (Kd / STEP) * 2.0 ** -24 * tsum)


def check_mx_rounding(name, gc, gs, v, delta):
    """GPU MXFP8 values (codes gc [R][C], row-layout scales gs) against
    reference values v [R][C] (float64), given the bound delta [R][C] on the
    GPU's error before it quantised.

    Round to nearest at the GPU's scale 2^X puts every dequantised value
    within half a code step of clamp(v', +-448 2^X) for the GPU's value v',
    |v' - v| <= delta, so |deq - clamp(v)| <= step / 2 + delta; and the block
    scale must be the shared exponent of some block maximum within the
    block's largest delta of the reference's."""
    deq = M.mx_dequantize(gc, gs, axis=1)
    X = np.repeat(gs.astype(np.int64) - 127, 32, axis=1)
    lim = 448.0 * np.exp2(X)
    vc = np.clip(v, -lim, lim)
    step, _ = step_of(gc, gs)
    ratio = np.abs(deq - vc) / (0.5 * step + delta)
    R, C = v.shape
    amax = np.abs(v).reshape(R, C // 32, 32).max(axis=2)
    dmax = delta.reshape(R, C // 32, 32).max(axis=2)
    lo = M.shared_exponent(np.maximum(amax - dmax, 0.0)) + 127
    hi = M.shared_exponent(amax + dmax) + 127
    ref_codes, _ = M.mx_quantize(v, axis=1)
    diff = gc != ref_codes
    mism = int(np.sum(diff))
    # how much of delta a differing code uses: (|deq - v| - step/2) / delta
    used = float(np.max((np.abs(deq - vc) - 0.5 * step)[diff] / np.maximum(delta[diff], 1e-300))) \
        if mism else 0.0
    say(f"  {name}: {v.size} values, {mism} codes differ from the reference's (using at most "
        f"{used:.2f} of delta); worst |deq - v| / (step/2 + delta) {float(ratio.max()):.3f}; "
        f"scales in range {float(np.mean((gs >= lo) & (gs <= hi))):.5%}; median delta / step "
        f"{float(np.median(delta / step)):.2e}")
    assert float(ratio.max()) <= 1.0, f"{name}: a value is not a rounding of the reference's"
    assert np.all((gs >= lo) & (gs <= hi)), f"{name}: a block scale off the reference's maximum"


def check_h_rounding(name, gc, gs, v, tmax, tsum, Kd):
    """The GELU output h = GELU(x W1) in MXFP8 against the oracle's
    unquantised h: delta is the GEMM bound through GELU's largest slope,
    plus 2^-18 sum|x w| for GELU evaluated in float32."""
    delta = GELU_SLOPE_MAX * gemm_delta(tmax, tsum, Kd) + 2.0 ** -18 * tsum
    check_mx_rounding(name, gc, gs, v, delta)


def check_out_rounding(name, gc, gs, v, tmax, tsum, Kd):
    """An expert output o = h W2 in MXFP8 against the float64 product of the
    GPU's own dequantised h and the dequantised weights (no activation)."""
    check_mx_rounding(name, gc, gs, v, gemm_delta(tmax, tsum, Kd))


def check_combine_definition(name, y, out_d, row_of, w, shared_d=None):
    """y (bf16, as float64 [T][H]) against combine's definition on the GPU's
    own dequantised expert outputs out_d [rows][H]: y = bf16(sum_k w out
    (+ shared)), accumulated in fp32.  Bound: one bf16 rounding of the sum
    plus fp32 rounding of its terms."""
    T, K = row_of.shape
    acc = np.zeros_like(y)
    mag = np.zeros_like(y)
    for k in range(K):
        m = row_of[:, k] >= 0
        o = out_d[row_of[m, k]]
        acc[m] += w[m, k][:, None] * o
        mag[m] += np.abs(w[m, k])[:, None] * np.abs(o)
    if shared_d is not None:
        acc += shared_d
        mag += np.abs(shared_d)
    err = np.abs(y - acc) / (2.0 ** -8 * np.abs(acc) + 2.0 ** -20 * mag + 1e-30)
    say(f"  {name}: {y.size} values, worst |y - bf16(sum w deq(out))| / bound {float(err.max()):.3f}")
    assert float(err.max()) <= 1.0, f"{name}: y is not combine of the GPU's outputs"
