"""CPU pins of the strict MXFP8 checks used by the GPU parity tests
(tests/mx_checks.py: check_h_rounding, check_out_rounding,
check_combine_definition, and the step-maximum bounds they rest on).

The check must accept any round-to-nearest quantisation of values within its
delta of the oracle's, and must reject the plausible mistakes: rounding
toward zero, the farther of the two neighbouring codes, and a block scale one
binade off.  Mistakes are planted in quantisers written here, on the CPU.
The direction of an exact tie is beyond any distance test (both codes lie
half a step away); ties are pinned by the bit-exact tests of the dispatch and
weight quantisation, which include them.
"""

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import mxfp8_oracle as M
from tests.mx_checks import (accum_bounds, accum_bounds_fast, check_combine_definition,
                             check_h_rounding, check_mx_close, check_out_rounding, gemm_delta)

R, KD, C = 24, 256, 96


def setup():
    g = np.random.default_rng(5)
    xd = M.mx_roundtrip(g.standard_normal((R, KD)), axis=1)
    wd = M.mx_roundtrip(0.05 * g.standard_normal((KD, C)), axis=0)
    v = O.gelu_tanh(xd @ wd)
    tmax, tsum = accum_bounds(xd, wd)
    return xd, wd, v, tmax, tsum


def quantize_with(v, pick):
    """MXFP8 of v with the oracle's block scales and a code chooser
    pick(scaled_magnitude) -> code index into the positive E4M3 values."""
    _, scales = M.mx_quantize(v, axis=1)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    a = np.minimum(np.abs(np.ldexp(v, -X)), 448.0)
    code = pick(a).astype(np.int64)
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    return code, scales


POS = M.e4m3_value(np.arange(0x7F))


def test_accum_bounds_brute_force():
    xd, wd, _, tmax, tsum = setup()
    i, n = 3, 7
    prods = np.abs(xd[i] * wd[:, n])
    assert np.isclose(tsum[i, n], prods.sum())
    assert np.isclose(tmax[i, n], sum(prods[k:k + 64].max() for k in range(0, KD, 64)))


def test_accepts_faithful_rounding_of_perturbed_values():
    _, _, v, tmax, tsum = setup()
    delta = 2.0 * (2.0 ** -11 * tmax + (KD / 64) * 2.0 ** -24 * tsum)
    g = np.random.default_rng(6)
    v2 = v + delta * g.uniform(-1.0, 1.0, v.shape)
    gc, gs = M.mx_quantize(v2, axis=1)
    check_h_rounding("perturbed", gc, gs, v, tmax, tsum, KD)


def test_rejects_rounding_toward_zero():
    _, _, v, tmax, tsum = setup()
    gc, gs = quantize_with(v, lambda a: np.searchsorted(POS, a, side="right") - 1)
    with pytest.raises(AssertionError, match="not a rounding"):
        check_h_rounding("truncated", gc, gs, v, tmax, tsum, KD)


def test_rejects_the_farther_neighbour():
    _, _, v, tmax, tsum = setup()
    # values 0.3 of a step above code 20, exactly representable, no
    # accumulation error: only code 20 is a rounding of them
    X = np.repeat(M.mx_quantize(v, axis=1)[1].astype(np.int64) - 127, 32, axis=1)
    vm = v.copy()
    vm[:, 5] = np.ldexp(POS[20] + 0.3 * (POS[21] - POS[20]), X[:, 5])
    tmax0 = np.zeros_like(tmax)
    tsum0 = np.zeros_like(tsum)
    gc, gs = M.mx_quantize(vm, axis=1)
    assert np.all((gc[:, 5] & 0x7F) == 20)
    check_h_rounding("nearest", gc, gs, vm, tmax0, tsum0, KD)
    bad = gc.copy()
    bad[:, 5] = (bad[:, 5] & 0x80) | 21
    with pytest.raises(AssertionError, match="not a rounding"):
        check_h_rounding("farther", bad, gs, vm, tmax0, tsum0, KD)


def test_rejects_scale_one_binade_off():
    _, _, v, tmax, tsum = setup()
    codes, scales = M.mx_quantize(v, axis=1)
    bad_s = scales + 1
    X = np.repeat(bad_s.astype(np.int64) - 127, 32, axis=1)
    bad_c = M.e4m3_encode(np.ldexp(v, -X))
    with pytest.raises(AssertionError):
        check_h_rounding("scale +1", bad_c, bad_s, v, tmax, tsum, KD)


# ---------------------------------------------------------------- out, y


def setup_out():
    """h as dequantised MXFP8 rows, W2 as dequantised MXFP8 columns, and
    their float64 product (the reference of the out check)."""
    g = np.random.default_rng(8)
    hd = M.mx_roundtrip(O.gelu_tanh(g.standard_normal((R, KD))), axis=1)
    wd = M.mx_roundtrip(0.05 * g.standard_normal((KD, C)), axis=0)
    return hd, wd, hd @ wd


def test_accum_bounds_fast_bounds_the_exact_step_maxima():
    hd, wd, _ = setup_out()
    tmax, tsum = accum_bounds(hd, wd)
    ub, tsum2 = accum_bounds_fast(hd, wd)
    assert np.allclose(tsum, tsum2, rtol=1e-12, atol=0)
    assert np.all(ub >= tmax * (1 - 1e-12))
    # brute force of one entry
    i, n = 5, 11
    want = sum(np.abs(hd[i, k:k + 64]).max() * np.abs(wd[k:k + 64, n]).max()
               for k in range(0, KD, 64))
    assert np.isclose(ub[i, n], want, rtol=1e-12)
    # a ragged last step (Kd not a multiple of 64) is still covered
    ub_r, _ = accum_bounds_fast(hd[:, :200], wd[:200])
    tmax_r, _ = accum_bounds(hd[:, :200], wd[:200])
    assert np.all(ub_r >= tmax_r * (1 - 1e-12))


def test_out_check_accepts_faithful_rounding_of_perturbed_values():
    hd, wd, v = setup_out()
    tmax, tsum = accum_bounds_fast(hd, wd)
    delta = gemm_delta(tmax, tsum, KD)
    v2 = v + delta * np.random.default_rng(9).uniform(-1.0, 1.0, v.shape)
    gc, gs = M.mx_quantize(v2, axis=1)
    check_out_rounding("perturbed out", gc, gs, v, tmax, tsum, KD)


def test_rounding_toward_zero_on_one_lane_in_16():
    """A rounding bug confined to one lane of 16 (here every column c with
    c % 16 == 3 truncated toward zero) passes the old closeness check (90%
    equal codes, one step plus 16 2^X) and fails the strict out check."""
    hd, wd, v = setup_out()
    tmax, tsum = accum_bounds_fast(hd, wd)
    good_c, good_s = M.mx_quantize(v, axis=1)
    rtz_c, _ = quantize_with(v, lambda a: np.searchsorted(POS, a, side="right") - 1)
    cols = np.arange(C) % 16 == 3
    bad = good_c.copy()
    bad[:, cols] = rtz_c[:, cols]
    assert np.mean(bad != good_c) > 0.01  # the bug changes codes
    check_mx_close("old check", bad, good_s, good_c, good_s, min_exact=0.9, units=16.0)
    with pytest.raises(AssertionError, match="not a rounding"):
        check_out_rounding("rtz on one lane", bad, good_s, v, tmax, tsum, KD)


def test_combine_definition_check():
    g = np.random.default_rng(10)
    T, K, H, rows = 40, 3, 64, 90
    out_d = g.standard_normal((rows, H))
    row_of = np.full((T, K), -1, np.int64)
    perm = g.permutation(rows)
    row_of.flat[g.choice(T * K, size=rows, replace=False)] = perm
    w = g.uniform(0.05, 1.0, (T, K)).astype(np.float32).astype(np.float64)
    sh = g.standard_normal((T, H))
    acc = np.zeros((T, H))
    for k in range(K):
        m = row_of[:, k] >= 0
        acc[m] += w[m, k][:, None] * out_d[row_of[m, k]]
    import torch
    y = torch.from_numpy(acc + sh).to(torch.bfloat16).to(torch.float64).numpy()
    check_combine_definition("exact", y, out_d, row_of, w, sh)
    # one slot's weight off by 1%
    w2 = w.copy()
    t0 = int(np.nonzero(row_of[:, 1] >= 0)[0][0])
    w2[t0, 1] *= 1.01
    with pytest.raises(AssertionError):
        check_combine_definition("weight off", y, out_d, row_of, w2, sh)
    # the shared expert's term left out
    with pytest.raises(AssertionError):
        check_combine_definition("no shared", y, out_d, row_of, w, None)
