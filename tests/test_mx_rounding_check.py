"""CPU pins of the strict MXFP8 rounding check used by the GPU parity tests
(tests/test_gpu_mxfp8.py: check_h_rounding).

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
from tests.test_gpu_mxfp8 import accum_bounds, check_h_rounding

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
