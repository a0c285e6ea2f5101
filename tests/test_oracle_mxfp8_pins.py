"""Pins of the MXFP8 oracle (all on the CPU).

Each test checks ``mxfp8_oracle`` against something other than itself: the
landmark values the OFP8 specification lists for E4M3, PyTorch's own
float8_e4m3fn type (an independent implementation of the same element
format, used here as a library routine for decoding and round-to-nearest-even
encoding inside the finite range), closed forms of the MX shared exponent,
the rounding error bound of the format, and structural cases whose answer is
fixed by the block axis (a block along the wrong axis fails them).
"""

import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import mxfp8_oracle as M


def _torch_decode(codes):
    t = torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(v32):
    return torch.tensor(np.asarray(v32, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_landmarks():
    """OFP8 E4M3: smallest subnormal 2^-9, largest subnormal 7 * 2^-9, smallest
    normal 2^-6, one, largest finite 448, NaN at S.1111.111, no infinity."""
    v = M.e4m3_value
    assert v(0x00) == 0.0 and v(0x80) == 0.0 and math.copysign(1, v(0x80)) < 0
    assert v(0x01) == 2.0 ** -9
    assert v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6
    assert v(0x38) == 1.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert np.isfinite(v(np.arange(256)[(np.arange(256) & 0x7F) != 0x7F])).all()


def test_e4m3_decode_matches_torch_float8():
    c = np.arange(256)
    a, b = M.e4m3_value(c), _torch_decode(c)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok])
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


def test_e4m3_encode_matches_torch_round_to_nearest_even():
    """Every tie (midpoint of two neighbouring values), the float32 values just
    either side of it, and random magnitudes over the whole finite range."""
    pos = M.e4m3_value(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2  # exact in float32 (few significant bits)
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(0))
    r = np.random.default_rng(0)
    rnd = (np.exp2(r.uniform(-14, 8.8, 20000)) * r.choice([-1, 1], 20000)).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    v = np.concatenate([m32, up, dn, -m32, -up, -dn, pos.astype(np.float32), rnd,
                        np.float32([0.0, -0.0, 1e-30, -1e-30])])
    assert np.array_equal(M.e4m3_encode(v), _torch_encode(v))


def test_e4m3_encode_saturates_past_448():
    """MX conversion saturates: magnitudes above 448 (the largest finite value)
    map to +-448, not NaN."""
    v = np.array([448.0, 449.0, 464.0, 479.9, 480.0, 511.0, 1e6, -500.0, -1e30])
    assert np.array_equal(M.e4m3_encode(v), np.uint8([0x7E] * 7 + [0xFE, 0xFE]))


def test_shared_exponent_closed_forms():
    """X = floor(log2 amax) - 8, clamped to [-127, 127], -127 for zero."""
    cases = {1.0: -8, 448.0: 0, 256.0: 0, 511.99: 0, 512.0: 1, 0.75: -9, 2.0 ** -20: -28,
             2.0 ** -119: -127, 2.0 ** -130: -127, 0.0: -127, 3.0e38: 119}
    for a, X in cases.items():
        assert int(M.shared_exponent(a)) == X, a


def test_mx_quantize_block_scales_and_range():
    """After scaling by 2^-X the block maximum lies in [256, 512) (saturating
    to 448 above 448); the scale code is X + 127; the block is 32 long."""
    r = np.random.default_rng(1)
    a = (r.standard_normal((64, 96)) * np.exp2(r.integers(-30, 30, (64, 1)))).astype(np.float32)
    codes, scales = M.mx_quantize(a, axis=1)
    assert codes.shape == a.shape and scales.shape == (64, 3)
    blk = a.reshape(64, 3, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    X = scales.astype(np.int64) - 127
    assert np.all(np.floor(np.log2(amax)) - 8 == X)
    s = amax / np.exp2(X)
    assert np.all((s >= 256) & (s < 512))


def test_mx_roundtrip_error_bound_and_exact_values():
    """Round-to-nearest error is at most half the spacing of E4M3 at the
    element's magnitude (2^-4 relative in the normal range, 2^(X-10) absolute in
    the subnormal range), except saturated elements (|v| > 448 * 2^X), which
    become 448 * 2^X.  Values already of the form E4M3 * 2^X come back
    exactly."""
    r = np.random.default_rng(2)
    a = (r.standard_normal((128, 64)) * np.exp2(r.integers(-8, 8, (128, 64)))).astype(np.float32)
    codes, scales = M.mx_quantize(a, axis=1)
    d = M.mx_dequantize(codes, scales, axis=1)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    v = a.astype(np.float64)
    sat = np.abs(v) > 448 * np.exp2(X)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, np.exp2(X - 10))
    assert np.all(np.abs(d - v)[~sat] <= bound[~sat])
    assert np.all(d[sat] == np.sign(v[sat]) * 448 * np.exp2(X[sat]))
    assert np.array_equal(M.mx_roundtrip(d, axis=1), d)


def test_mx_quantize_matches_torch_construction():
    """The same definition built from library primitives: frexp for the
    exponent, ldexp for the scaling, a clamp to +-448 and PyTorch's float8 cast
    for the rounding."""
    r = np.random.default_rng(3)
    a = torch.tensor((r.standard_normal((40, 128)) * np.exp2(r.integers(-20, 20, (40, 1))))
                     .astype(np.float32))
    blk = a.reshape(40, 4, 32).double()
    _, e = torch.frexp(blk.abs().amax(dim=2))
    X = (e - 1 - 8).clamp(-127, 127)
    scaled = torch.ldexp(blk, -X[..., None].double()).clamp(-448, 448).float()
    want = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(40, 128).numpy()
    codes, scales = M.mx_quantize(a.numpy(), axis=1)
    assert np.array_equal(codes, want)
    assert np.array_equal(scales.astype(np.int64), (X + 127).numpy())


def test_weight_blocks_run_along_the_contraction_dimension():
    """Weights whose magnitude changes by 2^4 from column to column but is
    constant down each column quantise exactly along K (one magnitude per
    block); blocks along N would flush the small columns to zero."""
    r = np.random.default_rng(4)
    E, Kd, N = 2, 64, 32
    mant = M.e4m3_value(r.integers(0x38, 0x3F, (E, Kd, N)))  # E4M3 values 1 .. 1.75
    w = mant * np.exp2(4.0 * (np.arange(N) % 8) - 16)[None, None, :]
    codes, scales = M.quantize_weights(w)
    assert codes.shape == (E, Kd, N) and scales.shape == (E, Kd // 32, N)
    assert np.array_equal(M.mx_dequantize(codes, scales, axis=1), w)
    along_n = M.mx_roundtrip(w, axis=2)
    assert np.max(np.abs(along_n - w) / np.abs(w)) == 1.0


def _layer_case(seed, T=40, H=64, E=4, h=96, hs=0, spread=0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H)).astype(np.float32)
    if spread:
        x *= np.exp2(r.integers(-spread, spread + 1, (T, 1))).astype(np.float32)
    p = dict(x=x, w_r=r.standard_normal((H, E)) * 0.2, b_r=None,
             w1=r.standard_normal((E, H, h)) * 0.15, w2=r.standard_normal((E, h, H)) * 0.15,
             ws1=r.standard_normal((H, hs)) * 0.15 if hs else None,
             ws2=r.standard_normal((hs, H)) * 0.15 if hs else None)
    return p


@pytest.mark.parametrize("hs", [0, 64])
def test_forward_mxfp8_close_to_float_forward_per_token(hs):
    """Token magnitudes spread over 2^-12 .. 2^12: every token's FP8 output is
    within the error of five E4M3 roundings (x, W1, h, W2, out: about 2.6% RMS
    each, so about 6% in all) of the float forward's (same routing).  A block
    taken across tokens instead of along the row would flush the small tokens
    (relative error 1)."""
    p = _layer_case(5, spread=12, hs=hs)
    f = O.forward(**p, K=2, cf=0.0)
    q = M.forward_mxfp8(**p, K=2, cf=0.0)
    assert np.array_equal(f["row_of"], q["row_of"])
    num = np.linalg.norm(q["y"] - f["y"], axis=1)
    den = np.linalg.norm(f["y"], axis=1)
    rel = num / den
    assert rel.max() < 0.15, rel.max()
    assert rel.min() > 1e-3  # it did quantise


def test_forward_mxfp8_exact_where_every_rounding_is_exact():
    """E = K = 1, no shared expert, x and W1 exact in MXFP8, and W2 = 0 except
    W2[j, j] = 1 for the first H columns of h: then out = h_fp8[:, :H] and y
    is exactly the MX round trip of GELU(x W1)[:, :H] (then of out again,
    which is already exact)."""
    r = np.random.default_rng(6)
    T, H, h = 16, 32, 64
    x = M.mx_roundtrip(r.standard_normal((T, H)).astype(np.float32), axis=1)
    w1 = M.mx_roundtrip(r.standard_normal((1, H, h)) * 0.3, axis=1)
    w2 = np.zeros((1, h, H))
    w2[0, np.arange(H), np.arange(H)] = 1.0
    q = M.forward_mxfp8(x, np.zeros((H, 1)), None, w1, w2, K=1, cf=0.0)
    g = O.gelu_tanh(x @ w1[0])
    want = M.mx_roundtrip(g, axis=1)[:, :H]
    assert np.array_equal(q["y"], want)
