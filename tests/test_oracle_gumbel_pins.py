"""Pins of the noisy-router oracle (all on the CPU).

The generator is checked against numpy's own Philox bit generator (an
independent implementation of the same published algorithm); the Gumbel
transform against the closed forms of the standard Gumbel distribution and
the Gumbel-max property (argmax of logits + noise is distributed as the
softmax of the logits), which fixes the transform's signs; the temperature
against closed forms; the backward with noise and temperature against
central differences.
"""

import math

import numpy as np
import pytest

from oracle import gumbel_oracle as G
from oracle import moe_oracle as O


@pytest.mark.parametrize("key,ctr", [
    ((7, 9), (0, 0, 0, 0)),
    ((0xFFFFFFFFFFFFFFFF, 0x123456789ABCDEF0), (5, 1, 0, 0)),
    ((123, 0), (0xFFFFFFFFFFFFFFFE, 3, 99, 0)),       # the counter's low word carries
    ((2 ** 63 + 1, 2 ** 40), (2 ** 62, 2 ** 63 - 1, 2 ** 64 - 1, 7)),
])
def test_philox_matches_numpy_bit_generator(key, ctr):
    """numpy's Philox (4x64, 10 rounds) increments its counter, then emits the
    block of the new counter, four 64-bit words at a time."""
    bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = bg.random_raw(12).astype(np.uint64)
    c = list(ctr)
    want = []
    for _ in range(3):
        # 256-bit increment with carries
        for i in range(4):
            c[i] = (c[i] + 1) % 2 ** 64
            if c[i] != 0:
                break
        want.append(G.philox4x64_10(np.array(c, dtype=np.uint64), np.array(key, dtype=np.uint64)))
    assert np.array_equal(raw, np.concatenate(want))


def test_mulhilo64_against_python_integers():
    r = np.random.default_rng(0)
    a = r.integers(0, 2 ** 63, 1000, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    b = r.integers(0, 2 ** 63, 1000, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    hi, lo = G.mulhilo64(a, b)
    for i in range(1000):
        p = int(a[i]) * int(b[i])
        assert int(hi[i]) == p >> 64 and int(lo[i]) == p & (2 ** 64 - 1)


def test_uniforms_are_24_bit_and_the_stream_layout():
    """U = (word >> 40) 2^-24, words of block (t, e // 4, offset, 0)."""
    T, E, seed, off = 5, 6, 42, 3
    u = G.uniforms(T, E, seed, off)
    assert u.shape == (T, E)
    assert np.all((u >= 0) & (u < 1)) and np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))
    w = G.philox4x64_10(np.array([2, 1, off, 0], dtype=np.uint64), np.array([seed, 0], dtype=np.uint64))
    assert u[2, 5] == float(int(w[1]) >> 40) * 2.0 ** -24  # t = 2, e = 5: block 1, word 1
    assert not np.array_equal(G.uniforms(T, E, seed, off + 1), u)
    assert not np.array_equal(G.uniforms(T, E, seed + 1, off), u)


def test_gumbel_moments_and_distribution():
    """Standard Gumbel: mean = Euler's gamma, variance = pi^2 / 6,
    CDF exp(-exp(-x)) (Kolmogorov-Smirnov distance)."""
    g = G.noise(250000, 4, seed=1, offset=0).ravel()
    n = g.size
    gamma = 0.5772156649015329
    sd = math.pi / math.sqrt(6)
    assert abs(g.mean() - gamma) < 5 * sd / math.sqrt(n)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    xs = np.sort(g)
    cdf = np.exp(-np.exp(-xs))
    ks = np.max(np.abs(cdf - np.arange(1, n + 1) / n))
    assert ks < 1.63 / math.sqrt(n)  # 1% level


def test_gumbel_max_samples_the_softmax():
    """argmax_e (l_e + g_e) is distributed as softmax(l): chi-square test.  A
    transform with a flipped sign (argmin) or the wrong nesting fails it."""
    l = np.array([0.5, -1.0, 1.2, 0.0, -0.3])
    n = 200000
    g = G.noise(n, 5, seed=2, offset=7)
    pick = np.argmax(l[None, :] + g, axis=1)
    counts = np.bincount(pick, minlength=5)
    p = O.softmax(l[None, :])[0]
    chi2 = np.sum((counts - n * p) ** 2 / (n * p))
    assert chi2 < 18.5  # 4 degrees of freedom, 0.1% level


def test_temperature_closed_forms():
    """K = E: the weights are softmax(z) with z = (l + g) / tau; the top-k set
    does not depend on tau (a positive scale is monotone)."""
    r = np.random.default_rng(3)
    T, E = 9, 4
    l = r.standard_normal((T, E))
    g = G.noise(T, E, seed=5, offset=0)
    for tau in (0.5, 0.8, 1.2, 2.0):
        z = G.scores(l, g, tau)
        rt = O.route(z, E, E, 0.0)
        w_full = np.exp(z - z.max(1, keepdims=True))
        w_full /= w_full.sum(1, keepdims=True)
        assert np.allclose(rt["w"], np.take_along_axis(w_full, rt["ids"].astype(np.int64), 1),
                           rtol=0, atol=1e-14)
        r2 = O.route(G.scores(l, g, tau), E, 2, 0.0)
        r1 = O.route(G.scores(l, g, 1.0), E, 2, 0.0)
        assert np.array_equal(r2["ids"], r1["ids"])


@pytest.mark.parametrize("tau,alpha,cf", [(0.7, 0.4, 0.0), (1.6, 0.0, 0.6)])
def test_backward_with_noise_and_temperature_matches_central_differences(tau, alpha, cf):
    r = np.random.default_rng(4)
    T, H, E, K, h = 7, 5, 4, 2, 3
    p = dict(x=r.standard_normal((T, H)), w_r=r.standard_normal((H, E)) * 0.7,
             b_r=r.standard_normal(E) * 0.3, w1=r.standard_normal((E, H, h)) * 0.6,
             w2=r.standard_normal((E, h, H)) * 0.6)
    dy = r.standard_normal((T, H))
    g = G.noise(T, E, seed=11, offset=2)

    def loss():
        z = G.scores(O.router_logits(p["x"], p["w_r"], p["b_r"]), g, tau)
        fw = O.forward(p["x"], p["w_r"], p["b_r"], p["w1"], p["w2"], K=K, cf=cf, logits=z)
        return float(np.sum(dy * fw["y"]) + alpha * fw["aux"]), fw["ids"].copy(), fw["row_of"].copy()

    z = G.scores(O.router_logits(p["x"], p["w_r"], p["b_r"]), g, tau)
    gr = O.backward(p["x"], p["w_r"], p["b_r"], p["w1"], p["w2"], dy=dy, K=K, cf=cf, alpha=alpha,
                    logits=z, tau=tau)
    _, ids0, ro0 = loss()
    eps = 1e-6
    for name, gname in (("x", "dx"), ("w_r", "dw_r"), ("b_r", "db_r"), ("w1", "dw1")):
        a = p[name]
        num = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + eps
            lp, i1, r1 = loss()
            a[idx] = old - eps
            lm, i2, r2 = loss()
            a[idx] = old
            assert np.array_equal(i1, ids0) and np.array_equal(i2, ids0)
            assert np.array_equal(r1, ro0) and np.array_equal(r2, ro0)
            num[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - gr[gname])) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, (gname, err)
