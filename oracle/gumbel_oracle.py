"""CPU oracle of the noisy router: Gumbel noise and temperature (test infrastructure).

This module is test infrastructure, not product code.  Only the tests, the
smoke check of ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it; the HIP path never does, and this module imports nothing from
the HIP path.

What it computes.  The router of section 3.1 of the dpshk.com "MoE module
infra notes": Gumbel noise g = -log(-log(U + 1e-9) + 1e-9), U uniform on
[0, 1), is added to the router logits and the sum is divided by a
temperature tau before the softmax and the top-k (tau about 1; lower is
sharper; the page runs 1.2 early in training and 0.8 later).  The same
section's listing for the layer (4.2) adds the noise with tau = 1.

Readings (also listed in the design notes):

* The uniforms come from a counter-based generator so that any token's noise
  can be recomputed anywhere: Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011), key (seed, 0),
  counter (t, e // 4, offset, 0) for token t; word e % 4 of the block is the
  uniform of expert e.  offset separates steps (the caller advances it).
* A 64-bit word x becomes U = (x >> 40) * 2^-24: 24 bits, so U is exact in
  float32 as well, on [0, 1) like the page's uniform draw.
* Selection scores z = (l + g) / tau, l the router logits (with bias).  Top-k
  and the softmax act on z exactly as they act on l without noise (the float
  oracle's route() on z); the aux loss uses the noisy probabilities and the
  noisy choices.
* Backward: g does not depend on the parameters, so dL/dl = dL/dz / tau.
"""

from __future__ import annotations

import numpy as np

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_PHILOX_M0 = np.uint64(0xD2E7470EE14C6C93)
_PHILOX_M1 = np.uint64(0xCA5A826395121157)
_PHILOX_W0 = np.uint64(0x9E3779B97F4A7C15)
_PHILOX_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def mulhilo64(a, b):
    """(high, low) 64-bit words of the 128-bit product a * b (uint64 arrays),
    from the four 32-bit partial products."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    a_lo, a_hi = a & _LO32, a >> _S32
    b_lo, b_hi = b & _LO32, b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _LO32) + (hl & _LO32)  # < 3 * 2^32, no overflow
    lo = (ll & _LO32) | ((mid & _LO32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds.  counter: uint64 [..., 4]; key: uint64 [..., 2].

    Each round multiplies words 0 and 2 by the two Philox multipliers and
    mixes:  c' = (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)),
    then bumps the key by the two Weyl constants.
    """
    c = np.array(counter, dtype=np.uint64, copy=True)
    k = np.array(key, dtype=np.uint64, copy=True)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = mulhilo64(_PHILOX_M0, c0)
            hi1, lo1 = mulhilo64(_PHILOX_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            k0 = k0 + _PHILOX_W0
            k1 = k1 + _PHILOX_W1
    return np.stack([c0, c1, c2, c3], axis=-1)


def uniforms(T: int, E: int, seed: int, offset: int) -> np.ndarray:
    """U[t, e] on [0, 1): word e % 4 of Philox block (t, e // 4, offset, 0)
    under key (seed, 0), as (x >> 40) * 2^-24."""
    nq = (E + 3) // 4
    t, q = np.meshgrid(np.arange(T, dtype=np.uint64), np.arange(nq, dtype=np.uint64),
                       indexing="ij")
    ctr = np.stack([t, q, np.full_like(t, np.uint64(offset)), np.zeros_like(t)], axis=-1)
    key = np.broadcast_to(np.array([seed, 0], dtype=np.uint64), ctr.shape[:-1] + (2,))
    words = philox4x64_10(ctr, key).reshape(T, nq * 4)[:, :E]
    return (words >> np.uint64(40)).astype(np.float64) * 2.0 ** -24


def gumbel(u) -> np.ndarray:
    """g = -log(-log(u + 1e-9) + 1e-9), the page's transform of a uniform."""
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u + 1e-9) + 1e-9)


def noise(T: int, E: int, seed: int, offset: int) -> np.ndarray:
    return gumbel(uniforms(T, E, seed, offset))


def scores(logits, g, tau: float) -> np.ndarray:
    """Selection scores z = (l + g) / tau (g = 0 for the noiseless router)."""
    return (np.asarray(logits, dtype=np.float64) + np.asarray(g, dtype=np.float64)) / float(tau)
