"""Property tests of the CPU oracle over random small shapes (hypothesis).

Shapes: T <= 64, E <= 16, K <= min(E, 4), capacity factor in {0 (no limit),
0.5, 1, 1.25, 0.3}.  Logits are drawn either as small integers (many exact
ties, signed zeros) or as Gaussians.  Every property is fixed by the
definition of the method, independently of how the oracle computes it:

  * selection equals a brute-force per-token sort by (logit desc, index asc);
  * renormalised weights sum to 1, and equal the softmax over the chosen
    logits (the two forms of the renormalisation agree);
  * counts sum to T*K, kept = min(counts, C), the drop count is the overflow,
    offsets are the exclusive sum of kept, row_of restricted to kept
    assignments is a bijection onto [0, N) with token_of its inverse, and
    tokens increase inside every segment;
  * the kept assignments to each expert are exactly its first C assignments
    in token order (brute force over the flattened assignment list);
  * the capacity is the exact ceiling of cf*T*K/E (rational arithmetic);
  * 0 <= aux <= E, and aux = 1 when all logits are equal;
  * y of the permutation-based forward equals the dense all-experts form to
    1e-12 (no permutation in the latter).

Inputs are seeded: hypothesis runs derandomised, so every run draws the
same examples.
"""

import fractions
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import moe_oracle as O

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def routing_case(draw):
    T = draw(st.integers(1, 64))
    E = draw(st.integers(1, 16))
    K = draw(st.integers(1, min(E, 4)))
    cf = draw(st.sampled_from([0.0, 0.5, 1.0, 1.25, 0.3]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    ties = draw(st.booleans())
    r = np.random.default_rng(seed)
    if ties:
        l = r.integers(-2, 3, size=(T, E)).astype(np.float64)
        l[r.random((T, E)) < 0.2] = -0.0  # signed zeros tie with +0
    else:
        l = r.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    return T, E, K, cf, l


def brute_ids(l, K):
    T, E = l.shape
    ids = np.zeros((T, K), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-l[t, e], e))
        ids[t] = order[:K]
    return ids


@SETTINGS
@given(routing_case())
def test_selection_and_weights(case):
    T, E, K, cf, l = case
    r = O.route(l, E, K, cf)
    assert np.array_equal(r["ids"], brute_ids(l, K))
    assert np.all(np.abs(r["w"].sum(1) - 1.0) <= 1e-12)
    assert np.allclose(r["w"], O.topk_weights_from_chosen_logits(l, r["ids"]), atol=1e-12, rtol=0)
    # slots in descending logit order
    chosen = np.take_along_axis(l, r["ids"], 1)
    assert np.all(np.diff(chosen, axis=1) <= 0)


@SETTINGS
@given(routing_case())
def test_capacity_and_row_map(case):
    T, E, K, cf, l = case
    r = O.route(l, E, K, cf)
    C = r["C"]
    if cf > 0:
        exact = fractions.Fraction(cf) * T * K / E
        assert C == math.ceil(exact)
    else:
        assert C == T
    counts, kept, off = r["counts"], r["kept"], r["offsets"]
    assert counts.sum() == T * K
    assert np.array_equal(kept, np.minimum(counts, C))
    assert r["n_dropped"] == int(np.maximum(counts - C, 0).sum())
    assert off[0] == 0 and np.array_equal(np.diff(off), kept)
    N = int(off[-1])
    rows = r["row_of"][r["row_of"] >= 0]
    assert np.array_equal(np.sort(rows), np.arange(N))
    t_idx = np.nonzero(r["row_of"] >= 0)[0]
    assert np.array_equal(r["token_of"][r["row_of"][r["row_of"] >= 0]], t_idx)
    for e in range(E):
        seg = r["token_of"][off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
    # brute force: the first C assignments to each expert in token order are kept
    flat = [(t, k, int(r["ids"][t, k])) for t in range(T) for k in range(K)]
    seen = np.zeros(E, dtype=np.int64)
    for t, k, e in flat:
        keep = seen[e] < C
        seen[e] += 1
        assert (r["row_of"][t, k] >= 0) == keep


@SETTINGS
@given(routing_case())
def test_aux_bounds(case):
    T, E, K, cf, l = case
    r = O.route(l, E, K, cf)
    assert -1e-12 <= r["aux"] <= E + 1e-12
    flat = O.route(np.zeros_like(l), E, K, cf)
    assert abs(flat["aux"] - 1.0) <= 1e-12


@settings(max_examples=60, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(routing_case(), st.integers(1, 12), st.integers(1, 12), st.booleans())
def test_forward_equals_dense_all_experts(case, H, h, shared):
    T, E, K, cf, l = case
    r = np.random.default_rng(T * 131 + E * 7 + K)
    x = r.standard_normal((T, H))
    w1 = r.standard_normal((E, H, h)) * 0.3
    w2 = r.standard_normal((E, h, H)) * 0.3
    ws1 = r.standard_normal((H, h)) * 0.3 if shared else None
    ws2 = r.standard_normal((h, H)) * 0.3 if shared else None
    w_r = r.standard_normal((H, E))
    f = O.forward(x, w_r, None, w1, w2, ws1, ws2, K=K, cf=cf, logits=l)
    dense = O.dense_all_experts(x, w1, w2, f, ws1, ws2)
    assert np.allclose(f["y"], dense, atol=1e-12, rtol=0)
