"""Pins of the oracle's temperature softmax and tie-closed top-p.

Closed forms, a hand-computed fixture (tests/golden/topp_v8.json) and an
O(V^2) brute-force statement of the top-p rule on small rows.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_constant_logits_uniform(oracle):
    for V in (1, 7, 1000):
        for T in (0.1, 1.0, 3.0):
            st, p, G, above, n = oracle.softmax_topp(np.full(V, 2.5), T, 1.0)
            assert st == 0 and n == V
            np.testing.assert_allclose(p, 1.0 / V, rtol=1e-14)


def test_two_level_closed_form(oracle):
    a, b, na, nb = 3.0, -1.25, 5, 11
    for T in (0.5, 1.0, 2.0):
        z = np.array([a] * na + [b] * nb)
        st, p, *_ = oracle.softmax_topp(z, T, 1.0)
        pa = math.exp(a / T) / (na * math.exp(a / T) + nb * math.exp(b / T))
        pb = math.exp(b / T) / (na * math.exp(a / T) + nb * math.exp(b / T))
        assert st == 0
        np.testing.assert_allclose(p[:na], pa, rtol=1e-14)
        np.testing.assert_allclose(p[na:], pb, rtol=1e-14)


def test_masked_entries_have_zero_mass(oracle):
    z = np.array([1.0, -np.inf, 0.5, -np.inf, 2.0])
    st, p, *_ = oracle.softmax_topp(z, 0.7, 1.0)
    assert st == 0
    assert p[1] == 0.0 and p[3] == 0.0
    ref = np.exp(np.array([1.0, 0.5, 2.0]) / 0.7)
    np.testing.assert_allclose(p[[0, 2, 4]], ref / ref.sum(), rtol=1e-14)


def test_shift_invariance_and_temperature(oracle):
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3, 500)
    _, p1, *_ = oracle.softmax_topp(z, 0.8, 1.0)
    _, p2, *_ = oracle.softmax_topp(z + 123.0, 0.8, 1.0)
    _, p3, *_ = oracle.softmax_topp(z / 0.8, 1.0, 1.0)
    np.testing.assert_allclose(p1, p2, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(p1, p3, rtol=1e-12, atol=1e-300)
    assert abs(p1.sum() - 1) < 1e-13


@pytest.mark.parametrize("z,T,P,bit", [
    ([0.0, np.nan, 1.0], 1.0, 1.0, 1),
    ([0.0, np.inf, 1.0], 1.0, 1.0, 1),
    ([-np.inf, -np.inf], 1.0, 1.0, 2),
    ([0.0, 1.0], 0.0, 1.0, 16),
    ([0.0, 1.0], -1.0, 1.0, 16),
    ([0.0, 1.0], np.inf, 1.0, 16),
    ([0.0, 1.0], np.nan, 1.0, 16),
    ([0.0, 1.0], 1.0, 0.0, 32),
    ([0.0, 1.0], 1.0, -0.5, 32),
    ([0.0, 1.0], 1.0, np.nan, 32),
])
def test_status_bits(oracle, z, T, P, bit):
    st, *_ = oracle.softmax_topp(np.array(z, dtype=np.float64), T, P)
    assert st & bit


def test_topp_hand_computed_fixture(oracle):
    fx = json.load(open(os.path.join(HERE, "golden", "topp_v8.json")))
    w = fx["weights"]
    z = np.array([math.log(x) if x > 0 else -math.inf for x in w])
    for case in fx["cases"]:
        st, p, G, above, n = oracle.softmax_topp(z, case["T"], case["top_p"])
        assert st == 0
        kept = sorted(np.nonzero(p > 0)[0].tolist())
        assert kept == case["kept"], case
        assert n == len(case["kept"])
        assert abs(G - float(Fraction(case["kept_mass"]))) < 1e-14
        # renormalised kept mass sums to one, and ratios inside are unchanged
        assert abs(p.sum() - 1.0) < 1e-14
        wt = np.array([x ** (1.0 / case["T"]) for x in w])
        ref = np.where(p > 0, wt, 0.0)
        np.testing.assert_allclose(p, ref / ref.sum(), rtol=1e-13)


def brute_force_kept(z, T, P):
    """Keep j iff sum over i with z_i > z_j of p_i is below P (O(V^2))."""
    zz = np.asarray(z, dtype=np.float64)
    w = np.exp(zz / T - np.max(zz / T))
    p = w / w.sum()
    return np.array([p[zz > zz[j]].sum() < P for j in range(zz.size)])


@pytest.mark.parametrize("seed", range(12))
def test_topp_matches_brute_force_with_ties(oracle, seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(2, 200))
    # a coarse grid makes ties common, as bf16 rows do
    z = np.round(rng.normal(0, 2, V) * 4) / 4
    if seed % 3 == 0:
        z[rng.integers(0, V, V // 5)] = -np.inf
        z[0] = 0.0
    T = float(rng.choice([0.3, 1.0, 1.7]))
    P = float(rng.choice([0.05, 0.5, 0.9, 0.99]))
    st, p, G, above, n = oracle.softmax_topp(z, T, P)
    assert st == 0
    kept = brute_force_kept(z, T, P)
    assert np.array_equal(p > 0, kept)
    # invariants: mass above the lowest kept group < P <= kept mass
    assert above < P <= G + 1e-15
    # equal logits are kept or dropped together
    for v in np.unique(z[np.isfinite(z)]):
        sel = z == v
        assert np.all(p[sel] > 0) or np.all(p[sel] == 0)


def test_signed_zeros_are_one_tie_group(oracle):
    z = np.array([1.0, 0.0, -0.0, -2.0])
    # mass above the zero group = e/(e + 2 + e^-2) = 0.5577; top_p 0.6 keeps both zeros
    st, p, G, above, n = oracle.softmax_topp(z, 1.0, 0.6)
    assert st == 0 and p[1] > 0 and p[2] > 0 and p[3] == 0 and n == 3


def test_topp_one_is_off(oracle):
    z = np.array([0.0, -50.0, -np.inf])
    for P in (1.0, 1.5):
        st, p, G, above, n = oracle.softmax_topp(z, 1.0, P)
        assert st == 0 and G == 1.0 and p[1] > 0 and p[2] == 0
