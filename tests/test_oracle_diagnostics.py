"""Pins of the oracle's boundary diagnostics and of the parity comparator's
use of them.

The parity bar excuses a GPU/oracle difference only where a decision lies
within a band of a floating-point boundary: the acceptance test (|u - rho| <
1e-5), an edge of the inverse CDF (1e-6, relative to the drawn mass) or the
top-p cut (1e-6).  The oracle reports those distances; these tests build rows
whose distances are known in closed form -- two- to four-token vocabularies
whose probabilities follow from the fp32 logits -- one inside and one
outside each band, and check

  * the reported distance against the closed form (the uniform u comes from
    numpy's independent Philox, as in the Philox pins);
  * that the comparator excuses a plausible different GPU result inside the
    band and rejects the same result outside it;
  * the what-if run (a forced accepted count, a probe token) on its own
    invariants.
"""
import numpy as np
import pytest

from tests.parity import ACC_BAND, CDF_BAND, TOPP_BAND, compare_sample
from tests.test_oracle_philox import numpy_block

SEED, OFF = 123, 7


def u_of(row, pos, draw, seed=SEED, offset=OFF):
    return (numpy_block((row, pos, draw, offset), (seed, 0))[0] >> 40) / 2.0 ** 24


def f32_logits(p):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.where(p > 0, np.log(np.where(p > 0, p, 1.0)), -np.inf).astype(np.float32)


def softmax64(z32, T=1.0):
    """The closed form the fp32 logits fix: exp(z/T - m) / sum, in fp64."""
    z = z32.astype(np.float64) / T
    w = np.exp(z - z.max())
    return w / w.sum()


def fake_gpu(out, K):
    """A GPU-shaped result dict built from an oracle result."""
    g = {"out_tokens": out["out_tokens"].copy(), "accepted": out["accepted"].copy(),
         "num_emitted": out["num_emitted"].copy(), "row_status": out["row_status"].copy(),
         "p_at_draft": out["p_at_draft"].astype(np.float32),
         "q_at_draft": out["q_at_draft"].astype(np.float32)}
    return g


def seed_with(pred):
    """An offset whose uniforms satisfy pred(u0, u1) for row 0."""
    for off in range(OFF, OFF + 1000):
        if pred(u_of(0, 0, 0, offset=off), u_of(0, 0, 1, offset=off), off):
            return off
    raise AssertionError("no offset found")


# --------------------------------------------------------------- acceptance

def acceptance_row(oracle, delta, T=0.7):
    """V = 2, k = 1: q(0) = 1/2 at position 0 and draft token 0, p(0) set so
    that rho = 2 p(0) = u0 - delta."""
    off = seed_with(lambda u0, u1, o: 0.2 < u0 < 0.9)
    u0 = u_of(0, 0, 0, offset=off)
    p0 = (u0 - delta) / 2
    a = np.float32(T * np.log(p0 / (1 - p0)))
    zt = np.array([[[a, 0.0], [0.3, -0.4]]], np.float32)       # [1, k+1, V]
    zd = np.array([[[0.0, 0.0]]], np.float32)                  # [1, k, V]
    toks = np.zeros((1, 1), np.int32)
    rho = 2.0 * softmax64(zt[0, 0], float(np.float32(T)))[0]  # T reaches the oracle as fp32
    out = oracle.verify_sample(zt, zd, toks, T, seed=SEED, offset=off)
    return out, u0 - rho


@pytest.mark.parametrize("delta", [5e-6, -5e-6, 3e-5, -3e-5, 0.1])
def test_acceptance_margin_is_u_minus_rho(oracle, delta):
    out, expect = acceptance_row(oracle, delta)
    m = out["acc_margin"][0, 0]
    assert abs(m - expect) < 1e-12 and abs(m - delta) < 1e-6
    assert out["accepted"][0] == (1 if m < 0 else 0)
    assert abs(out["rho"][0, 0] - (out["p_at_draft"][0, 0] / out["q_at_draft"][0, 0])) < 1e-15


@pytest.mark.parametrize("delta,inside", [(5e-6, True), (-5e-6, True), (3e-5, False),
                                          (-3e-5, False)])
def test_comparator_excuses_a_flipped_acceptance_only_inside_the_band(oracle, delta, inside):
    out, _ = acceptance_row(oracle, delta)
    a_o = int(out["accepted"][0])
    # the other decision at position 0, with the token the oracle draws there
    wi = out["rerun"](np.array([1 - a_o], np.int32), np.array([-1], np.int32), np.array([0]))
    g = fake_gpu(wi, 1)
    if inside:
        rep = compare_sample(g, out, None, 1)
        assert rep.excused_mismatches == 1 and rep.flags["accept"] == 1
    else:
        with pytest.raises(AssertionError):
            compare_sample(g, out, None, 1)


# ------------------------------------------------------------- CDF margins

def bonus_row(oracle, delta):
    """k = 1, q = p at position 0 (rho = 1: accepted); the bonus is drawn
    from p at position 1 = (p0, p1, p2) with p0 = u1 - delta, so token 1 is
    drawn and u sits delta above its lower edge."""

    off = seed_with(lambda u0, u1, o: 0.2 < u_of(0, 1, 1, offset=o) < 0.8)
    u1 = u_of(0, 1, 1, offset=off)
    p0 = u1 - delta
    p = [p0, (1 - p0) * 0.6, (1 - p0) * 0.4]
    zt = np.stack([f32_logits([0.5, 0.3, 0.2]), f32_logits(p)])[None]
    zd = zt[:, :1].copy()
    toks = np.zeros((1, 1), np.int32)
    out = oracle.verify_sample(zt, zd, toks, 1.0, seed=SEED, offset=off)
    pe = softmax64(zt[0, 1])
    C = np.cumsum(pe)  # left to right, as the inverse CDF sums
    R = C[-1]
    return out, u1, C, R


@pytest.mark.parametrize("delta", [5e-7, 3e-6, 0.05])
def test_cdf_margin_of_the_bonus_draw(oracle, delta):
    out, u1, C, R = bonus_row(oracle, delta)
    assert out["accepted"][0] == 1 and out["out_tokens"][0, 1] == 1
    expect = min(abs(C[0] / R - u1), abs(C[1] / R - u1))
    assert abs(out["cdf_margin"][0] - expect) < 1e-12
    assert abs(out["cdf_margin"][0] - delta) < 1e-6
    assert out["residual_mass"][0] == -1.0


@pytest.mark.parametrize("delta,inside", [(5e-7, True), (3e-6, False)])
def test_comparator_excuses_the_neighbour_across_a_flagged_edge(oracle, delta, inside):
    out, _, _, _ = bonus_row(oracle, delta)
    g = fake_gpu(out, 1)
    g["out_tokens"][0, 1] = 0  # the token just below the edge u sits on
    if inside:
        rep = compare_sample(g, out, None, 1)
        assert rep.excused_mismatches == 1 and rep.flags["cdf"] == 1
    else:
        with pytest.raises(AssertionError):
            compare_sample(g, out, None, 1)
    # a token whose interval is nowhere near u is never excused
    g["out_tokens"][0, 1] = 2
    with pytest.raises(AssertionError):
        compare_sample(g, out, None, 1)


def residual_row(oracle, delta):
    """k = 1, V = 3: q = (0.05, 0.05, 0.9), draft token 2, p = (p0, p1,
    0.05), so rho = 1/18 (rejected for u0 > 0.06) and the residual is
    (p0 - 0.05, p1 - 0.05, 0) with mass R = 0.85: its first edge, relative to
    R, sits delta below u1."""
    off = seed_with(lambda u0, u1, o: u0 > 0.1 and 0.2 < u1 < 0.8)
    u1 = u_of(0, 0, 1, offset=off)
    p0 = 0.05 + 0.85 * (u1 - delta)
    p = [p0, 0.95 - p0, 0.05]
    zt = np.stack([f32_logits(p), f32_logits([0.2, 0.3, 0.5])])[None]
    zd = f32_logits([0.05, 0.05, 0.9])[None, None]
    toks = np.full((1, 1), 2, np.int32)
    out = oracle.verify_sample(zt, zd, toks, 1.0, seed=SEED, offset=off)
    r = np.maximum(0.0, softmax64(zt[0, 0]) - softmax64(zd[0, 0]))
    C = np.cumsum(r)
    return out, u1, C, C[-1]


@pytest.mark.parametrize("delta", [5e-7, -5e-7, 3e-6])
def test_cdf_margin_of_the_residual_is_relative_to_its_mass(oracle, delta):
    out, u1, C, R = residual_row(oracle, delta)
    assert out["accepted"][0] == 0
    assert abs(out["residual_mass"][0] - R) < 1e-12 and abs(R - 0.85) < 1e-6
    y = int(out["out_tokens"][0, 0])
    assert y == (1 if delta > 0 else 0)
    expect = min(abs((C[y - 1] if y else 0.0) / R - u1), abs(C[y] / R - u1))
    assert abs(out["cdf_margin"][0] - expect) < 1e-12
    assert abs(out["cdf_margin"][0] - abs(delta)) < 1e-6


# ------------------------------------------------------------ top-p margins

def topp_row(oracle, p_target, P=0.9):
    zt = np.stack([f32_logits(p_target), f32_logits([0.4, 0.3, 0.2, 0.1])])[None]
    zd = np.stack([f32_logits([0.25, 0.25, 0.25, 0.25])])[None]
    toks = np.zeros((1, 1), np.int32)
    out = oracle.verify_sample(zt, zd, toks, 1.0, P, seed=SEED, offset=OFF)
    pe = softmax64(zt[0, 0])
    return out, pe


@pytest.mark.parametrize("delta", [5e-7, 3e-6])
def test_topp_margin_when_the_kept_mass_is_near_top_p(oracle, delta):
    # sorted masses 0.5, 0.4 + delta, ...: the first two are kept, G = 0.9 +
    # delta, and the mass above the lowest kept value is 0.5
    out, pe = topp_row(oracle, [0.5, 0.4 + delta, 0.06 - delta, 0.04])
    G = pe[0] + pe[1]
    P = float(np.float32(0.9))  # top_p reaches the oracle as fp32
    expect = min(abs(pe[0] - P), abs(G - P))
    m = out["topp_margin_t"][0, 0]
    assert abs(m - expect) < 1e-12 and abs(m - delta) < 1e-6
    st, _, G_o, above, n = oracle.softmax_topp(
        f32_logits([0.5, 0.4 + delta, 0.06 - delta, 0.04]), 1.0, P)
    assert n == 2 and abs(G_o - G) < 1e-15 and abs(above - pe[0]) < 1e-15


@pytest.mark.parametrize("delta", [5e-7, 3e-6])
def test_topp_margin_when_the_mass_above_the_cut_is_near_top_p(oracle, delta):
    # sorted masses 0.9 - delta, 0.05, ...: token 1 is still kept (the mass
    # above it is below 0.9), so the mass above the lowest kept value is
    # 0.9 - delta while G = 0.95 - delta is far from 0.9
    out, pe = topp_row(oracle, [0.9 - delta, 0.05, 0.03, 0.02 + delta])
    P = float(np.float32(0.9))  # top_p reaches the oracle as fp32
    expect = min(abs(pe[0] - P), abs(pe[0] + pe[1] - P))
    m = out["topp_margin_t"][0, 0]
    assert abs(m - expect) < 1e-12 and abs(m - delta) < 1e-6


@pytest.mark.parametrize("delta,inside", [(5e-7, True), (3e-6, False)])
def test_comparator_excuses_decisions_on_a_flagged_top_p_vector(oracle, delta, inside):
    out, _ = topp_row(oracle, [0.9 - delta, 0.05, 0.03, 0.02 + delta])
    a_o = int(out["accepted"][0])
    wi = out["rerun"](np.array([1 - a_o], np.int32), np.array([-1], np.int32), np.array([0]))
    g = fake_gpu(wi, 1)
    if inside:
        rep = compare_sample(g, out, None, 1)
        assert rep.excused_mismatches == 1 and rep.flags["topp"] == 1
    else:
        with pytest.raises(AssertionError):
            compare_sample(g, out, None, 1)


# ------------------------------------------------------------- what-if run

def test_forcing_the_oracles_own_count_changes_nothing(oracle):
    rng = np.random.default_rng(5)
    B, K, V = 40, 4, 50
    zt = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    zd = (zt[:, :K] + rng.normal(0, 1, (B, K, V))).astype(np.float32)
    toks, _ = oracle.draft_sample(zd, 0.9, 0.8, seed=3, offset=1)
    out = oracle.verify_sample(zt, zd, toks, 0.9, 0.8, seed=3, offset=1)
    wi = out["rerun"](out["accepted"], out["out_tokens"][np.arange(B), out["accepted"]],
                      np.arange(B))
    for k in ("out_tokens", "accepted", "acc_margin", "cdf_margin", "topp_margin_t"):
        assert np.array_equal(wi[k], out[k]), k
    # the probe of the oracle's own token: its interval holds u, its share is
    # the interval's width
    lo, hi, mass, u = wi["probe"].T
    assert np.all((lo <= u) & (u < hi)) and np.all(mass > 0)
    assert np.allclose(hi - lo, mass, rtol=0, atol=1e-12)


def test_forced_count_draws_where_it_is_told(oracle):
    # q = p at every position: the scan accepts all k, so forcing a = 0 must
    # draw from the residual max(0, p - q) = 0 -- the zero-residual fallback,
    # a draw from p at position 0 with u(b, 0, 1)
    rng = np.random.default_rng(6)
    B, K, V = 30, 3, 20
    zt = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    zd = zt[:, :K].copy()
    toks, _ = oracle.draft_sample(zd, 1.0, seed=4, offset=0)
    out = oracle.verify_sample(zt, zd, toks, 1.0, seed=4, offset=0)
    assert np.all(out["accepted"] == K)
    wi = out["rerun"](np.zeros(B, np.int32), np.full(B, -1, np.int32), np.arange(B))
    assert np.all(wi["accepted"] == 0) and np.all(wi["residual_mass"] == 0.0)
    for b in range(B):
        p = softmax64(zt[b, 0])
        u = u_of(b, 0, 1, seed=4, offset=0)
        assert wi["out_tokens"][b, 0] == int(np.searchsorted(np.cumsum(p), u * p.sum(),
                                                             side="right"))


def test_draft_probe_holds_the_draws_uniform(oracle):
    rng = np.random.default_rng(7)
    B, K, V = 20, 3, 30
    zd = rng.normal(0, 2, (B, K, V)).astype(np.float32)
    toks, st, cdf, topp, probe = oracle.draft_sample(zd, 1.2, 0.7, seed=9, offset=2,
                                                     diagnostics=True,
                                                     probe_tokens=np.zeros((B, K), np.int32) + 0)
    toks2, _, _, _, probe2 = oracle.draft_sample(zd, 1.2, 0.7, seed=9, offset=2,
                                                 diagnostics=True, probe_tokens=toks)
    lo, hi, mass, u = np.moveaxis(probe2, -1, 0)
    assert np.array_equal(toks, toks2)
    assert np.all((lo <= u) & (u < hi)) and np.all(mass > 0)
    assert np.allclose(np.minimum(u - lo, hi - u), cdf, rtol=0, atol=1e-15)
    for b in range(B):
        for i in range(K):
            assert u[b, i] == u_of(b, i, 2, seed=9, offset=2)
