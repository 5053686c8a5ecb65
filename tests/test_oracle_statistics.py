"""Statistical pins of the oracle's sampled verification.

What the pages fix about the method, checked on the oracle without any
implementation to compare against:
  * the output law equals the target's whatever the draft is ([SD] §2.1 and
    [SSD] §2.4 derive it): exact brute-force pmf on V <= 4, chi-square of the
    emitted token at each reached position on V <= 16;
  * the mean number of emitted tokens per round is E(k) = (1 - a^(k+1))/(1 - a)
    when each position accepts with probability a ([SSD] §3.2, [SD] §2.3);
  * q = p accepts everything; disjoint supports accept nothing;
  * a zero residual falls back to p ([SSD] §4.3).
Every run is seeded, so each test is deterministic.
"""
import json
import math
import os
from fractions import Fraction
from itertools import product

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))
NT = 8


def logits_of(w):
    w = np.asarray(w, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), -np.inf).astype(np.float32)


def exact_p(z32, T=1.0):
    """p of fp32 logits as exact rationals of the fp64 values."""
    z = z32.astype(np.float64) / T
    w = np.exp(z - z.max())
    p = w / w.sum()
    return [Fraction(float(x)) for x in p]


def run_mc(zt, zd, n_rows, n_rounds, T=1.0, top_p=None, flags=0, seed=11, oracle=None):
    """zt [k+1, V], zd [k, V] fp32 logits; every row of every round holds the
    same distributions, with draft tokens drawn by the oracle's draft sampler."""
    K1, V = zt.shape
    k = K1 - 1
    tgt = np.ascontiguousarray(np.broadcast_to(zt, (n_rows, K1, V)))
    dft = np.ascontiguousarray(np.broadcast_to(zd, (n_rows, k, V)))
    toks_all, acc_all = [], []
    for r in range(n_rounds):
        toks, st = oracle.draft_sample(dft, T, top_p, seed=seed, offset=r, flags=flags, nthreads=NT)
        assert np.all(st == 0)
        out = oracle.verify_sample(tgt, dft, toks, T, top_p, seed=seed, offset=r, flags=flags,
                                   nthreads=NT)
        assert np.all(out["row_status"] == 0)
        toks_all.append(out["out_tokens"])
        acc_all.append(out["accepted"])
    return np.concatenate(toks_all), np.concatenate(acc_all)


def brute_force_pmf(p, q):
    """Exact law of (accepted, emitted tokens) by enumerating the draft tokens
    and the accept / reject branch at each position.  p: k+1 lists, q: k lists
    of Fractions."""
    k, V = len(q), len(p[0])
    pmf = {}

    def add(key, pr):
        if pr:
            pmf[key] = pmf.get(key, Fraction(0)) + pr

    def walk(i, prefix, pr):
        if i == k:
            for y in range(V):
                add((k, tuple(prefix) + (y,)), pr * p[k][y])
            return
        for x in range(V):
            if q[i][x] == 0:
                continue
            acc = min(Fraction(1), p[i][x] / q[i][x])
            walk(i + 1, prefix + [x], pr * q[i][x] * acc)
            rej = pr * q[i][x] * (1 - acc)
            if rej:
                r = [max(Fraction(0), p[i][j] - q[i][j]) for j in range(V)]
                R = sum(r)
                dist = [x_ / R for x_ in r] if R else p[i]
                for y in range(V):
                    add((i, tuple(prefix) + (y,)), rej * dist[y])

    walk(0, [], Fraction(1))
    return pmf


def chi2_against(counts, probs, min_expected=5.0):
    """Chi-square p-value of observed counts vs probabilities, merging rare cells."""
    n = counts.sum()
    exp = probs * n
    big = exp >= min_expected
    obs = np.append(counts[big], counts[~big].sum())
    ex = np.append(exp[big], exp[~big].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    ex = ex * obs.sum() / ex.sum()
    return stats.chisquare(obs, ex).pvalue


BRUTE_CASES = [
    # (target weights per position k+1, draft weights per position k)
    ([[1, 2, 3], [3, 1, 1], [1, 1, 2]], [[3, 2, 1], [1, 1, 3]]),
    ([[5, 1, 0, 2], [1, 1, 1, 1]], [[1, 1, 4, 2]]),
    ([[2, 1, 1, 0], [0, 1, 1, 4], [1, 2, 3, 4]], [[0, 1, 1, 2], [1, 0, 2, 2]]),
]


@pytest.mark.parametrize("case", range(len(BRUTE_CASES)))
def test_exact_pmf_brute_force(oracle, case):
    pw, qw = BRUTE_CASES[case]
    zt = np.stack([logits_of(w) for w in pw])
    zd = np.stack([logits_of(w) for w in qw])
    p = [exact_p(z) for z in zt]
    q = [exact_p(z) for z in zd]
    pmf = brute_force_pmf(p, q)
    assert abs(sum(pmf.values()) - 1) < Fraction(1, 10**12)
    toks, acc = run_mc(zt, zd, 20000, 50, oracle=oracle, seed=100 + case)
    keys = sorted(pmf)
    index = {kk: n for n, kk in enumerate(keys)}
    counts = np.zeros(len(keys))
    for t, a in zip(toks, acc):
        key = (int(a), tuple(int(x) for x in t[: a + 1]))
        assert key in index, key  # every observed outcome has positive exact mass
        counts[index[key]] += 1
    probs = np.array([float(pmf[kk]) for kk in keys])
    assert chi2_against(counts, probs) > 0.01
    # the marginal of the first emitted token is exactly p_0 in the brute force
    first = {}
    for (a, ts), pr in pmf.items():
        first[ts[0]] = first.get(ts[0], Fraction(0)) + pr
    for y, pr in first.items():
        assert abs(pr - p[0][y]) < Fraction(1, 10**12)


def emitted_marginals_ok(toks, acc, p_primes):
    """Emitted token at output index j, given the row got that far, ~ p'_j."""
    k = len(p_primes) - 1
    for j in range(k + 1):
        sel = acc >= j
        ys = toks[sel, j]
        V = p_primes[j].size
        counts = np.bincount(ys, minlength=V).astype(float)
        assert counts[p_primes[j] == 0].sum() == 0
        pv = chi2_against(counts, p_primes[j])
        if pv <= 0.01:
            return False, j, pv
    return True, None, None


CHI_CASES = [
    dict(V=16, k=3, T=1.0, top_p=None, flags=0, seed=1),
    dict(V=16, k=3, T=0.7, top_p=0.8, flags=0, seed=2),
    dict(V=12, k=2, T=1.3, top_p=0.6, flags=1, seed=3),
    dict(V=8, k=4, T=1.0, top_p=None, flags=0, seed=4),
]


@pytest.mark.parametrize("cfg", CHI_CASES)
def test_chi_square_output_law_is_target(oracle, cfg):
    rng = np.random.default_rng(cfg["seed"])
    V, k = cfg["V"], cfg["k"]
    zt = rng.normal(0, 1.5, (k + 1, V)).astype(np.float32)
    zd = (zt[:k] + rng.normal(0, 1.5, (k, V))).astype(np.float32)
    P = cfg["top_p"] if cfg["top_p"] is not None else 1.0
    pp = [oracle.softmax_topp(zt[j].astype(np.float64), cfg["T"], P)[1] for j in range(k + 1)]
    toks, acc = run_mc(zt, zd, 25000, 40, T=cfg["T"], top_p=cfg["top_p"], flags=cfg["flags"],
                       seed=cfg["seed"], oracle=oracle)
    ok, j, pv = emitted_marginals_ok(toks, acc, pp)
    assert ok, (j, pv)


@pytest.mark.parametrize("alpha,k", [(0.6, 4), (0.8, 6), (0.9, 8), (0.35, 2)])
def test_mean_emitted_matches_E_k(oracle, alpha, k):
    p = [alpha / 2, alpha / 2, 1 - alpha, 0.0]
    q = [alpha / 2, alpha / 2, 0.0, 1 - alpha]
    zt = np.stack([logits_of(p)] * (k + 1))
    zd = np.stack([logits_of(q)] * k)
    rows, rounds = 20000, 10
    toks, acc = run_mc(zt, zd, rows, rounds, oracle=oracle, seed=int(alpha * 100) + k)
    emitted = acc + 1
    E = (1 - alpha ** (k + 1)) / (1 - alpha)
    pa = np.array([alpha ** j * (1 - alpha) for j in range(k)] + [alpha ** k])
    vals = np.arange(1, k + 2)
    var = (pa * vals ** 2).sum() - (pa * vals).sum() ** 2
    assert abs((pa * vals).sum() - E) < 1e-12
    assert abs(emitted.mean() - E) < 4 * math.sqrt(var / emitted.size)
    # each draft position accepts with probability alpha, independently
    for j in range(k):
        reached = acc >= j
        frac = (acc[reached] > j).mean()
        assert abs(frac - alpha) < 4 * math.sqrt(alpha * (1 - alpha) / reached.sum())


def test_q_equal_p_accepts_everything(oracle):
    rng = np.random.default_rng(5)
    for top_p in (None, 0.7):
        zt = rng.normal(0, 2, (7, 50)).astype(np.float32)
        zd = zt[:6].copy()
        toks, acc = run_mc(zt, zd, 2000, 3, top_p=top_p, oracle=oracle, seed=6)
        assert np.all(acc == 6)
        pbonus = oracle.softmax_topp(zt[6].astype(np.float64), 1.0, top_p or 1.0)[1]
        counts = np.bincount(toks[:, 6], minlength=50).astype(float)
        assert chi2_against(counts, pbonus) > 0.01


def test_disjoint_supports_accept_nothing(oracle):
    p = [3, 1, 0, 0, 2, 0]
    q = [0, 0, 1, 1, 0, 5]
    zt = np.stack([logits_of(p)] * 3)
    zd = np.stack([logits_of(q)] * 2)
    toks, acc = run_mc(zt, zd, 20000, 5, oracle=oracle, seed=7)
    assert np.all(acc == 0)
    counts = np.bincount(toks[:, 0], minlength=6).astype(float)
    assert chi2_against(counts, np.array(p) / sum(p)) > 0.01
    assert np.all(toks[:, 1:] == -1)


def test_zero_residual_falls_back_to_p(oracle):
    """p = q exactly, draft token outside the support: rho = 0 rejects, the
    residual max(0, p - q) is identically zero, and the token comes from p."""
    w = [4, 0, 1, 2, 2]
    z = logits_of(w)
    B = 30000
    tgt = np.ascontiguousarray(np.broadcast_to(np.stack([z, z]), (B, 2, 5)))
    dft = np.ascontiguousarray(np.broadcast_to(z[None], (B, 1, 5)))
    toks = np.ones((B, 1), np.int32)  # token 1 has zero mass on both sides
    out = oracle.verify_sample(tgt, dft, toks, 1.0, seed=9, nthreads=NT)
    assert np.all(out["accepted"] == 0)
    assert np.all(out["residual_mass"] == 0.0)
    counts = np.bincount(out["out_tokens"][:, 0], minlength=5).astype(float)
    assert counts[1] == 0
    assert chi2_against(counts, np.array(w) / sum(w)) > 0.01


def test_speedup_table_reading_of_the_page():
    fx = json.load(open(os.path.join(HERE, "golden", "ssd_speedup_c03.json")))
    c = fx["c"]
    bad = []
    for k, vals in fx["rows"].items():
        k = int(k)
        for a, printed in zip(fx["alpha"], vals):
            E = (1 - a ** (k + 1)) / (1 - a)
            if abs(E / (c * k + 1) - printed) > 0.0051:
                bad.append([str(k), a])
    assert sorted(bad) == sorted(fx["known_mismatches"])
