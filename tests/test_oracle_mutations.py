"""Plants plausible mistakes in copies of the oracle and checks that a pin
catches each one.  Everything runs on the CPU: each mutant is the oracle
source with one textual change, built with gcc into a temporary directory.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import build as obuild

import tests.test_oracle_philox as T_philox
import tests.test_oracle_statistics as T_stats
import tests.test_oracle_greedy_rollback as T_gr
import tests.test_oracle_softmax_topp as T_sm
import tests.test_oracle_dynk as T_dk

SRC = open(obuild.SRC).read()


def _pins_pmf(o):
    for case in range(len(T_stats.BRUTE_CASES)):
        T_stats.test_exact_pmf_brute_force(o, case)


def _pins_chi(o):
    for cfg in T_stats.CHI_CASES[:2]:
        T_stats.test_chi_square_output_law_is_target(o, cfg)


MUTANTS = [
    ("residual without the clamp at zero",
     "c->qa[j] = d > 0.0 ? d : 0.0; /* reuse qa as r */", "c->qa[j] = d; /* reuse qa as r */",
     _pins_pmf),
    ("ratio inverted (q/p)",
     "double rho = qx[i] > 0.0 ? px[i] / qx[i] : 0.0;\n    double u",
     "double rho = px[i] > 0.0 ? qx[i] / px[i] : 0.0;\n    double u", _pins_pmf),
    ("accept when u > rho",
     "if (!(u < rho)) { acc = i; break; }", "if (!(u > rho)) { acc = i; break; }", _pins_pmf),
    ("bonus drawn from the last draft position",
     "    load_target(c, b, k);\n    svref_softmax_topp(c->z, V, T, P, c->pa, NULL, NULL, NULL);\n    y = inverse_cdf",
     "    load_target(c, b, k - 1);\n    svref_softmax_topp(c->z, V, T, P, c->pa, NULL, NULL, NULL);\n    y = inverse_cdf",
     _pins_pmf),
    ("draft side softmax at temperature 1",
     "svref_softmax_topp(c->z, V, T, Pq, c->qa, &G, &above, NULL);",
     "svref_softmax_topp(c->z, V, 1.0, Pq, c->qa, &G, &above, NULL);", _pins_chi),
    ("Philox mixes the wrong high half",
     "uint64_t y0 = hi1 ^ x1 ^ k0;", "uint64_t y0 = hi0 ^ x1 ^ k0;",
     lambda o: [T_philox.test_philox_block_matches_numpy(o, *c) for c in T_philox.CASES]),
    ("uniform from output word 1",
     "return (double)(out[0] >> 40)", "return (double)(out[1] >> 40)",
     lambda o: T_philox.test_uniform_is_top24_bits_of_word0(o)),
    ("greedy keeps the last maximal index",
     "if (z[j] > z[best]) best = j;", "if (z[j] >= z[best]) best = j;",
     lambda o: T_gr.test_greedy_matches_numpy_argmax_with_ties(o)),
    ("rollback one slot too far",
     "newlen[b] = old - (k - acc);", "newlen[b] = old - (k - acc) - 1;",
     lambda o: T_gr.test_worked_example_k5_three_accepted(o)),
    ("top-p compares the mass including the token itself",
     "if (before < top_p) { tau = v; tau_before = before; }\n    else break;\n    before += group;",
     "before += group;\n    if (before < top_p) { tau = v; tau_before = before - group; }\n    else break;",
     lambda o: T_sm.test_topp_hand_computed_fixture(o)),
    ("softmax without the max shift divides by the wrong sum",
     "for (int32_t j = 0; j < V; ++j) p_out[j] /= S;", "for (int32_t j = 0; j < V; ++j) p_out[j] /= (S + 1e-3);",
     lambda o: T_sm.test_two_level_closed_form(o)),
    ("controller raises k at exactly 85 %",
     "if (sa * a->up_den > (int64_t)a->up_num * sp) next = k + 1;",
     "if (sa * a->up_den >= (int64_t)a->up_num * sp) next = k + 1;",
     lambda o: T_dk.test_thresholds_are_strict()),
    ("controller acts before its window is full",
     "if (st[0] == W) {\n      const int64_t sa", "if (st[0] >= W - 1) {\n      const int64_t sa",
     lambda o: T_dk.test_all_accepted_climbs_to_k_max_after_the_window_fills()),
]


@pytest.fixture(scope="module")
def tmpdir_mut():
    d = tempfile.mkdtemp(prefix="svref_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(oracle, tmpdir_mut, name, old, new, pin):
    assert SRC.count(old) == 1, "mutation anchor not found: " + name
    d = os.path.join(tmpdir_mut, str(abs(hash(name))))
    os.makedirs(d, exist_ok=True)
    src = os.path.join(d, "svref.c")
    open(src, "w").write(SRC.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(obuild.SRC), "svref.h"), d)
    lib = os.path.join(d, "libsvref_mut.so")
    subprocess.run(["gcc", *obuild.CFLAGS, src, "-o", lib, "-lm"], check=True,
                   capture_output=True)
    with oracle.using_library(lib):
        with pytest.raises(AssertionError):
            pin(oracle)
