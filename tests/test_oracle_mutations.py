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
import tests.test_oracle_diagnostics as T_dg

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
     "    load_target(c, b, k);\n    svref_softmax_topp(c->z, V, T, P, c->pa, NULL, NULL, NULL);\n    drawn = c->pa;",
     "    load_target(c, b, k - 1);\n    svref_softmax_topp(c->z, V, T, P, c->pa, NULL, NULL, NULL);\n    drawn = c->pa;",
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
     "if (n >= W) {", "if (n >= W - 1) {",
     lambda o: T_dk.test_all_accepted_climbs_to_k_max_after_the_window_fills()),
    ("controller window one round short",
     "for (int32_t r = n - W; r < n; ++r)", "for (int32_t r = n - W + 1; r < n; ++r)",
     lambda o: T_dk.test_window_forgets_the_oldest_round()),
    ("controller records a k outside its range",
     "if (k < a->k_min || k > a->k_max || acc < 0 || acc > k) continue;",
     "if (acc < 0 || acc > k) continue;",
     lambda o: [T_dk.test_k_outside_the_controllers_range_is_not_recorded(k) for k in (0, 9)]),
    ("acceptance margin with its sign reversed",
     "a->diag_acc_margin[(int64_t)b * K + i] = u - rho;\n    if (!(u < rho))",
     "a->diag_acc_margin[(int64_t)b * K + i] = rho - u;\n    if (!(u < rho))",
     lambda o: T_dg.test_acceptance_margin_is_u_minus_rho(o, 5e-6)),
    ("CDF margin not relative to the drawn mass",
     "double lo = fabs(prev / R - u), hi = fabs(C / R - u);",
     "double lo = fabs(prev - u), hi = fabs(C - u);",
     lambda o: T_dg.test_cdf_margin_of_the_residual_is_relative_to_its_mass(o, 5e-7)),
    ("CDF margin to the upper edge only",
     "*margin = lo < hi ? lo : hi;", "*margin = hi;",
     lambda o: T_dg.test_cdf_margin_of_the_bonus_draw(o, 5e-7)),
    ("top-p margin from the kept mass only",
     "return m1 < m2 ? m1 : m2;", "return m2;",
     lambda o: T_dg.test_topp_margin_when_the_mass_above_the_cut_is_near_top_p(o, 5e-7)),
    ("top-p margin from the mass above the cut only",
     "return m1 < m2 ? m1 : m2;", "return m1;",
     lambda o: T_dg.test_topp_margin_when_the_kept_mass_is_near_top_p(o, 5e-7)),
    ("probe interval starts after the token's own mass",
     "    if (j == t) below = C;\n    C += r[j];", "    C += r[j];\n    if (j == t) below = C;",
     lambda o: T_dg.test_forcing_the_oracles_own_count_changes_nothing(o)),
    ("what-if run ignores the forced count",
     "if (f >= 0 && f <= k) acc = f;", "if (f >= 0 && f < 0) acc = f;",
     lambda o: T_dg.test_forced_count_draws_where_it_is_told(o)),
    ("page check only near the rolled-back positions",
     "        if (pg < used) {\n          if (e < 0",
     "        if (pg < used && pg >= used - 1) {\n          if (e < 0",
     lambda o: T_gr.test_rollback_flags_every_page_table_corruption(o, True)),
    ("page check only just past the length",
     "} else if (a->free_pages && e != -1) {",
     "} else if (a->free_pages && e != -1 && pg == used) {",
     lambda o: T_gr.test_rollback_flags_every_page_table_corruption(o, True)),
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
