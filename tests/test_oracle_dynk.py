"""Pins of the oracle's dynamic draft-length controller ([SSD] §3.2: raise k
when the acceptance rate is above 85 %, lower it below 70 %; the window of
recent rounds, the start value and the clamp to [2, 8] are this build's
readings of that passage).  The expected trajectories are worked out by hand
from the rule."""
import numpy as np
import pytest

from oracle import svref


def run(acc_seq, k0=5, window=4, **kw):
    k = np.array([k0], np.int32)
    h = svref.DynkHistory(1, len(acc_seq) + 1)
    out = []
    for a in acc_seq:
        a = k[0] if a == "all" else a
        svref.dynamic_k(np.array([a], np.int32), k, h, window=window, **kw)
        out.append(int(k[0]))
    return out, h


def test_all_accepted_climbs_to_k_max_after_the_window_fills():
    out, _ = run(["all"] * 8)
    assert out == [5, 5, 5, 6, 7, 8, 8, 8]


def test_nothing_accepted_falls_to_k_min():
    out, _ = run([0] * 8)
    assert out == [5, 5, 5, 4, 3, 2, 2, 2]


def test_thresholds_are_strict():
    # 17 of 20 proposed = exactly 85 %: no raise; 18 of 20: raise
    out, _ = run([5, 4, 4, 4, 5, 5])
    assert out == [5, 5, 5, 5, 5, 6]
    # 14 of 20 = exactly 70 %: no cut; 13 of 20: cut
    out, _ = run([4, 3, 3, 4, 3])
    assert out == [5, 5, 5, 5, 4]


def test_window_holds_the_proposed_k_of_each_round():
    # after a raise to 6 the next round proposes 6: the window 4 of
    # (5,5),(5,5),(5,5),(5,5) gives 6; then (6,6) pushes one (5,5) out:
    # 21/21 gives 7
    out, h = run(["all"] * 5)
    assert out == [5, 5, 5, 6, 7]
    assert h.window(0, 4) == [(5, 5), (5, 5), (5, 5), (6, 6)]
    assert int(h.length[0]) == 5


def test_window_forgets_the_oldest_round():
    # window 3: (0,5) then (5,5),(5,5),(5,5): the first full window is
    # 10/15 < 70 % (k falls to 4); once the zero round has left, 14/14 raises
    out, h = run([0, 5, 5, 4], window=3)
    assert out == [5, 5, 4, 5]
    assert h.window(0, 3) == [(5, 5), (5, 5), (4, 4)]


@pytest.mark.parametrize("bad", [-1, 6, 9])
def test_invalid_accepted_leaves_the_row_untouched(bad):
    k = np.array([5, 5], np.int32)
    h = svref.DynkHistory(2, 10)
    for _ in range(3):
        svref.dynamic_k(np.array([5, 5], np.int32), k, h, window=4)
    svref.dynamic_k(np.array([bad, 5], np.int32), k, h, window=4)
    assert k[0] == 5 and int(h.length[0]) == 3
    assert k[1] == 6 and int(h.length[1]) == 4


@pytest.mark.parametrize("k0", [0, 1, 9, 40000])
def test_k_outside_the_controllers_range_is_not_recorded(k0):
    # a draft length the controller could not have chosen ([2, 8]) teaches
    # it nothing, and k stays where the caller put it
    k = np.array([k0, 5], np.int32)
    h = svref.DynkHistory(2, 10)
    for _ in range(6):
        svref.dynamic_k(np.array([min(k0, 1), 5], np.int32), k, h, window=4)
    assert k[0] == k0 and int(h.length[0]) == 0
    assert k[1] == 8 and int(h.length[1]) == 6


def test_history_records_exactly_the_valid_rounds_in_order():
    rng = np.random.default_rng(0)
    B, W, R = 16, 5, 200
    k = np.full(B, 5, np.int32)
    h = svref.DynkHistory(B, R)
    seen = [[] for _ in range(B)]
    for _ in range(R):
        acc = np.minimum(rng.integers(0, 9, B), k).astype(np.int32)
        acc[rng.random(B) < 0.05] = -1
        for b in range(B):
            if acc[b] >= 0:
                seen[b].append((int(acc[b]), int(k[b])))
        svref.dynamic_k(acc, k, h, window=W)
        assert np.all((k >= 2) & (k <= 8))
    for b in range(B):
        assert h.window(b, R) == seen[b]


def test_empty_batch_full_history_and_argument_checks():
    svref.dynamic_k(np.zeros(0, np.int32), np.zeros(0, np.int32), svref.DynkHistory(0, 4),
                    window=4)
    with pytest.raises(ValueError):
        svref.dynamic_k(np.zeros(1, np.int32), np.full(1, 4, np.int32),
                        svref.DynkHistory(1, 4), window=4, k_min=5, k_max=4)
    h = svref.DynkHistory(1, 2)
    k = np.full(1, 5, np.int32)
    svref.dynamic_k(np.zeros(1, np.int32), k, h, window=4)
    svref.dynamic_k(np.zeros(1, np.int32), k, h, window=4)
    with pytest.raises(ValueError):
        svref.dynamic_k(np.zeros(1, np.int32), k, h, window=4)
