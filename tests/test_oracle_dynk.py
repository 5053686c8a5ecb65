"""Pins of the oracle's dynamic draft-length controller ([SSD] §3.2: raise k
when the acceptance rate is above 85 %, lower it below 70 %; window, start
value and clamp are the readings of the design doc).  The expected trajectories
are worked out by hand from that rule."""
import numpy as np
import pytest

from oracle import svref


def run(acc_seq, k0=5, window=4, **kw):
    k = np.array([k0], np.int32)
    st = svref.dynk_state(1, window)
    out = []
    for a in acc_seq:
        a = k[0] if a == "all" else a
        svref.dynamic_k(np.array([a], np.int32), k, st, window=window, **kw)
        out.append(int(k[0]))
    return out, st


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
    # after a raise to 6 the next rounds propose 6: window 4 of
    # (5,5),(5,5),(5,5),(5,5) -> 6; then (6,6) pushes (5,5) out: 21/21 -> 7
    out, st = run(["all"] * 5)
    assert out == [5, 5, 5, 6, 7]
    assert st[0, 0] == 4 and st[0, 2] == 5 + 5 + 5 + 6 and st[0, 3] == 5 + 5 + 5 + 6


@pytest.mark.parametrize("bad", [-1, 6, 9])
def test_invalid_accepted_leaves_the_row_untouched(bad):
    k = np.array([5, 5], np.int32)
    st = svref.dynk_state(2, 4)
    for _ in range(3):
        svref.dynamic_k(np.array([5, 5], np.int32), k, st, window=4)
    before_k, before_st = k.copy(), st.copy()
    svref.dynamic_k(np.array([bad, 5], np.int32), k, st, window=4)
    assert k[0] == before_k[0] and np.array_equal(st[0], before_st[0])
    assert k[1] == 6 and st[1, 0] == 4


def test_ring_sums_match_the_slots_over_a_long_run():
    rng = np.random.default_rng(0)
    B, W = 16, 5
    k = np.full(B, 5, np.int32)
    st = svref.dynk_state(B, W)
    for _ in range(200):
        acc = np.minimum(rng.integers(0, 9, B), k).astype(np.int32)
        acc[rng.random(B) < 0.05] = -1
        svref.dynamic_k(acc, k, st, window=W)
        slots = st[:, 4:]
        assert np.array_equal(st[:, 2], (slots & 0xFFFF).sum(axis=1))
        assert np.array_equal(st[:, 3], (slots >> 16).sum(axis=1))
        assert np.all((k >= 2) & (k <= 8))
        assert np.all(st[:, 0] <= W) and np.all((st[:, 1] >= 0) & (st[:, 1] < W))


def test_k_too_large_for_a_slot_is_not_a_draft_length():
    # a slot stores proposed k in 15 bits; a larger k leaves the row alone
    k = np.array([40000, 5], np.int32)
    st = svref.dynk_state(2, 4)
    for _ in range(6):
        svref.dynamic_k(np.array([3, 5], np.int32), k, st, window=4)
    assert k[0] == 40000 and np.all(st[0] == 0)
    assert k[1] == 8 and st[1, 0] == 4


def test_empty_batch_and_argument_checks():
    k = np.zeros(0, np.int32)
    st = svref.dynk_state(0, 4)
    svref.dynamic_k(np.zeros(0, np.int32), k, st, window=4)
    with pytest.raises(ValueError):
        svref.dynamic_k(np.zeros(1, np.int32), np.ones(1, np.int32), svref.dynk_state(1, 4),
                        window=4, k_min=5, k_max=4)
