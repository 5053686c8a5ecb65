"""Parity comparator between the GPU library and the CPU oracle.

Bars (from the definition of the task):
  * greedy tokens, accepted lengths, row status, rollback state: bit-exact;
  * sampled tokens: identical, except where a decision of the row lies on a
    floating-point boundary the oracle flags:
      - acceptance boundary: |u - rho| < 1e-5,
      - CDF boundary: u within 1e-6 of an edge of a token's interval,
      - top-p boundary: the decisive top-p masses within 1e-6 of top_p;
  * probabilities p'(x_i), q'(x_i): within 1e-5 absolute, except on a vector
    with a top-p boundary flag.

A row that differs from the oracle's is not excused wholesale: the oracle is
run again with the GPU's accepted count forced on it (the "what-if" run) and
every decision the GPU took is checked against the oracle's own values:
  * each draft the GPU accepted has u < rho, or |u - rho| within the band;
  * a draft the GPU rejected has u >= rho, or |u - rho| within the band;
  * the emitted token is the oracle's draw at the GPU's position, or a token
    with positive mass in that distribution whose CDF interval lies within
    the band of u (the neighbour across a flagged edge);
  * a decision on a vector with a top-p boundary flag is excused (the kept
    set itself may differ there), and is counted.
Flags and excused rows are counted and returned so tests can bound them.
"""
from dataclasses import dataclass, field

import numpy as np

ACC_BAND = 1e-5
CDF_BAND = 1e-6
TOPP_BAND = 1e-6
PROB_TOL = 1e-5


@dataclass
class Report:
    rows: int = 0
    error_rows: int = 0
    exact_rows: int = 0
    flagged_rows: int = 0        # rows with a flag on the oracle's own path
    excused_mismatches: int = 0  # rows that differ and were validated
    flags: dict = field(default_factory=lambda: {"accept": 0, "cdf": 0, "topp": 0})

    def merge(self, o):
        self.rows += o.rows
        self.error_rows += o.error_rows
        self.exact_rows += o.exact_rows
        self.flagged_rows += o.flagged_rows
        self.excused_mismatches += o.excused_mismatches
        for k in self.flags:
            self.flags[k] += o.flags[k]
        return self

    def bound(self, max_flagged=None, max_excused=None):
        """Caps a test puts on its boundary cases: rows with a flag on the
        oracle's path (by default 10 % of the rows plus 2: a margin that
        flagged everything would trip it; how many draws land among tokens
        of mass below the band depends on the workload), and rows that differ
        from the oracle, each validated decision by decision (by default 1 %
        of the rows plus 1)."""
        mf = self.rows // 10 + 2 if max_flagged is None else max_flagged
        me = self.rows // 100 + 1 if max_excused is None else max_excused
        assert self.flagged_rows <= mf, "%d flagged rows > %d: %s" % (self.flagged_rows, mf, self)
        assert self.excused_mismatches <= me, \
            "%d excused rows > %d: %s" % (self.excused_mismatches, me, self)
        return self


def _np(x):
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy()
    return np.asarray(x)


def _interval_near(probe, band):
    """probe = {C_(t-1)/R, C_t/R, r_t/R, u}: t has mass and its interval lies
    within `band` of u."""
    lo, hi, mass, u = probe
    if not np.isfinite(lo) or not (mass > 0):
        return False
    return (lo - band) <= u < (hi + band)


def _topp_flag(ora, o, i, kb):
    t = ora["topp_margin_t"][o, i] < TOPP_BAND
    d = i < kb and ora["topp_margin_d"][o, i] < TOPP_BAND
    return bool(t or d)


def validate_row(ora, o, what_if, w, kb, a_g, out_g, draft_tokens):
    """Checks every decision of a row the GPU decided differently from the
    oracle, against the oracle's values (`what_if` = the oracle rerun with the
    GPU's accepted count forced and its token as probe, row w).  Returns the
    reasons the row is excused; raises AssertionError on a decision outside
    every band."""
    why = set()
    assert 0 <= a_g <= kb, "accepted %d outside [0, %d]" % (a_g, kb)
    assert np.array_equal(out_g[:a_g], draft_tokens[:a_g]), \
        "accepted prefix %s is not the draft %s" % (out_g[:a_g], draft_tokens[:a_g])
    assert np.all(out_g[a_g + 1:] == -1), "padding after the emitted token: %s" % out_g
    m = ora["acc_margin"][o]
    for i in range(a_g + (1 if a_g < kb else 0)):
        accepted_here = i < a_g
        if _topp_flag(ora, o, i, kb):
            why.add("topp")
            continue
        agrees = (m[i] < 0) if accepted_here else (m[i] >= 0)
        if not agrees:
            assert abs(m[i]) < ACC_BAND, \
                "position %d: GPU %s with u - rho = %.3g" % (
                    i, "accepted" if accepted_here else "rejected", m[i])
            why.add("accept")
    y_g = int(out_g[a_g])
    if y_g != int(what_if["out_tokens"][w, a_g]):
        if _topp_flag(ora, o, a_g, kb):
            why.add("topp")
        else:
            pr = what_if["probe"][w]
            assert _interval_near(pr, CDF_BAND), \
                "token %d at %d: interval [%.9g, %.9g) mass %.3g, u = %.9g" % (
                    y_g, a_g, pr[0], pr[1], pr[2], pr[3])
            why.add("cdf")
    return why


def compare_sample(gpu, ora, k_per_row, K, rows=None):
    """gpu: dict of tensors from the library; ora: dict from oracle.verify_sample
    computed on the same inputs (possibly on a subset of rows, given by
    `rows` = the GPU row index of each oracle row).  Raises AssertionError
    on a difference no band explains; returns a Report."""
    g = {k: _np(v) for k, v in gpu.items()}
    n = ora["accepted"].shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    kk = np.full(n, K) if k_per_row is None else _np(k_per_row)[rows]
    rep = Report()
    differ = []
    for o, b in enumerate(rows):
        rep.rows += 1
        st_o, st_g = int(ora["row_status"][o]), int(g["row_status"][b])
        assert st_g == st_o, "row %d: status %#x vs oracle %#x" % (b, st_g, st_o)
        if st_o:
            rep.error_rows += 1
            assert np.all(g["out_tokens"][b] == -1) and g["accepted"][b] == -1
            assert g["num_emitted"][b] == 0
            if "p_at_draft" in g:
                assert np.all(np.isnan(g["p_at_draft"][b])) and np.all(np.isnan(g["q_at_draft"][b]))
            continue
        kb = int(kk[o])
        a_o = int(ora["accepted"][o])
        # flags on the oracle's own path (counted, and bounded by the tests)
        flagged = None
        for i in range(a_o + 1):
            if _topp_flag(ora, o, i, kb):
                flagged = "topp"
            elif i < kb and abs(ora["acc_margin"][o, i]) < ACC_BAND:
                flagged = "accept"
            elif i == a_o and ora["cdf_margin"][o] < CDF_BAND:
                flagged = "cdf"
            if flagged:
                break
        if flagged:
            rep.flagged_rows += 1
            rep.flags[flagged] += 1
        a_g = int(g["accepted"][b])
        if a_g == a_o and np.array_equal(g["out_tokens"][b], ora["out_tokens"][o]):
            rep.exact_rows += 1
        else:
            differ.append((o, b, kb, a_g))
        assert int(g["num_emitted"][b]) == a_g + 1, "row %d: num_emitted" % b
        # probabilities at the draft tokens
        if "p_at_draft" in g:
            for i in range(K):
                if i >= kb:
                    assert g["p_at_draft"][b, i] == 0.0 and g["q_at_draft"][b, i] == 0.0
                    continue
                if ora["topp_margin_t"][o, i] >= TOPP_BAND:
                    assert abs(g["p_at_draft"][b, i] - ora["p_at_draft"][o, i]) <= PROB_TOL, (b, i)
                if ora["topp_margin_d"][o, i] >= TOPP_BAND:
                    assert abs(g["q_at_draft"][b, i] - ora["q_at_draft"][o, i]) <= PROB_TOL, (b, i)
    if differ:
        assert "rerun" in ora, "rows %s differ and the oracle result cannot be rerun" % (
            [d[1] for d in differ])
        sel = np.array([d[0] for d in differ])
        forced = np.array([d[3] for d in differ], np.int32)
        probe = np.array([g["out_tokens"][d[1], d[3]] if 0 <= d[3] <= K else -1
                          for d in differ], np.int32)
        wi = ora["rerun"](forced, probe, sel)
        for w, (o, b, kb, a_g) in enumerate(differ):
            toks = wi["draft_tokens_in"][w] if "draft_tokens_in" in wi else None
            if toks is None:
                raise AssertionError("what-if run lacks the draft tokens")
            try:
                validate_row(ora, o, wi, w, kb, a_g, g["out_tokens"][b], toks)
            except AssertionError as e:
                raise AssertionError("row %d (oracle accepted %d, GPU %d; GPU %s vs oracle %s): %s"
                                     % (b, ora["accepted"][o], a_g, g["out_tokens"][b].tolist(),
                                        ora["out_tokens"][o].tolist(), e))
            rep.excused_mismatches += 1
    return rep


def compare_draft(g_toks, g_st, o_toks, o_st, cdf, topp, probe):
    """Draft-sampler parity: status bit-exact; tokens identical except where
    the oracle flags the draw (CDF edge or top-p boundary), and there the
    GPU's token must have mass in q' with an interval within the band of u
    (probe = the oracle's intervals of the GPU's tokens), or sit on a flagged
    top-p vector.  Returns the number of differing positions."""
    g_toks, g_st = _np(g_toks), _np(g_st)
    assert np.array_equal(g_st, o_st), "draft status differs"
    diff = np.argwhere(g_toks != o_toks)
    for b, i in diff:
        if topp[b, i] < TOPP_BAND:
            continue
        assert cdf[b, i] < CDF_BAND and _interval_near(probe[b, i], CDF_BAND), \
            "draft (%d, %d): GPU %d vs oracle %d, probe %s" % (b, i, g_toks[b, i], o_toks[b, i],
                                                              probe[b, i])
    return len(diff)


def window_from_device_state(state_row, W):
    """The device controller's packed state row [filled, oldest, sum accepted,
    sum proposed, W slots of accepted | proposed << 16] as the list of
    (accepted, proposed) pairs of its window, oldest first; also checks the
    two running sums against the slots."""
    s = [int(x) for x in state_row]
    filled, oldest = s[0], s[1]
    assert 0 <= filled <= W and 0 <= oldest < W
    slots = s[4:4 + W]
    pairs = [(slots[(oldest + j) % W] & 0xFFFF, slots[(oldest + j) % W] >> 16)
             for j in range(filled)]
    assert s[2] == sum(a for a, _ in pairs) and s[3] == sum(p for _, p in pairs)
    return pairs


def windows_from_device_states(state, W):
    """All rows of a device controller state at once, in the form of
    DynkHistory.windows: [B][W] accepted and proposed (oldest first, -1 past
    the filled count) and the filled counts; checks the running sums."""
    st = _np(state).astype(np.int64)
    B = st.shape[0]
    filled, oldest = st[:, 0], st[:, 1]
    assert np.all((filled >= 0) & (filled <= W)) and np.all((oldest >= 0) & (oldest < W))
    j = np.arange(W)[None, :]
    slots = np.take_along_axis(st[:, 4:4 + W], (oldest[:, None] + j) % W, axis=1)
    live = j < filled[:, None]
    acc = np.where(live, slots & 0xFFFF, -1)
    prop = np.where(live, slots >> 16, -1)
    assert np.array_equal(st[:, 2], np.where(live, acc, 0).sum(axis=1))
    assert np.array_equal(st[:, 3], np.where(live, prop, 0).sum(axis=1))
    return acc.astype(np.int32), prop.astype(np.int32), filled.astype(np.int32)


def compare_exact(gpu, ora, keys):
    for k in keys:
        a, b = _np(gpu[k]), np.asarray(ora[k])
        assert np.array_equal(a, b), "%s differs at %s" % (k, np.argwhere(a != b)[:5].tolist())
