"""Parity comparator between the GPU library and the CPU oracle.

Bars (from the definition of the task):
  * greedy tokens, accepted lengths, row status, rollback state: bit-exact;
  * sampled tokens: identical, except at a position the oracle flags as a
    boundary case and everywhere after it in the row:
      - acceptance boundary: |u - rho| < 1e-5,
      - CDF boundary: u within 1e-6 of an edge of the chosen token's interval,
      - top-p boundary: the decisive top-p masses within 1e-6 of top_p;
  * probabilities p'(x_i), q'(x_i): within 1e-5 absolute, except on a vector
    with a top-p boundary flag.
Flags are counted and returned so tests can report them.
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
    flagged_rows: int = 0
    excused_mismatches: int = 0
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


def _np(x):
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy()
    return np.asarray(x)


def compare_sample(gpu, ora, k_per_row, K, rows=None):
    """gpu: dict of tensors from the library; ora: dict from oracle.verify_sample
    computed on the same inputs (possibly on a subset of rows, given by
    `rows` = the GPU row index of each oracle row).  Raises AssertionError
    on an unexcused difference; returns a Report."""
    g = {k: _np(v) for k, v in gpu.items()}
    n = ora["accepted"].shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    kk = np.full(n, K) if k_per_row is None else _np(k_per_row)[rows]
    rep = Report()
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
        # first flagged position on the oracle's path
        f = None
        for i in range(a_o + 1):
            why = None
            if ora["topp_margin_t"][o, i] < TOPP_BAND:
                why = "topp"
            if i < kb and ora["topp_margin_d"][o, i] < TOPP_BAND:
                why = "topp"
            if i < kb and abs(ora["acc_margin"][o, i]) < ACC_BAND:
                why = why or "accept"
            if i == a_o and ora["cdf_margin"][o] < CDF_BAND:
                why = why or "cdf"
            if why:
                f = i
                rep.flags[why] += 1
                break
        out_g, out_o = g["out_tokens"][b], ora["out_tokens"][o]
        a_g = int(g["accepted"][b])
        if f is None:
            assert a_g == a_o, "row %d: accepted %d vs oracle %d" % (b, a_g, a_o)
            assert np.array_equal(out_g, out_o), "row %d: %s vs oracle %s" % (b, out_g, out_o)
            assert int(g["num_emitted"][b]) == a_o + 1
            rep.exact_rows += 1
        else:
            rep.flagged_rows += 1
            assert a_g >= f, "row %d: rejected at %d before the flagged position %d" % (b, a_g, f)
            assert np.array_equal(out_g[:f], out_o[:f]), "row %d: prefix differs before %d" % (b, f)
            if a_g != a_o or not np.array_equal(out_g, out_o):
                rep.excused_mismatches += 1
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
    return rep


def compare_exact(gpu, ora, keys):
    for k in keys:
        a, b = _np(gpu[k]), np.asarray(ora[k])
        assert np.array_equal(a, b), "%s differs at %s" % (k, np.argwhere(a != b)[:5].tolist())
