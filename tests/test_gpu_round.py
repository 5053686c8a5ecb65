"""GPU parity of the on-device round: the dynamic draft-length controller
(sv_dynamic_k) against the oracle's, and a whole round -- draft sampling,
verification, KV rollback, controller update and round-counter advance --
run eagerly and as a captured HIP graph replayed round after round, both
against the oracle's chain of the same steps.

Between rounds the test plays the models' part on the host: it writes the
next round's logits into the fixed input buffers and grows every row's KV
length by its k + 1 speculative positions, mapping pages from the free
stack.  Everything inside a round runs in the library's kernels; the graph
replays read the round counter, k and the KV state from device memory.
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_11_amd as sv
from rejection_sampling_verify_11_amd import workloads as W
from tests.parity import compare_draft, compare_sample, window_from_device_state

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NT = 8


def check_windows(g_state, hist, W, rows=None):
    """The device controller's packed windows against the oracle's plain
    histories, row by row."""
    st = g_state.cpu().numpy()
    for b in (range(st.shape[0]) if rows is None else rows):
        assert window_from_device_state(st[b], W) == hist.window(b, W), "row %d" % b


def test_dynamic_k_matches_oracle_over_many_rounds(oracle):
    rng = np.random.default_rng(11)
    B, Wn, R = 1000, 8, 300
    k0 = np.full(B, 5, np.int32)
    k0[7] = 40000          # outside [k_min, k_max]: the row must never move
    k0[8] = 0              # likewise, with accepted 0
    k0[9] = 9              # one above k_max
    rate = rng.uniform(0.3, 1.0, B)
    o_k, o_h = k0.copy(), oracle.DynkHistory(B, R)
    g_k = torch.from_numpy(k0.copy()).to(DEV)
    g_st = sv.dynk_state(B, Wn, DEV)
    for r in range(R):
        acc = rng.binomial(o_k.clip(0, 8), rate).astype(np.int32)
        acc[8] = 0
        bad = rng.random(B) < 0.05
        acc[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, o_k[bad] + 1)
        oracle.dynamic_k(acc, o_k, o_h, window=Wn)
        sv.dynamic_k(torch.from_numpy(acc).to(DEV), g_k, g_st, window=Wn)
        assert np.array_equal(g_k.cpu().numpy(), o_k), "round %d" % r
        if r % 37 == 0 or r == R - 1:
            check_windows(g_st, o_h, Wn)
    assert o_k[7] == 40000 and o_k[8] == 0 and o_k[9] == 9
    assert np.all(o_h.length[7:10] == 0) and np.all(g_st[7:10].cpu().numpy() == 0)
    assert len(np.unique(o_k)) >= 5  # the controller really moved


def test_dynamic_k_other_thresholds_and_window_one(oracle):
    rng = np.random.default_rng(12)
    B, R = 300, 150
    for Wn, kmin, kmax, up, down in ((1, 1, 32, (1, 2), (1, 3)), (64, 3, 6, (9, 10), (1, 2))):
        o_k = rng.integers(kmin, kmax + 1, B).astype(np.int32)
        o_h = oracle.DynkHistory(B, R)
        g_k = torch.from_numpy(o_k.copy()).to(DEV)
        g_st = sv.dynk_state(B, Wn, DEV)
        for r in range(R):
            acc = rng.integers(0, o_k + 1).astype(np.int32)
            kw = dict(window=Wn, k_min=kmin, k_max=kmax, up=up, down=down)
            oracle.dynamic_k(acc, o_k, o_h, **kw)
            sv.dynamic_k(torch.from_numpy(acc).to(DEV), g_k, g_st, **kw)
            assert np.array_equal(g_k.cpu().numpy(), o_k)
        check_windows(g_st, o_h, Wn)


def test_close_round_is_the_two_calls():
    """sv_close_round against sv_dynamic_k then sv_advance_offset, round after
    round (k, state and counter bit for bit), eagerly and replayed from a
    captured graph; with no rows only the counter moves."""
    rng = np.random.default_rng(5)
    B, Wn, R = 700, 4, 40
    k0 = torch.from_numpy(rng.integers(1, 10, B).astype(np.int32)).to(DEV)
    two = dict(k=k0.clone(), st=sv.dynk_state(B, Wn, DEV),
               off=torch.tensor([2**63 - 3], dtype=torch.int64, device=DEV))
    one = dict(k=k0.clone(), st=sv.dynk_state(B, Wn, DEV), off=two["off"].clone())
    rep = dict(k=k0.clone(), st=sv.dynk_state(B, Wn, DEV), off=two["off"].clone())
    acc = torch.zeros(B, dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.close_round(acc, rep["k"], rep["st"], rep["off"], 3, window=Wn)
    for r in range(R):
        kk = two["k"].cpu().numpy()
        a = rng.binomial(np.clip(kk, 0, 8), 0.8).astype(np.int32)
        a[rng.random(B) < 0.03] = -1
        acc.copy_(torch.from_numpy(a))
        sv.dynamic_k(acc, two["k"], two["st"], window=Wn)
        sv.advance_offset(two["off"], 3)
        sv.close_round(acc, one["k"], one["st"], one["off"], 3, window=Wn)
        g.replay()
        torch.cuda.synchronize()
        for n in ("k", "st", "off"):
            assert torch.equal(two[n], one[n]), (r, n)
            assert torch.equal(two[n], rep[n]), (r, n)
    assert len(np.unique(two["k"].cpu().numpy())) >= 3  # the controller moved
    empty = torch.zeros(0, dtype=torch.int32, device=DEV)
    off = torch.zeros(1, dtype=torch.int64, device=DEV)
    sv.close_round(empty, empty.clone(), sv.dynk_state(0, Wn, DEV), off, 7, window=Wn)
    assert int(off.item()) == 7


def test_advance_offset_wraps():
    off = torch.tensor([-3], dtype=torch.int64, device=DEV)  # 2^64 - 3 as a word
    sv.advance_offset(off, 5)
    assert int(off.item()) == 2
    sv.advance_offset(off, 2**64 - 1)
    assert int(off.item()) == 1


# ------------------------------------------------------------------ the round

PS, K, WIN = 16, 8, 4
POOL = (2, 1, 8)  # layers, KV heads, head dim of a small pool (poisoning on)


def grow(st, k):
    """The target forward's k_b + 1 speculative KV writes: lengths grow and
    the new logical pages are mapped from the top of the free stack."""
    B = st["kv_len"].shape[0]
    for b in range(B):
        old = int(st["kv_len"][b])
        new = old + int(k[b]) + 1
        for lp in range((old + PS - 1) // PS, (new + PS - 1) // PS):
            top = int(st["free_top"][0])
            assert top > 0, "the test pool ran out of pages"
            st["page_table"][b, lp] = st["free_pages"][top - 1]
            st["free_pages"][top - 1] = -1
            st["free_top"][0] = top - 1
        st["kv_len"][b] = new


class Chain:
    """One device-resident chain of rounds over fixed buffers."""

    def __init__(self, target, draft, temperature, state, k0, close_in_one_launch=False):
        B = temperature.shape[0]
        self.close_in_one_launch = close_in_one_launch
        self.offset = torch.zeros(1, dtype=torch.int64, device=DEV)
        self.k = torch.from_numpy(k0.copy()).to(DEV)
        self.toks = torch.full((B, K), -1, dtype=torch.int32, device=DEV)
        self.dyn = sv.dynk_state(B, WIN, DEV)
        self.kv = {n: torch.from_numpy(v.copy()).to(DEV) for n, v in state.items()
                   if n != "kv_pool"}
        self.pool = torch.from_numpy(state["kv_pool"].view(np.int16).copy()).to(DEV)
        self.draft_call = sv.VerifyCall("draft", None, draft, self.toks, temperature, None,
                                        self.k, seed=7, offset=self.offset)
        self.verify_call = sv.VerifyCall("sample", target, draft, self.toks, temperature, None,
                                         self.k, seed=7, offset=self.offset)
        self.roll = sv.RollbackCall(
            self.kv["kv_len"], self.verify_call.outputs["accepted"], self.kv["page_table"], PS,
            K, self.k, self.kv["free_pages"], self.kv["free_top"],
            self.pool.view(torch.bfloat16), state["kv_pool"].shape[0], *POOL)

    def round(self):
        self.draft_call.run()
        self.verify_call.run()
        self.roll.run()
        if self.close_in_one_launch:
            sv.close_round(self.verify_call.outputs["accepted"], self.k, self.dyn, self.offset,
                           1, window=WIN)
        else:
            sv.dynamic_k(self.verify_call.outputs["accepted"], self.k, self.dyn, window=WIN)
            sv.advance_offset(self.offset, 1)

    def host_state(self):
        s = {n: t.cpu().numpy() for n, t in self.kv.items()}
        s["kv_pool"] = self.pool.cpu().numpy().view(np.uint16)
        return s

    def load_kv(self, st):
        for n, t in self.kv.items():
            t.copy_(torch.from_numpy(st[n]))
        self.pool.copy_(torch.from_numpy(st["kv_pool"].view(np.int16)))


def test_captured_round_matches_eager_and_oracle(oracle):
    """Ragged per-row temperature batch (bf16 target N(0, 3^2), draft =
    target + per-row noise, V = 128256, no top-p), 16 rows with contexts of
    512..4096 tokens, k from the controller (start 5, window 4, k in [2, 8]),
    8 rounds.  Every round the graph replay equals the eager round bit for
    bit, the draft tokens and the verification are checked against the
    oracle on the same inputs, and the oracle's rollback and controller,
    fed the GPU's accepted counts, must give the device's state exactly.
    The captured round closes with sv_close_round, the eager one with the
    controller and counter calls apart."""
    B, R = 16, 8
    rows = W.workload5_rows(3, B=B)
    T = rows.temperature
    MP = (4096 + (K + 1) * (R + 1) + PS - 1) // PS
    kv = W.paged_kv(rows.kv_len0, PS, MP, spare_pages=B * (R + 1) + 8, seed=3)
    o = {"kv_len": rows.kv_len0.numpy().copy(), "page_table": kv.page_table.numpy().copy(),
         "free_pages": kv.free_pages.numpy().copy(), "free_top": kv.free_top.numpy().copy()}
    o["kv_pool"] = np.random.default_rng(3).integers(
        0, 60000, (kv.num_pages,) + (POOL[0], 2, POOL[1], PS, POOL[2])).astype(np.uint16)
    o_k, o_h = np.full(B, 5, np.int32), oracle.DynkHistory(B, R)
    grow(o, o_k)

    tgt = torch.empty((B, K + 1, 128256), dtype=torch.bfloat16, device=DEV)
    dft = torch.empty((B, K, 128256), dtype=torch.bfloat16, device=DEV)
    T_d = T.to(DEV)
    eager = Chain(tgt, dft, T_d, o, o_k)
    graph = Chain(tgt, dft, T_d, o, o_k, close_in_one_launch=True)

    inp = W.workload5(0, rows, torch.from_numpy(o_k))
    tgt.copy_(inp.target)
    dft.copy_(inp.draft)
    eager.round()  # also loads every kernel before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph.round()
    n_draft_diff = 0
    for r in range(R):
        if r > 0:
            inp = W.workload5(r, rows, torch.from_numpy(o_k))
            tgt.copy_(inp.target)
            dft.copy_(inp.draft)
            eager.round()
        g.replay()
        torch.cuda.synchronize()
        # graph replay == eager round, bit for bit
        for a, b in ((eager.toks, graph.toks), (eager.k, graph.k), (eager.dyn, graph.dyn),
                     (eager.offset, graph.offset), (eager.pool, graph.pool)):
            assert torch.equal(a, b), "round %d" % r
        for n in eager.kv:
            assert torch.equal(eager.kv[n], graph.kv[n]), "round %d: %s" % (r, n)
        for n, t in eager.verify_call.outputs.items():
            assert torch.equal(t, graph.verify_call.outputs[n]), "round %d: %s" % (r, n)
        assert int(graph.offset.item()) == r + 1
        # the oracle on the same inputs: draft tokens, then the verification
        # of the GPU's draft tokens
        g_toks = graph.toks.cpu().numpy()
        o_toks, o_st, cdf, topp, probe = oracle.draft_sample(
            W.host_logits(inp.draft), T.numpy(), None, o_k, seed=7, offset=r, nthreads=NT,
            diagnostics=True, probe_tokens=g_toks)
        assert np.all(o_st == 0)
        n_draft_diff += compare_draft(g_toks, graph.draft_call.outputs["row_status"], o_toks,
                                      o_st, cdf, topp, probe)
        ov = oracle.verify_sample(W.host_logits(inp.target), W.host_logits(inp.draft), g_toks,
                                  T.numpy(), None, o_k, seed=7, offset=r, nthreads=NT)
        compare_sample(graph.verify_call.outputs, ov, o_k, K).bound()
        # rollback and controller on the GPU's accepted counts
        acc = graph.verify_call.outputs["accepted"].cpu().numpy().astype(np.int32)
        ost = oracle.kv_rollback(o["kv_len"], acc, o["page_table"], PS, K, k_per_row=o_k,
                                 free_pages=o["free_pages"], free_top=o["free_top"],
                                 free_capacity=o["free_pages"].size, kv_pool=o["kv_pool"],
                                 num_layers=POOL[0], kv_heads=POOL[1], head_dim=POOL[2],
                                 num_pages=kv.num_pages)
        assert np.all(ost == 0)
        assert np.array_equal(graph.roll.row_status.cpu().numpy(), ost)
        oracle.dynamic_k(acc, o_k, o_h, window=WIN)
        gs = graph.host_state()
        for n in o:
            assert np.array_equal(gs[n], o[n]), "round %d: %s" % (r, n)
        assert np.array_equal(graph.k.cpu().numpy(), o_k), "round %d" % r
        check_windows(graph.dyn, o_h, WIN)
        # the models' part: the next round's speculative KV writes, mapped
        # from the free stack (applied to the oracle's state, found equal to
        # the device chains' above, then loaded into both chains)
        grow(o, o_k)
        for c in (eager, graph):
            c.load_kv(o)
    assert n_draft_diff <= 2
    assert len(set(o_h.accepted[:, :R].sum(axis=1).tolist())) > 1  # rows accepted differently
