"""GPU parity of vocabulary-sharded statistics (sv_shard_stats per shard,
sv_shard_combine, then sv_verify_sample / sv_draft_sample on the merged
records) against the oracle, which sees the whole vocabulary at once, and
against the unsharded path: the merge adds exact integer counts and runs the
unsharded epilogue, so the records of vectors the count table holds are the
unsharded pass's, bit for bit.  Shards here are column views of one logits
tensor on one GPU, from 1 to 16 of them, aligned or not."""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_11_amd as sv
from rejection_sampling_verify_11_amd import workloads as W
from tests.parity import compare_sample
from tests.test_gpu_sample import NT, check_draft, oracle_tokens, oracle_verify, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def records(call, B, K):
    """The per-vector records of a call's workspace, as raw 32-byte rows."""
    n = B * (2 * K + 1) * 32
    return call.workspace[:n].view(B * (2 * K + 1), 32).cpu().numpy()


def sharded_and_plain(inp, toks, shards, seed=3, offset=1, flags=0, sharded_draw=False):
    d = to_dev(inp)
    t = torch.as_tensor(toks, dtype=torch.int32).to(DEV)
    plain = sv.VerifyCall("sample", d.target, d.draft, t, d.temperature, d.top_p, d.k_per_row,
                          seed, offset, flags)
    shard = sv.ShardedCall("sample", d.target, d.draft, t, d.temperature, d.top_p, d.k_per_row,
                           shards, seed, offset, flags, sharded_draw)
    po = plain.run()
    so = shard.run()
    torch.cuda.synchronize()
    return plain, po, shard, so


@pytest.mark.parametrize("shards", [1, 2, 3, 8, 16])
def test_merged_records_are_the_unsharded_records(oracle, shards):
    """Zipf-shaped bf16 logits with top-p 0.9 (V = 151936): every record the
    merge writes equals the unsharded pass's bit for bit, so the outputs are
    identical too; and both match the oracle."""
    inp = W.workload4(3, B=4)
    toks = oracle_tokens(oracle, inp, 3, 1)
    plain, po, shard, so = sharded_and_plain(inp, toks, shards)
    B, K = 4, inp.draft.shape[1]
    assert np.array_equal(records(plain, B, K), records(shard.call, B, K))
    for k in po:
        assert torch.equal(po[k], so[k]), k
    rep = compare_sample(so, oracle_verify(oracle, inp, toks, 3, 1), None, K)
    assert rep.excused_mismatches <= 1


@pytest.mark.parametrize("case", range(12))
def test_random_shardings_match_the_oracle(oracle, case):
    """Random B, k, V, per-row k and temperature, top-p mode and shard
    layouts, including shards that do not start on 8-column boundaries."""
    rng = np.random.default_rng(500 + case)
    B, K = int(rng.integers(1, 12)), int(rng.integers(1, 7))
    V = int(rng.choice([17, 100, 1000, 4097, 16385, 40000]))
    G = int(rng.integers(1, min(16, V) + 1))
    if rng.random() < 0.5:
        cuts = np.sort(rng.choice(np.arange(1, V), G - 1, replace=False)) if G > 1 else []
        edges = [0] + [int(c) for c in cuts] + [V]
        shards = [(edges[g], edges[g + 1] - edges[g]) for g in range(G)]
    else:
        shards = G
    g = torch.Generator().manual_seed(600 + case)
    zt = (torch.randn((B, K + 1, V), generator=g) * float(rng.uniform(0.5, 4))).to(torch.bfloat16)
    zd = (zt[:, :K].float() + torch.randn((B, K, V), generator=g)).to(torch.bfloat16)
    T = torch.from_numpy(rng.uniform(0.3, 1.5, B).astype(np.float32))
    mode = int(rng.integers(0, 3))
    P = None if mode == 0 else torch.from_numpy(rng.uniform(0.5, 0.99, B).astype(np.float32))
    flags = sv.FLAG_TOPP_TARGET_ONLY if mode == 2 else 0
    kk = None if rng.random() < 0.5 else torch.from_numpy(rng.integers(1, K + 1, B).astype(np.int32))
    inp = W.SampleInputs(zt, zd, T, P, kk)
    toks = oracle_tokens(oracle, inp, 8, case, flags)
    sharded_draw = case % 2 == 1
    plain, po, shard, so = sharded_and_plain(inp, toks, shards, 8, case, flags, sharded_draw)
    rep = compare_sample(so, oracle_verify(oracle, inp, toks, 8, case, flags), kk, K)
    assert rep.excused_mismatches <= 1
    for k in po:  # the same records (and draws up to rounding order), so the same outputs
        assert torch.equal(po[k], so[k]), k


@pytest.mark.parametrize("shards", [2, 8])
def test_sharded_draft_sampler(oracle, shards):
    inp = W.workload4(4, B=6, V=50000)
    d = to_dev(inp)
    g_toks, g_st = sv.draft_sample_sharded(d.draft, d.temperature, d.top_p, shards=shards,
                                           seed=2, offset=5)
    p_toks, _ = sv.draft_sample(d.draft, d.temperature, d.top_p, seed=2, offset=5)
    torch.cuda.synchronize()
    assert torch.equal(g_toks, p_toks) and not g_st.any()
    _, nd = check_draft(oracle, W.host_logits(inp.draft), inp.temperature.numpy(),
                        inp.top_p.numpy(), None, 2, 5, g_toks, g_st)
    assert nd <= 1


def test_vectors_the_table_cannot_hold(oracle):
    """Rows built to leave the count table: a logit of magnitude >= 2^16 in
    one shard, 80 nonzero values below 2^-24 spread over the shards (more
    than the merged list holds), 70000 equal logits split over shards (a
    merged count past 16 bits, which the merge's 32-bit table keeps), NaN in
    one shard (a row error), an all -inf draft vector (a row error), and
    draft tokens on shard edges.  The first two are redone from the shards'
    logits."""
    B, K, V, G = 6, 2, 100000, 4
    g = torch.Generator().manual_seed(77)
    zt = torch.randn((B, K + 1, V), generator=g) * 2
    zd = zt[:, :K] + torch.randn((B, K, V), generator=g)
    zt[0, 1, 60000] = 70000.0                        # above the window, shard 2
    tiny = torch.arange(80) * 1237 + 11
    zd[1, 0, tiny] = 1e-9 * (1 + torch.arange(80, dtype=torch.float32))
    zt[2, 0, :70000] = 0.5                           # 70000 equal values
    zt[3, 2, 30000] = float("nan")
    zd[4, 1, :] = float("-inf")
    inp = W.SampleInputs(zt.to(torch.bfloat16), zd.to(torch.bfloat16), torch.ones(B),
                         torch.full((B,), 0.9))
    toks = oracle_tokens(oracle, W.SampleInputs(inp.target[:4], inp.draft[:4],
                                                inp.temperature[:4], inp.top_p[:4]), 4, 0)
    edges = [b for b, _ in sv.shard_bounds(V, G)]
    toks = np.concatenate([toks, np.array([[edges[1] - 1, edges[1]], [edges[2], V - 1]],
                                          np.int32)])
    plain, po, shard, so = sharded_and_plain(inp, toks, G, 4, 0)
    st = so["row_status"].cpu().numpy()
    assert st[3] & sv.ROW_NONFINITE_LOGIT and st[4] & sv.ROW_NO_FINITE
    assert np.all(st[[0, 1, 2, 5]] == 0)
    ok = [0, 1, 2, 5]
    o = oracle_verify(oracle, inp, toks, 4, 0, rows=ok)
    rep = compare_sample(so, o, None, K, rows=ok)
    assert rep.excused_mismatches == 0
    # row 2 takes the generic path unsharded (its count wraps 16 bits) and
    # the table path sharded; every other row takes the same path both ways
    same = [0, 1, 3, 4, 5]
    for k in po:
        a, b = po[k][same].float(), so[k][same].float()
        assert torch.equal(torch.nan_to_num(a), torch.nan_to_num(b)), k


@pytest.mark.parametrize("T", [1.0, 1000.0])
def test_negative_logits_above_the_window_sharded(oracle, T):
    """Masks at the most negative bf16 and scattered values such as -7e4,
    above the count table's window in every shard: the merge redoes such a
    vector from the shards' logits, as the unsharded pass redoes it from the
    whole vector, so the records are bit for bit the same (T = 1 and
    T = 1000), and both match the oracle."""
    B, K, V, G = 4, 3, 60000, 5
    g = torch.Generator().manual_seed(81)
    zt = torch.randn((B, K + 1, V), generator=g) * 3
    zd = zt[:, :K] + torch.randn((B, K, V), generator=g)
    for z in (zt, zd):
        z[torch.rand(z.shape, generator=g) < 0.3] = -3.3895313892515355e38
        z[torch.rand(z.shape, generator=g) < 0.01] = -7e4
    inp = W.SampleInputs(zt.to(torch.bfloat16), zd.to(torch.bfloat16), torch.full((B,), T),
                         torch.full((B,), 0.9))
    toks = oracle_tokens(oracle, inp, 5, 0)
    plain, po, shard, so = sharded_and_plain(inp, toks, G, 5, 0)
    assert np.array_equal(records(plain, B, K), records(shard.call, B, K))
    for k in po:
        assert torch.equal(torch.nan_to_num(po[k].float()), torch.nan_to_num(so[k].float())), k
    rep = compare_sample(so, oracle_verify(oracle, inp, toks, 5, 0), None, K)
    assert rep.excused_mismatches <= 1


@pytest.mark.parametrize("shards", [1, 2, 3, 8, 16])
def test_sharded_draw(oracle, shards):
    """The draw split over the shards (each sums its columns' residual and p'
    masses; the shard holding u R draws from its own columns) on the bench
    logits: the same outputs as the unsharded call, and the oracle's."""
    inp = W.workload4(5, B=8)
    toks = oracle_tokens(oracle, inp, 6, 2)
    plain, po, shard, so = sharded_and_plain(inp, toks, shards, 6, 2, sharded_draw=True)
    for k in po:
        assert torch.equal(po[k], so[k]), k
    rep = compare_sample(so, oracle_verify(oracle, inp, toks, 6, 2), None, inp.draft.shape[1])
    assert rep.excused_mismatches <= 1
    assert shard.masses.sum().item() > 0


def test_sharded_draw_degenerate_rows(oracle):
    """q = p (every draft accepted: the bonus from p'), disjoint supports
    (every first draft rejected), a zero residual (the draw falls back to p'
    across shards), mass only in the last shard, and a row error, over 5
    unaligned shards."""
    V, B = 4096, 10
    g = torch.Generator().manual_seed(21)
    zt = torch.randn((B, 3, V), generator=g) * 2
    zd = zt[:, :2].clone()                                   # rows 0-1: q = p
    zt[2:4, :, : V // 2] = float("-inf")                     # rows 2-3: disjoint supports
    zd[2:4, :, V // 2:] = float("-inf")
    zd[4:6] = zt[4:6, :2]                                    # rows 4-5: zero residual
    zt[4:6, :, 7] = zd[4:6, :, 7] = float("-inf")
    zt[6:8, :, : V - 100] = float("-inf")                    # rows 6-7: target mass at the end
    zt[8, 0, 3] = float("nan")                               # row 8: an error
    inp = W.SampleInputs(zt.to(torch.bfloat16), zd.to(torch.bfloat16), torch.ones(B), None)
    toks = np.zeros((B, 2), np.int32)
    ok = [0, 1, 2, 3, 6, 7, 9]
    sub = W.SampleInputs(inp.target[ok], inp.draft[ok], inp.temperature[ok], None)
    toks[ok] = oracle_tokens(oracle, sub, 9, 0)
    toks[4:6] = 7                                            # outside both supports: rejected
    toks[8] = 0
    shards = [(0, 999), (999, 1), (1000, 1501), (2501, 1000), (3501, 595)]
    plain, po, shard, so = sharded_and_plain(inp, toks, shards, 9, 0, sharded_draw=True)
    st = so["row_status"].cpu().numpy()
    assert st[8] & sv.ROW_NONFINITE_LOGIT and np.all(np.delete(st, 8) == 0)
    for k in po:
        a, b = torch.nan_to_num(po[k].float()), torch.nan_to_num(so[k].float())
        assert torch.equal(a, b), k
    acc = so["accepted"].cpu().numpy()
    assert np.all(acc[[0, 1]] == 2) and np.all(acc[[2, 3, 4, 5]] == 0)
    rows = [r for r in range(B) if r != 8]
    rep = compare_sample(so, oracle_verify(oracle, inp, toks, 9, 0, rows=rows), None, 2, rows=rows)
    assert rep.excused_mismatches == 0



@pytest.mark.parametrize("V,G", [(1, 1), (5, 5), (9, 4)])
def test_tiny_vocabularies(oracle, V, G):
    """One-column shards and vocabularies smaller than a 16-byte load."""
    B, K = 3, 2
    g = torch.Generator().manual_seed(V * 31 + G)
    zt = (torch.randn((B, K + 1, V), generator=g) * 2).to(torch.bfloat16)
    zd = (zt[:, :K].float() + torch.randn((B, K, V), generator=g)).to(torch.bfloat16)
    inp = W.SampleInputs(zt, zd, torch.ones(B), torch.full((B,), 0.95))
    toks = oracle_tokens(oracle, inp, 12, 3)
    plain, po, shard, so = sharded_and_plain(inp, toks, G, 12, 3, sharded_draw=True)
    for k in po:
        assert torch.equal(po[k], so[k]), k
    rep = compare_sample(so, oracle_verify(oracle, inp, toks, 12, 3), None, K)
    assert rep.excused_mismatches == 0
