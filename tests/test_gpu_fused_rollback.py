"""GPU: verification fused with the KV rollback (sv_verify_sample_rollback)
against the two calls it stands for -- sv_verify_sample, then sv_kv_rollback
on the accepted counts -- bit for bit in every output and in the cache state.
The two calls are checked against the oracle elsewhere.

Without a free stack or pool each row's rollback needs nothing from the
other rows and is committed by its verification workgroup; with one, each
workgroup writes its row's decision and the rollback's scan kernels place
the releases.  Both must give the same state as the two calls.
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_11_amd as sv
from rejection_sampling_verify_11_amd import workloads as W
from tests.test_gpu_sample import oracle_tokens, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def page_table(lens, ps, MP):
    """Each row maps ceil(len / ps) distinct pages (at most MP); -1 elsewhere."""
    B = len(lens)
    pt = np.full((B, MP), -1, np.int32)
    nxt = 0
    for b in range(B):
        n = min(-(-max(int(lens[b]), 0) // ps), MP)
        pt[b, :n] = np.arange(nxt, nxt + n)
        nxt += n
    return pt, nxt


def run_both(inp, toks, kpr, lens, ps, pt, num_pages, free_spare=None, pool_dims=None):
    d = to_dev(inp)
    K = inp.draft.shape[1]
    t = torch.as_tensor(toks, dtype=torch.int32, device=DEV)
    k = None if kpr is None else torch.as_tensor(kpr, dtype=torch.int32, device=DEV)
    res = []
    for fused in (False, True):
        call = sv.VerifyCall("sample", d.target, d.draft, t, d.temperature, d.top_p, k, 9, 2)
        kv = torch.as_tensor(np.asarray(lens, np.int32), device=DEV).clone()
        ptd = torch.as_tensor(pt, device=DEV).clone()
        extra = {}
        if free_spare is not None:
            fp = torch.full((free_spare + 4 * len(lens),), -1, dtype=torch.int32, device=DEV)
            fp[:free_spare] = torch.arange(num_pages, num_pages + free_spare, dtype=torch.int32)
            extra = dict(free_pages=fp, free_top=torch.tensor([free_spare], dtype=torch.int32,
                                                              device=DEV))
        if pool_dims is not None:
            L, H, D = pool_dims
            g = torch.Generator(device=DEV).manual_seed(5)
            pool = torch.randint(0, 30000, (num_pages + (free_spare or 0), L, 2, H, ps, D),
                                 generator=g, device=DEV, dtype=torch.int16)
            extra.update(kv_pool=pool.view(torch.bfloat16), num_layers=L, kv_heads=H,
                         head_dim=D)
        roll = sv.RollbackCall(kv, call.outputs["accepted"], ptd, ps, K, k_per_row=k,
                               num_pages=num_pages + (free_spare or 0), **extra)
        if fused:
            call.run_with_rollback(roll)
        else:
            call.run()
            roll.run()
        torch.cuda.synchronize()
        state = {n: x.clone() for n, x in call.outputs.items()}
        state.update(kv_len=kv.clone(), page_table=ptd.clone(), roll_status=roll.row_status.clone())
        for n, x in extra.items():
            if isinstance(x, torch.Tensor):
                state[n] = x.view(torch.int16).clone() if n == "kv_pool" else x.clone()
        res.append(state)
    a, b = res
    for n in a:
        x, y = a[n], b[n]
        if x.is_floating_point():
            x, y = torch.nan_to_num(x, nan=-7.0), torch.nan_to_num(y, nan=-7.0)
        assert torch.equal(x, y), n
    return b


def test_fused_rollback_bench_shape(oracle):
    """B=256, k=6, V=151936 Zipf logits with top-p 0.9; contexts of
    512..4096 tokens plus the round's 7 writes, page size 16."""
    inp = W.workload4(1)
    toks = sv.draft_sample(inp.draft.to(DEV), inp.temperature.to(DEV), inp.top_p.to(DEV),
                           seed=0, offset=1)[0].cpu().numpy()
    rng = np.random.default_rng(5)
    lens = rng.integers(512, 4097, 256) + 7
    ps, MP = 16, (4096 + 7 + 15) // 16
    pt, n = page_table(lens, ps, MP)
    out = run_both(inp, toks, None, lens, ps, pt, n)
    assert torch.all(out["roll_status"] == 0)
    acc = out["accepted"].cpu().numpy()
    assert np.array_equal(out["kv_len"].cpu().numpy(), lens - (6 - acc))


@pytest.mark.parametrize("ps", [1, 16])
def test_fused_rollback_bad_rows(oracle, ps):
    """Per-row k (some outside [1, K]), a draft token out of range, lengths
    too short for the dropped positions, a negative length, too many pages,
    an unmapped page and a page past num_pages among the dropped ones: every
    such row is flagged by both paths alike and keeps its length."""
    B, K = 48, 5
    inp = W.workload2(3, B=B, V=32000)
    rng = np.random.default_rng(ps)
    kpr = rng.integers(1, K + 1, B).astype(np.int32)
    toks = oracle_tokens(oracle, W.SampleInputs(inp.target, inp.draft, inp.temperature,
                                                inp.top_p, torch.from_numpy(kpr)), 4, 2)
    kpr[3], kpr[4] = 0, K + 1
    toks[5, 0] = 32000
    lens = rng.integers(40, 200, B).astype(np.int32)
    lens[6], lens[7] = 0, 2
    lens[8] = -3
    MP = -(-260 // ps)
    lens[9] = MP * ps + 1
    pt, n = page_table(lens, ps, MP)
    last = [(b, -(-int(lens[b]) // ps) - 1) for b in (10, 11)]
    pt[last[0]] = -1
    pt[last[1]] = n + 100
    out = run_both(inp, toks, kpr, lens, ps, pt, n)
    st = out["roll_status"].cpu().numpy()
    acc = out["accepted"].cpu().numpy()
    assert st[3] & sv.ROW_BAD_K and st[4] & sv.ROW_BAD_K
    assert st[5] & sv.ROW_BAD_ACCEPTED
    assert st[8] & sv.ROW_BAD_PAGES and st[9] & sv.ROW_BAD_PAGES
    for b in (10, 11):
        # the whole row of the table is checked against the length
        assert st[b] & sv.ROW_BAD_PAGES, b
    assert np.all(out["kv_len"].cpu().numpy()[st != 0] == lens[st != 0])


@pytest.mark.parametrize("pool", [False, True])
def test_fused_entry_with_a_free_stack(oracle, pool):
    """With a free stack (and optionally a pool to poison) each verification
    workgroup takes its row's rollback decision, whole page-table check
    included, and the rollback's scan places the releases: lengths, pages
    released, stack, pool and status match the two calls, also on rows whose
    table maps a page past the length or leaves one below it unmapped."""
    B, K = 32, 4
    inp = W.workload2(4, B=B, k=K, V=32000)
    toks = oracle_tokens(oracle, inp, 6, 2)
    rng = np.random.default_rng(9)
    lens = rng.integers(17, 120, B).astype(np.int32)
    ps, MP = 4, 32
    pt, n = page_table(lens, ps, MP)
    used = -(-lens // ps)
    pt[2, min(used[2] + 3, MP - 1)] = 5   # mapped far past the length
    pt[3, 0] = -1                   # unmapped below it
    pt[4, used[4]] = -2             # not -1 past the length
    out = run_both(inp, toks, None, lens, ps, pt, n, free_spare=6,
                   pool_dims=(2, 1, 8) if pool else None)
    st = out["roll_status"].cpu().numpy()
    assert list(np.nonzero(st)[0]) == [2, 3, 4]
    assert np.all(st[[2, 3, 4]] == sv.ROW_BAD_PAGES)


def test_fused_rollback_in_a_replayed_graph(oracle):
    """Rounds of (k + 1 KV writes, fused verification + rollback) captured
    once as a HIP graph and replayed, against the same rounds run eagerly as
    two calls: every replay leaves the same lengths and outputs."""
    B, K, ps = 64, 4, 16
    inp = W.workload2(6, B=B, k=K, V=32000)
    toks = torch.as_tensor(oracle_tokens(oracle, inp, 7, 1), dtype=torch.int32, device=DEV)
    d = to_dev(inp)
    MP = (300 + 8 * (K + 1) + ps - 1) // ps
    lens0 = torch.as_tensor(np.random.default_rng(2).integers(100, 300, B), dtype=torch.int32)

    def chain():
        call = sv.VerifyCall("sample", d.target, d.draft, toks, d.temperature, d.top_p, None, 7, 1)
        kv = lens0.to(DEV).clone()
        pt = torch.arange(B * MP, dtype=torch.int32, device=DEV).view(B, MP)
        roll = sv.RollbackCall(kv, call.outputs["accepted"], pt, ps, K, num_pages=B * MP)
        return call, kv, roll

    g_call, g_kv, g_roll = chain()
    e_call, e_kv, e_roll = chain()

    def fused_round():
        g_kv.add_(K + 1)
        g_call.run_with_rollback(g_roll)

    fused_round()  # loads the kernels before the capture
    torch.cuda.synchronize()
    g_kv.copy_(lens0.to(DEV))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fused_round()
    for r in range(5):
        e_kv.add_(K + 1)
        e_call.run()
        e_roll.run()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_kv, e_kv), r
        assert torch.equal(g_roll.row_status, e_roll.row_status), r
        for n in ("out_tokens", "accepted", "num_emitted", "row_status"):
            assert torch.equal(g_call.outputs[n], e_call.outputs[n]), (r, n)
