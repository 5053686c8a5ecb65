"""GPU parity of greedy verification (sv_verify_greedy) and KV rollback
(sv_kv_rollback) against the CPU oracle: bit-exact tokens, accepted
lengths, row status, lengths, page tables, free stacks and KV poisoning."""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_11_amd as sv
from rejection_sampling_verify_11_amd import workloads as W
from tests.parity import compare_exact

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

GREEDY_KEYS = ("out_tokens", "accepted", "num_emitted", "row_status")


def greedy_pair(oracle, target, toks=None, draft=None, k_per_row=None):
    g = sv.verify_greedy(target.to(DEV), None if toks is None else toks.to(DEV),
                         None if draft is None else draft.to(DEV),
                         None if k_per_row is None else k_per_row.to(DEV))
    torch.cuda.synchronize()
    o = oracle.verify_greedy(W.host_logits(target),
                             draft=None if draft is None else W.host_logits(draft),
                             draft_tokens=None if toks is None else toks.cpu().numpy(),
                             k_per_row=None if k_per_row is None else k_per_row.cpu().numpy(),
                             nthreads=8)
    return g, o


def test_workload3_greedy_full_size(oracle):
    """B=64, k=8, V=128256 bf16 N(0, 2^2); draft = target argmax w.p. 0.85."""
    emitted = []
    for r in range(4):
        zt, toks = W.workload3(r, device=DEV)
        g, o = greedy_pair(oracle, zt, toks)
        compare_exact(g, o, GREEDY_KEYS)
        emitted.append(o["num_emitted"])
    mean = np.concatenate(emitted).mean()
    a = 0.85 + 0.15 / 128256
    assert abs(mean - (1 - a ** 9) / (1 - a)) < 0.5


def test_greedy_ties_lowest_index(oracle):
    B, K, V = 32, 4, 20000
    g = torch.Generator().manual_seed(1)
    z = (torch.randn((B, K + 1, V), generator=g) * 2).round() / 2  # many exact ties
    z[:, :, 100] = 9.0
    z[:, :, 7] = 9.0      # tie with index 100: 7 must win
    z[::2, :, 3] = -0.0
    zb = z.to(torch.bfloat16)
    toks = torch.full((B, K), 7, dtype=torch.int32)
    toks[::3, 1] = 100    # the later index of the tie is a mismatch
    kk = torch.randint(1, K + 1, (B,), generator=g, dtype=torch.int32)
    gg, o = greedy_pair(oracle, zb, toks, k_per_row=kk)
    compare_exact(gg, o, GREEDY_KEYS)
    assert np.all(o["out_tokens"][:, 0] == 7)


@pytest.mark.parametrize("dtype,V,pad", [(torch.float32, 33333, 0), (torch.bfloat16, 16385, 5),
                                         (torch.bfloat16, 3, 0)])
def test_greedy_draft_logits_and_strides(oracle, dtype, V, pad):
    B, K = 9, 5
    g = torch.Generator().manual_seed(V)
    zt = torch.randn((B, K + 1, V + pad), generator=g)
    zd = zt[:, :K] + 0.3 * torch.randn((B, K, V + pad), generator=g)
    zt_d = zt.to(dtype).to(DEV)[:, :, :V]
    zd_d = zd.to(dtype).to(DEV)[:, :, :V]
    out = sv.verify_greedy(zt_d, draft=zd_d)
    torch.cuda.synchronize()
    o = oracle.verify_greedy(W.host_logits(zt.to(dtype)[:, :, :V].contiguous()),
                             draft=W.host_logits(zd.to(dtype)[:, :, :V].contiguous()))
    compare_exact(out, o, GREEDY_KEYS)


def test_greedy_row_errors(oracle):
    B, K, V = 8, 3, 5000
    z = torch.randn((B, K + 1, V))
    z[1, 2, 9] = float("nan")
    z[2, 0, 9] = float("inf")
    z[3, 1, :] = float("-inf")
    toks = torch.randint(0, V, (B, K), dtype=torch.int32)
    toks[4, 2] = V
    toks[5, 0] = -1
    kk = torch.full((B,), K, dtype=torch.int32)
    kk[6] = 0
    kk[7] = 1
    z[7, 3, :] = float("nan")  # beyond k: ignored
    g, o = greedy_pair(oracle, z.to(torch.bfloat16), toks, k_per_row=kk)
    compare_exact(g, o, GREEDY_KEYS)
    assert list(o["row_status"]) == [0, 1, 1, 2, 4, 4, 8, 0]


# ------------------------------------------------------ greedy in one launch

def one_launch_matches(target, toks=None, draft=None, k_per_row=None, calls=3):
    """sv_verify_greedy_one_launch against sv_verify_greedy on the same
    inputs, bit for bit, over several calls on one state buffer; the state
    is all zero after every call."""
    two = sv.VerifyCall("greedy", target, draft, toks, k_per_row=k_per_row)
    one = sv.VerifyCall("greedy", target, draft, toks, k_per_row=k_per_row, one_launch=True)
    ref = {k: v.clone() for k, v in two.run().items()}
    for c in range(calls):
        out = one.run()
        torch.cuda.synchronize()
        for k in GREEDY_KEYS:
            assert torch.equal(out[k], ref[k]), (c, k)
        assert int(one.state.count_nonzero()) == 0, c
    return ref


def test_one_launch_greedy_full_size(oracle):
    """Workload 3 (B=64, k=8, V=128256) through the one-launch path, four
    rounds on one state buffer, against the oracle and the two launches."""
    zt, toks = W.workload3(0, device=DEV)
    one = sv.VerifyCall("greedy", zt, None, toks, one_launch=True)
    for r in range(4):
        z, t = W.workload3(r, device=DEV)
        zt.copy_(z)
        toks.copy_(t)
        out = one.run()
        torch.cuda.synchronize()
        o = oracle.verify_greedy(W.host_logits(z), draft_tokens=t.cpu().numpy(), nthreads=8)
        compare_exact(out, o, GREEDY_KEYS)
        assert int(one.state.count_nonzero()) == 0
    one_launch_matches(zt, toks)


def test_one_launch_greedy_edge_rows():
    """Ties (lowest index), +0 and -0 as one value, NaN, +inf, vectors of
    -inf or of NaN only, k_b outside [1, k], tokens out of range, draft
    logits instead of tokens, and a layout that takes the two launches."""
    B, K, V = 40, 5, 24576
    g = torch.Generator().manual_seed(3)
    z = (torch.randn((B, K + 1, V), generator=g) * 2).round() / 2
    z[:, :, 9000] = 9.0
    z[:, :, 4100] = 9.0          # tie across chunks: 4100 wins
    z[1, 2, :] = 0.0
    z[1, 2, 5] = -0.0            # the zeros tie: index 0
    z[2, 0, 8191] = float("nan")
    z[3, 1, 12288] = float("inf")
    z[4, 2, :] = float("-inf")
    z[5, 3, :] = float("nan")
    z[6, 0, :] = -1.0
    z[6, 0, 20000] = -0.5
    z[6, 0, 7] = -0.5            # a negative tie: 7
    zb = z.to(torch.bfloat16).to(DEV)
    toks = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    toks[:, 0] = 4100
    toks[7, 1] = V
    kk = torch.randint(1, K + 1, (B,), generator=g, dtype=torch.int32)
    kk[8], kk[9] = 0, K + 1
    kk[1:7] = K
    one_launch_matches(zb, toks.to(DEV), k_per_row=kk.to(DEV))
    one_launch_matches(zb, toks.to(DEV))
    zd = (zb[:, :K].float() + 0.25 * torch.randn((B, K, V), device=DEV)).to(torch.bfloat16)
    one_launch_matches(zb, draft=zd, k_per_row=kk.to(DEV))
    # unaligned vectors (V not a multiple of 8): the two launches, state untouched
    one_launch_matches(zb[:, :, :V - 3], toks.to(DEV))


@pytest.mark.parametrize("B,K,V", [(512, 8, 8192), (3, 1, 4096 * 40), (1000, 2, 4096),
                                   (7, 32, 12296)])
def test_one_launch_greedy_shapes(B, K, V):
    """Many rows with few chunks each (the row counters see many rows'
    chunks at once), few rows with many chunks (one counter sees them all),
    k at its limit, and a last chunk shorter than the others."""
    g = torch.Generator(device=DEV).manual_seed(B + K)
    zt = (torch.randn((B, K + 1, V), generator=g, device=DEV) * 2).to(torch.bfloat16)
    top = zt[:, :K].float().argmax(dim=2).to(torch.int32)
    toks = torch.where(torch.rand((B, K), generator=g, device=DEV) < 0.8, top,
                       torch.randint(0, V, (B, K), generator=g, device=DEV, dtype=torch.int32))
    one_launch_matches(zt, toks, calls=2)


def test_one_launch_greedy_in_a_replayed_graph():
    """The one-launch call captured once and replayed: every replay gives
    the eager result and leaves the state zero."""
    zt, toks = W.workload3(5, device=DEV, B=16)
    one = sv.VerifyCall("greedy", zt, None, toks, one_launch=True)
    ref = {k: v.clone() for k, v in sv.VerifyCall("greedy", zt, None, toks).run().items()}
    one.run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one.run()
    for r in range(4):
        for k in GREEDY_KEYS:
            one.outputs[k].fill_(-9)
        graph.replay()
        torch.cuda.synchronize()
        for k in GREEDY_KEYS:
            assert torch.equal(one.outputs[k], ref[k]), (r, k)
        assert int(one.state.count_nonzero()) == 0


# ------------------------------------------------------------------ rollback

def rollback_pair(oracle, lens, acc, kk, K, ps, MP, spare=8, capacity=None, pool_dims=None,
                  keep_pages=False, seed=0, top=None):
    kv = W.paged_kv(torch.as_tensor(lens, dtype=torch.int32), ps, MP, spare_pages=spare,
                    seed=seed)
    pt = kv.page_table.numpy().copy()
    free = kv.free_pages.numpy().copy()
    if capacity is not None:
        free = np.full(capacity, -1, np.int32)
        free[: min(spare, capacity)] = kv.free_pages.numpy()[: min(spare, capacity)]
    ftop = kv.free_top.numpy().copy() if top is None else np.array([top], np.int32)
    lens = np.asarray(lens, np.int32)
    acc = np.asarray(acc, np.int32)
    kk = np.asarray(kk, np.int32)
    pool = None
    if pool_dims is not None:
        L, H, D = pool_dims
        pool = np.random.default_rng(seed).integers(0, 60000, (kv.num_pages, L, 2, H, ps, D)
                                                    ).astype(np.uint16)
    # GPU
    d_len = torch.from_numpy(lens.copy()).to(DEV)
    d_pt = torch.from_numpy(pt.copy()).to(DEV)
    d_free = None if keep_pages else torch.from_numpy(free.copy()).to(DEV)
    d_top = None if keep_pages else torch.from_numpy(ftop.copy()).to(DEV)
    d_pool = None if pool is None else torch.from_numpy(pool.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    st = sv.kv_rollback(d_len, torch.from_numpy(acc).to(DEV), d_pt, ps, K,
                        k_per_row=torch.from_numpy(kk).to(DEV), free_pages=d_free,
                        free_top=d_top, kv_pool=d_pool, num_pages=kv.num_pages,
                        num_layers=0 if pool is None else pool_dims[0],
                        kv_heads=0 if pool is None else pool_dims[1],
                        head_dim=0 if pool is None else pool_dims[2])
    torch.cuda.synchronize()
    # oracle
    o_len, o_pt, o_free, o_top = lens.copy(), pt.copy(), free.copy(), ftop.copy()
    o_pool = None if pool is None else pool.copy()
    o_st = oracle.kv_rollback(o_len, acc, o_pt, ps, K, k_per_row=kk,
                              free_pages=None if keep_pages else o_free,
                              free_top=None if keep_pages else o_top,
                              free_capacity=free.size, kv_pool=o_pool,
                              num_layers=0 if pool is None else pool_dims[0],
                              kv_heads=0 if pool is None else pool_dims[1],
                              head_dim=0 if pool is None else pool_dims[2],
                              num_pages=kv.num_pages)
    assert np.array_equal(st.cpu().numpy(), o_st)
    assert np.array_equal(d_len.cpu().numpy(), o_len)
    assert np.array_equal(d_pt.cpu().numpy(), o_pt)
    if not keep_pages:
        assert np.array_equal(d_top.cpu().numpy(), o_top)
        assert np.array_equal(d_free.cpu().numpy(), o_free)
    if pool is not None:
        assert np.array_equal(d_pool.view(torch.int16).cpu().numpy().view(np.uint16), o_pool)
    return o_st, o_len


def test_rollback_workload3_rows(oracle):
    """64 rows, contexts U[512, 4096] after k+1 = 9 writes, page size 16,
    accepted counts from a greedy round."""
    rng = np.random.default_rng(3)
    B, K, ps = 64, 8, 16
    lens = rng.integers(512, 4097, B) + 9
    MP = int((lens.max() + ps - 1) // ps)
    zt, toks = W.workload3(0, device=DEV, B=B, V=4096)
    acc = sv.verify_greedy(zt, toks)["accepted"].cpu().numpy()
    st, new = rollback_pair(oracle, lens, acc, np.full(B, K), K, ps, MP, spare=32)
    assert np.all(st == 0) and np.array_equal(new, lens - (K - acc))


def test_rollback_small_pool_poison_exact(oracle):
    rng = np.random.default_rng(4)
    B, K, ps = 10, 5, 4
    lens = rng.integers(6, 40, B)
    kk = rng.integers(1, K + 1, B)
    acc = np.array([rng.integers(0, k + 1) for k in kk])
    rollback_pair(oracle, lens, acc, kk, K, ps, 12, spare=6, pool_dims=(3, 2, 8), seed=4)


@pytest.mark.parametrize("D", [8, 6])
def test_rollback_pool_bad_rows_overflow_and_many_rows(oracle, D):
    """Poisoning with the commit done by each row's last poisoning
    workgroup: 1100 rows (two tiles of the scan), rows with a bad accepted
    count or k, rows that roll nothing back, a free stack that overflows,
    and a pool without a free stack.  D = 8 takes the 16-byte stores, D = 6
    the one-value path."""
    rng = np.random.default_rng(7 + D)
    B, K, ps = 1100, 4, 4
    lens = rng.integers(5, 60, B)
    kk = rng.integers(1, K + 1, B)
    acc = np.array([rng.integers(0, k + 1) for k in kk])
    acc[::9] = kk[::9]  # nothing rolled back
    acc[3], acc[4], kk[5] = -1, kk[4] + 1, 0
    MP = 16
    st, _ = rollback_pair(oracle, lens, acc, kk, K, ps, MP, spare=40, pool_dims=(2, 3, D),
                          seed=8)
    assert (st == 0).sum() > B // 2
    st, _ = rollback_pair(oracle, lens, acc, kk, K, ps, MP, spare=0, capacity=30,
                          pool_dims=(2, 3, D), seed=9)
    assert (st & sv.ROW_FREE_OVERFLOW).any()
    rollback_pair(oracle, lens, acc, kk, K, ps, MP, keep_pages=True, pool_dims=(1, 2, D),
                  seed=10)


def test_rollback_keep_pages_overflow_and_bad_rows(oracle):
    rng = np.random.default_rng(5)
    B, K, ps = 300, 4, 8
    lens = rng.integers(5, 200, B)
    kk = rng.integers(1, K + 1, B)
    acc = np.array([rng.integers(0, k + 1) for k in kk])
    acc[3], acc[4], kk[5] = -1, kk[4] + 1, 0
    MP = 26
    rollback_pair(oracle, lens, acc, kk, K, ps, MP, keep_pages=True)
    st, _ = rollback_pair(oracle, lens, acc, kk, K, ps, MP, spare=0, capacity=20)
    assert (st & sv.ROW_FREE_OVERFLOW).any()
    st, _ = rollback_pair(oracle, lens, acc, kk, K, ps, MP, spare=0, capacity=20, top=25)
    assert ((st & sv.ROW_FREE_OVERFLOW) != 0).sum() > 0


def test_rollback_keep_pages_over_rounds(oracle):
    """Without a free stack pages past the length stay mapped; three rounds
    in a row on the same table, each checked against the oracle's."""
    rng = np.random.default_rng(8)
    B, K, ps = 300, 6, 16
    lens = (rng.integers(40, 400, B) + K + 1).astype(np.int32)
    MP = int((lens.max() + ps - 1) // ps)
    kv = W.paged_kv(torch.from_numpy(lens), ps, MP, seed=8)
    o_len, o_pt = lens.copy(), kv.page_table.numpy().copy()
    d_len, d_pt = torch.from_numpy(lens.copy()).to(DEV), kv.page_table.to(DEV)
    for r in range(3):
        kk = rng.integers(1, K + 1, B).astype(np.int32)
        acc = np.array([rng.integers(0, k + 1) for k in kk], np.int32)
        st = sv.kv_rollback(d_len, torch.from_numpy(acc).to(DEV), d_pt, ps, K,
                            k_per_row=torch.from_numpy(kk).to(DEV))
        o_st = oracle.kv_rollback(o_len, acc, o_pt, ps, K, k_per_row=kk)
        assert np.all(o_st == 0), "round %d" % r
        assert np.array_equal(st.cpu().numpy(), o_st)
        assert np.array_equal(d_len.cpu().numpy(), o_len)
        assert np.array_equal(d_pt.cpu().numpy(), o_pt)


def test_rollback_full_size_pool_poison(oracle):
    """The workload's real pool: 32 layers x 8 KV heads x 128 dims bf16, page
    size 16 (2 MiB per page), 64 rows of 512..4096 tokens.  The oracle gives
    the new lengths; every rolled-back slot must hold the poison pattern and
    nothing else may change."""
    rng = np.random.default_rng(6)
    B, K, ps, L, H, D = 64, 8, 16, 32, 8, 128
    lens = (rng.integers(512, 4097, B) + 9).astype(np.int32)
    MP = int((lens.max() + ps - 1) // ps)
    acc = rng.integers(0, K + 1, B).astype(np.int32)
    kv = W.paged_kv(torch.from_numpy(lens), ps, MP, spare_pages=16, seed=6)
    pool = torch.zeros((kv.num_pages, L, 2, H, ps, D), dtype=torch.bfloat16, device=DEV)
    pt0 = kv.page_table.numpy().copy()
    d_len = torch.from_numpy(lens.copy()).to(DEV)
    st = sv.kv_rollback(d_len, torch.from_numpy(acc).to(DEV), kv.page_table.to(DEV), ps, K,
                        free_pages=kv.free_pages.to(DEV), free_top=kv.free_top.to(DEV),
                        kv_pool=pool, num_layers=L, kv_heads=H, head_dim=D)
    torch.cuda.synchronize()
    o_len = lens.copy()
    o_st = oracle.kv_rollback(o_len, acc, pt0.copy(), ps, K)
    assert np.array_equal(st.cpu().numpy(), o_st) and np.array_equal(d_len.cpu().numpy(), o_len)
    pool16 = pool.view(torch.int16)
    poisoned = int((pool16 == -1).sum())
    assert poisoned == int((lens - o_len).sum()) * L * 2 * H * D
    for b in range(0, B, 7):
        for pos in range(o_len[b], lens[b]):
            page = pt0[b, pos // ps]
            assert bool((pool16[page, :, :, :, pos % ps, :] == -1).all())


@pytest.mark.parametrize("case", range(16))
def test_greedy_random_configuration_sweep(oracle, case):
    """Seeded random greedy shapes: V from 1 to 70000 (chunk tails of every
    kind), bf16 and fp32, padded strides, draft tokens or draft logits,
    per-row k, values rounded so that ties are common; bit-exact."""
    rng = np.random.default_rng(3000 + case)
    B, K = int(rng.integers(1, 20)), int(rng.integers(1, 10))
    V = int(rng.choice([1, 3, 8, 9, 100, 16383, 16384, 16385, 40000, 70000]))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    pad = int(rng.choice([0, 0, 1, 5, 8]))
    g = torch.Generator().manual_seed(4000 + case)
    base_t = ((torch.randn((B, K + 1, V + pad), generator=g) * 3).round() / 2).to(dtype)
    use_draft = rng.random() < 0.5
    base_d = ((torch.randn((B, K, V + pad), generator=g) * 3).round() / 2).to(dtype)
    toks = torch.from_numpy(rng.integers(0, V, (B, K)).astype(np.int32))
    top = torch.argmax(base_t[:, :K, :V].float(), dim=2).to(torch.int32)
    toks = torch.where(torch.from_numpy(rng.random((B, K)) < 0.7), top, toks)
    kk = None if rng.random() < 0.5 else torch.from_numpy(rng.integers(1, K + 1, B).astype(np.int32))
    d_t = base_t.to(DEV)[:, :, :V]
    d_d = base_d.to(DEV)[:, :, :V] if use_draft else None
    gg = sv.verify_greedy(d_t, None if use_draft else toks.to(DEV), d_d,
                          None if kk is None else kk.to(DEV))
    torch.cuda.synchronize()
    og = oracle.verify_greedy(W.host_logits(base_t[:, :, :V].contiguous()),
                              draft=W.host_logits(base_d[:, :, :V].contiguous()) if use_draft else None,
                              draft_tokens=None if use_draft else toks.numpy(),
                              k_per_row=None if kk is None else kk.numpy(), nthreads=8)
    compare_exact(gg, og, GREEDY_KEYS)


def test_pool_rollback_in_a_replayed_graph():
    """The rollback with a free stack and poisoning, captured once as a HIP
    graph (state restored inside the graph first) and replayed with other
    accepted counts each time: every replay equals the eager call on the
    same state.  The poisoning's per-row commit counters are zeroed by the
    scan in every call, so replays start clean."""
    rng = np.random.default_rng(11)
    B, K, ps, L, H, D = 96, 6, 8, 3, 2, 16
    lens = (rng.integers(20, 200, B) + K + 1).astype(np.int32)
    MP = int((lens.max() + ps - 1) // ps)
    kv = W.paged_kv(torch.from_numpy(lens), ps, MP, spare_pages=16, seed=11)
    init = [torch.from_numpy(lens).to(DEV), kv.page_table.to(DEV), kv.free_pages.to(DEV),
            kv.free_top.to(DEV),
            torch.zeros((kv.num_pages, L, 2, H, ps, D), dtype=torch.bfloat16, device=DEV)]

    def state():
        return [t.clone() for t in init]

    g, e = state(), state()
    g_acc = torch.zeros(B, dtype=torch.int32, device=DEV)
    e_acc = torch.zeros(B, dtype=torch.int32, device=DEV)

    def call(st, acc):
        return sv.RollbackCall(st[0], acc, st[1], ps, K, free_pages=st[2], free_top=st[3],
                               kv_pool=st[4], num_pages=kv.num_pages, num_layers=L, kv_heads=H,
                               head_dim=D)

    g_call, e_call = call(g, g_acc), call(e, e_acc)

    def graphed():
        for t, t0 in zip(g, init):
            t.copy_(t0)
        g_call.run()

    graphed()  # loads the kernels before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed()
    for r in range(4):
        acc = torch.from_numpy(rng.integers(0, K + 1, B).astype(np.int32)).to(DEV)
        g_acc.copy_(acc)
        e_acc.copy_(acc)
        for t, t0 in zip(e, init):
            t.copy_(t0)
        e_call.run()
        graph.replay()
        torch.cuda.synchronize()
        assert not e_call.row_status.any(), r
        assert torch.equal(g_call.row_status, e_call.row_status), r
        for a, b in zip(g, e):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), r
        assert int((g[4].view(torch.int16) == -1).sum()) == \
            int((torch.from_numpy(lens).to(DEV) - g[0]).sum()) * L * 2 * H * D, r
