"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random inputs: logits, draft tokens that stand in for a
draft model's choices, per-row parameters and KV page tables.  It holds none
of the verification arithmetic, so it can feed both the GPU library and the
CPU oracle.  Every generator is keyed by (seed, workload, round) through its
own torch.Generator; the same call on the same device gives the same bits.
Logits are drawn in fp32 and rounded to bf16 once (round-to-nearest-even).

The workloads stand in for the pages' models and datasets, which are not
available: a 7B target with a 1.5B draft on CNN/DailyMail, GSM8K and code
([FS] §4.1-§4.2), and a 7B self-speculative model on mixed code/chat traffic
([SSD] §4.6).  Vocabulary sizes 32000, 128256 and 151936 and draft lengths
2..8 bracket what those models use.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_TAGS = {"w1": 1, "w2": 2, "w3": 3, "w4": 4, "w5": 5, "kv": 6, "misc": 7}


def generator(seed: int, tag: str, round_idx: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + _TAGS[tag] * 7919 + int(round_idx) * 104729)
                  & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> host numpy uint16 bit patterns (what the oracle takes)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host_logits(t: torch.Tensor) -> np.ndarray:
    """Logits in the form the oracle takes: float32 array or bf16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    assert t.dtype == torch.float32
    return t.detach().contiguous().cpu().numpy()


@dataclass
class SampleInputs:
    target: torch.Tensor        # [B, k_max+1, V] fp32 or bf16
    draft: torch.Tensor         # [B, k_max, V]
    temperature: torch.Tensor   # [B] float32
    top_p: Optional[torch.Tensor]  # [B] float32 or None
    k_per_row: Optional[torch.Tensor] = None  # [B] int32 or None
    draft_tokens: Optional[torch.Tensor] = None  # [B, k_max] int32


def _normal(shape, g, device, std=1.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def workload1(round_idx=0, seed=0, device="cpu", B=1, k=4, V=32000) -> SampleInputs:
    """fp32; target N(0, 3^2), draft = target + N(0, 1); T = 1; no top-p.
    Draft tokens are drawn by the draft sampler (draw 2), not here."""
    g = generator(seed, "w1", round_idx, device)
    zt = _normal((B, k + 1, V), g, device, 3.0)
    zd = zt[:, :k] + _normal((B, k, V), g, device, 1.0)
    T = torch.ones(B, dtype=torch.float32, device=device)
    return SampleInputs(zt.contiguous(), zd.contiguous(), T, None)


def workload2(round_idx=0, seed=0, device="cpu", B=32, k=5, V=32000) -> SampleInputs:
    """bf16; target N(0, 3^2) with 1% of entries raised by 8; draft =
    0.7*target + N(0, 1.5^2); T = 0.8 on both sides; no top-p."""
    g = generator(seed, "w2", round_idx, device)
    zt = _normal((B, k + 1, V), g, device, 3.0)
    boost = torch.rand((B, k + 1, V), generator=g, device=device) < 0.01
    zt = zt + 8.0 * boost.float()
    zd = 0.7 * zt[:, :k] + _normal((B, k, V), g, device, 1.5)
    T = torch.full((B,), 0.8, dtype=torch.float32, device=device)
    return SampleInputs(zt.to(torch.bfloat16), zd.to(torch.bfloat16), T, None)


def workload3(round_idx=0, seed=0, device="cpu", B=64, k=8, V=128256):
    """Greedy: bf16 target N(0, 2^2) at k+1 positions; each draft token is the
    target's top token with probability 0.85, else uniform over V.  Returns
    (target bf16 [B,k+1,V], draft_tokens int32 [B,k]).  The top token is found
    with torch.argmax on the rounded values; only the draft inputs depend on
    it."""
    g = generator(seed, "w3", round_idx, device)
    zt = _normal((B, k + 1, V), g, device, 2.0).to(torch.bfloat16)
    top = torch.argmax(zt[:, :k].float(), dim=2).to(torch.int32)
    rnd = torch.randint(0, V, (B, k), generator=g, device=device, dtype=torch.int32)
    keep = torch.rand((B, k), generator=g, device=device) < 0.85
    toks = torch.where(keep, top, rnd).to(torch.int32)
    return zt.contiguous(), toks.contiguous()


def workload4(round_idx=0, seed=0, device="cpu", B=256, k=6, V=151936) -> SampleInputs:
    """bf16 Zipf-shaped target: per (row, position) the sorted log-weights
    -1.1*ln(rank) + N(0, 0.5^2), randomly permuted over the vocabulary; draft
    = target + N(0, 1); T = 1 and top-p 0.9 on both sides."""
    g = generator(seed, "w4", round_idx, device)
    n = B * (k + 1)
    ranks = torch.arange(1, V + 1, device=device, dtype=torch.float32)
    base = -1.1 * torch.log(ranks)
    out = torch.empty((n, V), dtype=torch.float32, device=device)
    chunk = max(1, (1 << 26) // V)  # bound temporary memory
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        vals = base.unsqueeze(0) + _normal((e - s, V), g, device, 0.5)
        perm = torch.rand((e - s, V), generator=g, device=device).argsort(dim=1)
        out[s:e] = torch.gather(vals, 1, perm)
    zt = out.view(B, k + 1, V)
    zd = zt[:, :k] + _normal((B, k, V), g, device, 1.0)
    T = torch.ones(B, dtype=torch.float32, device=device)
    P = torch.full((B,), 0.9, dtype=torch.float32, device=device)
    return SampleInputs(zt.to(torch.bfloat16), zd.to(torch.bfloat16), T, P)


@dataclass
class Workload5Rows:
    temperature: torch.Tensor  # [B] U[0.1, 1]
    sigma: torch.Tensor        # [B] U[0.3, 2]
    kv_len0: torch.Tensor      # [B] int32 U[512, 4096]


def workload5_rows(seed=0, B=512, device="cpu", ctx_lo=512, ctx_hi=4096) -> Workload5Rows:
    g = generator(seed, "w5", 0, device)
    T = 0.1 + 0.9 * torch.rand(B, generator=g, device=device)
    sig = 0.3 + 1.7 * torch.rand(B, generator=g, device=device)
    ctx = torch.randint(ctx_lo, ctx_hi + 1, (B,), generator=g, device=device, dtype=torch.int32)
    return Workload5Rows(T.float(), sig.float(), ctx)


def workload5(round_idx, rows: Workload5Rows, k_per_row: torch.Tensor, k_max=8,
              seed=0, device="cpu", V=128256) -> SampleInputs:
    """Ragged batch: bf16 target N(0, 3^2); draft = target + N(0, sigma_b^2)
    with a per-row sigma; per-row temperature; no top-p.  Positions beyond a
    row's k are filled too (the verifier must ignore them)."""
    B = rows.temperature.shape[0]
    g = generator(seed, "w5", round_idx + 1, device)
    zt = _normal((B, k_max + 1, V), g, device, 3.0)
    zd = zt[:, :k_max] + _normal((B, k_max, V), g, device, 1.0) * rows.sigma.to(device).view(B, 1, 1)
    return SampleInputs(zt.to(torch.bfloat16), zd.to(torch.bfloat16),
                        rows.temperature.to(device), None,
                        k_per_row.to(device=device, dtype=torch.int32))


def gumbel_draft_tokens(draft: torch.Tensor, temperature: torch.Tensor, seed: int,
                        round_idx: int) -> torch.Tensor:
    """Stand-in for a draft model's sampled choices when no draft sampler is
    run: x_i = argmax(z_i / T + Gumbel noise), i.e. a sample of the untruncated
    temperature softmax of the draft logits, drawn with torch's generator."""
    g = generator(seed, "misc", round_idx, draft.device)
    B, K, V = draft.shape
    toks = torch.empty((B, K), dtype=torch.int32, device=draft.device)
    for b in range(B):
        u = torch.rand((K, V), generator=g, device=draft.device).clamp_(1e-20, 1.0)
        gum = -torch.log(-torch.log(u))
        toks[b] = torch.argmax(draft[b].float() / temperature[b].float() + gum, dim=1).to(torch.int32)
    return toks


@dataclass
class PagedKV:
    page_table: torch.Tensor  # [B, max_pages] int32, -1 unmapped
    free_pages: torch.Tensor  # [capacity] int32 stack storage
    free_top: torch.Tensor    # [1] int32
    num_pages: int


def paged_kv(kv_len: torch.Tensor, page_size: int, max_pages: int, spare_pages: int = 0,
             seed=0, device="cpu") -> PagedKV:
    """A page table mapping each row's first ceil(len/page_size) logical pages
    to distinct physical pages (shuffled), plus a free stack holding the
    physical pages nobody maps, with room for every page in the pool."""
    B = kv_len.shape[0]
    used = ((kv_len.cpu().long() + page_size - 1) // page_size)
    assert int(used.max()) <= max_pages
    total_used = int(used.sum())
    num_pages = total_used + spare_pages
    g = generator(seed, "kv", 0, "cpu")
    phys = torch.randperm(num_pages, generator=g).to(torch.int32)
    pt = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        n = int(used[b])
        pt[b, :n] = phys[off:off + n]
        off += n
    free = torch.full((num_pages,), -1, dtype=torch.int32)
    free[:spare_pages] = phys[total_used:]
    top = torch.tensor([spare_pages], dtype=torch.int32)
    return PagedKV(pt.to(device), free.to(device), top.to(device), num_pages)
