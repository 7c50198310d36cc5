"""Seeded synthetic inputs for GQLA decode (shared by tests, bench and smoke).

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle consume what it
returns, so it must stay free of anything either side computes.

Workloads (shapes follow the GQLA pages' running examples):

* ``tiny``    -- 16 heads, 2 groups, latent 64 + rope 16, nope/v 32, batch 2,
                 context 256 (small enough for the oracle in seconds).
* ``llama3_8b`` -- LLaMA-3-8B-shaped TransGQLA layer: 32 heads, 8 groups,
                 latent 512 + rope 64, nope/v 128, batch 32, context 2048.
* ``dsv3``    -- DeepSeek-V3-shaped GQLA: 128 heads, 8 groups, latent 512 +
                 rope 64, nope/v 128, batch 64, context 4096.
* ``dsv3_ragged`` -- same dims, batch 16, contexts log-uniform in
                 [1024, 32768], random page table.

Recipe: one ``torch.Generator`` seeded per case; draw order is context
lengths, page permutation, W_UK, W_UV, latent page pool (c and k_rope
together, one N(0,1) draw per page row), q_nope, q_rope.  Activations are
N(0,1); weights are N(0, std = 1/sqrt(r)).  Every tensor is rounded to bf16
(round-to-nearest-even, torch's conversion) unless ``dtype=torch.float32``.
Unused page slots and the spare "poison" page are NaN when ``poison`` is set
(they must never be read), else 0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK_SIZE = 64

CONFIGS = {
    "tiny":        dict(h_q=16, g=2, r=64, d_R=16, d_nope=32, d_v=32, batch=2, ctx=256),
    "llama3_8b":   dict(h_q=32, g=8, r=512, d_R=64, d_nope=128, d_v=128, batch=32, ctx=2048),
    "dsv3":        dict(h_q=128, g=8, r=512, d_R=64, d_nope=128, d_v=128, batch=64, ctx=4096),
    "dsv3_ragged": dict(h_q=128, g=8, r=512, d_R=64, d_nope=128, d_v=128, batch=16,
                        ctx=("loguniform", 1024, 32768)),
    # the pages' other ridge-optimal GQA configuration, (g, s_q) = (4, 1): 32 heads per
    # group, 2176 B per token in the expanded cache
    "dsv3_g4":     dict(h_q=128, g=4, r=512, d_R=64, d_nope=128, d_v=128, batch=64, ctx=4096),
}


@dataclass
class Case:
    """One decode problem: dims, weights, paged latent cache, queries (CPU tensors)."""
    h_q: int
    g: int
    r: int
    d_R: int
    d_nope: int
    d_v: int
    s_q: int
    bs: int
    seqlens: torch.Tensor          # int32 [B]
    block_table: torch.Tensor      # int32 [B, max_blocks]; unused entries -> poison page
    pages: torch.Tensor            # [n_pages, bs, r + d_R]; last page is the poison page
    w_uk: torch.Tensor             # [g, r, d_nope]
    w_uv: torch.Tensor             # [g, r, d_v]
    q_nope: torch.Tensor           # [B, s_q, h_q, d_nope]
    q_rope: torch.Tensor           # [B, s_q, h_q, d_R]
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.seqlens.numel())

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def dims(self) -> dict:
        return dict(h_q=self.h_q, g=self.g, r=self.r, d_R=self.d_R, d_nope=self.d_nope,
                    d_v=self.d_v, s_q=self.s_q, bs=self.bs)


def draw_seqlens(gen: torch.Generator, batch: int, ctx) -> torch.Tensor:
    """Uniform context, or log-uniform in [lo, hi]: round(exp(U(ln lo, ln hi))) clamped."""
    if isinstance(ctx, (tuple, list)) and ctx[0] == "loguniform":
        lo, hi = ctx[1], ctx[2]
        u = torch.rand(batch, generator=gen, dtype=torch.float64)
        lens = torch.round(torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
        return lens.clamp(lo, hi).to(torch.int32)
    if isinstance(ctx, (tuple, list)):
        return torch.tensor(list(ctx), dtype=torch.int32)
    return torch.full((batch,), int(ctx), dtype=torch.int32)


def make_case(h_q, g, r, d_R, d_nope, d_v, batch, ctx, s_q, seed, *, table="identity",
              poison=False, dtype=torch.bfloat16, bs=BLOCK_SIZE, q_scale=1.0) -> Case:
    gen = torch.Generator().manual_seed(seed)
    seqlens = draw_seqlens(gen, batch, ctx)
    if int(seqlens.min()) < s_q:
        raise ValueError("every context must hold at least s_q tokens")
    nblk = [(int(L) + bs - 1) // bs for L in seqlens]
    used = sum(nblk)
    n_pages = used + 1                                   # + the poison page
    max_blocks = max(nblk)
    perm = torch.randperm(used, generator=gen) if table == "random" else torch.arange(used)
    block_table = torch.full((batch, max_blocks), n_pages - 1, dtype=torch.int32)
    k = 0
    for b, n in enumerate(nblk):
        block_table[b, :n] = perm[k:k + n].to(torch.int32)
        k += n
    w_std = 1.0 / math.sqrt(r)
    w_uk = torch.randn(g, r, d_nope, generator=gen) * w_std
    w_uv = torch.randn(g, r, d_v, generator=gen) * w_std
    pages = torch.randn(n_pages, bs, r + d_R, generator=gen)
    q_nope = torch.randn(batch, s_q, h_q, d_nope, generator=gen) * q_scale
    q_rope = torch.randn(batch, s_q, h_q, d_R, generator=gen) * q_scale
    fill = float("nan") if poison else 0.0
    pages[n_pages - 1] = fill
    for b, n in enumerate(nblk):
        tail = int(seqlens[b]) - (n - 1) * bs          # used slots of the last page
        if tail < bs:
            pages[int(block_table[b, n - 1]), tail:] = fill
    cast = (lambda t: t.to(dtype))
    return Case(h_q=h_q, g=g, r=r, d_R=d_R, d_nope=d_nope, d_v=d_v, s_q=s_q, bs=bs,
                seqlens=seqlens, block_table=block_table, pages=cast(pages),
                w_uk=cast(w_uk), w_uv=cast(w_uv), q_nope=cast(q_nope), q_rope=cast(q_rope),
                meta=dict(seed=seed, table=table, poison=poison))


def config_case(name: str, s_q: int, *, seed=None, batch=None, ctx=None, table=None,
                poison=False, dtype=torch.bfloat16) -> Case:
    """A case shaped like one of CONFIGS (batch/ctx may be overridden for smaller runs)."""
    c = dict(CONFIGS[name])
    base_seed = {"tiny": 1000, "llama3_8b": 1001, "dsv3": 1002, "dsv3_ragged": 1004, "dsv3_g4": 1005}[name]
    if table is None:
        table = "random" if name == "dsv3_ragged" else "identity"
    return make_case(c["h_q"], c["g"], c["r"], c["d_R"], c["d_nope"], c["d_v"],
                     batch if batch is not None else c["batch"],
                     ctx if ctx is not None else c["ctx"], s_q,
                     seed if seed is not None else base_seed + 10 * s_q,
                     table=table, poison=poison, dtype=dtype)


def random_partials(n_splits_per_seq, s_q, h_q, d_v, seed, empty_frac=0.0):
    """Random fp32 split partials (normalized outputs + lse) for testing the merge alone."""
    gen = torch.Generator().manual_seed(seed)
    offsets = [0]
    for n in n_splits_per_seq:
        offsets.append(offsets[-1] + int(n))
    total = offsets[-1]
    part_out = torch.randn(total, s_q, h_q, d_v, generator=gen)
    part_lse = torch.randn(total, s_q, h_q, generator=gen) * 4.0 + 2.0
    if empty_frac > 0:
        mask = torch.rand(total, s_q, h_q, generator=gen) < empty_frac
        part_lse[mask] = float("-inf")
        part_out[mask] = 0.0
    return part_out, part_lse, torch.tensor(offsets, dtype=torch.int32)


def sparse_indices(seqlens, g, topk, seed, *, invalid_frac=0.0, dup_frac=0.0):
    """Per-group token selections for the sparse decode: int32 [batch][g][topk].

    Recipe: for each (sequence b, group G), independently, min(topk, L_b)
    distinct positions drawn uniformly from [0, L_b) in random order (a
    stand-in for an indexer's top-k, which the pages leave open); slots past
    L_b are -1.  With ``invalid_frac`` that share of the entries is replaced by
    -1 or by a position at or past L_b, and with ``dup_frac`` that share by a
    copy of another entry of the same list.
    """
    gen = torch.Generator().manual_seed(seed)
    batch = len(seqlens)
    idx = torch.full((batch, g, topk), -1, dtype=torch.int32)
    for b in range(batch):
        L = int(seqlens[b])
        n = min(topk, L)
        for G in range(g):
            if n > 0:
                idx[b, G, :n] = torch.randperm(L, generator=gen)[:n].to(torch.int32)
            if dup_frac > 0 and n > 1:
                m = torch.rand(topk, generator=gen) < dup_frac
                src = torch.randint(0, n, (topk,), generator=gen)
                idx[b, G][m] = idx[b, G][src[m]]
            if invalid_frac > 0:
                m = torch.rand(topk, generator=gen) < invalid_frac
                bad = torch.where(torch.rand(topk, generator=gen) < 0.5,
                                  torch.full((topk,), -1),
                                  L + torch.randint(0, 1 << 20, (topk,), generator=gen))
                idx[b, G][m] = bad[m].to(torch.int32)
    return idx
