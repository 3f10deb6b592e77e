"""Seeded cohorts shaped like WeNet-style Conformer encoders (no attention arithmetic here).

Value recipe (the same for every workload):

* q, k, v, the new chunk K/V and the pre-filled pool contents are N(0, 1);
* pos_bias_u and pos_bias_v are N(0, 0.02^2) (0.02 is the standard deviation);
* positional tables are sinusoidal embeddings of signed distances, projected by a seeded linear map
  W of shape [d_model, d_model] with entries N(0, 1/d_model), d_model = n_head * head_dim;
* every value is drawn in float32 and rounded once (round to nearest even) to the storage dtype.

Structure recipe: each stream gets ceil((cache + C) / block_size) pages, whose physical IDs come
from a seeded random permutation of the pool; table columns past a stream's pages hold -1. The
whole pool is filled with N(0, 1), so whatever a stream's table points at is its cached K/V.

Page layout: k_pool [num_blocks, n_kv_head, head_dim / 32, block_size, 32] (32-dim column blocks)
and v_pool [num_blocks, n_kv_head, head_dim, block_size] (V transposed inside each page).

Table layout: row r of a table with centre ``center`` holds the embedding of distance center - r.
A shared table has 2 (max_cache + C) - 1 rows. Per-row tables are packed as
[B, 2 (max_cache + C) - 1, H, D]; stream b uses the first 2 T_b - 1 rows, centred at T_b - 1.
Packed varlen tables put segment s's 2 L_s - 1 rows at row 2 cu_seqlens[s] (2 L_s rows reserved).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BF16 = torch.bfloat16
F32 = torch.float32


def sinusoidal_embedding(distances, d_model):
    """Sinusoidal encoding of signed integer distances, float64 [n, d_model].

    Column 2k is sin(d * w_k) and column 2k + 1 is cos(d * w_k) with w_k = 10000^(-2k / d_model).
    """
    d = torch.as_tensor(distances, dtype=torch.float64).reshape(-1, 1)
    k = torch.arange(0, d_model, 2, dtype=torch.float64)
    w = torch.exp(-math.log(10000.0) * k / d_model)
    out = torch.zeros(d.shape[0], d_model, dtype=torch.float64)
    out[:, 0::2] = torch.sin(d * w)
    out[:, 1::2] = torch.cos(d * w)
    return out


def relpos_projection(d_model, gen):
    """Seeded linear map [d_model, d_model] with N(0, 1/d_model) entries (drawn on the CPU)."""
    return torch.randn(d_model, d_model, generator=gen, dtype=torch.float32).double() / math.sqrt(d_model)


def embed_distances(distances, proj, n_head, head_dim):
    """Projected embeddings of the given distances, float64 [n, n_head, head_dim]."""
    e = sinusoidal_embedding(distances, n_head * head_dim) @ proj
    return e.reshape(-1, n_head, head_dim)


def descending_table(center, proj, n_head, head_dim):
    """Table of 2 center + 1 rows, row r holding the embedding of distance center - r."""
    dist = center - torch.arange(2 * center + 1)
    return embed_distances(dist, proj, n_head, head_dim)


def column_blocked(k_pool):
    """A K pool [N, Hk, S, D] (D a multiple of 32) re-laid out in 32-dim column blocks
    [N, Hk, D / 32, S, 32], the layout the kernels read: the same frames, another order."""
    n, hk, s, d = k_pool.shape
    return k_pool.reshape(n, hk, s, d // 32, 32).permute(0, 1, 3, 2, 4).contiguous()


def column_blocked_table(pos, per_row):
    """A positional table stored in 32-dim column blocks per head (a layout change only):
    [P, H, D] -> [H, D / 32, P, 32], or per row [B, P, H, D] -> [B, H, D / 32, P, 32]. Element
    (r, h, d) lands at (h, d // 32, r, d % 32)."""
    if per_row:
        B, P, H, D = pos.shape
        return pos.reshape(B, P, H, D // 32, 32).permute(0, 2, 3, 1, 4).contiguous()
    P, H, D = pos.shape
    return pos.reshape(P, H, D // 32, 32).permute(1, 2, 0, 3).contiguous()


def add_blocked_table(co):
    """Give a cohort the column-blocked copy of its positional table (co.pos stays row-major,
    as the oracle reads it)."""
    co.pos_cb = column_blocked_table(co.pos, co.per_row_pos)
    return co


def key_position_tables(proj, starts, width, n_head, head_dim):
    """Per-key tables (WeNet's convention): row j of table b is the projected sinusoid of the
    absolute position starts[b] + j; float64 [len(starts), width, n_head, head_dim]."""
    return torch.stack([embed_distances(torch.arange(s0, s0 + width), proj, n_head, head_dim)
                        for s0 in starts])


def use_key_position_tables(co, starts, per_row=True):
    """Replace a chunk cohort's tables by per-key tables whose keys start at absolute positions
    ``starts`` (one per stream; ``per_row=False`` takes starts[0] for one shared table), each of
    max_cache_seqlen + C rows."""
    B, C, H, D = co.q.shape
    width = co.max_cache_seqlen + C
    tabs = key_position_tables(co.meta["proj"], starts if per_row else starts[:1], width, H, D)
    co.pos = (tabs if per_row else tabs[0]).to(co.q.dtype).to(co.q.device)
    co.per_row_pos = per_row
    co.per_key_pos = True
    co.pos_cb = None
    return co


def _randn(shape, gen, device, dtype, std=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def linear_weights(n_out, d_in, *, seed=0, dtype=BF16, device="cpu", bias=True):
    """Seeded weights of a linear layer: W [n_out, d_in] with N(0, 1/d_in) entries (unit-variance
    outputs for unit-variance inputs) and, if ``bias``, b [n_out] with N(0, 0.02^2) entries.
    Drawn on the CPU. Returns (W, b or None)."""
    gen = torch.Generator().manual_seed(seed)
    w = (torch.randn(n_out, d_in, generator=gen) / math.sqrt(d_in)).to(dtype).to(device)
    b = (torch.randn(n_out, generator=gen) * 0.02).to(dtype).to(device) if bias else None
    return w, b


def activations(shape, *, seed=0, dtype=BF16, device="cpu"):
    """Seeded N(0, 1) activations of the given shape (drawn on the CPU)."""
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=gen).to(dtype).to(device)


@dataclass
class ChunkCohort:
    """One layer's inputs for a cohort of streams (all tensors on one device)."""

    q: torch.Tensor               # [B, C, H, D]
    k_new: torch.Tensor           # [B, C, Hk, D]
    v_new: torch.Tensor           # [B, C, Hk, D]
    k_pool: torch.Tensor          # [N, Hk, D / 32, S, 32] (32-dim column blocks)
    v_pool: torch.Tensor          # [N, Hk, D, S]
    block_tables: torch.Tensor    # [B, M] int32
    cache_seqlens: torch.Tensor   # [B] int32
    pos: torch.Tensor             # shared [P, H, D] or per-row [B, P, H, D]
    pos_bias_u: torch.Tensor      # [H, D]
    pos_bias_v: torch.Tensor      # [H, D]
    per_row_pos: bool
    block_size: int
    max_cache_seqlen: int
    meta: dict = field(default_factory=dict)
    per_key_pos: bool = False     # pos rows are keys (WeNet), not distances
    pos_cb: torch.Tensor = None   # the same table in 32-dim column blocks (add_blocked_table)

    @property
    def shape(self):
        B, C, H, D = self.q.shape
        return dict(B=B, C=C, H=H, Hk=self.k_new.shape[2], D=D, S=self.block_size,
                    N=self.k_pool.shape[0], M=self.block_tables.shape[1])


def make_chunk_cohort(B, H, D, C, block_size, cache_seqlens, *, Hk=None, dtype=BF16,
                      per_row_pos=False, num_blocks=None, pool_factor=1.25,
                      max_blocks_per_seq=None, seed=0, device="cpu", pos_noise=0.0,
                      max_cache_seqlen=None, proj_seed=None):
    """Draw one layer of a streaming cohort.

    cache_seqlens: per-stream cached frames before this chunk. The block table covers each
    stream's cached frames and its chunk. ``pos_noise`` > 0 adds N(0, pos_noise^2) to each per-row
    table so that rows' tables differ (a sensitivity aid for tests; 0 for the named workloads).
    """
    Hk = H if Hk is None else Hk
    cache = torch.as_tensor(cache_seqlens, dtype=torch.int64).reshape(-1)
    if cache.numel() != B:
        raise ValueError("cache_seqlens must have B entries")
    max_cache = int(cache.max()) if max_cache_seqlen is None else int(max_cache_seqlen)
    gen = torch.Generator().manual_seed(seed)
    pages = [(int(c) + C + block_size - 1) // block_size for c in cache]
    need = sum(pages)
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need))
    if num_blocks < need:
        raise ValueError("pool too small for the cohort")
    if max_blocks_per_seq is None:
        max_blocks_per_seq = (max_cache + C + block_size - 1) // block_size
    perm = torch.randperm(num_blocks, generator=gen)
    bt = torch.full((B, max_blocks_per_seq), -1, dtype=torch.int32)
    at = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[at: at + n].to(torch.int32)
        at += n

    dgen = torch.Generator(device=device).manual_seed(seed + 1)
    q = _randn((B, C, H, D), dgen, device, dtype)
    k_new = _randn((B, C, Hk, D), dgen, device, dtype)
    v_new = _randn((B, C, Hk, D), dgen, device, dtype)
    k_pool = column_blocked(_randn((num_blocks, Hk, block_size, D), dgen, device, dtype))
    v_pool = _randn((num_blocks, Hk, D, block_size), dgen, device, dtype)
    u = _randn((H, D), gen, "cpu", dtype, 0.02).to(device)
    w = _randn((H, D), gen, "cpu", dtype, 0.02).to(device)
    proj_gen = gen if proj_seed is None else torch.Generator().manual_seed(proj_seed)
    proj = relpos_projection(H * D, proj_gen)
    center = max_cache + C - 1
    full = descending_table(center, proj, H, D)             # [2 center + 1, H, D]
    if per_row_pos:
        P = 2 * center + 1
        pos = torch.zeros((B, P, H, D), dtype=dtype)
        for b in range(B):
            T = int(cache[b]) + C
            lo = center - (T - 1)                            # distance T - 1 sits at row lo of full
            rows = full[lo: lo + 2 * T - 1]
            if pos_noise > 0:
                rows = rows + pos_noise * torch.randn((2 * T - 1, H, D), generator=gen,
                                                      dtype=torch.float32).double()
            pos[b, : 2 * T - 1] = rows.to(dtype)
        pos = pos.to(device)
    else:
        pos = full.to(dtype).to(device)
    return ChunkCohort(q=q, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool,
                       block_tables=bt.to(device), cache_seqlens=cache.to(torch.int32).to(device),
                       pos=pos, pos_bias_u=u, pos_bias_v=w, per_row_pos=per_row_pos,
                       block_size=block_size, max_cache_seqlen=max_cache,
                       meta=dict(pages=pages, seed=seed, proj=proj))


@dataclass
class VarlenCohort:
    q: torch.Tensor            # [total, H, D]
    k: torch.Tensor            # [total, Hk, D]
    v: torch.Tensor            # [total, Hk, D]
    cu_seqlens: torch.Tensor   # [S + 1] int32
    pos: torch.Tensor          # [2 total, H, D]
    pos_bias_u: torch.Tensor   # [H, D]
    pos_bias_v: torch.Tensor   # [H, D]
    lengths: list
    meta: dict = field(default_factory=dict)


def make_varlen_cohort(lengths, H, D, *, Hk=None, dtype=BF16, seed=0, device="cpu"):
    """Packed, gapless utterances with one relative-position table per utterance."""
    Hk = H if Hk is None else Hk
    lengths = [int(x) for x in lengths]
    total = sum(lengths)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    gen = torch.Generator().manual_seed(seed)
    dgen = torch.Generator(device=device).manual_seed(seed + 1)
    q = _randn((total, H, D), dgen, device, dtype)
    k = _randn((total, Hk, D), dgen, device, dtype)
    v = _randn((total, Hk, D), dgen, device, dtype)
    u = _randn((H, D), gen, "cpu", dtype, 0.02).to(device)
    w = _randn((H, D), gen, "cpu", dtype, 0.02).to(device)
    proj = relpos_projection(H * D, gen)
    n_rows = 2 * total
    pos = torch.zeros((n_rows, H, D), dtype=torch.float64)
    lmax = max(lengths) if lengths else 1
    full = descending_table(max(lmax - 1, 0), proj, H, D)
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        row0 = 2 * int(cu[s])
        lo = (lmax - 1) - (n - 1)
        pos[row0: row0 + 2 * n - 1] = full[lo: lo + 2 * n - 1]
    return VarlenCohort(q=q, k=k, v=v, cu_seqlens=cu.to(device), pos=pos.to(dtype).to(device),
                        pos_bias_u=u, pos_bias_v=w, lengths=lengths, meta=dict(seed=seed, proj=proj))


# The five named workloads: Conformer-shaped streaming cohorts and one packed offline batch.
WORKLOADS = {
    0: dict(kind="chunk", name="tiny fp32 oracle check", B=2, H=4, D=64, C=16, block_size=16,
            cache=64, dtype=F32, num_blocks=32, max_blocks_per_seq=8, n_layers=1),
    1: dict(kind="chunk", name="d_model 256 streaming cohort", B=64, H=4, D=64, C=16,
            block_size=16, cache=256, dtype=BF16, pool_factor=1.25, max_blocks_per_seq=512,
            n_layers=12),
    2: dict(kind="chunk", name="d_model 512 large cohort", B=256, H=8, D=64, C=16, block_size=16,
            cache=512, dtype=BF16, pool_factor=1.25, max_blocks_per_seq=512, n_layers=12),
    3: dict(kind="chunk", name="ragged cohort, per-row tables", B=128, H=8, D=64, C=16,
            block_size=32, cache="ragged", cache_max=1024, new_fraction=0.1, dtype=BF16,
            pool_factor=1.25, max_blocks_per_seq=512, per_row_pos=True, n_layers=1),
    4: dict(kind="varlen", name="offline packed varlen", n_seqs=32, len_lo=100, len_hi=1500,
            H=8, D=64, dtype=BF16, n_layers=1),
}


def ragged_cache(B, cache_max, new_fraction, seed, step=16):
    """Cache lengths uniform over {0, step, ..., cache_max}; a seeded subset of rows set to 0."""
    gen = torch.Generator().manual_seed(seed + 7)
    c = step * torch.randint(0, cache_max // step + 1, (B,), generator=gen)
    n_new = int(new_fraction * B)
    c[torch.randperm(B, generator=gen)[:n_new]] = 0
    return c


def make_config(index, layer=0, seed=0, device="cpu"):
    """Inputs of one layer of a named workload."""
    cfg = WORKLOADS[index]
    s = 1_000_003 * seed + 1009 * index + 7919 * layer
    if cfg["kind"] == "varlen":
        gen = torch.Generator().manual_seed(s + 3)
        lengths = torch.randint(cfg["len_lo"], cfg["len_hi"] + 1, (cfg["n_seqs"],), generator=gen)
        return make_varlen_cohort(lengths.tolist(), cfg["H"], cfg["D"], dtype=cfg["dtype"],
                                  seed=s, device=device)
    if cfg["cache"] == "ragged":
        cache = ragged_cache(cfg["B"], cfg["cache_max"], cfg["new_fraction"], s)
        max_cache = cfg["cache_max"]
    else:
        cache = torch.full((cfg["B"],), cfg["cache"], dtype=torch.int64)
        max_cache = cfg["cache"]
    return make_chunk_cohort(cfg["B"], cfg["H"], cfg["D"], cfg["C"], cfg["block_size"], cache,
                             dtype=cfg["dtype"], per_row_pos=cfg.get("per_row_pos", False),
                             num_blocks=cfg.get("num_blocks"),
                             pool_factor=cfg.get("pool_factor", 1.25),
                             max_blocks_per_seq=cfg.get("max_blocks_per_seq"), seed=s,
                             device=device, max_cache_seqlen=max_cache)
