"""Helpers for the GPU parity tests: host copies, poisoning of unused storage, compaction of a
sample of streams, and the oracle run on exactly the tensors the GPU saw."""

import numpy as np
import torch

import oracle

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def host64(t):
    """Exact float64 host copy of a bf16 / fp32 tensor."""
    return t.detach().cpu().double().numpy()


def bits(t):
    """Integer view of the storage, for bit-exact comparisons."""
    it = {torch.bfloat16: torch.int16, torch.float32: torch.int32}[t.dtype]
    return t.detach().cpu().contiguous().view(it).numpy()


def live_slot_mask(co):
    """Boolean [N, S] mask of the pool slots that hold some stream's frames [0, cache + C)."""
    bt = co.block_tables.cpu().numpy()
    cs = co.cache_seqlens.cpu().numpy()
    N, S = co.k_pool.shape[0], co.block_size
    C = co.q.shape[1]
    live = np.zeros((N, S), dtype=bool)
    for b in range(bt.shape[0]):
        for t in range(int(cs[b]) + C):
            live[bt[b, t // S], t % S] = True
    return live


def poison(co):
    """NaN everything the path must never read: pool slots no stream owns and per-row table rows
    past each stream's 2 T_b - 1."""
    live = torch.from_numpy(live_slot_mask(co)).to(co.k_pool.device)
    nan = float("nan")
    co.k_pool.masked_fill_(~live[:, None, None, :, None], nan)     # [N, Hk, D/32, S, 32]
    co.v_pool.masked_fill_(~live[:, None, None, :], nan)
    if co.per_row_pos:
        C = co.q.shape[1]
        cs = co.cache_seqlens.cpu().numpy()
        for b in range(len(cs)):
            co.pos[b, 2 * (int(cs[b]) + C) - 1:] = nan
    return co


def compact(co, streams):
    """The sub-cohort of `streams` with only their pages, renumbered 0..n-1 (block relabelling
    does not change the result). Returns host float64 arrays for the oracle."""
    C = co.q.shape[1]
    S = co.block_size
    bt = co.block_tables.cpu().numpy()[streams]
    cs = co.cache_seqlens.cpu().numpy()[streams]
    used = []
    for r, c in zip(bt, cs):
        used.extend(int(x) for x in r[: (int(c) + C + S - 1) // S])
    ids = np.array(sorted(set(used)))
    remap = {int(x): i for i, x in enumerate(ids)}
    bt2 = np.full_like(bt, -1)
    for r in range(bt.shape[0]):
        n = (int(cs[r]) + C + S - 1) // S
        bt2[r, :n] = [remap[int(x)] for x in bt[r, :n]]
    idx = torch.from_numpy(ids).to(co.k_pool.device)
    sel = torch.as_tensor(streams, device=co.q.device)
    return dict(
        q=host64(co.q[sel]), k_new=host64(co.k_new[sel]), v_new=host64(co.v_new[sel]),
        k_pool=host64(co.k_pool.index_select(0, idx)), v_pool=host64(co.v_pool.index_select(0, idx)),
        bt=bt2, cs=cs, pos=host64(co.pos[sel] if co.per_row_pos else co.pos),
        u=host64(co.pos_bias_u), w=host64(co.pos_bias_v), per_row=co.per_row_pos,
        per_key=getattr(co, "per_key_pos", False))


def oracle_chunk(co, streams=None, chunk_lens=None):
    """Oracle append + attention for `streams` (default all) of a cohort whose pools have not been
    appended to yet (chunk_lens: optional real frames per stream of the whole cohort). Returns
    float64 [len(streams), C, H, D]."""
    if streams is None:
        streams = list(range(co.q.shape[0]))
    h = compact(co, streams)
    lens = None if chunk_lens is None else np.asarray(chunk_lens)[streams]
    kp, vp = oracle.paged_kv_append(h["k_pool"], h["v_pool"], h["k_new"], h["v_new"], h["bt"], h["cs"],
                                    lens)
    return oracle.chunk_relpos_attn(h["q"], kp, vp, h["bt"], h["cs"], h["pos"], h["u"], h["w"],
                                    per_row_pos=h["per_row"], chunk_lens=lens,
                                    per_key_pos=h["per_key"])


def poison_padding(co, chunk_lens):
    """NaN the frames a stream's chunk does not have: its padded rows of q, k_new and v_new, and
    the pool slots they would have been appended to."""
    C = co.q.shape[1]
    S = co.block_size
    bt = co.block_tables.cpu().numpy()
    cs = co.cache_seqlens.cpu().numpy()
    nan = float("nan")
    for b, n in enumerate(chunk_lens):
        n = int(n)
        co.q[b, n:] = nan
        co.k_new[b, n:] = nan
        co.v_new[b, n:] = nan
        for t in range(int(cs[b]) + n, int(cs[b]) + C):
            blk, slot = int(bt[b, t // S]), t % S
            co.k_pool[blk, :, :, slot, :] = nan
            co.v_pool[blk, :, :, slot] = nan
    return co


def max_err(gpu, ref):
    g = gpu.detach().cpu().double().numpy() if torch.is_tensor(gpu) else gpu
    assert np.isfinite(g).all(), "non-finite output"
    return float(np.abs(g - ref).max())


def ring_tables(co, seed, wraps=3):
    """Window starts and ring-rotated table rows for a cohort: stream b's window starts at
    k_b S (k_b drawn in [0, wraps M)) and its row is rotated so that absolute position
    k_b S + t finds the block the plain row gives frame t. Returns (starts as a list, ring
    tables on the cohort's device)."""
    rng = np.random.default_rng(seed)
    bt = co.block_tables.cpu().numpy()
    M = bt.shape[1]
    S = co.block_size
    ring = np.full_like(bt, -1)
    starts = []
    for b in range(bt.shape[0]):
        k = int(rng.integers(0, wraps * M))
        starts.append(k * S)
        for i in range(M):
            ring[b, (k + i) % M] = bt[b, i]
    return starts, torch.from_numpy(ring).to(co.block_tables.device)
