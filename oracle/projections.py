"""Plain float64 definitions of the GEMMs either side of the paged attention (test
infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use this
module. It shares no code with the HIP path and imports nothing from it.

Sources, cited by page title and section (OASR documentation):

* "ASR Engine", section 9 "Performance Considerations" (the streaming graph ladder): the
  positional projection of the relative-position table is sized by the cache rung - one
  projected row per table row.
* "Model Layer", "Three optional encoder declarations" (fixed_attention_window): a uniform
  cache_seqlens lets one shared Transformer-XL table serve the cohort; otherwise the positional
  projection runs per row.
* "Scheduler", section 4.3 "Heterogeneous-offset batching": the positional embedding is built per
  stream from its offset when offsets differ.
* "ASR Engine", section 9, and "Model Layer", the Nemotron encoder notes: WeNet's convention
  takes absolute positions starting at offset - cache_seqlens per row.
* "Model Layer", the decoder notes (WeNet's linear_q / linear_k / linear_v / linear_out over the
  shared attention core, an activation folded into the GEMM epilogue) and "Heads" (projections at
  a GEMM-aligned width).
* "ASR Engine", section 4.3 "Batched paged forward": the chunk's K/V go into the stream's pages
  before the attention reads them (the append, ``relpos_attn.paged_kv_append``).

Readings where the pages are silent (each is listed in the design notes):

* A linear layer is y = x W^T + b with W stored [out_features, in_features].
* The sinusoidal embedding of position p (any real p, negative included) has, for d_model d and
  i in [0, d/2), entry 2i = sin(p w_i) and entry 2i + 1 = cos(p w_i), w_i = 10000^(-2i/d)
  (interleaved, as in the WeNet positional encoding the pages name).
* The positional projection has no bias.
* The fused Q/K/V weight stacks the rows of linear_q, linear_k and linear_v, in that order:
  [H D + 2 Hk D, d_model], bias likewise.
"""

from __future__ import annotations

import numpy as np

from .relpos_attn import paged_kv_append


def linear(x, w, bias=None):
    """y = x W^T (+ b) in float64: x [..., K], w [N, K], bias [N] or None -> [..., N]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


def sinusoid(positions, d_model):
    """Sinusoidal embeddings [len(positions), d_model] of the given positions (float64)."""
    p = np.asarray(positions, dtype=np.float64)[:, None]
    i = np.arange(d_model // 2, dtype=np.float64)[None, :]
    freq = np.power(10000.0, -2.0 * i / d_model)
    out = np.empty((p.shape[0], d_model), dtype=np.float64)
    out[:, 0::2] = np.sin(p * freq)
    out[:, 1::2] = np.cos(p * freq)
    return out


def table_positions(pos_start, pos_step, rows):
    """Position of row r of table t: pos_start[t] + pos_step * r -> [n_tables, rows] (int64).

    A Transformer-XL table centred at ``center`` (row r holds distance center - r) is
    pos_start = center, pos_step = -1; WeNet's per-key table of a stream (row j holds the key's
    absolute position offset - cache + j) is pos_start = offset - cache, pos_step = +1.
    """
    start = np.asarray(pos_start, dtype=np.int64).reshape(-1, 1)
    return start + int(pos_step) * np.arange(rows, dtype=np.int64)[None, :]


def rel_pos_projection(w_pos, pos_start, pos_step, rows):
    """linear_pos over sinusoidal tables: [n_tables, rows, N] = sinusoid(positions) W_pos^T.

    w_pos: [N, d_model] (N = H D, the table's heads and dims); no bias.
    """
    w_pos = np.asarray(w_pos, dtype=np.float64)
    pos = table_positions(pos_start, pos_step, rows)
    n_tables = pos.shape[0]
    d_model = w_pos.shape[1]
    emb = sinusoid(pos.reshape(-1), d_model)
    return linear(emb, w_pos).reshape(n_tables, rows, w_pos.shape[0])


def qkv_project(x, w_qkv, b_qkv, n_head, n_kv_head, head_dim):
    """The chunk's Q/K/V projection: x [B, C, d_model] -> q [B, C, H, D], k, v [B, C, Hk, D]."""
    y = linear(x, w_qkv, b_qkv)
    n_streams, chunk = y.shape[0], y.shape[1]
    hq = n_head * head_dim
    hk = n_kv_head * head_dim
    q = y[..., :hq].reshape(n_streams, chunk, n_head, head_dim)
    k = y[..., hq:hq + hk].reshape(n_streams, chunk, n_kv_head, head_dim)
    v = y[..., hq + hk:hq + 2 * hk].reshape(n_streams, chunk, n_kv_head, head_dim)
    return q, k, v


def qkv_append(x, w_qkv, b_qkv, k_pool, v_pool, block_tables, cache_seqlens, n_head, n_kv_head,
               head_dim, chunk_lens=None, window_start=None, round_kv=None):
    """The Q/K/V projection with the append as its epilogue.

    Returns (q, k_pool', v_pool'): q [B, C, H, D] in float64 and the pools after the chunk's
    projected K/V rows are appended (``relpos_attn.paged_kv_append``: frames past chunk_lens are
    not written, window starts address the ring). ``round_kv`` (optional) maps the float64 K/V to
    the pool's storage type before the append, the way the kernels store them.
    """
    q, k, v = qkv_project(x, w_qkv, b_qkv, n_head, n_kv_head, head_dim)
    if round_kv is not None:
        k, v = round_kv(k), round_kv(v)
    k_out, v_out = paged_kv_append(k_pool, v_pool, k, v, block_tables, cache_seqlens,
                                   chunk_lens=chunk_lens, window_start=window_start)
    return q, k_out, v_out
