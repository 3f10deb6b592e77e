"""Plain float64 definition of the paged chunk attention path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use this
module. It shares no code with the HIP path and imports nothing from it.

Sources, cited by page title and section (OASR documentation):

* "ASR Engine", section 4.3 "Batched paged forward": a cohort of B streams shares one block pool;
  each stream has a block table (B, blocks_per_seq) and a cache_seqlens entry (B,); the chunk's K/V
  are written into the stream's pages, and cache_seqlens is advanced by commit_chunk_paged only
  after the forward, so during the forward it counts the frames cached *before* the chunk.
  One PagedKVCache per layer shares the block table and cache_seqlens.
* "Scheduler", section 4.3 "Heterogeneous-offset batching": the attention runs over the paged pool
  with a per-stream length mask built from cache_seqlens, and the Conformer relative-position bias
  matrix_bd is added to the scores scaled by 1/sqrt(d_k); the positional embedding is built per
  stream when offsets differ and collapses to one broadcast table when they match.
* "Model Layer", "Three optional encoder declarations" (fixed_attention_window): the query at
  chunk row i and the key at index j sit cache + i - j frames apart, and that offset selects the
  Transformer-XL table row; when every stream has the same cache_seqlens a single table serves
  the cohort, and otherwise each stream gets a table of its own.
* "Model Layer", "The engine-facing surface" (forward_offline_packed) and "ASR Engine" section 4.1
  (sequence packing): the offline forward packs utterances into one gapless varlen row and
  attention never crosses an utterance boundary.

Readings where the pages are silent (each is listed, with its reason, in the design notes):

* Score: s[i, j] = ((q_i + u) . k_j + (q_i + v) . p[cache + i - j]) * scale, scale = 1/sqrt(D)
  applied to the sum (the pages scale matrix_bd by 1/sqrt(d_k); the content term carries the same
  scale in standard scaled dot-product attention).
* No mask inside the window: each of the C chunk queries sees every cached frame and every chunk
  frame (unlimited left context, no causality inside the chunk).
* Table orientation: row r of a table with centre ``center`` holds the embedding of the signed
  distance ``center - r`` (row 0 is the largest positive distance). A shared table is centred at
  (P - 1) / 2; a per-row table of stream b holds 2 T_b - 1 rows centred at T_b - 1, T_b = c_b + C.
* GQA: query head h reads kv head h * Hk // H.
* Page layout (the pages give none): v_pool[n, g, d, s] (V transposed inside each page), and K
  either k_pool[n, g, s, d] or, in column blocks of w dims, k_pool[n, g, c, s, e] holding dim
  c w + e of slot s (the kernels' layout, w = 32: a page keeps each 32-dim half of every slot's
  row together); logical frame t of stream b sits in block block_tables[b, t // S], slot t % S.
* Bounded history ("ASR Engine", section 6, num_left_chunks and recycle_streaming_history;
  section 9, cached_frames held at max_logical_blocks - 1 blocks, positions unaffected): a stream
  may carry a window start w_b, the absolute position of its first cached frame, a multiple of S.
  Absolute position p then sits in block block_tables[b, (p // S) % M], slot p % S (the table row
  is a ring of M pages, so a recycled page is reused without rewriting the table); the cached
  frames are p in [w_b, w_b + cache_b) and the chunk follows them. Distances are taken inside the
  window (cache + i - j with j the key's index in the window), which a table by distance makes
  independent of w_b.
* Other conventions ("Model Layer", the Nemotron encoder notes): WeNet's relative position needs no
  shift - its table has one row per key, the embedding of the key's absolute position, and the
  position term is (q_i + v) . p[j]. The chunked_limited mask lets a query see its own chunk and
  a fixed number of earlier chunks, offline too.
"""

from __future__ import annotations

import numpy as np

DEFAULT_LAYOUT = {"k_pool": "[num_blocks, n_kv_head, head_dim / 32, block_size, 32]",
                  "v_pool": "[num_blocks, n_kv_head, head_dim, block_size]"}


def _k_put(k_pool, block, slot, rows):
    """Write one slot's K rows [Hk, D] into a plain or column-blocked K pool."""
    if k_pool.ndim == 5:
        n_kv, nb, w = k_pool.shape[1], k_pool.shape[2], k_pool.shape[4]
        k_pool[block, :, :, slot, :] = np.asarray(rows).reshape(n_kv, nb, w)
    else:
        k_pool[block, :, slot, :] = rows


def _k_get(k_pool, block, slot):
    """One slot's K rows [Hk, D] from a plain or column-blocked K pool."""
    if k_pool.ndim == 5:
        n_kv, nb, w = k_pool.shape[1], k_pool.shape[2], k_pool.shape[4]
        return k_pool[block, :, :, slot, :].reshape(n_kv, nb * w)
    return k_pool[block, :, slot, :]


def _slot(block_table_row, p, block_size):
    """Block and slot of absolute position p in a stream's ring of pages."""
    n_entries = len(block_table_row)
    return int(block_table_row[(p // block_size) % n_entries]), p % block_size


def paged_kv_append(k_pool, v_pool, k_new, v_new, block_tables, cache_seqlens, chunk_lens=None,
                    window_start=None):
    """Write each stream's chunk K/V into its pages ("ASR Engine" section 4.3, steps 1 and 5).

    k_new, v_new: [B, C, Hk, D]. Frame t of the chunk of stream b is logical frame
    L = cache_seqlens[b] + t, stored in block block_tables[b, L // S] at slot L % S.
    ``chunk_lens`` (default: C for every stream) gives each stream's real frames n_b <= C: only
    frames t < n_b are written ("ASR Engine" section 4.3 step 6: a stream commits its actual
    frames; the final window is short). A stream with n_b = 0 (the padding lane) writes nothing.
    ``window_start`` (default 0): frame t goes to absolute position w_b + cache_b + t, addressed
    through the ring of the stream's table row (see the module notes).
    Returns new pools; every element that is not written is copied unchanged. Works on any dtype
    (pass integer views of the storage to compare bit patterns).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    n_streams, chunk = k_new.shape[0], k_new.shape[1]
    block_size = v_pool.shape[3]
    for b in range(n_streams):
        n_real = chunk if chunk_lens is None else int(chunk_lens[b])
        start = 0 if window_start is None else int(window_start[b])
        for t in range(n_real):
            frame = start + int(cache_seqlens[b]) + t
            block, slot = _slot(block_tables[b], frame, block_size)
            _k_put(k_out, block, slot, k_new[b, t])
            v_out[block, :, :, slot] = v_new[b, t]
    return k_out, v_out


def commit_chunk(cache_seqlens, chunk, chunk_lens=None, window_start=None, max_cached_frames=None,
                 block_size=None):
    """After a step: cache_b += n_b ("ASR Engine" section 4.3 step 6, commit_chunk_paged). With a
    window start and a cap (bounded history, "ASR Engine" sections 6 and 9), the oldest whole
    blocks are then dropped while cache_b exceeds the cap: w_b += S, cache_b -= S, as long as a
    whole filled block is left to drop (cache_b >= S; a cap below one block then keeps the
    partial last block rather than dropping frames that are still to be written). Returns the new
    (cache_seqlens, window_start) as int64 arrays (window_start None when not given)."""
    cache = np.array(cache_seqlens, dtype=np.int64, copy=True)
    lens = np.full(cache.shape, chunk) if chunk_lens is None else np.asarray(chunk_lens)
    cache += lens
    if window_start is None:
        return cache, None
    start = np.array(window_start, dtype=np.int64, copy=True)
    if max_cached_frames is not None:
        for b in range(len(cache)):
            # only whole blocks that are already filled can leave: the next chunk's frames are
            # written right after the cached ones, so a block they reach stays in the window
            while cache[b] > max_cached_frames and cache[b] >= block_size:
                start[b] += block_size
                cache[b] -= block_size
    return cache, start


def gather_stream(k_pool, v_pool, block_table_row, n_frames, start=0):
    """Read the frames at absolute positions [start, start + n_frames) of one stream through its
    block table (a ring of pages when start > 0).

    Returns K, V as [n_frames, Hk, D] arrays in the pool's dtype ("Scheduler" section 4.3: the
    attention reads the paged pool through each stream's table).
    """
    block_size = v_pool.shape[3]
    ks, vs = [], []
    for t in range(start, start + n_frames):
        block, slot = _slot(block_table_row, t, block_size)
        ks.append(_k_get(k_pool, block, slot))
        vs.append(v_pool[block, :, :, slot])
    return np.stack(ks), np.stack(vs)


def table_row(center, cache, i, j):
    """Row of a Transformer-XL table that holds the distance cache + i - j ("Model Layer",
    fixed_attention_window declaration), with rows in descending distance order."""
    return center - (cache + i - j)


def _attend(q, k, v, pos_rows, u, w, center, cache, scale, query_rows=None, per_key=False,
            keep=None):
    """Attention of C queries at absolute positions cache + i over T = cache + C keys (one stream).

    q: [C, H, D]; k, v: [T, Hk, D]; pos_rows: [P_b, H, D] table of this stream. Returns the output
    and the probabilities for the queries in ``query_rows`` (default: all C), as
    [len(query_rows), H, D] and [H, len(query_rows), T].
    per_key: WeNet's convention - row j of the table is key j's own embedding (no shift), the
    position term is (q_i + v) . p[j]. keep: optional callable (i, j array) -> bool array, the
    keys query i may see (the others get no weight).
    """
    n_q, n_head, _ = q.shape
    n_k, n_kv_head = k.shape[0], k.shape[1]
    if query_rows is None:
        query_rows = np.arange(n_q)
    query_rows = np.asarray(query_rows)
    j = np.arange(n_k)
    out = np.empty((len(query_rows), n_head, v.shape[2]))
    probs = np.empty((n_head, len(query_rows), n_k))
    for x, i in enumerate(query_rows):
        if per_key:
            if pos_rows.shape[0] < n_k:
                raise ValueError("per-key table shorter than the keys")
            emb = pos_rows[:n_k]                                              # p[j]: [T, H, D]
        else:
            rows = table_row(center, cache, int(i), j)                        # [T]
            if rows.min() < 0 or rows.max() >= pos_rows.shape[0]:
                raise ValueError("relative-position table too short for distances cache + i - j")
            emb = pos_rows[rows]                                              # p[cache + i - j]: [T, H, D]
        seen = np.ones(n_k, dtype=bool) if keep is None else keep(int(i), j)
        for h in range(n_head):
            g = h * n_kv_head // n_head
            content = k[:, g, :] @ (q[i, h, :] + u[h])                       # (q + u) . k_j
            position = emb[:, h, :] @ (q[i, h, :] + w[h])                    # (q + v) . p
            s = (content + position) * scale
            s = np.where(seen, s, -np.inf)
            s = s - s.max()
            a = np.exp(s)
            a = a / a.sum()
            probs[h, x] = a
            out[x, h, :] = a @ v[:, g, :]
    return out, probs


def chunk_relpos_attn(q, k_pool, v_pool, block_tables, cache_seqlens, pos, pos_bias_u, pos_bias_v,
                      per_row_pos=False, scale=None, return_probs=False, streams=None,
                      chunk_lens=None, window_start=None, per_key_pos=False):
    """Chunk attention of every stream over its cached frames plus its own chunk.

    q: [B, C, H, D]. The chunk's K/V must already be in the pools (append first, then attend).
    pos: one shared table [P, H, D] centred at (P - 1) / 2, or per-row tables [B, P_max, H, D],
    row b centred at T_b - 1 with 2 T_b - 1 meaningful rows, T_b = c_b + C. pos_bias_u,
    pos_bias_v: [H, D]. Returns out [B, C, H, D] in float64 (and the per-stream probabilities
    when asked). ``streams`` (default: all) restricts the work to a sample of streams; other rows
    are NaN.

    ``chunk_lens`` (default: C for every stream) gives each stream's real frames n_b <= C (a short
    final window, "ASR Engine" section 4.3 step 6 and section 8; a padding lane has n_b = 0,
    "ASR Engine" section 9). Reading: frames t >= n_b do not exist, so query i < n_b attends over
    keys j < c_b + n_b, and output rows i >= n_b are zero. Tables keep the geometry of the full
    chunk width (a per-row table stays centred at c_b + C - 1).

    ``window_start`` (default 0): stream b's cached frames are the absolute positions
    [w_b, w_b + c_b) of its ring of pages (bounded history); the keys are those frames and the
    chunk's, and distances are counted inside the window, so the result depends on w_b only
    through which pages are read.

    ``per_key_pos`` (WeNet's convention): the table holds one row per key instead of one per
    distance - shared [P, H, D] or per-row [B, P_max, H, D], row j the embedding of key j's absolute
    position (the caller builds it from positions starting at offset - cache_b) - and the position
    term is (q_i + v) . p[j].
    """
    q = np.asarray(q, dtype=np.float64)
    u = np.asarray(pos_bias_u, dtype=np.float64)
    w = np.asarray(pos_bias_v, dtype=np.float64)
    n_streams, chunk, _, head_dim = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    out = np.full(q.shape, np.nan)
    all_probs = []
    for b in (range(n_streams) if streams is None else streams):
        cache = int(cache_seqlens[b])
        n_real = chunk if chunk_lens is None else int(chunk_lens[b])
        out[b] = 0.0
        if n_real == 0:
            all_probs.append(np.zeros((q.shape[2], 0, cache)))
            continue
        n_k = cache + n_real
        start = 0 if window_start is None else int(window_start[b])
        k, v = gather_stream(k_pool, v_pool, block_tables[b], n_k, start)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        if per_key_pos:
            center = 0
            rows = np.asarray(pos[b] if per_row_pos else pos, dtype=np.float64)
        elif per_row_pos:
            center = cache + chunk - 1
            rows = np.asarray(pos[b][: 2 * (cache + chunk) - 1], dtype=np.float64)
        else:
            if pos.shape[0] % 2 != 1:
                raise ValueError("a shared relative-position table has an odd number of rows")
            center = (pos.shape[0] - 1) // 2
            rows = np.asarray(pos, dtype=np.float64)
        out[b, :n_real], probs = _attend(q[b, :n_real], k, v, rows, u, w, center, cache, scale,
                                         per_key=per_key_pos)
        all_probs.append(probs)
    if return_probs:
        return out, all_probs
    return out


def chunked_limited_keep(chunk, left_chunks):
    """The chunked_limited mask ("Model Layer", Nemotron encoder notes): query i sees the keys of
    its own chunk and of the ``left_chunks`` chunks before it (chunks of ``chunk`` frames counted
    from the utterance's first frame)."""
    def keep(i, j):
        a, kc = i // chunk, np.asarray(j) // chunk
        return (kc <= a) & (kc >= a - left_chunks)
    return keep


def varlen_relpos_attn(q, k, v, cu_seqlens, pos, pos_bias_u, pos_bias_v, scale=None,
                       return_probs=False, segments=None, query_rows=None, chunk=None,
                       left_chunks=None):
    """Full-context attention inside each packed segment ("Model Layer", forward_offline_packed).

    q: [total, H, D], k, v: [total, Hk, D], packed gapless; segment s is frames
    [cu_seqlens[s], cu_seqlens[s+1]). Its table has 2 L_s - 1 rows centred at L_s - 1 and starts at
    row 2 cu_seqlens[s] of pos [2 total, H, D] (each utterance owns 2 L_s rows, the last one
    unused, so empty utterances keep every offset consistent). Each segment is the chunk case with
    cache = 0 and C = L_s. Returns out [total, H, D] in float64.

    ``segments`` (default: all) and ``query_rows`` (a callable L -> rows of the segment, default
    all) restrict the work to a sample; rows not computed are NaN in ``out``.
    ``chunk`` and ``left_chunks`` (both or neither): apply the chunked_limited mask inside each
    segment (see chunked_limited_keep); the table is still the segment's 2 L - 1 rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    u = np.asarray(pos_bias_u, dtype=np.float64)
    w = np.asarray(pos_bias_v, dtype=np.float64)
    head_dim = q.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    out = np.full(q.shape, np.nan)
    all_probs = []
    n_seg = len(cu_seqlens) - 1
    for s in (range(n_seg) if segments is None else segments):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        n = hi - lo
        if n == 0:
            all_probs.append(np.zeros((q.shape[1], 0, 0)))
            continue
        row0 = 2 * lo
        rows = np.asarray(pos[row0: row0 + 2 * n - 1], dtype=np.float64)
        qr = np.arange(n) if query_rows is None else np.asarray(query_rows(n))
        keep = None if chunk is None else chunked_limited_keep(chunk, left_chunks)
        out[lo + qr], probs = _attend(q[lo:hi], k[lo:hi], v[lo:hi], rows, u, w, n - 1, 0, scale, qr,
                                      keep=keep)
        all_probs.append(probs)
    if return_probs:
        return out, all_probs
    return out
