"""Benchmark of the paged chunk attention hot path on one MI355X.

A step is one pass of the whole hot path over one synthetic cohort: for each of the 12 encoder
layers, the paged append of the chunk's K/V and the chunk attention with the Transformer-XL term,
launched as one fused kernel per layer on one HIP stream. The headline workload is the d_model 256
streaming cohort (B = 64 streams, 4 heads, head_dim 64, chunk 16, uniform cache 256 frames,
block size 16, one shared relative-position table, 12 layers, bf16 storage, fp32 accumulation).

Inputs are resident in HBM before timing starts. To measure HBM rather than the 256 MB
Infinity Cache, every step rotates over --rotate independent cohorts (each with its own pools,
queries and tables; 4 sets are about 1 GB for the headline workload).

Each cohort's 12-layer chain is captured once as a HIP graph and a step replays it, as a
streaming engine replays its captured encoder step; launching kernels one by one from Python
would time the host, not the GPU (the line's `eager` object does that, with HIP events around
every launch).

Prints one JSON line. `value` is chunk*heads per second per layer: B * H * layers / step time.
`roofline` prices the fused kernel's algorithmic bytes per launch against 8 TB/s; the kernel's
average launch duration is the graph-replay time of the timed region, measured with HIP events on
the replay stream, divided by the number of kernel launches in it (gaps between the graph's
kernels count against the kernel). `roofline.ceiling` is the same-run time of a kernel that moves
the same bytes through the same tables with no arithmetic, `roofline.launch_floor_us` that of
the same grid writing only its output, and `roofline.copy` that of a plain device copy of the
same bytes (with the kernel's rate as a fraction of it). `configs` holds the other workloads of the same run (the
d_model 512 cohort, the ragged cohort, the packed offline batch) with their own rooflines.
`cpu_baseline` times the float64 oracle on a bounded sample on the host; `cpu_baselines` does so
for every workload.
"""

from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged chunk-attention chunk·heads/sec per layer + % of HBM roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0


KERNEL_SOURCES = {
    "chunk": ["chunk_attn.hip", "pkc_step.h", "pkc_device.h", "pkc_launch.h"],
    "varlen": ["varlen_attn.hip", "pkc_step.h", "pkc_device.h", "pkc_launch.h"],
    "gemm": ["gemm.hip", "pkc_device.h", "pkc_launch.h"],
}


def kernel_source_hash(kernel="chunk"):
    """Hash of the code one kernel is compiled from: stored counter readings are used only while
    it matches. Line comments and blank lines are left out, so a comment edit keeps the readings;
    any change to the code itself drops them."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        for line in open(os.path.join(ROOT, "paged_kv_chunk_amd", "csrc", name), encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def stored_traffic(key, kernel):
    """HBM bytes per launch from the committed counter summary, or None once the kernel changed."""
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(tpath):
        return None
    rec = json.load(open(tpath)).get(key)
    if rec and rec.get("source_hash") == kernel_source_hash(kernel):
        return rec.get("bytes_per_launch")
    return None


def algorithmic_bytes(co):
    """Bytes the fused append + attention must move for one layer of a cohort: read q, k_new,
    v_new, the cached K/V and the positional band rows in use, u and v, the block-table entries
    and cache lengths; write the new K/V into the pool and the output. With per-stream chunk
    lengths n_b (``co.chunk_lens``) only real frames are read and appended (every output row is
    still written; a padding lane, n_b = 0, reads nothing)."""
    B, C, H, D = co.q.shape
    Hk = co.k_new.shape[2]
    eb = co.q.element_size()
    cache = co.cache_seqlens.cpu().tolist()
    lens = co.chunk_lens.cpu().tolist() if getattr(co, "chunk_lens", None) is not None else [C] * B
    live = [(c, n) for c, n in zip(cache, lens) if n > 0]
    S = co.block_size
    qo = sum(lens) * H * D * eb + B * C * H * D * eb
    new = 4 * sum(lens) * Hk * D * eb
    cached = 2 * sum(c for c, _ in live) * Hk * D * eb
    if getattr(co, "per_key_pos", False):
        # one table row per key: c + n rows per stream, or the longest for a shared table
        rows = [c + n for c, n in live]
        band = (sum(rows) if co.per_row_pos else max(rows, default=0)) * H * D * eb
    elif co.per_row_pos:
        band = sum(c + C + n - 1 for c, n in live) * H * D * eb
    else:
        band = max((c + C + n - 1 for c, n in live), default=0) * H * D * eb
    uv = 2 * H * D * eb
    tables = sum((c + n + S - 1) // S for c, n in live) * 4 + B * 4 * (2 if lens != [C] * B else 1)
    return qo + new + cached + band + uv + tables


def build_sets(cfg_index, n_sets, n_layers, device, blocked=True):
    """n_sets independent cohorts, each of n_layers layers sharing one block table and cache
    lengths (one block ID addresses every layer's pool). ``blocked``: each layer also gets its
    positional table in 32-dim column blocks, the layout the timed kernels read."""
    from synth import make_config, add_blocked_table
    sets = []
    for r in range(n_sets):
        layers = []
        base = make_config(cfg_index, layer=0, seed=r, device=device)
        for l in range(n_layers):
            co = base if l == 0 else make_config(cfg_index, layer=l, seed=r, device=device)
            co.block_tables = base.block_tables
            co.cache_seqlens = base.cache_seqlens
            co.out = torch.empty_like(co.q)
            if blocked:
                add_blocked_table(co)
            layers.append(co)
        sets.append(layers)
    return sets


def launch_layer(pkc, co, stream):
    blocked = co.pos_cb is not None
    pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool,
                                    co.block_tables, co.cache_seqlens,
                                    co.pos_cb if blocked else co.pos, co.pos_bias_u,
                                    co.pos_bias_v, co.max_cache_seqlen,
                                    per_row_pos=co.per_row_pos, per_key_pos=co.per_key_pos,
                                    out=co.out, chunk_lens=getattr(co, "chunk_lens", None),
                                    pos_blocked=blocked, stream=stream)


def set_chunk_lens(sets, pad_lanes, short_frac, seed=0):
    """Production cohort shapes: the last ``pad_lanes`` streams become padding lanes (chunk
    length 0) and a seeded fraction ``short_frac`` of the real streams carry a short final window
    (1..C-1 real frames). One lengths vector per cohort, shared by its layers."""
    for r, layers in enumerate(sets):
        co = layers[0]
        B, C = co.q.shape[0], co.q.shape[1]
        rng = np.random.default_rng(1000 + 17 * seed + r)
        lens = np.full(B, C, dtype=np.int32)
        real = B - pad_lanes
        short = rng.choice(real, size=int(round(short_frac * real)), replace=False)
        lens[short] = rng.integers(1, C, size=len(short))
        lens[real:] = 0
        t = torch.from_numpy(lens).to(co.q.device)
        for co in layers:
            co.chunk_lens = t


def blas_info():
    """The BLAS library numpy calls (named in the CPU baseline's record)."""
    try:
        from threadpoolctl import threadpool_info
        for rec in threadpool_info():
            if rec.get("user_api") == "blas":
                return (f"{rec.get('internal_api')} {rec.get('version')} "
                        f"({rec.get('threading_layer')}, {rec.get('filepath', '').split('/')[-1]})")
    except Exception:  # pragma: no cover
        pass
    return "unknown"


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        return None


def host_sample(co, streams):
    """Host float64 copies of a sample of a cohort's streams with only their pages (block IDs
    renumbered 0..n-1 in first-use order; relabelling blocks changes no result), as the oracle's
    arguments. Layout handling only."""
    C = co.q.shape[1]
    S = co.block_size
    bt = co.block_tables.cpu().numpy()[streams]
    cs = co.cache_seqlens.cpu().numpy()[streams]
    ids, remap = [], {}
    bt2 = np.full_like(bt, -1)
    for r in range(bt.shape[0]):
        n = (int(cs[r]) + C + S - 1) // S
        for x in range(n):
            blk = int(bt[r, x])
            if blk not in remap:
                remap[blk] = len(ids)
                ids.append(blk)
            bt2[r, x] = remap[blk]
    idx = torch.tensor(ids, device=co.k_pool.device)
    sel = torch.as_tensor(streams, device=co.q.device)
    h = lambda t: t.detach().cpu().double().numpy()
    lens = getattr(co, "chunk_lens", None)
    return dict(q=h(co.q[sel]), k_new=h(co.k_new[sel]), v_new=h(co.v_new[sel]),
                k_pool=h(co.k_pool.index_select(0, idx)), v_pool=h(co.v_pool.index_select(0, idx)),
                bt=bt2, cs=cs, pos=h(co.pos[sel] if co.per_row_pos else co.pos),
                u=h(co.pos_bias_u), w=h(co.pos_bias_v), per_row=co.per_row_pos,
                per_key=getattr(co, "per_key_pos", False),
                lens=None if lens is None else lens.cpu().numpy()[streams])


def _oracle_streams(x):
    import oracle
    kp, vp = oracle.paged_kv_append(x["k_pool"], x["v_pool"], x["k_new"], x["v_new"], x["bt"],
                                    x["cs"], x["lens"])
    oracle.chunk_relpos_attn(x["q"], kp, vp, x["bt"], x["cs"], x["pos"], x["u"], x["w"],
                             per_row_pos=x["per_row"], chunk_lens=x["lens"],
                             per_key_pos=x["per_key"])


def cpu_baseline(co, min_seconds, name=None):
    """The float64 oracle (append + attention) on one layer of a cohort, one BLAS thread: streams
    in batches of 8 (host copies of just their pages), in order, for at least ``min_seconds``,
    and again from the first stream when the layer is done. chunk·heads per second."""
    limiter = _one_blas_thread()
    B, C, H, D = co.q.shape
    lens = co.chunk_lens.cpu().numpy() if getattr(co, "chunk_lens", None) is not None else None
    batches = [list(range(b, min(B, b + 8))) for b in range(0, B, 8)]
    units, el, done = 0, 0.0, 0
    t_prep = 0.0
    while el < min_seconds:
        streams = batches[done % len(batches)]
        t0 = time.perf_counter()
        x = host_sample(co, streams)
        t1 = time.perf_counter()
        _oracle_streams(x)
        el += time.perf_counter() - t1
        t_prep += t1 - t0
        units += H * (len(streams) if lens is None else int((lens[streams] > 0).sum()))
        done += 1
    if limiter is not None:
        limiter.restore_original_limits()
    covered = sum(len(x) for x in batches[:min(done, len(batches))])
    return dict(value=units / el, unit="chunk·heads/s", cores=1, threads=1, blas=blas_info(),
                kind="oracle",
                sample=f"{name + ': ' if name else ''}{covered} of {B} streams x {H} heads of one "
                       f"layer ({units} chunk·heads), append + attention in float64 numpy, "
                       f"{el:.1f} s of oracle time (host copies of the streams' pages excluded)")


def cpu_baseline_varlen(co, min_seconds, name=None):
    """The float64 oracle on whole utterances of a packed batch (every head), in order, for at
    least ``min_seconds``, one BLAS thread. utterance·heads per second."""
    import oracle
    limiter = _one_blas_thread()
    h = lambda t: t.detach().cpu().double().numpy()
    q, k, v, pos, u, w = h(co.q), h(co.k), h(co.v), h(co.pos), h(co.pos_bias_u), h(co.pos_bias_v)
    cu = co.cu_seqlens.cpu().numpy()
    H = q.shape[1]
    n_seg = len(cu) - 1
    segs, el = 0, 0.0
    frames = 0
    while el < min_seconds and segs < n_seg:
        t0 = time.perf_counter()
        oracle.varlen_relpos_attn(q, k, v, cu, pos, u, w, segments=[segs])
        el += time.perf_counter() - t0
        frames += int(cu[segs + 1] - cu[segs])
        segs += 1
    if limiter is not None:
        limiter.restore_original_limits()
    return dict(value=segs * H / el, unit="utterance·heads/s", cores=1, threads=1,
                blas=blas_info(), kind="oracle",
                sample=f"{name + ': ' if name else ''}the first {segs} of {n_seg} utterances "
                       f"({frames} frames) x {H} heads, float64 numpy, {el:.1f} s")


def _oracle_slice(args):
    """Child process: the oracle (append + attention) on a slice of the cohort's streams, repeated
    for at least ``seconds``; returns (repetitions, elapsed). Imports no GPU code."""
    x, seconds = args
    import time as _t
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    reps, t0 = 0, _t.perf_counter()
    while True:
        _oracle_streams(x)
        reps += 1
        el = _t.perf_counter() - t0
        if el >= seconds:
            return reps, el


def cpu_baseline_all_cores(co, seconds, workers):
    """The same oracle on every host core: the cohort's streams split into ``workers`` slices, one
    child process (started fresh, one BLAS thread) per slice; chunk·heads per second summed."""
    import multiprocessing as mp
    B, C, H, D = co.q.shape
    groups = [g for g in np.array_split(np.arange(B), workers) if len(g)]
    jobs = [(host_sample(co, list(g)), seconds) for g in groups]
    with mp.get_context("spawn").Pool(len(groups)) as pool:
        out = pool.map(_oracle_slice, jobs)
    rate = sum(len(g) * H * r / el for g, (r, el) in zip(groups, out))
    return dict(value=rate, unit="chunk·heads/s", cores=len(groups), threads=len(groups),
                blas=blas_info(), kind="oracle",
                sample=f"one layer of the timed cohort (B={B}, H={H}) split over {len(groups)} "
                       f"processes by streams, each the float64 numpy oracle (append + attention) "
                       f"repeated for {seconds:.0f} s on one thread")


def visible_pairs(L, chunk=0, left=0):
    """(query, key) pairs of one utterance: all L^2, or under the chunked_limited mask the keys of
    each query's own chunk and of the ``left`` chunks before it."""
    if chunk <= 0:
        return L * L
    i = np.arange(L)
    a = i // chunk
    return int((np.minimum(L, (a + 1) * chunk) - np.maximum(0, (a - left) * chunk)).sum())


def varlen_flops(co, chunk=0, left=0):
    """Algorithmic FLOPs of the packed offline attention: per utterance and head, one dot product
    of length D for each of the content term, the position term and the PV product per visible
    (query, key) pair (L^2 without a mask)."""
    H, D = co.q.shape[1], co.q.shape[2]
    return sum(6 * visible_pairs(L, chunk, left) * D * H for L in co.lengths)


def varlen_bytes(co):
    """Algorithmic bytes: read q, k, v and each utterance's 2L - 1 table rows, write out."""
    total, H, D = co.q.shape
    Hk = co.k.shape[1]
    eb = co.q.element_size()
    rows = sum(2 * L - 1 for L in co.lengths if L > 0)
    return (2 * total * H + 2 * total * Hk) * D * eb + rows * H * D * eb + 2 * H * D * eb


def varlen_workload(args, pkc, mask_chunk=0, mask_left=0):
    """Packed offline attention: whole calls replayed from HIP graphs over rotated batches.
    Returns (result dict, the first batch)."""
    from synth import make_config
    sets = [make_config(4, seed=r, device="cuda") for r in range(args.rotate)]
    for co in sets:
        co.out = torch.empty_like(co.q)

    def call(co, st):
        pkc.varlen_packed_relpos_attn(co.q, co.k, co.v, co.cu_seqlens, co.pos, co.pos_bias_u,
                                      co.pos_bias_v, max(co.lengths), out=co.out,
                                      mask_chunk=mask_chunk, mask_left_chunks=mask_left,
                                      stream=st)

    # (one graph over every batch: a graph per call would also time the graph's own launch)
    graphs = capture_graphs([list(sets)], call)
    ms = replay_ms(graphs, args.steps, args.warmup) / len(sets)
    flops = sum(varlen_flops(co, mask_chunk, mask_left) for co in sets) / len(sets)
    nbytes = sum(varlen_bytes(co) for co in sets) / len(sets)
    units = sum(len(co.lengths) * co.q.shape[1] for co in sets) / len(sets)
    tflops = flops / (ms / 1e3) / 1e12
    from synth import WORKLOADS
    cfg = WORKLOADS[4]
    res = {
        "workload": f"{cfg['name']}: {cfg['n_seqs']} utterances, lengths uniform in "
                    f"[{cfg['len_lo']}, {cfg['len_hi']}], H={cfg['H']}, head_dim={cfg['D']}, "
                    "per-utterance tables, no cache" + (
                        f", chunked_limited mask (chunk {mask_chunk} frames, {mask_left} left "
                        "chunks)" if mask_chunk else ""),
        "value": units / (ms / 1e3), "unit": "utterance·heads/s", "ms_per_call": ms,
        "rotated_batches": len(sets), "launch": f"graph of {len(sets)} calls, one per batch",
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tflops / 2500.0,
                     "traffic": None if mask_chunk else stored_traffic("varlen_cfg4", "varlen"),
                     "kernel": "varlen_attn_kernel<bf16>", "kernel_us": ms * 1e3,
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes,
                     "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS},
    }
    first = sets[0]
    del graphs
    return res, first


def bench_varlen(args, cfg, pkc):
    """The packed offline workload alone, as its own JSON line."""
    r, _ = varlen_workload(args, pkc, args.mask_chunk, args.mask_left)
    result = {
        "metric": "packed offline rel-pos attention utterance·heads/sec + % of bf16 MFMA roofline, 1 GPU",
        "value": r["value"], "unit": r["unit"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_call"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["workload"], "rotated_batches": r["rotated_batches"],
                   "launch": "graph", "mask_chunk": args.mask_chunk,
                   "mask_left_chunks": args.mask_left},
        "roofline": r["roofline"],
    }
    print(json.dumps(result), flush=True)


def proj_layer_shapes(co):
    """(M, N, K) of one layer's three projections: the chunk's Q/K/V projection, linear_pos over
    the shared table (2 (max_cache + C) - 1 rows, the cache rung's width) and linear_out."""
    B, C, H, D = co.q.shape
    Hk = co.k_new.shape[2]
    dm = H * D
    rows = 2 * (co.max_cache_seqlen + C) - 1
    return {"qkv": (B * C, (H + 2 * Hk) * D, dm), "pos": (rows, H * D, dm), "out": (B * C, dm, H * D)}


def proj_bytes(co, kind):
    """Algorithmic bytes of one projection launch: read x (not for the generated sinusoid) and W
    (and b), write y; the Q/K/V epilogue writes q and the chunk's K/V into the pages."""
    (M, N, K) = proj_layer_shapes(co)[kind]
    eb = co.q.element_size()
    x = 0 if kind == "pos" else M * K * eb
    bias = 0 if kind == "pos" else N * eb
    return x + N * K * eb + bias + M * N * eb


def bench_proj(args, cfg, pkc):
    """The GEMMs either side of the attention for a cohort workload: per layer, the chunk's Q/K/V
    projection with the paged append as its epilogue, linear_pos over the shared table and
    linear_out. Each kind is timed alone (12 launches replayed from HIP graphs over the rotated
    sets), then all three together per step."""
    from synth import activations, linear_weights
    n_layers = cfg["n_layers"]
    sets = build_sets(args.config, args.rotate, n_layers, "cuda")
    co0 = sets[0][0]
    B, C, H, D = co0.q.shape
    Hk = co0.k_new.shape[2]
    dm = H * D
    shapes = proj_layer_shapes(co0)
    rows = shapes["pos"][0]
    center = (rows - 1) // 2
    for r, layers in enumerate(sets):
        for l, co in enumerate(layers):
            sd = 1000 * r + 10 * l
            co.x = activations((B, C, dm), seed=sd, device="cuda")
            co.w_qkv, co.b_qkv = linear_weights((H + 2 * Hk) * D, dm, seed=sd + 1, device="cuda")
            co.w_pos, _ = linear_weights(H * D, dm, seed=sd + 2, device="cuda", bias=False)
            co.w_out, co.b_out = linear_weights(dm, H * D, seed=sd + 3, device="cuda")
            co.attn = activations((B * C, H * D), seed=sd + 4, device="cuda")
            co.q_out = torch.empty_like(co.q)
            co.pos_out = torch.empty(1, rows, H * D, dtype=co.q.dtype, device="cuda")
            co.y_out = torch.empty(B * C, dm, dtype=co.q.dtype, device="cuda")

    def launch(co, kind, st):
        if kind == "qkv":
            pkc.paged_kv_qkv_append(co.x, co.w_qkv, co.b_qkv, co.k_pool, co.v_pool, co.block_tables,
                                    co.cache_seqlens, co.max_cache_seqlen, H, q_out=co.q_out,
                                    stream=st)
        elif kind == "pos":
            pkc.rel_pos_projection(co.w_pos, rows, pos_first=center, pos_step=-1, out=co.pos_out,
                                   stream=st)
        else:
            pkc.linear(co.attn, co.w_out, co.b_out, out=co.y_out, stream=st)

    stream = torch.cuda.current_stream()
    kinds = ("qkv", "pos", "out")

    def timed(kind_list):
        for layers in sets:
            for co in layers:
                for k in kind_list:
                    launch(co, k, stream)
        torch.cuda.synchronize()
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for layers in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    for co in layers:
                        for k in kind_list:
                            launch(co, k, cap)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    per_kind = {}
    for k in kinds:
        ms = timed([k])
        (M, N, K) = shapes[k]
        us = ms * 1e3 / n_layers
        per_kind[k] = dict(us=us, M=M, N=N, K=K, flops=2.0 * M * N * K, bytes=proj_bytes(co0, k),
                           tflops=2.0 * M * N * K / (us * 1e-6) / 1e12)
        per_kind[k]["hbm_frac"] = per_kind[k]["bytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
    ms_step = timed(list(kinds))
    flops_layer = sum(v["flops"] for v in per_kind.values())
    dom = max(kinds, key=lambda k: per_kind[k]["us"])
    d = per_kind[dom]
    kernel_name = {"qkv": "gemm_dma_kernel<bf16, Q/K/V paged epilogue>",
                   "pos": "gemm_dma_kernel<bf16, generated sinusoid>",
                   "out": "gemm_dma_kernel<bf16, plain>"}
    result = {
        "metric": "Q/K/V, positional and output projections per layer: tokens/sec + % of bf16 MFMA roofline, 1 GPU",
        "value": B * C * n_layers / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: the projections either side of the attention "
                               f"(B={B}, C={C}, d_model={dm}, H={H}, head_dim={D}, {n_layers} layers; "
                               f"Q/K/V + append, linear_pos over {rows} table rows, linear_out)",
                   "rotated_cohorts": len(sets), "launch": "graph",
                   "per_kind_us": {k: round(v["us"], 3) for k, v in per_kind.items()},
                   "per_kind_tflops": {k: round(v["tflops"], 1) for k, v in per_kind.items()},
                   "per_kind_hbm_frac": {k: round(v["hbm_frac"], 3) for k, v in per_kind.items()},
                   "flops_per_layer": flops_layer},
        "roofline": {"bound": "mfma", "achieved": d["tflops"], "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": d["tflops"] / 2500.0,
                     "traffic": stored_traffic(f"proj_{dom}_cfg{args.config}", "gemm"),
                     "kernel": kernel_name[dom], "kernel_us": d["us"],
                     "algorithmic_flops_per_launch": d["flops"],
                     "algorithmic_bytes_per_launch": d["bytes"], "hbm_frac": d["hbm_frac"]},
    }
    print(json.dumps(result), flush=True)


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def capture_graphs(sets, launch):
    """One HIP graph per cohort set, replaying launch(co, stream) over the set's layers (after
    one eager pass that also warms the code)."""
    stream = torch.cuda.current_stream()
    for layers in sets:
        for co in layers:
            launch(co, stream)
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        for layers in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for co in layers:
                    launch(co, cap)
            graphs.append(g)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    return graphs


def replay_ms(graphs, steps, warmup):
    """Mean milliseconds per replay over ``steps`` replays that cycle through the graphs, timed
    with HIP events on the replay stream after ``warmup`` untimed replays."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def copy_reference(nbytes, steps, warmup):
    """Same-run time of a plain device copy moving a launch's bytes (half read, half written),
    rotated over buffer pairs that together exceed the 256 MB last-level cache and replayed from
    one HIP graph like the kernels: the HBM rate one launch of this size reaches with no gather
    and no arithmetic. Returns the roofline's `copy` object (without the kernel's share)."""
    half = -(-max(nbytes // 2, 1 << 20) // 256) * 256
    pairs = max(2, -(-(512 << 20) // (2 * half)))
    bufs = []
    for _ in range(pairs):
        src = torch.empty(half, dtype=torch.uint8, device="cuda").random_(0, 255)
        bufs.append((src, torch.empty_like(src)))
    graphs = capture_graphs([bufs], lambda sd, st: sd[1].copy_(sd[0]))
    us = replay_ms(graphs, max(steps // 4, 10), max(warmup // 4, 3)) * 1e3 / pairs
    del graphs, bufs
    torch.cuda.empty_cache()
    moved = 2 * half
    return {"kernel": f"device copy (the runtime's copy kernel, one launch per copy) of "
                      f"{half / 2**20:.1f} MiB read + {half / 2**20:.1f} MiB written, over {pairs} "
                      f"buffer pairs ({pairs * moved / 2**20:.0f} MiB) in turn, graph replay",
            "bytes_per_copy": moved, "us": us, "achieved": moved / (us * 1e-6) / 1e9,
            "frac": moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


# launch shapes of the memory-path ceiling kernel: (waves per workgroup, workgroups per stream
# and head); the attention kernel's own grids are (4, 1) and, for cohorts whose grid fills every
# wave slot with one wave per unit, (1, 1)
CEILING_SHAPES = ((4, 1), (8, 1), (4, 2), (1, 1))


def chains_of(sets):
    """The launch chains to capture: one graph per cohort set for multi-layer workloads; for
    one-layer workloads one graph over every set's layer (one graph per launch would time the
    graph's own launch, some 15 us, more than most of these kernels)."""
    return sets if len(sets[0]) > 1 else [[layers[0] for layers in sets]]


def longest_first(co):
    """The cohort with its streams reordered by decreasing cache length (stable): the same
    pools, each stream's rows, table row, cache length and positional table moved together."""
    import copy
    perm = torch.argsort(-co.cache_seqlens.long(), stable=True)
    c = copy.copy(co)
    for f in ("q", "k_new", "v_new", "block_tables", "cache_seqlens", "out"):
        setattr(c, f, getattr(co, f)[perm].contiguous())
    if co.per_row_pos:
        c.pos = co.pos[perm].contiguous()
        if co.pos_cb is not None:
            c.pos_cb = co.pos_cb[perm].contiguous()
    return c


def ceiling_and_floor(sets, pkc, steps, warmup, n_layers, nbytes):
    """Same-run times of pkc_gather_read on the same cohorts: the fused launch's bytes through
    the same tables with no arithmetic, at each ceiling shape (the fastest is the ceiling), and
    the attention kernel's grid writing only its output (the launch floor)."""
    def gr(w, sp, reads):
        def launch(co, st):
            blocked = co.pos_cb is not None
            pkc.gather_read(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool, co.block_tables,
                            co.cache_seqlens, co.pos_cb if blocked else co.pos, co.pos_bias_u,
                            co.pos_bias_v, co.max_cache_seqlen, co.out,
                            per_row_pos=co.per_row_pos, pos_blocked=blocked, waves=w, split=sp,
                            reads=reads, stream=st)
        return launch
    variants = {}
    chains = chains_of(sets)
    per_graph = len(chains[0])
    for w, sp in CEILING_SHAPES:
        graphs = capture_graphs(chains, gr(w, sp, True))
        variants[f"{w} waves x {sp} workgroup(s)"] = replay_ms(graphs, steps, warmup) * 1e3 / per_graph
        del graphs
    # Ragged cohorts: the attention runs multi-pass grids longest cache first, so the ceiling is
    # also timed on the same cohorts with their streams reordered that way on the host (no
    # ranking cost: a bound from below).
    if any(bool((layers[0].cache_seqlens != layers[0].cache_seqlens[0]).any()) for layers in sets):
        ordered = [[longest_first(co) for co in layers] for layers in sets]
        ochains = chains_of(ordered)
        for w, sp in CEILING_SHAPES:
            graphs = capture_graphs(ochains, gr(w, sp, True))
            variants[f"{w} waves x {sp} workgroup(s), longest first"] = (
                replay_ms(graphs, steps, warmup) * 1e3 / per_graph)
            del graphs
        del ordered, ochains
    graphs = capture_graphs(chains, gr(4, 1, False))
    floor_us = replay_ms(graphs, steps, warmup) * 1e3 / per_graph
    del graphs
    best = min(variants, key=variants.get)
    us = variants[best]
    return {"kernel": "pkc_gather_read: the fused launch's bytes through the same block tables "
                      "and layouts, every page request of a step group issued before any wait, "
                      "no arithmetic",
            "us": us, "shape": best, "achieved": nbytes / (us * 1e-6) / 1e9,
            "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "variants_us": {k: round(v, 3) for k, v in variants.items()}}, floor_us


def chunk_workload(cfg_index, args, pkc, measure_ceiling=True, lens_mode=False):
    """One cohort workload: fused append + attention per layer, each cohort set's layer chain
    replayed from a HIP graph. Returns (result dict, sets, graphs)."""
    from synth import WORKLOADS
    cfg = WORKLOADS[cfg_index]
    n_layers = cfg["n_layers"]
    progress(f"workload {cfg_index} ({cfg['name']}): building {args.rotate} cohort sets")
    sets = build_sets(cfg_index, args.rotate, n_layers, "cuda", blocked=not args.pos_row_major)
    if lens_mode:
        set_chunk_lens(sets, args.pad_lanes, args.short_frac)
    if args.per_key:
        from synth import use_key_position_tables, add_blocked_table
        for layers in sets:
            for co in layers:
                # keys' absolute positions start at offset - cache; here every stream's offset
                # is its cache length (unlimited history), so positions start at 0
                use_key_position_tables(co, [0] * co.q.shape[0], per_row=co.per_row_pos)
                if not args.pos_row_major:
                    add_blocked_table(co)
    co0 = sets[0][0]
    B, C, H, D = co0.q.shape
    chains = chains_of(sets)
    graphs = capture_graphs(chains, lambda co, st: launch_layer(pkc, co, st))
    kernel_us = replay_ms(graphs, args.steps, args.warmup) * 1e3 / len(chains[0])
    ms = kernel_us * n_layers / 1e3     # one step: every layer of one cohort
    nbytes = algorithmic_bytes(co0)
    achieved = nbytes / (kernel_us * 1e-6) / 1e9
    real = B - (args.pad_lanes if lens_mode else 0)
    res = {
        "workload": f"{cfg['name']}: B={B} streams, H={H}, head_dim={D}, chunk={C}, "
                    f"cache={'ragged up to ' if cfg['cache'] == 'ragged' else ''}"
                    f"{co0.max_cache_seqlen} frames, block_size={co0.block_size}, "
                    f"{'per-row' if co0.per_row_pos else 'shared'} rel-pos table"
                    f"{'s' if co0.per_row_pos else ''}, {n_layers} layer"
                    f"{'s' if n_layers > 1 else ''}, fused append+attention per layer",
        "value": real * H * n_layers / (ms / 1e3), "unit": "chunk·heads/s",
        "ms_per_step": ms, "layers": n_layers, "rotated_cohorts": len(sets),
        "launch": "graph" if n_layers > 1 else f"graph of {len(chains[0])} launches, one per set",
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (None if lens_mode or args.per_key or args.pos_row_major
                        else stored_traffic(f"fused_cfg{cfg_index}", "chunk")),
            "kernel": "chunk_attn_kernel<bf16, fused>", "kernel_us": kernel_us,
            "kernel_time_from": "graph replay, timed-region time / kernel launches",
            "algorithmic_bytes_per_launch": nbytes,
        },
    }
    progress(f"workload {cfg_index}: {kernel_us:.2f} us per layer, {achieved / HBM_PEAK_GBS:.3f} "
             "of HBM peak")
    if measure_ceiling and not (lens_mode or args.per_key) and co0.q.dtype == torch.bfloat16:
        ceil, floor_us = ceiling_and_floor(sets, pkc, args.steps, args.warmup, n_layers, nbytes)
        res["roofline"]["ceiling"] = ceil
        res["roofline"]["kernel_over_ceiling"] = kernel_us / ceil["us"]
        res["roofline"]["launch_floor_us"] = floor_us
        # the survey's "% of a measured copy bandwidth": the same bytes through a plain copy
        copy = copy_reference(nbytes, args.steps, args.warmup)
        copy["kernel_frac_of_copy"] = achieved / copy["achieved"]
        res["roofline"]["copy"] = copy
        # (the ceiling kernel appended the same K/V again and left garbage in out; restore a
        # clean state for what follows by replaying the attention once more)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    return res, sets, graphs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1,
                    help="workload index (1, 2, 3: cohorts; 4: the packed offline batch); with "
                         "the default 1 the line also carries the other workloads under configs")
    ap.add_argument("--rotate", type=int, default=4, help="independent cohort sets cycled per step")
    ap.add_argument("--no-configs", action="store_true",
                    help="headline workload only (no configs object)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the same-run ceiling and launch-floor kernels")
    ap.add_argument("--eager", action="store_true",
                    help="launch layer by layer from Python with HIP events around each launch "
                         "instead of replaying captured graphs")
    ap.add_argument("--no-events", action="store_true", help="eager mode without per-launch events")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-seconds-other", type=float, default=6.0,
                    help="oracle time per workload for the cpu_baselines of the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pad-lanes", type=int, default=0,
                    help="the last N streams of the cohort are padding lanes (chunk length 0)")
    ap.add_argument("--short-frac", type=float, default=0.0,
                    help="fraction of the real streams in a short final window (1..C-1 frames)")
    ap.add_argument("--mask-chunk", type=int, default=0,
                    help="packed offline workload: chunked_limited mask chunk (frames); 0 = none")
    ap.add_argument("--mask-left", type=int, default=0,
                    help="packed offline workload: left chunks of the chunked_limited mask")
    ap.add_argument("--pos-row-major", action="store_true",
                    help="cohort workloads: positional tables row-major [P, H, D] instead of in "
                         "32-dim column blocks per head")
    ap.add_argument("--per-key", action="store_true",
                    help="cohort workloads: WeNet per-key tables instead of Transformer-XL ones")
    ap.add_argument("--proj", action="store_true",
                    help="cohort workloads: time the projections either side of the attention "
                         "(Q/K/V with the paged append, linear_pos, linear_out) instead")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the workload, time a plain device copy of this many MiB "
                         "(reference for HBM counters and achievable bandwidth)")
    ap.add_argument("--copy-rotate", type=int, default=1,
                    help="with --copy-mib: copy over this many buffer pairs in turn (enough to "
                         "exceed the last-level cache makes every copy come from HBM)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the path has "
              "no cross-GPU exchange; the figure is one GPU's throughput.", file=sys.stderr)
        sys.exit(2)

    global torch
    import torch
    import paged_kv_chunk_amd as pkc
    from synth import WORKLOADS, make_config

    if args.copy_mib:
        # plain device copies (torch's copy kernel): the calibration of the HBM counters, and
        # with --copy-rotate K over K buffer pairs in turn, so that a small copy comes from HBM
        # and not the last-level cache (a single launch's reference for the same bytes)
        n = args.copy_mib << 20
        pairs = []
        for _ in range(max(args.copy_rotate, 1)):
            src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
            pairs.append((src, torch.empty_like(src)))
        for i in range(args.warmup):
            d, s = pairs[i % len(pairs)][1], pairs[i % len(pairs)][0]
            d.copy_(s)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(args.steps):
            d, s = pairs[i % len(pairs)][1], pairs[i % len(pairs)][0]
            d.copy_(s)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "buffer_pairs": len(pairs),
                          "ms_per_copy": ms, "read_plus_write_GBps": 2 * n / (ms / 1e3) / 1e9}),
              flush=True)
        return

    cfg = WORKLOADS[args.config]
    if cfg["kind"] == "varlen":
        return bench_varlen(args, cfg, pkc)
    if args.proj:
        return bench_proj(args, cfg, pkc)
    lens_mode = bool(args.pad_lanes or args.short_frac)
    stream = torch.cuda.current_stream()
    n_layers = cfg["n_layers"]
    if args.eager:
        sets = build_sets(args.config, args.rotate, n_layers, "cuda",
                          blocked=not args.pos_row_major)
        if lens_mode:
            set_chunk_lens(sets, args.pad_lanes, args.short_frac)
        co0 = sets[0][0]
        B, C, H, D = co0.q.shape
        use_events = not args.no_events
        for i in range(max(args.warmup, len(sets))):
            for co in sets[i % len(sets)]:
                launch_layer(pkc, co, stream)
        ev = ([[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_layers)]
               for _ in range(args.steps)] if use_events else None)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            for li, co in enumerate(sets[i % len(sets)]):
                if use_events:
                    ev[i][2 * li].record(stream)
                launch_layer(pkc, co, stream)
                if use_events:
                    ev[i][2 * li + 1].record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / args.steps
        if use_events:
            durs = [ev[i][2 * l].elapsed_time(ev[i][2 * l + 1]) for i in range(args.steps)
                    for l in range(n_layers)]
            kernel_ms = sum(durs) / len(durs)
            src = "eager launches, HIP events around each launch"
        else:
            kernel_ms = ms_step / n_layers
            src = "eager launches, step time / launches"
        nbytes = algorithmic_bytes(co0)
        achieved = nbytes / (kernel_ms / 1e3) / 1e9
        real = B - args.pad_lanes
        res = {"workload": f"{cfg['name']} (eager)", "value": real * H * n_layers / (ms_step / 1e3),
               "unit": "chunk·heads/s", "ms_per_step": ms_step, "layers": n_layers,
               "rotated_cohorts": len(sets), "launch": "eager",
               "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                            "kernel": "chunk_attn_kernel<bf16, fused>",
                            "kernel_us": kernel_ms * 1e3, "kernel_time_from": src,
                            "algorithmic_bytes_per_launch": nbytes}}
        graphs = None
    else:
        res, sets, graphs = chunk_workload(args.config, args, pkc,
                                           measure_ceiling=not args.no_ceiling,
                                           lens_mode=lens_mode)
        co0 = sets[0][0]
        B, C, H, D = co0.q.shape
        ms_step = res["ms_per_step"]
    result = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "chunk·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": res["workload"],
            "streams": B, "heads": H, "head_dim": D, "chunk": C,
            "cache_frames": co0.max_cache_seqlen, "block_size": co0.block_size,
            "layers": n_layers, "rotated_cohorts": len(sets), "launch": res["launch"],
            "shared_pos_table": not co0.per_row_pos,
            "pos_convention": "per-key (WeNet, no shift)" if args.per_key else "Transformer-XL",
            "pos_layout": "row-major [P, H, D]" if args.pos_row_major
                          else "32-dim column blocks per head [H, D/32, P, 32]",
        },
        "roofline": res["roofline"],
    }
    if graphs is not None:
        # the spread of single steps: a separate pass with events around every replay
        n_pct = min(args.steps, 100)
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_pct)]
        for i, (a0, a1) in enumerate(pev):
            a0.record(stream)
            graphs[i % len(graphs)].replay()
            a1.record(stream)
        torch.cuda.synchronize()
        # (a one-layer workload's graph holds one step of every set)
        steps_per_graph = 1 if n_layers > 1 else len(sets)
        per_step = np.array([a0.elapsed_time(a1) for a0, a1 in pev]) / steps_per_graph
        result["step_ms_percentiles"] = {"graph_replays": n_pct,
                                         "steps_per_replay": steps_per_graph,
                                         "p10": float(np.percentile(per_step, 10)),
                                         "p50": float(np.percentile(per_step, 50)),
                                         "p90": float(np.percentile(per_step, 90))}
        # the same chain launched layer by layer from the host, with HIP events around each
        # launch: reported beside the replay figure, labelled, never as `value`
        n_eager = min(args.steps, 50)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_layers)]
              for _ in range(n_eager)]
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n_eager):
            for li, co in enumerate(sets[i % len(sets)]):
                ev[i][2 * li].record(stream)
                launch_layer(pkc, co, stream)
                ev[i][2 * li + 1].record(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        durs = [ev[i][2 * l].elapsed_time(ev[i][2 * l + 1]) for i in range(n_eager)
                for l in range(n_layers)]
        result["eager"] = {"steps": n_eager, "ms_per_step": e0.elapsed_time(e1) / n_eager,
                           "kernel_us_mean": 1e3 * sum(durs) / len(durs),
                           "kernel_us_median": 1e3 * float(np.median(durs)),
                           "timed_from": "eager launches, HIP events around each launch"}
    if lens_mode:
        lens0 = co0.chunk_lens.cpu().numpy()
        result["config"]["workload"] += (f"; {args.pad_lanes} padding lanes, "
                                          f"{int(((lens0 > 0) & (lens0 < C)).sum())} streams in a "
                                          "short final window")
        result["config"].update(real_streams=B - args.pad_lanes, padding_lanes=args.pad_lanes,
                                short_windows=int(((lens0 > 0) & (lens0 < C)).sum()))
    if not args.no_cpu_baseline:
        progress("CPU oracle baselines of the headline workload")
        result["cpu_baseline"] = cpu_baseline(co0, args.cpu_seconds,
                                              name=WORKLOADS[args.config]["name"])
        if not lens_mode and not args.per_key:
            # host cores this process may run on (the machine's CPU share, at most 16)
            n_cores = min(len(os.sched_getaffinity(0)), 16)
            if n_cores > 1:
                result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(
                    co0, args.cpu_seconds, n_cores)
    del sets, graphs
    torch.cuda.empty_cache()

    if args.config == 1 and not (args.no_configs or args.eager or lens_mode or args.per_key):
        # the other workloads of the same run, each with its own roofline (and oracle baseline)
        configs, cpu_other = {}, {}
        for idx in (2, 3):
            r, sets, graphs = chunk_workload(idx, args, pkc, measure_ceiling=not args.no_ceiling)
            configs[f"cfg{idx}"] = r
            if not args.no_cpu_baseline:
                cpu_other[f"cfg{idx}"] = cpu_baseline(sets[0][0], args.cpu_seconds_other,
                                                      name=WORKLOADS[idx]["name"])
            del sets, graphs
            torch.cuda.empty_cache()
        progress("workload 4 (packed offline batch)")
        r, first = varlen_workload(args, pkc)
        configs["cfg4"] = r
        if not args.no_cpu_baseline:
            cpu_other["cfg4"] = cpu_baseline_varlen(first, args.cpu_seconds_other,
                                                    name=WORKLOADS[4]["name"])
            cpu_other["cfg0"] = cpu_baseline(make_config(0, device="cuda"),
                                             args.cpu_seconds_other, name=WORKLOADS[0]["name"])
            cpu_other["cfg1"] = result["cpu_baseline"]
            result["cpu_baselines"] = cpu_other
        del first
        torch.cuda.empty_cache()
        result["configs"] = configs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
