"""A whole streaming step - the fused append + attention of every layer, then the device-side
commit of the cache lengths - captured once in a HIP graph and replayed step after step while the
streams grow ("ASR Engine", section 4.3: one PagedKVCache per layer sharing the block table and
cache_seqlens, commit_chunk_paged after the forward; section 9: the graph is keyed by batch width
and cache rung, so one capture must serve every cache length up to its rung).

Every replay is checked bitwise against the same sequence run eagerly, with eager work and
synchronisations between replays, and the last step against the oracle.
"""

import copy

import numpy as np
import pytest
import torch

import oracle
import paged_kv_chunk_amd as pkc
from synth import make_chunk_cohort
from gpu_helpers import TOL, bits, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"

B, H, D, C, S, L = 3, 2, 64, 16, 16, 3
RUNG = 96                                  # max_cache_seqlen the step is captured with
START = [0, 16, 37]                        # cache lengths at the first step
STEP_LENS = [[C, C, C], [C, C, C], [C, 11, C], [C, 5, 0]]   # real frames per step (0: padding lane)


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def make_layers():
    layers = []
    base = None
    for l in range(L):
        co = make_chunk_cohort(B, H, D, C, S, [RUNG] * B, dtype=torch.bfloat16, seed=50 + l,
                               device=DEV)
        if base is None:
            base = co
        co.block_tables = base.block_tables          # one table for every layer's pool
        co.out = torch.empty_like(co.q)
        layers.append(co)
    cs = torch.tensor(START, dtype=torch.int32, device=DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    return layers, base.block_tables, cs, lens


def step_inputs(step):
    """The chunk inputs of one step, per layer (seeded, drawn on the host)."""
    g = torch.Generator().manual_seed(1000 + step)
    shape = (B, C, H, D)
    return [[torch.randn(shape, generator=g).to(torch.bfloat16) for _ in range(3)] for _ in range(L)]


def load_step(layers, lens, step):
    for co, (q, k, v) in zip(layers, step_inputs(step)):
        co.q.copy_(q)
        co.k_new.copy_(k)
        co.v_new.copy_(v)
    lens.copy_(torch.tensor(STEP_LENS[step], dtype=torch.int32))


def test_captured_step_replays_a_growing_stream():
    layers, bt, cs, lens = make_layers()
    # eager reference on a copy of the whole state
    ref_layers = [copy.copy(co) for co in layers]
    for co, r in zip(layers, ref_layers):
        for n in ["q", "k_new", "v_new", "k_pool", "v_pool", "out"]:
            setattr(r, n, getattr(co, n).clone())
    ref_cs, ref_lens = cs.clone(), lens.clone()
    ref_out = []
    before_last = None
    for step in range(len(STEP_LENS)):
        load_step(ref_layers, ref_lens, step)
        if step == len(STEP_LENS) - 1:
            before_last = (host64(ref_layers[0].k_pool), host64(ref_layers[0].v_pool),
                           ref_cs.cpu().numpy().copy())
        for co in ref_layers:
            pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool, bt,
                                            ref_cs, co.pos, co.pos_bias_u, co.pos_bias_v, RUNG,
                                            out=co.out, chunk_lens=ref_lens)
        pkc.paged_kv_commit(ref_cs, C, chunk_lens=ref_lens)
        torch.cuda.synchronize()
        ref_out.append([bits(co.out) for co in ref_layers])

    # capture one step on the real state, then replay it
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            pkc.paged_kv_append_relpos_attn_layers(layers, bt, cs, RUNG, chunk_lens=lens,
                                                   stream=side)
            pkc.paged_kv_commit(cs, C, chunk_lens=lens, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert cs.cpu().tolist() == START            # capturing ran nothing

    for step in range(len(STEP_LENS)):
        load_step(layers, lens, step)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l, co in enumerate(layers):
            np.testing.assert_array_equal(bits(co.out), ref_out[step][l], err_msg=f"step {step} layer {l}")
    expect = np.array(START) + np.array(STEP_LENS).sum(axis=0)
    assert cs.cpu().tolist() == expect.tolist() == ref_cs.cpu().tolist()
    for co, r in zip(layers, ref_layers):
        np.testing.assert_array_equal(bits(co.k_pool), bits(r.k_pool))
        np.testing.assert_array_equal(bits(co.v_pool), bits(r.v_pool))

    # the last step of layer 0 against the oracle
    kp, vp, c_last = before_last
    q, k, v = [host64(x) for x in step_inputs(len(STEP_LENS) - 1)[0]]
    co = layers[0]
    lens_last = np.array(STEP_LENS[-1])
    kp2, vp2 = oracle.paged_kv_append(kp, vp, k, v, bt.cpu().numpy(), c_last, lens_last)
    ref = oracle.chunk_relpos_attn(q, kp2, vp2, bt.cpu().numpy(), c_last, host64(co.pos),
                                   host64(co.pos_bias_u), host64(co.pos_bias_v),
                                   chunk_lens=lens_last)
    out = co.out.detach().cpu().double().numpy()
    assert np.abs(out - ref).max() <= TOL[torch.bfloat16]


def test_layers_entry_equals_per_layer_calls_bitwise():
    layers, bt, cs, lens = make_layers()
    lens.fill_(C)
    twin = [copy.copy(co) for co in layers]
    for co, r in zip(layers, twin):
        for n in ["k_pool", "v_pool", "out"]:
            setattr(r, n, getattr(co, n).clone())
    pkc.paged_kv_append_relpos_attn_layers(layers, bt, cs, RUNG)
    for co in twin:
        pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool, bt, cs,
                                        co.pos, co.pos_bias_u, co.pos_bias_v, RUNG, out=co.out)
    torch.cuda.synchronize()
    for co, r in zip(layers, twin):
        np.testing.assert_array_equal(bits(co.out), bits(r.out))
        np.testing.assert_array_equal(bits(co.k_pool), bits(r.k_pool))


def test_bounded_history_stream_from_one_graph():
    """num_left_chunks = 3 over a ring of 4 pages: eight steps (the ring wraps twice) replayed
    from one captured step - layers plus the evicting commit - equal the eager sequence bitwise
    and, on the last step, the oracle's bounded-history streaming."""
    Bq, Lq, K, steps = 2, 2, 3, 8
    cap = K * C
    M = (cap + C) // S
    layers = []
    base = None
    for l in range(Lq):
        co = make_chunk_cohort(Bq, H, D, C, S, [cap] * Bq, dtype=torch.bfloat16, seed=70 + l,
                               device=DEV, max_blocks_per_seq=M)
        if base is None:
            base = co
        co.block_tables = base.block_tables
        co.out = torch.empty_like(co.q)
        layers.append(co)
    bt = base.block_tables
    assert (bt >= 0).all()                                  # every ring entry is a page
    cs = torch.zeros(Bq, dtype=torch.int32, device=DEV)
    ws = torch.tensor([0, 5 * S], dtype=torch.int32, device=DEV)    # stream 1 starts mid-ring
    ref = [copy.copy(co) for co in layers]
    for co, r in zip(layers, ref):
        for n in ["q", "k_new", "v_new", "k_pool", "v_pool", "out"]:
            setattr(r, n, getattr(co, n).clone())
    ref_cs, ref_ws = cs.clone(), ws.clone()

    def inputs(step):
        g = torch.Generator().manual_seed(2000 + step)
        return [[torch.randn((Bq, C, H, D), generator=g).to(torch.bfloat16) for _ in range(3)]
                for _ in range(Lq)]

    def load(ls, step):
        for co, (q, k, v) in zip(ls, inputs(step)):
            co.q.copy_(q)
            co.k_new.copy_(k)
            co.v_new.copy_(v)

    ref_out, snap = [], None
    for step in range(steps):
        load(ref, step)
        if step == steps - 1:
            snap = (host64(ref[0].k_pool), host64(ref[0].v_pool), ref_cs.cpu().numpy().copy(),
                    ref_ws.cpu().numpy().copy())
        pkc.paged_kv_append_relpos_attn_layers(ref, bt, ref_cs, cap, window_start=ref_ws)
        pkc.paged_kv_commit(ref_cs, C, window_start=ref_ws, max_cached_frames=cap, block_size=S)
        torch.cuda.synchronize()
        ref_out.append([bits(co.out) for co in ref])
        assert int(ref_cs.max()) <= cap

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            pkc.paged_kv_append_relpos_attn_layers(layers, bt, cs, cap, window_start=ws,
                                                   stream=side)
            pkc.paged_kv_commit(cs, C, window_start=ws, max_cached_frames=cap, block_size=S,
                                stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for step in range(steps):
        load(layers, step)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l, co in enumerate(layers):
            np.testing.assert_array_equal(bits(co.out), ref_out[step][l], err_msg=f"step {step}")
    assert cs.cpu().tolist() == ref_cs.cpu().tolist() == [cap] * Bq
    assert ws.cpu().tolist() == ref_ws.cpu().tolist() == [steps * C - cap, 5 * S + steps * C - cap]

    kp, vp, c_last, w_last = snap
    q, k, v = [host64(x) for x in inputs(steps - 1)[0]]
    btn = bt.cpu().numpy()
    kp2, vp2 = oracle.paged_kv_append(kp, vp, k, v, btn, c_last, window_start=w_last)
    co = layers[0]
    expect = oracle.chunk_relpos_attn(q, kp2, vp2, btn, c_last, host64(co.pos),
                                      host64(co.pos_bias_u), host64(co.pos_bias_v),
                                      window_start=w_last)
    assert np.abs(co.out.detach().cpu().double().numpy() - expect).max() <= TOL[torch.bfloat16]
