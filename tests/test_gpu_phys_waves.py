"""GPU: the chunk attention's launch choices - physical waves per workgroup and stream order.

The kernel splits a unit's keys over four virtual waves and merges them in a fixed order; a
large cohort runs them on fewer physical waves (more units per CU at once). A grid that takes more
than one pass over the CUs runs its streams longest cache first. Both are launch choices only:
outputs and pools must be bit-identical under every choice, and match the oracle.
PKC_CHUNK_WAVES and PKC_CHUNK_ORDER force them (read by the library at each launch).
"""

import os

import numpy as np
import pytest
import torch

import paged_kv_chunk_amd as pkc
from synth import make_chunk_cohort, make_config
from gpu_helpers import TOL, bits, max_err, oracle_chunk, poison

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = torch.bfloat16

# bf16, fused, no chunk lengths or window starts: the variants that run at fewer physical waves.
# Cache lengths put the virtual waves' boundaries at every offset inside a physical wave's range,
# with empty virtual waves (short caches), a partial last page and caches of 0.
COHORTS = {
    "ragged_S16": dict(B=6, H=2, D=64, C=16, block_size=16,
                       cache_seqlens=[0, 5, 37, 100, 257, 640], dtype=BF16),
    "ragged_S32_per_row": dict(B=5, H=2, D=64, C=16, block_size=32,
                               cache_seqlens=[0, 31, 96, 161, 1024], dtype=BF16,
                               per_row_pos=True, pos_noise=0.5),
    "gqa_odd_chunk": dict(B=4, H=4, Hk=2, D=64, C=13, block_size=16,
                          cache_seqlens=[3, 64, 200, 513], dtype=BF16),
    "chunk32": dict(B=3, H=2, D=64, C=32, block_size=16, cache_seqlens=[31, 250, 0], dtype=BF16),
    "single_query": dict(B=3, H=2, D=64, C=1, block_size=16, cache_seqlens=[0, 1, 255],
                         dtype=BF16),
    "steps_1_to_9": dict(B=9, H=1, D=64, C=16, block_size=16,
                         cache_seqlens=[32 * k for k in range(1, 10)], dtype=BF16),
}


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu] {request.node.nodeid}", flush=True)
    yield
    os.environ.pop("PKC_CHUNK_WAVES", None)
    os.environ.pop("PKC_CHUNK_ORDER", None)
    torch.cuda.synchronize()


def clone(co):
    import copy
    c2 = copy.copy(co)
    c2.k_pool = co.k_pool.clone()
    c2.v_pool = co.v_pool.clone()
    return c2


def fused(co, waves):
    os.environ["PKC_CHUNK_WAVES"] = str(waves)
    out = pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool,
                                          co.block_tables, co.cache_seqlens, co.pos,
                                          co.pos_bias_u, co.pos_bias_v, co.max_cache_seqlen,
                                          per_row_pos=co.per_row_pos)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", sorted(COHORTS))
def test_physical_waves_bit_identical_and_match_oracle(name):
    co = poison(make_chunk_cohort(seed=11, device=DEV, **COHORTS[name]))
    ref = oracle_chunk(co)
    runs = {}
    for w in (4, 2, 1):
        c = clone(co)
        runs[w] = (fused(c, w), c)
    out4, c4 = runs[4]
    assert max_err(out4, ref) <= TOL[BF16], max_err(out4, ref)
    for w in (2, 1):
        out, c = runs[w]
        np.testing.assert_array_equal(bits(out), bits(out4), err_msg=f"{w} waves: out")
        np.testing.assert_array_equal(bits(c.k_pool), bits(c4.k_pool), err_msg=f"{w} waves: k")
        np.testing.assert_array_equal(bits(c.v_pool), bits(c4.v_pool), err_msg=f"{w} waves: v")


@pytest.mark.parametrize("cfg", [2, 3])
def test_physical_waves_bit_identical_on_workloads(cfg):
    """The d_model 512 cohort (where one physical wave is chosen by default on MI355X) and the
    ragged per-row cohort (four): every count gives the same bits as four, and so does the
    default choice."""
    co = make_config(cfg, device=DEV)
    base = fused(clone(co), 4)
    for w in (2, 1):
        np.testing.assert_array_equal(bits(fused(clone(co), w)), bits(base), err_msg=f"{w} waves")
    os.environ.pop("PKC_CHUNK_WAVES", None)
    np.testing.assert_array_equal(bits(fused_default(clone(co))), bits(base))


def fused_default(co):
    out = pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool,
                                          co.block_tables, co.cache_seqlens, co.pos,
                                          co.pos_bias_u, co.pos_bias_v, co.max_cache_seqlen,
                                          per_row_pos=co.per_row_pos)
    torch.cuda.synchronize()
    return out


def test_one_wave_graph_replays_match_eager():
    """The one-wave launch captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, gives the four-wave eager bits."""
    co = make_chunk_cohort(seed=12, device=DEV, **COHORTS["ragged_S16"])
    eager = fused(clone(co), 4)
    os.environ["PKC_CHUNK_WAVES"] = "1"
    c = clone(co)
    out = torch.empty_like(co.q)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            pkc.paged_kv_append_relpos_attn(c.q, c.k_new, c.v_new, c.k_pool, c.v_pool,
                                            c.block_tables, c.cache_seqlens, c.pos,
                                            c.pos_bias_u, c.pos_bias_v, c.max_cache_seqlen,
                                            out=out, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out), bits(eager), err_msg=f"replay {r}")
        _ = (co.q.float() * 2).sum().item()   # unrelated eager work between replays


def ordered(co, waves, order):
    os.environ["PKC_CHUNK_ORDER"] = str(order)
    return fused(co, waves)


@pytest.mark.parametrize("name", sorted(COHORTS))
def test_longest_first_order_bit_identical(name):
    """Streams run longest cache first (ranked inside each workgroup, at four physical waves)
    give the bits of index order, pools included; at one physical wave the order switch is
    ignored and the bits are the same again."""
    co = make_chunk_cohort(seed=13, device=DEV, **COHORTS[name])
    c0 = clone(co)
    base = ordered(c0, 4, 0)
    for waves in (4, 1):
        c = clone(co)
        out = ordered(c, waves, 1)
        np.testing.assert_array_equal(bits(out), bits(base), err_msg=f"{waves} waves")
        np.testing.assert_array_equal(bits(c.k_pool), bits(c0.k_pool))
        np.testing.assert_array_equal(bits(c.v_pool), bits(c0.v_pool))


def test_longest_first_order_many_streams():
    """More than 64 streams (the ranking walks them in groups of 64), cache lengths with ties
    and empty caches: every order gives the same bits, and the oracle's values."""
    rng = np.random.default_rng(5)
    cache = (rng.integers(0, 40, size=150) * 16).tolist()
    cache[::7] = [0] * len(cache[::7])
    co = poison(make_chunk_cohort(150, 2, 64, 16, 16, cache, dtype=BF16, seed=14, device=DEV))
    ref = oracle_chunk(co)
    base = ordered(clone(co), 4, 0)
    assert max_err(base, ref) <= TOL[BF16]
    np.testing.assert_array_equal(bits(ordered(clone(co), 4, 1)), bits(base))
    # the unfused entry (append, then attention over the pool) ranks the same way
    c = clone(co)
    os.environ["PKC_CHUNK_ORDER"] = "1"
    pkc.paged_kv_append(c.k_new, c.v_new, c.k_pool, c.v_pool, c.block_tables, c.cache_seqlens,
                        c.max_cache_seqlen)
    out = pkc.chunk_paged_relpos_attn(c.q, c.k_pool, c.v_pool, c.block_tables, c.cache_seqlens,
                                      c.pos, c.pos_bias_u, c.pos_bias_v, c.max_cache_seqlen)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(base))


@pytest.mark.parametrize("cfg", [2, 3])
def test_longest_first_order_on_workloads(cfg):
    co = make_config(cfg, device=DEV)
    base = ordered(clone(co), 4, 0)
    np.testing.assert_array_equal(bits(ordered(clone(co), 4, 1)), bits(base))
