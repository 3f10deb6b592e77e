"""GPU parity of the positional tables stored in 32-dim column blocks per head, of the
bounded-history commit when the cap is below one block, and of the memory-path ceiling kernel's
writes.

A column-blocked table holds the same values as the row-major one at other addresses, so every
output must be bitwise equal to the row-major run; the full workloads are also checked against the
float64 oracle in the launch configuration the benchmark times (the fused entry, blocked tables).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_chunk_amd as pkc
from synth import add_blocked_table, make_chunk_cohort, make_config, use_key_position_tables
from gpu_helpers import TOL, bits, max_err, oracle_chunk, poison

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def run(co, fused, blocked, chunk_lens=None):
    """One layer on the GPU with the row-major or the column-blocked table (pools updated)."""
    pos = co.pos_cb if blocked else co.pos
    kw = dict(per_row_pos=co.per_row_pos, per_key_pos=co.per_key_pos, chunk_lens=chunk_lens,
              pos_blocked=blocked)
    if fused:
        return pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool,
                                               co.block_tables, co.cache_seqlens, pos,
                                               co.pos_bias_u, co.pos_bias_v, co.max_cache_seqlen,
                                               **kw)
    pkc.paged_kv_append(co.k_new, co.v_new, co.k_pool, co.v_pool, co.block_tables,
                        co.cache_seqlens, co.max_cache_seqlen, chunk_lens=chunk_lens)
    return pkc.chunk_paged_relpos_attn(co.q, co.k_pool, co.v_pool, co.block_tables,
                                       co.cache_seqlens, pos, co.pos_bias_u, co.pos_bias_v,
                                       co.max_cache_seqlen, **kw)


def twin(co):
    import copy
    c2 = copy.copy(co)
    c2.k_pool = co.k_pool.clone()
    c2.v_pool = co.v_pool.clone()
    return c2


CASES = {
    "bf16_shared": dict(B=3, H=2, D=64, C=16, block_size=16, cache_seqlens=[0, 37, 100], dtype=BF16),
    "fp32_shared": dict(B=3, H=2, D=64, C=16, block_size=16, cache_seqlens=[0, 37, 100], dtype=F32),
    "bf16_per_row": dict(B=4, H=2, D=64, C=16, block_size=32, cache_seqlens=[0, 16, 48, 272],
                         dtype=BF16, per_row_pos=True, pos_noise=0.5),
    "fp32_per_row": dict(B=4, H=2, D=64, C=16, block_size=32, cache_seqlens=[0, 16, 48, 272],
                         dtype=F32, per_row_pos=True, pos_noise=0.5),
    "gqa_odd": dict(B=4, H=4, Hk=2, D=64, C=13, block_size=8, cache_seqlens=[5, 11, 1, 90],
                    dtype=BF16),
    "chunk32": dict(B=3, H=2, D=64, C=32, block_size=16, cache_seqlens=[31, 63, 0], dtype=BF16),
    "long_chunk": dict(B=3, H=2, D=64, C=80, block_size=16, cache_seqlens=[45, 128, 0],
                       dtype=BF16),
    "long_cache": dict(B=1, H=2, D=64, C=16, block_size=64, cache_seqlens=[1000], dtype=BF16),
}


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", sorted(CASES))
def test_blocked_tables_equal_row_major_bitwise(name, fused):
    co = poison(make_chunk_cohort(seed=31, device=DEV, **CASES[name]))
    add_blocked_table(co)
    ref = oracle_chunk(co)
    co2 = twin(co)
    out_r = run(co, fused, blocked=False)
    out_b = run(co2, fused, blocked=True)
    assert max_err(out_b, ref) <= TOL[co.q.dtype], (name, max_err(out_b, ref))
    np.testing.assert_array_equal(bits(out_r), bits(out_b))
    np.testing.assert_array_equal(bits(co.k_pool), bits(co2.k_pool))
    np.testing.assert_array_equal(bits(co.v_pool), bits(co2.v_pool))


@pytest.mark.parametrize("per_row", [False, True])
def test_blocked_per_key_tables_equal_row_major_bitwise(per_row):
    co = make_chunk_cohort(seed=32, device=DEV, **CASES["gqa_odd"])
    use_key_position_tables(co, [5, 0, 100, 7], per_row=per_row)
    add_blocked_table(co)
    lens = torch.tensor([13, 4, 0, 9], dtype=torch.int32, device=DEV)
    co2 = twin(co)
    out_r = run(co, True, blocked=False, chunk_lens=lens)
    out_b = run(co2, True, blocked=True, chunk_lens=lens)
    np.testing.assert_array_equal(bits(out_r), bits(out_b))


@pytest.mark.parametrize("cfg,streams", [(0, None), (1, None), (2, "sample"), (3, None)])
def test_workloads_blocked_fused_against_the_oracle(cfg, streams):
    """The benchmark's launch configuration (fused entry, column-blocked tables) at each
    workload's full size: every stream against the oracle (16 sampled streams for the d_model 512
    cohort), and bitwise equal to the row-major run."""
    co = add_blocked_table(make_config(cfg, device=DEV))
    B = co.q.shape[0]
    if streams == "sample":
        streams = sorted(np.random.default_rng(cfg).choice(B, size=16, replace=False).tolist())
    ref = oracle_chunk(co, streams)
    co2 = twin(co)
    out = run(co, True, blocked=True)
    sel = slice(None) if streams is None else torch.as_tensor(streams, device=DEV)
    err = max_err(out[sel], ref)
    assert err <= TOL[co.q.dtype], (cfg, err)
    np.testing.assert_array_equal(bits(out), bits(run(co2, True, blocked=False)))


def test_commit_with_a_cap_below_one_block_matches_the_oracle():
    """Bounded history with max_cached_frames below a block: only filled blocks leave, cache
    lengths stay >= 0 and the window start never passes the next frame's position."""
    rng = np.random.default_rng(37)
    B, C, S = 300, 16, 8
    for cap in (0, 3, 7, 8, 13):
        cache = rng.integers(0, 3 * S, size=B).astype(np.int32)
        start = (rng.integers(0, 1000, size=B) * S).astype(np.int32)
        lens = rng.integers(0, C + 1, size=B).astype(np.int32)
        ec, es = oracle.commit_chunk(cache, C, chunk_lens=lens, window_start=start,
                                     max_cached_frames=cap, block_size=S)
        c_t, s_t = torch.from_numpy(cache).to(DEV), torch.from_numpy(start).to(DEV)
        pkc.paged_kv_commit(c_t, C, chunk_lens=torch.from_numpy(lens).to(DEV), window_start=s_t,
                            max_cached_frames=cap, block_size=S)
        got_c, got_s = c_t.cpu().numpy(), s_t.cpu().numpy()
        assert got_c.tolist() == ec.tolist(), cap
        assert got_s.tolist() == es.tolist(), cap
        assert (got_c >= 0).all()
        assert (got_s <= start + cache + lens).all()


@pytest.mark.parametrize("cfg", [1, 3])
@pytest.mark.parametrize("waves,split", [(4, 1), (8, 1), (4, 2), (1, 1)])
def test_gather_read_writes_the_pools_as_the_append(cfg, waves, split):
    """The memory-path ceiling kernel appends the chunk exactly as paged_kv_append does (it
    touches no other pool element); its `out` is unspecified and not checked."""
    co = add_blocked_table(make_config(cfg, device=DEV))
    kb, vb = bits(co.k_pool), bits(co.v_pool)
    ek, ev = oracle.paged_kv_append(kb, vb, bits(co.k_new), bits(co.v_new),
                                    co.block_tables.cpu().numpy(), co.cache_seqlens.cpu().numpy())
    out = torch.empty_like(co.q)
    for blocked in (False, True):
        pkc.gather_read(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool, co.block_tables,
                        co.cache_seqlens, co.pos_cb if blocked else co.pos, co.pos_bias_u,
                        co.pos_bias_v, co.max_cache_seqlen, out, per_row_pos=co.per_row_pos,
                        pos_blocked=blocked, waves=waves, split=split)
        torch.cuda.synchronize()
        assert (bits(co.k_pool) == ek).all()
        assert (bits(co.v_pool) == ev).all()
