"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Tolerances (max-abs over every compared output): 2e-2 for bf16 storage, 1e-4 for fp32; the
append and the block indexing are compared bit for bit. Every input is seeded and synthetic.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_chunk_amd as pkc
from synth import make_chunk_cohort, make_config, make_varlen_cohort, use_key_position_tables
from gpu_helpers import TOL, bits, compact, host64, max_err, oracle_chunk, poison, poison_padding

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def gpu_chunk(co, fused=False, chunk_lens=None):
    """Run one layer on the GPU (append then attention, or the fused entry). Pools are updated."""
    if fused:
        return pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool,
                                               co.block_tables, co.cache_seqlens, co.pos,
                                               co.pos_bias_u, co.pos_bias_v, co.max_cache_seqlen,
                                               per_row_pos=co.per_row_pos, chunk_lens=chunk_lens,
                                               per_key_pos=co.per_key_pos)
    pkc.paged_kv_append(co.k_new, co.v_new, co.k_pool, co.v_pool, co.block_tables,
                        co.cache_seqlens, co.max_cache_seqlen, chunk_lens=chunk_lens)
    return pkc.chunk_paged_relpos_attn(co.q, co.k_pool, co.v_pool, co.block_tables,
                                       co.cache_seqlens, co.pos, co.pos_bias_u, co.pos_bias_v,
                                       co.max_cache_seqlen, per_row_pos=co.per_row_pos,
                                       chunk_lens=chunk_lens, per_key_pos=co.per_key_pos)


def clone(co):
    import copy
    c2 = copy.copy(co)
    c2.k_pool = co.k_pool.clone()
    c2.v_pool = co.v_pool.clone()
    return c2


# --------------------------------------------------------------------------------------------
# Paged append: bit-exact on the whole pool
# --------------------------------------------------------------------------------------------

SMALL = {
    "fp32_ragged": dict(B=3, H=2, D=64, C=16, block_size=16, cache_seqlens=[0, 37, 100], dtype=F32),
    "bf16_ragged": dict(B=3, H=2, D=64, C=16, block_size=16, cache_seqlens=[0, 37, 100], dtype=BF16),
    "partial_tile_S8": dict(B=3, H=2, D=64, C=5, block_size=8, cache_seqlens=[3, 0, 64], dtype=BF16),
    "two_tiles_per_row": dict(B=2, H=2, D=64, C=20, block_size=32, cache_seqlens=[7, 50],
                              dtype=BF16, per_row_pos=True, pos_noise=0.5),
    "gqa_h4_k2": dict(B=3, H=4, Hk=2, D=64, C=16, block_size=16, cache_seqlens=[31, 8, 129],
                      dtype=BF16),
    "gqa_h4_k1_fp32": dict(B=2, H=4, Hk=1, D=64, C=16, block_size=16, cache_seqlens=[31, 8],
                           dtype=F32),
    "single_query": dict(B=3, H=2, D=64, C=1, block_size=16, cache_seqlens=[0, 1, 255], dtype=BF16),
    "long_cache": dict(B=1, H=2, D=64, C=16, block_size=64, cache_seqlens=[1000], dtype=BF16),
    "per_row_ragged_fp32": dict(B=4, H=2, D=64, C=16, block_size=32, cache_seqlens=[0, 16, 48, 272],
                                dtype=F32, per_row_pos=True, pos_noise=0.5),
    "odd_lengths": dict(B=4, H=2, D=64, C=13, block_size=8, cache_seqlens=[5, 11, 1, 90],
                        dtype=BF16),
    # the largest tail the register-held staging takes (31 pool keys + 32 chunk frames) ...
    "chunk32_full_tail": dict(B=3, H=2, D=64, C=32, block_size=16, cache_seqlens=[31, 63, 0],
                              dtype=BF16),
    # ... and bf16 chunks past it, staged by the loop
    "long_chunk_bf16": dict(B=3, H=2, D=64, C=80, block_size=16, cache_seqlens=[45, 128, 0],
                            dtype=BF16),
    # the longest chunks the LDS staging takes (dynamic LDS past 64 KB)
    "max_chunk_bf16": dict(B=2, H=2, D=64, C=512, block_size=32, cache_seqlens=[40, 0],
                           dtype=BF16),
    "max_chunk_fp32": dict(B=1, H=2, D=64, C=256, block_size=16, cache_seqlens=[77], dtype=F32),
    # pages near the 128-entry block-ID window each wave keeps in LDS: blocks of 16 and 32 whose
    # last pages (125 of 126) still lie in it, and blocks of 16 past it (133 pages: IDs past the
    # window read from the table)
    "window_edge_S16": dict(B=2, H=2, D=64, C=16, block_size=16, cache_seqlens=[2000, 9],
                            dtype=BF16),
    "window_edge_S32": dict(B=2, H=2, D=64, C=16, block_size=32, cache_seqlens=[4000, 70],
                            dtype=BF16),
    "past_window_S16": dict(B=2, H=2, D=64, C=16, block_size=16, cache_seqlens=[2100, 33],
                            dtype=BF16),
}


def small_cohort(name, seed=0):
    return make_chunk_cohort(seed=seed, device=DEV, **SMALL[name])


@pytest.mark.parametrize("name", sorted(SMALL))
def test_append_bit_exact_small(name):
    co = small_cohort(name)
    kb, vb = bits(co.k_pool), bits(co.v_pool)
    ek, ev = oracle.paged_kv_append(kb, vb, bits(co.k_new), bits(co.v_new),
                                    co.block_tables.cpu().numpy(), co.cache_seqlens.cpu().numpy())
    pkc.paged_kv_append(co.k_new, co.v_new, co.k_pool, co.v_pool, co.block_tables,
                        co.cache_seqlens, co.max_cache_seqlen)
    np.testing.assert_array_equal(bits(co.k_pool), ek)
    np.testing.assert_array_equal(bits(co.v_pool), ev)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_append_bit_exact_workloads(cfg):
    co = make_config(cfg, device=DEV)
    kb, vb = bits(co.k_pool), bits(co.v_pool)
    ek, ev = oracle.paged_kv_append(kb, vb, bits(co.k_new), bits(co.v_new),
                                    co.block_tables.cpu().numpy(), co.cache_seqlens.cpu().numpy())
    pkc.paged_kv_append(co.k_new, co.v_new, co.k_pool, co.v_pool, co.block_tables,
                        co.cache_seqlens, co.max_cache_seqlen)
    assert (bits(co.k_pool) == ek).all()
    assert (bits(co.v_pool) == ev).all()


# --------------------------------------------------------------------------------------------
# Attention parity
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", sorted(SMALL))
def test_attention_parity_small(name):
    co = poison(small_cohort(name, seed=3))
    ref = oracle_chunk(co)
    out = gpu_chunk(co)
    err = max_err(out, ref)
    assert err <= TOL[co.q.dtype], (name, err)


@pytest.mark.parametrize("name", ["bf16_ragged", "two_tiles_per_row", "gqa_h4_k2", "odd_lengths",
                                  "per_row_ragged_fp32", "chunk32_full_tail", "long_chunk_bf16",
                                  "max_chunk_bf16"])
def test_fused_equals_append_then_attend(name):
    """The fused entry writes the same pool bits and produces the same output bits (both entries
    split the keys and assign them to waves by the cache length alone)."""
    co = small_cohort(name, seed=4)
    ref = oracle_chunk(co)
    co2 = clone(co)
    out_a = gpu_chunk(co)
    out_f = gpu_chunk(co2, fused=True)
    tol = TOL[co.q.dtype]
    assert max_err(out_a, ref) <= tol, ("append+attend", max_err(out_a, ref))
    assert max_err(out_f, ref) <= tol, ("fused", max_err(out_f, ref))
    np.testing.assert_array_equal(bits(co.k_pool), bits(co2.k_pool))
    np.testing.assert_array_equal(bits(co.v_pool), bits(co2.v_pool))
    np.testing.assert_array_equal(bits(out_a), bits(out_f))


@pytest.mark.parametrize("cfg,streams", [(0, None), (1, None), (2, "sample"), (3, None)])
def test_attention_parity_workloads(cfg, streams):
    co = make_config(cfg, device=DEV)
    B = co.q.shape[0]
    if streams == "sample":
        rng = np.random.default_rng(cfg)
        streams = sorted(rng.choice(B, size=16, replace=False).tolist())
    ref = oracle_chunk(co, streams)
    co_f = clone(co)
    out = gpu_chunk(co)
    sel = slice(None) if streams is None else torch.as_tensor(streams, device=DEV)
    err = max_err(out[sel], ref)
    assert err <= TOL[co.q.dtype], (cfg, err)
    out_f = gpu_chunk(co_f, fused=True)
    np.testing.assert_array_equal(bits(out), bits(out_f))


def test_attention_random_cohorts():
    """A seeded sweep of cohort shapes: streams, heads (GQA), chunk sizes from 1 to 96, block
    sizes from 8 to 64, ragged cache lengths (empty caches and partial blocks included), shared
    or per-row tables, bf16 and fp32. Each cohort against the oracle, with the fused entry and
    the append + attention pair bitwise equal, pools included."""
    rng = np.random.default_rng(71)
    for i in range(12):
        dtype = torch.float32 if i % 4 == 3 else torch.bfloat16
        Hk = int(rng.choice([1, 2, 4]))
        H = Hk * int(rng.choice([1, 2]))
        C = int(rng.choice([1, 5, 16, 17, 32, 48, 96]))
        S = int(rng.choice([8, 16, 32, 64]))
        B = int(rng.integers(1, 24))
        caches = rng.integers(0, 400, size=B).tolist()
        per_row = bool(rng.integers(0, 2))
        co = poison(make_chunk_cohort(B, H, 64, C, S, caches, Hk=Hk, dtype=dtype,
                                      per_row_pos=per_row, pos_noise=0.5 if per_row else 0.0,
                                      seed=80 + i, device=DEV))
        what = f"B={B} H={H} Hk={Hk} C={C} S={S} per_row={per_row} {dtype}"
        ref = oracle_chunk(co)
        co2 = clone(co)
        out_a = gpu_chunk(co)
        out_f = gpu_chunk(co2, fused=True)
        torch.cuda.synchronize()
        assert max_err(out_f, ref) <= TOL[dtype], (what, max_err(out_f, ref))
        np.testing.assert_array_equal(bits(out_a), bits(out_f), err_msg=what)
        np.testing.assert_array_equal(bits(co.k_pool), bits(co2.k_pool), err_msg=what)
        np.testing.assert_array_equal(bits(co.v_pool), bits(co2.v_pool), err_msg=what)


def test_block_relabelling_is_bitwise_invariant():
    co = small_cohort("bf16_ragged", seed=5)
    N = co.k_pool.shape[0]
    pi = torch.randperm(N, generator=torch.Generator().manual_seed(1)).to(DEV)
    co2 = clone(co)
    co2.k_pool[pi] = co.k_pool
    co2.v_pool[pi] = co.v_pool
    bt = co.block_tables.long()
    co2.block_tables = torch.where(bt >= 0, pi[bt.clamp(min=0)], bt).to(torch.int32)
    np.testing.assert_array_equal(bits(gpu_chunk(co)), bits(gpu_chunk(co2)))


def test_row_results_do_not_depend_on_the_cohort():
    """Row-locality: a stream's output bits are the same alone, in a cohort, and after the
    cohort's rows are permuted."""
    co = small_cohort("bf16_ragged", seed=6)
    full = gpu_chunk(clone(co))
    for b in range(co.q.shape[0]):
        one = clone(co)
        one.q = co.q[b:b + 1].contiguous()
        one.k_new = co.k_new[b:b + 1].contiguous()
        one.v_new = co.v_new[b:b + 1].contiguous()
        one.block_tables = co.block_tables[b:b + 1].contiguous()
        one.cache_seqlens = co.cache_seqlens[b:b + 1].contiguous()
        np.testing.assert_array_equal(bits(gpu_chunk(one))[0], bits(full)[b])
    perm = torch.tensor([2, 0, 1], device=DEV)
    pc = clone(co)
    pc.q = co.q[perm].contiguous()
    pc.k_new = co.k_new[perm].contiguous()
    pc.v_new = co.v_new[perm].contiguous()
    pc.block_tables = co.block_tables[perm].contiguous()
    pc.cache_seqlens = co.cache_seqlens[perm].contiguous()
    np.testing.assert_array_equal(bits(gpu_chunk(pc)), bits(full)[perm.cpu().numpy()])


def test_uniform_cache_shared_and_per_row_tables_agree():
    co = make_chunk_cohort(3, 2, 64, 16, 16, [48, 48, 48], dtype=BF16, seed=9, device=DEV)
    per = clone(co)
    per.pos = co.pos[None].expand(3, *co.pos.shape).contiguous()
    per.per_row_pos = True
    np.testing.assert_array_equal(bits(gpu_chunk(co)), bits(gpu_chunk(per)))


# --------------------------------------------------------------------------------------------
# Packed varlen
# --------------------------------------------------------------------------------------------

def gpu_varlen(co):
    return pkc.varlen_packed_relpos_attn(co.q, co.k, co.v, co.cu_seqlens, co.pos, co.pos_bias_u,
                                         co.pos_bias_v, max(co.lengths))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_varlen_parity_small(dtype):
    # 1 to 9 key steps of 32: even and odd step counts (bf16 stages two steps, fp32 pairs its
    # one-step stages), every way a length ends - whole stages only, a last stage of one or two
    # steps, its last step whole or cut - and one to three query tiles
    co = make_varlen_cohort([1, 5, 0, 16, 17, 32, 40, 64, 70, 96, 100, 128, 150, 257], 2, 64,
                            dtype=dtype, seed=2, device=DEV)
    ref = oracle.varlen_relpos_attn(host64(co.q), host64(co.k), host64(co.v),
                                    co.cu_seqlens.cpu().numpy(), host64(co.pos),
                                    host64(co.pos_bias_u), host64(co.pos_bias_v))
    err = max_err(gpu_varlen(co), ref)
    assert err <= TOL[dtype], err


def test_varlen_longer_than_max_seqlen_is_cut_in_bounds():
    # Out of contract: utterances longer than max_seqlen. Each is cut to its first max_seqlen
    # frames; frames past them keep what the output held, an utterance within the bound is exact,
    # and every written value is finite (the cut utterances' values are otherwise unspecified).
    lengths = [40, 100, 70]
    co = make_varlen_cohort(lengths, 2, 64, dtype=BF16, seed=5, device=DEV)
    sentinel = 7.0
    out = torch.full_like(co.q, sentinel)
    pkc.varlen_packed_relpos_attn(co.q, co.k, co.v, co.cu_seqlens, co.pos, co.pos_bias_u,
                                  co.pos_bias_v, 64, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu()
    cu = co.cu_seqlens.cpu().tolist()
    for s, n in enumerate(lengths):
        seg = got[cu[s]:cu[s + 1]]
        assert torch.isfinite(seg[:64]).all()
        assert (seg[64:] == sentinel).all()
    ref = oracle.varlen_relpos_attn(host64(co.q), host64(co.k), host64(co.v),
                                    co.cu_seqlens.cpu().numpy(), host64(co.pos),
                                    host64(co.pos_bias_u), host64(co.pos_bias_v))
    assert max_err(got[:40], ref[:40]) <= TOL[BF16]


def test_varlen_gqa_parity():
    co = make_varlen_cohort([33, 64, 7], 4, 64, Hk=2, dtype=BF16, seed=3, device=DEV)
    ref = oracle.varlen_relpos_attn(host64(co.q), host64(co.k), host64(co.v),
                                    co.cu_seqlens.cpu().numpy(), host64(co.pos),
                                    host64(co.pos_bias_u), host64(co.pos_bias_v))
    assert max_err(gpu_varlen(co), ref) <= TOL[BF16]


def test_varlen_random_batches():
    """A seeded sweep of packed batches: 1 to 10 utterances of 0 to 700 frames, heads with GQA,
    bf16 and fp32, each against the oracle."""
    rng = np.random.default_rng(73)
    for i in range(8):
        dtype = F32 if i % 4 == 3 else BF16
        Hk = int(rng.choice([1, 2, 4]))
        H = Hk * int(rng.choice([1, 2]))
        lengths = rng.integers(0, 700, size=int(rng.integers(1, 11))).tolist()
        co = make_varlen_cohort(lengths, H, 64, Hk=Hk, dtype=dtype, seed=90 + i, device=DEV)
        ref = oracle.varlen_relpos_attn(host64(co.q), host64(co.k), host64(co.v),
                                        co.cu_seqlens.cpu().numpy(), host64(co.pos),
                                        host64(co.pos_bias_u), host64(co.pos_bias_v))
        err = max_err(gpu_varlen(co), ref)
        assert err <= TOL[dtype], (lengths, H, Hk, dtype, err)


def test_varlen_workload_sampled():
    co = make_config(4, device=DEV)
    out = gpu_varlen(co)
    lengths = co.lengths
    segs = sorted({int(np.argmax(lengths)), int(np.argmin(lengths)), 0, len(lengths) - 1})
    rng = np.random.default_rng(4)

    def rows(n):
        pick = set(range(min(16, n))) | set(range(max(0, n - 16), n))
        pick |= set(rng.choice(n, size=min(16, n), replace=False).tolist())
        return sorted(pick)
    ref = oracle.varlen_relpos_attn(host64(co.q), host64(co.k), host64(co.v),
                                    co.cu_seqlens.cpu().numpy(), host64(co.pos),
                                    host64(co.pos_bias_u), host64(co.pos_bias_v),
                                    segments=segs, query_rows=rows)
    have = ~np.isnan(ref[:, 0, 0])
    assert have.sum() > 0
    g = out.detach().cpu().double().numpy()
    assert np.isfinite(g).all()
    err = float(np.abs(g[have] - ref[have]).max())
    assert err <= TOL[BF16], err


def test_varlen_segment_equals_chunk_at_zero_cache():
    """A packed utterance of 16 frames is the chunk case with cache 0 and C = 16."""
    vc = make_varlen_cohort([16], 2, 64, dtype=BF16, seed=5, device=DEV)
    ch = make_chunk_cohort(1, 2, 64, 16, 16, [0], dtype=BF16, seed=5, device=DEV)
    ch.q = vc.q[None].contiguous()
    ch.k_new = vc.k[None].contiguous()
    ch.v_new = vc.v[None].contiguous()
    ch.pos = vc.pos[:31].contiguous()
    ch.pos_bias_u = vc.pos_bias_u
    ch.pos_bias_v = vc.pos_bias_v
    a = gpu_varlen(vc)
    b = gpu_chunk(ch)[0]
    # the two kernels round differently (bf16 operands), so they agree to the bf16 tolerance
    assert float((a.double() - b.double()).abs().max()) <= TOL[BF16]


def test_graph_replays_match_eager():
    """The fused entry captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bit for bit."""
    co = small_cohort("gqa_h4_k2", seed=7)
    eager = gpu_chunk(clone(co), fused=True)
    torch.cuda.synchronize()
    out = torch.empty_like(co.q)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool,
                                            co.block_tables, co.cache_seqlens, co.pos,
                                            co.pos_bias_u, co.pos_bias_v, co.max_cache_seqlen,
                                            out=out, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out), bits(eager), err_msg=f"replay {r}")
        _ = (co.q.float() * 2).sum().item()   # unrelated eager work between replays


# --------------------------------------------------------------------------------------------
# Per-row chunk lengths (short final windows) and padding lanes
# --------------------------------------------------------------------------------------------

def _lens_for(co, seed):
    """Seeded real-frame counts covering 0 (padding lane), 1, C and values in between."""
    B, C = co.q.shape[0], co.q.shape[1]
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, C + 1, size=B)
    for x, v in enumerate([0, C, 1]):
        if x < B:
            lens[x] = v
    return lens.astype(np.int32)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["bf16_ragged", "gqa_h4_k2", "odd_lengths", "per_row_ragged_fp32",
                                  "chunk32_full_tail", "long_chunk_bf16"])
def test_chunk_lens_parity(name, fused):
    """Streams with fewer real frames than the chunk width: the GPU writes exactly the oracle's
    pool bits (nothing past the real frames) and matches its output; padded rows are exactly
    zero. Padded frames are NaN everywhere, so any read of one shows."""
    co = poison(small_cohort(name, seed=6))
    lens = _lens_for(co, 7)
    poison_padding(co, lens)
    ref = oracle_chunk(co, chunk_lens=lens)
    kb, vb = bits(co.k_pool), bits(co.v_pool)
    ek, ev = oracle.paged_kv_append(kb, vb, bits(co.k_new), bits(co.v_new),
                                    co.block_tables.cpu().numpy(), co.cache_seqlens.cpu().numpy(), lens)
    out = gpu_chunk(co, fused=fused, chunk_lens=torch.from_numpy(lens).to(DEV))
    np.testing.assert_array_equal(bits(co.k_pool), ek)
    np.testing.assert_array_equal(bits(co.v_pool), ev)
    o = out.detach().cpu().double().numpy()
    C = co.q.shape[1]
    for b, n in enumerate(lens):
        assert (o[b, n:] == 0).all(), b
    assert np.abs(o - ref).max() <= TOL[co.q.dtype], (name, np.abs(o - ref).max())


def test_chunk_lens_fused_equals_unfused_bitwise():
    co = small_cohort("odd_lengths", seed=8)
    lens = _lens_for(co, 9)
    co2 = clone(co)
    t = torch.from_numpy(lens).to(DEV)
    a = gpu_chunk(co, chunk_lens=t)
    f = gpu_chunk(co2, fused=True, chunk_lens=t)
    np.testing.assert_array_equal(bits(a), bits(f))
    np.testing.assert_array_equal(bits(co.k_pool), bits(co2.k_pool))


def test_full_chunk_lens_equal_no_lens_bitwise():
    co = small_cohort("bf16_ragged", seed=10)
    co2 = clone(co)
    full = torch.full((co.q.shape[0],), co.q.shape[1], dtype=torch.int32, device=DEV)
    np.testing.assert_array_equal(bits(gpu_chunk(co, fused=True)),
                                  bits(gpu_chunk(co2, fused=True, chunk_lens=full)))


def test_padding_lanes_are_inert_and_leave_other_rows_bitwise_unchanged():
    """A cohort padded with lanes of chunk length 0, whose tables point only at a NaN scratch
    block: the real rows' outputs and pool bits are those of the unpadded cohort, the padding
    rows' outputs are zero and the scratch block is untouched."""
    co = make_config(0, device=DEV)
    base = clone(co)
    out_base = gpu_chunk(base, fused=True).clone()
    B, C, H, D = co.q.shape
    P = 3
    N = co.k_pool.shape[0]
    nan = float("nan")
    kp = torch.cat([co.k_pool, torch.full_like(co.k_pool[:1], nan)])
    vp = torch.cat([co.v_pool, torch.full_like(co.v_pool[:1], nan)])
    bt = torch.cat([co.block_tables, torch.full((P, co.block_tables.shape[1]), N, dtype=torch.int32,
                                                device=DEV)])
    cs = torch.cat([co.cache_seqlens, torch.tensor([0, 7, int(co.max_cache_seqlen)], dtype=torch.int32,
                                                   device=DEV)])
    pad = lambda x: torch.cat([x, torch.full((P,) + tuple(x.shape[1:]), nan, dtype=x.dtype, device=DEV)])
    q, k_new, v_new = pad(co.q), pad(co.k_new), pad(co.v_new)
    lens = torch.tensor([C] * B + [0] * P, dtype=torch.int32, device=DEV)
    out = pkc.paged_kv_append_relpos_attn(q, k_new, v_new, kp, vp, bt, cs, co.pos, co.pos_bias_u,
                                          co.pos_bias_v, co.max_cache_seqlen, chunk_lens=lens)
    np.testing.assert_array_equal(bits(out[:B]), bits(out_base))
    assert (out[B:] == 0).all()
    np.testing.assert_array_equal(bits(kp[:N]), bits(base.k_pool))
    np.testing.assert_array_equal(bits(vp[:N]), bits(base.v_pool))
    assert torch.isnan(kp[N:]).all() and torch.isnan(vp[N:]).all()


# --------------------------------------------------------------------------------------------
# Bounded history: window starts and ring-addressed tables
# --------------------------------------------------------------------------------------------

def _as_ring(co, seed, wraps=3):
    """The same cohort addressed through rings: stream b gets a window start w_b (a whole number
    of blocks, several times round the ring) and its table row rotated so that the window's
    pages land on the same physical blocks. Returns (window_start tensor, ring tables)."""
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
    return (torch.tensor(starts, dtype=torch.int32, device=DEV),
            torch.from_numpy(ring).to(DEV))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["bf16_ragged", "odd_lengths", "per_row_ragged_fp32",
                                  "long_chunk_bf16"])
def test_ring_tables_with_window_starts_equal_plain_tables_bitwise(name, fused):
    """A window start that moves the stream's pages round its ring, with the table row rotated to
    match, addresses the same frames: outputs and pools are bitwise those of the plain table, and
    match the oracle's ring addressing."""
    co = poison(small_cohort(name, seed=12))
    co2 = clone(co)
    ws, ring = _as_ring(co, 13)
    lens = _lens_for(co, 14)
    t = torch.from_numpy(lens).to(DEV)
    plain = gpu_chunk(co, fused=fused, chunk_lens=t)
    co2.block_tables = ring
    if fused:
        out = pkc.paged_kv_append_relpos_attn(co2.q, co2.k_new, co2.v_new, co2.k_pool, co2.v_pool,
                                              ring, co2.cache_seqlens, co2.pos, co2.pos_bias_u,
                                              co2.pos_bias_v, co2.max_cache_seqlen,
                                              per_row_pos=co2.per_row_pos, chunk_lens=t,
                                              window_start=ws)
    else:
        pkc.paged_kv_append(co2.k_new, co2.v_new, co2.k_pool, co2.v_pool, ring, co2.cache_seqlens,
                            co2.max_cache_seqlen, chunk_lens=t, window_start=ws)
        out = pkc.chunk_paged_relpos_attn(co2.q, co2.k_pool, co2.v_pool, ring, co2.cache_seqlens,
                                          co2.pos, co2.pos_bias_u, co2.pos_bias_v,
                                          co2.max_cache_seqlen, per_row_pos=co2.per_row_pos,
                                          chunk_lens=t, window_start=ws)
    np.testing.assert_array_equal(bits(out), bits(plain))
    np.testing.assert_array_equal(bits(co2.k_pool), bits(co.k_pool))
    np.testing.assert_array_equal(bits(co2.v_pool), bits(co.v_pool))


def test_ring_addressing_matches_the_oracle():
    co = poison(small_cohort("gqa_h4_k2", seed=15))
    ws, ring = _as_ring(co, 16)
    co.block_tables = ring
    h = {k: host64(getattr(co, k)) for k in ["q", "k_new", "v_new", "k_pool", "v_pool", "pos",
                                             "pos_bias_u", "pos_bias_v"]}
    bt, cs, w = ring.cpu().numpy(), co.cache_seqlens.cpu().numpy(), ws.cpu().numpy()
    kp, vp = oracle.paged_kv_append(h["k_pool"], h["v_pool"], h["k_new"], h["v_new"], bt, cs,
                                    window_start=w)
    ref = oracle.chunk_relpos_attn(h["q"], kp, vp, bt, cs, h["pos"], h["pos_bias_u"],
                                   h["pos_bias_v"], window_start=w)
    out = pkc.paged_kv_append_relpos_attn(co.q, co.k_new, co.v_new, co.k_pool, co.v_pool, ring,
                                          co.cache_seqlens, co.pos, co.pos_bias_u, co.pos_bias_v,
                                          co.max_cache_seqlen, window_start=ws)
    assert max_err(out, ref) <= TOL[co.q.dtype]


def test_commit_with_eviction_matches_the_oracle():
    rng = np.random.default_rng(17)
    B, C, S, cap = 257, 16, 8, 40
    cache = rng.integers(0, cap + 1, size=B).astype(np.int32)
    start = (rng.integers(0, 1000, size=B) * S).astype(np.int32)
    lens = rng.integers(0, C + 1, size=B).astype(np.int32)
    ec, es = oracle.commit_chunk(cache, C, chunk_lens=lens, window_start=start,
                                 max_cached_frames=cap, block_size=S)
    c_t, s_t = torch.from_numpy(cache).to(DEV), torch.from_numpy(start).to(DEV)
    pkc.paged_kv_commit(c_t, C, chunk_lens=torch.from_numpy(lens).to(DEV), window_start=s_t,
                        max_cached_frames=cap, block_size=S)
    assert c_t.cpu().numpy().tolist() == ec.tolist()
    assert s_t.cpu().numpy().tolist() == es.tolist()
    c2 = torch.from_numpy(cache).to(DEV)
    pkc.paged_kv_commit(c2, C)
    assert c2.cpu().numpy().tolist() == (cache + C).tolist()


# --------------------------------------------------------------------------------------------
# WeNet's convention: per-key tables, no shift
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name,per_row", [("bf16_ragged", True), ("bf16_ragged", False),
                                          ("gqa_h4_k2", True), ("odd_lengths", True),
                                          ("per_row_ragged_fp32", True), ("long_chunk_bf16", True),
                                          ("chunk32_full_tail", False)])
def test_per_key_tables_parity(name, per_row, fused):
    """Tables with one row per key (the keys' absolute positions start at offset - cache per
    stream): the GPU matches the oracle, with short windows and padding lanes mixed in."""
    co = poison(small_cohort(name, seed=20))
    B = co.q.shape[0]
    starts = np.random.default_rng(21).integers(0, 500, size=B).tolist()
    use_key_position_tables(co, starts, per_row=per_row)
    if per_row:
        C = co.q.shape[1]
        for b, c in enumerate(co.cache_seqlens.cpu().tolist()):
            co.pos[b, c + C:] = float("nan")              # rows past the stream's keys
    lens = _lens_for(co, 22)
    poison_padding(co, lens)
    ref = oracle_chunk(co, chunk_lens=lens)
    out = gpu_chunk(co, fused=fused, chunk_lens=torch.from_numpy(lens).to(DEV))
    assert max_err(out, ref) <= TOL[co.q.dtype], (name, max_err(out, ref))


def test_per_key_fused_equals_unfused_bitwise():
    co = small_cohort("odd_lengths", seed=23)
    use_key_position_tables(co, [5, 0, 100, 7], per_row=True)
    co2 = clone(co)
    np.testing.assert_array_equal(bits(gpu_chunk(co)), bits(gpu_chunk(co2, fused=True)))


# --------------------------------------------------------------------------------------------
# The chunked_limited mask in the packed offline kernel
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,chunk,left", [(BF16, 16, 4), (BF16, 14, 5), (BF16, 4, 0),
                                              (BF16, 100, 1), (BF16, 8, 1000), (F32, 13, 2)])
def test_varlen_chunked_limited_parity(dtype, chunk, left):
    """Utterances of many lengths (shorter than a chunk, not a multiple of it, several query
    blocks) under the chunked_limited mask, against the oracle."""
    co = make_varlen_cohort([1, 37, 0, 130, 64, 200, 5], 2, 64, dtype=dtype, seed=30, device=DEV)
    ref = oracle.varlen_relpos_attn(host64(co.q), host64(co.k), host64(co.v),
                                    co.cu_seqlens.cpu().numpy(), host64(co.pos),
                                    host64(co.pos_bias_u), host64(co.pos_bias_v), chunk=chunk,
                                    left_chunks=left)
    out = pkc.varlen_packed_relpos_attn(co.q, co.k, co.v, co.cu_seqlens, co.pos, co.pos_bias_u,
                                        co.pos_bias_v, max(co.lengths), mask_chunk=chunk,
                                        mask_left_chunks=left)
    assert max_err(out, ref) <= TOL[dtype], (chunk, left, max_err(out, ref))


def test_varlen_chunked_limited_sampled_workload():
    """The packed offline workload under a 16-frame chunk with 4 left chunks, checked on sampled
    rows of the longest, shortest, first and last utterances."""
    co = make_config(4, device=DEV)
    out = pkc.varlen_packed_relpos_attn(co.q, co.k, co.v, co.cu_seqlens, co.pos, co.pos_bias_u,
                                        co.pos_bias_v, max(co.lengths), mask_chunk=16,
                                        mask_left_chunks=4)
    lengths = co.lengths
    segs = sorted({int(np.argmax(lengths)), int(np.argmin(lengths)), 0, len(lengths) - 1})
    rng = np.random.default_rng(31)

    def rows(n):
        pick = set(range(min(20, n))) | set(range(max(0, n - 20), n))
        pick |= set(rng.choice(n, size=min(20, n), replace=False).tolist())
        return sorted(pick)
    ref = oracle.varlen_relpos_attn(host64(co.q), host64(co.k), host64(co.v),
                                    co.cu_seqlens.cpu().numpy(), host64(co.pos),
                                    host64(co.pos_bias_u), host64(co.pos_bias_v),
                                    segments=segs, query_rows=rows, chunk=16, left_chunks=4)
    have = ~np.isnan(ref[:, 0, 0])
    o = out.detach().cpu().double().numpy()
    assert np.abs(o[have] - ref[have]).max() <= TOL[BF16]
