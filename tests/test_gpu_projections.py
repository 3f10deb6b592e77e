"""GPU parity of the GEMMs either side of the attention - the linear layer, the chunk's Q/K/V
projection with the paged append as its epilogue, and linear_pos over sinusoidal tables - through
the C ABI against the float64 oracle (oracle/projections.py). Every input is seeded and synthetic.

Tolerances follow from the arithmetic. The kernels multiply stored values exactly and accumulate
in fp32 over K terms (error below K 2^-24 sum_k |x_k w_k|), then round once to the output dtype
(half an ulp: 2^-9 |y| in bf16, 2^-24 |y| in fp32). Elementwise:
    bf16:  |gpu - oracle| <= 2^-8 |y| + 2^-14 sum_k |x_k w_k|
    fp32:  |gpu - oracle| <= 2^-22 |y| + K 2^-23 sum_k |x_k w_k|
With the generated sinusoid, each table entry e_k is rounded to the dtype before the product
(bf16: 2^-9 |e_k|); in fp32 the phase p f_k is itself rounded (2^-24 relative), moving e_k by up
to |p f_k| 2^-23 (plus the sincos error, a few 2^-24):
    bf16:  + 2^-8 sum_k |e_k w_k|
    fp32:  + sum_k (|p f_k| + 4) 2^-23 |w_k|
The pools are compared bit for bit everywhere the append must not write.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_chunk_amd as pkc
from synth import activations, linear_weights, make_chunk_cohort
from gpu_helpers import bits, host64, ring_tables

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def bound(y_ref, absprod, dtype, K):
    """Elementwise tolerance of a GEMM output (see the module notes)."""
    if dtype == BF16:
        return 2.0 ** -8 * np.abs(y_ref) + 2.0 ** -14 * absprod
    return 2.0 ** -22 * np.abs(y_ref) + K * 2.0 ** -23 * absprod


def assert_within(got, ref, tol, what):
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside the bound; worst "
                           f"excess {float((err - tol).max()):.3g} (max err {float(err.max()):.3g})")


# --------------------------------------------------------------------------------------------
# linear
# --------------------------------------------------------------------------------------------

LINEAR = {
    "tiny": (3, 16, 32),
    "ragged_rows_partial_tile": (1000, 48, 64),
    # the directly loaded bf16 path (K of 256 / 512 / 1024), with a half pair of 16 features
    # at the end (N = 16 mod 32) and ragged rows
    "direct_k256_half_pair": (1000, 48, 256),
    "direct_k1024_half_pair": (77, 1040, 1024),
    "direct_k512_one_row": (1, 512, 512),
    "dmodel256_qkv_shape": (1024, 768, 256),
    # K = 256 on more than 256 tiles: the three-slot ring (at most 256 tiles: all stages in
    # flight at once)
    "direct_k256_ring": (4096, 1536, 256),
    "dmodel512_qkv_shape_large_tiles": (4096, 1536, 512),
    # the 128 x 192 tile (one per CU, the deep ring) with a ragged last row of tiles
    "direct_k512_wide_tiles_ragged_rows": (4000, 1536, 512),
    # 128 x 192 tiles on more than one per CU: the three-slot ring
    "direct_k512_wide_tiles_ring": (8192, 1536, 512),
    "out_proj_dmodel512": (4096, 512, 512),
}


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("case", list(LINEAR))
def test_linear_parity(case, with_bias, dtype):
    M, N, K = LINEAR[case]
    x = activations((M, K), seed=1, dtype=dtype, device=DEV)
    w, b = linear_weights(N, K, seed=2, dtype=dtype, device=DEV, bias=with_bias)
    y = pkc.linear(x, w, b)
    torch.cuda.synchronize()
    xh, wh = host64(x), host64(w)
    ref = oracle.linear(xh, wh, host64(b) if with_bias else None)
    assert_within(host64(y), ref, bound(ref, np.abs(xh) @ np.abs(wh).T, dtype, K), f"linear {case}")


def _random_shapes(seed, n):
    """Seeded GEMM shapes over the launcher's choices: every tile shape, ring depth and staging
    path (K of 256, 512 and 1024 load directly in bf16), ragged M and N (N a multiple of 16)."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        K = int(rng.choice([32, 96, 256, 512, 1024]))
        M = int(rng.integers(1, 4200))
        N = 16 * int(rng.integers(1, 100))
        shapes.append((M, N, K))
    return shapes


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
def test_linear_random_shapes(dtype):
    for i, (M, N, K) in enumerate(_random_shapes(21, 16)):
        x = activations((M, K), seed=100 + i, dtype=dtype, device=DEV)
        w, b = linear_weights(N, K, seed=200 + i, dtype=dtype, device=DEV, bias=i % 2 == 0)
        y = pkc.linear(x, w, b)
        torch.cuda.synchronize()
        xh, wh = host64(x), host64(w)
        ref = oracle.linear(xh, wh, host64(b) if b is not None else None)
        assert_within(host64(y), ref, bound(ref, np.abs(xh) @ np.abs(wh).T, dtype, K),
                      f"linear M={M} N={N} K={K}")


def test_linear_batched_leading_dims():
    x = activations((4, 16, 256), seed=3, device=DEV)
    w, b = linear_weights(256, 256, seed=4, device=DEV)
    y = pkc.linear(x, w, b)
    y2 = pkc.linear(x.reshape(64, 256), w, b)
    torch.cuda.synchronize()
    assert y.shape == (4, 16, 256)
    assert np.array_equal(bits(y.reshape(64, 256)), bits(y2))


# --------------------------------------------------------------------------------------------
# the Q/K/V projection with the append as its epilogue
# --------------------------------------------------------------------------------------------

QKV = {
    "bf16_ragged": dict(B=3, H=2, Hk=2, D=64, C=16, S=16, caches=[0, 37, 100], dm=128, dtype=BF16),
    "fp32_ragged": dict(B=3, H=2, Hk=2, D=64, C=16, S=16, caches=[0, 37, 100], dm=128, dtype=F32),
    "gqa_short_chunk": dict(B=4, H=4, Hk=2, D=64, C=5, S=8, caches=[3, 0, 64, 11], dm=256, dtype=BF16),
    "dmodel256_cohort": dict(B=64, H=4, Hk=4, D=64, C=16, S=16, caches=[256] * 64, dm=256, dtype=BF16),
    # d_model 256 with 256 streams: 384 tiles, the ring path of the K = 256 epilogue
    "dmodel256_wide_cohort": dict(B=256, H=4, Hk=4, D=64, C=16, S=16, caches=[64, 0, 17, 255] * 64,
                                  dm=256, dtype=BF16),
    # the d_model 512 cohort at full size, in the launch configuration the projection bench times
    "dmodel512_cohort": dict(B=256, H=8, Hk=8, D=64, C=16, S=16, caches=[512] * 256, dm=512, dtype=BF16),
    # head sizes other than 64 (the append takes any multiple of 32): the pair and page offsets
    "head_dim32": dict(B=5, H=4, Hk=2, D=32, C=16, S=16, caches=[0, 15, 16, 100, 33], dm=128, dtype=BF16),
    "head_dim128_gqa": dict(B=3, H=4, Hk=1, D=128, C=16, S=32, caches=[0, 37, 100], dm=256, dtype=BF16),
}


def _written_mask(k_pool, v_pool, bt, cs, C, Hk, D, lens, ws):
    """Pool elements the append writes (the oracle's own addressing, on marker pools)."""
    B = bt.shape[0]
    kz, vz = np.zeros(k_pool.shape), np.zeros(v_pool.shape)
    ones = np.ones((B, C, Hk, D))
    km, vm = oracle.paged_kv_append(kz, vz, ones, ones, bt, cs, chunk_lens=lens, window_start=ws)
    return km != 0, vm != 0


def _qkv_case(case, seed=0):
    c = QKV[case]
    co = make_chunk_cohort(c["B"], c["H"], c["D"], c["C"], c["S"], c["caches"], Hk=c["Hk"],
                           dtype=c["dtype"], seed=seed, device=DEV)
    x = activations((c["B"], c["C"], c["dm"]), seed=seed + 7, dtype=c["dtype"], device=DEV)
    w, b = linear_weights((c["H"] + 2 * c["Hk"]) * c["D"], c["dm"], seed=seed + 8, dtype=c["dtype"], device=DEV)
    return c, co, x, w, b


def _check_qkv(c, co, x, w, b, lens=None, ws=None):
    k0, v0 = host64(co.k_pool), host64(co.v_pool)
    kb0, vb0 = bits(co.k_pool), bits(co.v_pool)
    bt, cs = co.block_tables.cpu().numpy(), co.cache_seqlens.cpu().numpy()
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws_t = None if ws is None else torch.tensor(ws, dtype=torch.int32, device=DEV)
    q = pkc.paged_kv_qkv_append(x, w, b, co.k_pool, co.v_pool, co.block_tables, co.cache_seqlens,
                                co.max_cache_seqlen, c["H"], chunk_lens=lens_t, window_start=ws_t)
    torch.cuda.synchronize()
    xh, wh, bh = host64(x), host64(w), host64(b)
    q_ref, k_ref, v_ref = oracle.qkv_append(xh, wh, bh, k0, v0, bt, cs, c["H"], c["Hk"], c["D"],
                                            chunk_lens=lens, window_start=ws)
    absprod = (np.abs(xh) @ np.abs(wh).T).reshape(c["B"], c["C"], -1)
    K = c["dm"]
    HD, HkD = c["H"] * c["D"], c["Hk"] * c["D"]
    assert_within(host64(q), q_ref, bound(q_ref, absprod[..., :HD].reshape(q_ref.shape), c["dtype"], K), "q")
    km, vm = _written_mask(k0, v0, bt, cs, c["C"], c["Hk"], c["D"], lens, ws)
    # untouched pool elements: bit for bit
    assert np.array_equal(bits(co.k_pool)[~km], kb0[~km])
    assert np.array_equal(bits(co.v_pool)[~vm], vb0[~vm])
    # written ones: the projected rows, within the bound (the oracle places them itself)
    _, ka, va = oracle.qkv_append(np.zeros_like(xh), np.zeros_like(wh), None, np.zeros(k0.shape),
                                  np.zeros(v0.shape), bt, cs, c["H"], c["Hk"], c["D"], chunk_lens=lens,
                                  window_start=ws)
    # tolerance planes placed like the values: append the per-element bounds as "K/V rows"
    kb = absprod[..., HD:HD + HkD].reshape(c["B"], c["C"], c["Hk"], c["D"])
    vb = absprod[..., HD + HkD:].reshape(c["B"], c["C"], c["Hk"], c["D"])
    kt, vt = oracle.paged_kv_append(np.zeros(k0.shape), np.zeros(v0.shape), kb, vb, bt, cs,
                                    chunk_lens=lens, window_start=ws)
    assert_within(host64(co.k_pool)[km], k_ref[km], bound(k_ref[km], kt[km], c["dtype"], K), "K pages")
    assert_within(host64(co.v_pool)[vm], v_ref[vm], bound(v_ref[vm], vt[vm], c["dtype"], K), "V pages")
    return q


@pytest.mark.parametrize("case", list(QKV))
def test_qkv_append_parity(case):
    c, co, x, w, b = _qkv_case(case)
    _check_qkv(c, co, x, w, b)


def test_qkv_append_chunk_lens_and_padding_lane():
    c, co, x, w, b = _qkv_case("gqa_short_chunk", seed=3)
    _check_qkv(c, co, x, w, b, lens=[5, 0, 2, 4])


def test_qkv_append_window_start_ring():
    # each stream's table row is a ring of M pages, its window start several times round it
    c, co, x, w, b = _qkv_case("bf16_ragged", seed=5)
    starts, co.block_tables = ring_tables(co, 13)
    _check_qkv(c, co, x, w, b, ws=starts, lens=[16, 9, 16])


def test_qkv_append_wide_tiles_chunk_lens_and_window_starts():
    """The d_model 512 cohort's launch (128 x 192 tiles, one per CU, the deep ring) with
    per-stream chunk lengths from 0 to C frames and ring-rotated table rows: each row's stream
    entries, loaded ahead of the contraction, place its K/V in the right page and slot."""
    c, co, x, w, b = _qkv_case("dmodel512_cohort", seed=9)
    starts, co.block_tables = ring_tables(co, 17)
    lens = np.random.default_rng(19).integers(0, c["C"] + 1, size=c["B"]).tolist()
    _check_qkv(c, co, x, w, b, ws=starts, lens=lens)


def test_qkv_append_random_cohorts():
    """A seeded sweep of cohort shapes: streams, chunk size, heads (GQA), head size (32, 64, 128),
    block size, d_model and ragged cache lengths, with and without chunk lengths."""
    rng = np.random.default_rng(31)
    for i in range(10):
        Hk = int(rng.choice([1, 2, 4]))
        H = Hk * int(rng.choice([1, 2]))
        D = int(rng.choice([32, 64, 128]))
        C = int(rng.integers(1, 33))
        S = int(rng.choice([8, 16, 32]))
        B = int(rng.integers(1, 40))
        dm = 32 * int(rng.integers(2, 17))
        caches = rng.integers(0, 300, size=B).tolist()
        c = dict(B=B, H=H, Hk=Hk, D=D, C=C, S=S, caches=caches, dm=dm, dtype=BF16)
        co = make_chunk_cohort(B, H, D, C, S, caches, Hk=Hk, dtype=BF16, seed=40 + i, device=DEV)
        x = activations((B, C, dm), seed=50 + i, dtype=BF16, device=DEV)
        w, b = linear_weights((H + 2 * Hk) * D, dm, seed=60 + i, dtype=BF16, device=DEV)
        lens = rng.integers(0, C + 1, size=B).tolist() if i % 2 else None
        _check_qkv(c, co, x, w, b, lens=lens)


def test_qkv_append_then_attention_equals_append_of_projected_rows():
    """The epilogue writes exactly what paged_kv_append writes for the same K/V rows: project with
    the plain linear layer, split, append, and compare the pools bit for bit."""
    c, co, x, w, b = _qkv_case("gqa_short_chunk", seed=9)
    k2, v2 = co.k_pool.clone(), co.v_pool.clone()
    pkc.paged_kv_qkv_append(x, w, b, co.k_pool, co.v_pool, co.block_tables, co.cache_seqlens,
                            co.max_cache_seqlen, c["H"])
    y = pkc.linear(x, w, b)
    HD, HkD = c["H"] * c["D"], c["Hk"] * c["D"]
    k_new = y[..., HD:HD + HkD].reshape(c["B"], c["C"], c["Hk"], c["D"]).contiguous()
    v_new = y[..., HD + HkD:].reshape(c["B"], c["C"], c["Hk"], c["D"]).contiguous()
    pkc.paged_kv_append(k_new, v_new, k2, v2, co.block_tables, co.cache_seqlens, co.max_cache_seqlen)
    torch.cuda.synchronize()
    assert np.array_equal(bits(co.k_pool), bits(k2))
    assert np.array_equal(bits(co.v_pool), bits(v2))


# --------------------------------------------------------------------------------------------
# linear_pos over sinusoidal tables
# --------------------------------------------------------------------------------------------

def _pos_bound(w64, pos, dtype, d_model, ref):
    """Per-element tolerance of a projected sinusoid table [n, rows, N]."""
    emb = oracle.sinusoid(pos.reshape(-1), d_model)
    absprod = np.abs(emb) @ np.abs(w64).T
    if dtype == BF16:
        extra = 2.0 ** -8 * absprod
    else:
        # the phase is reduced exactly (fp64) before fp32 sees it, so its error, about 2^-25
        # turns, and the fp32 sine's own few ulps do not grow with |p|
        extra = np.broadcast_to(2.0 ** -21 * np.abs(w64).sum(axis=1), absprod.shape)
    return bound(ref, absprod.reshape(ref.shape), dtype, d_model) + extra.reshape(ref.shape)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("case", ["txl_shared_dmodel256", "txl_shared_dmodel512", "wenet_per_stream",
                                  "dmodel1024_ragged_tables",
                                  # a width whose rows the kernel stages through registers
                                  "txl_shared_dmodel384",
                                  # many per-row tables: more tiles than CUs, the three-slot ring
                                  "many_tables_dmodel512",
                                  # 1536 output features over 4096 rows: 128 x 192 tiles
                                  "wide_tiles_dmodel512"])
def test_rel_pos_projection_parity(case, dtype):
    if case == "dmodel1024_ragged_tables":
        # tables whose rows do not fill whole 64-row tiles, crossing table boundaries in a tile
        dm, rows = 1024, 37
        w, _ = linear_weights(512, dm, seed=13, dtype=dtype, device=DEV, bias=False)
        starts = np.array([40, -7, 3000])
        st = torch.tensor(starts, dtype=torch.int32, device=DEV)
        got = pkc.rel_pos_projection(w, rows, pos_start=st, pos_step=-1)
        step = -1
    elif case == "wide_tiles_dmodel512":
        dm, rows = 512, 512
        w, _ = linear_weights(1536, dm, seed=17, dtype=dtype, device=DEV, bias=False)
        starts = np.random.default_rng(18).integers(-3000, 3000, size=8)
        st = torch.tensor(starts, dtype=torch.int32, device=DEV)
        got = pkc.rel_pos_projection(w, rows, pos_start=st, pos_step=-1)
        step = -1
    elif case == "many_tables_dmodel512":
        dm, rows = 512, 300
        w, _ = linear_weights(dm, dm, seed=15, dtype=dtype, device=DEV, bias=False)
        starts = np.random.default_rng(16).integers(-5000, 5000, size=40)
        st = torch.tensor(starts, dtype=torch.int32, device=DEV)
        got = pkc.rel_pos_projection(w, rows, pos_start=st, pos_step=1)
        step = 1
    elif case.startswith("txl"):
        dm = int(case.rsplit("dmodel", 1)[1])
        # max cache + C - 1 of the streaming workloads
        center = {256: 271, 512: 527}.get(dm, 100)
        w, _ = linear_weights(dm, dm, seed=11, dtype=dtype, device=DEV, bias=False)
        rows = 2 * center + 1
        got = pkc.rel_pos_projection(w, rows, pos_first=center, pos_step=-1)
        starts, step = np.array([center]), -1
    else:
        dm, rows = 256, 300
        w, _ = linear_weights(dm, dm, seed=12, dtype=dtype, device=DEV, bias=False)
        starts = np.array([-250, 0, 17, 1000, -3])          # offset - cache per stream
        st = torch.tensor(starts, dtype=torch.int32, device=DEV)
        got = pkc.rel_pos_projection(w, rows, pos_start=st, pos_step=1)
        step = 1
    torch.cuda.synchronize()
    w64 = host64(w)
    ref = oracle.rel_pos_projection(w64, starts, step, rows)
    pos = oracle.table_positions(starts, step, rows)
    assert got.shape == ref.shape
    assert_within(host64(got), ref, _pos_bound(w64, pos, dtype, dm, ref), case)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("step", [-1, 1])
def test_rel_pos_projection_at_large_positions(dtype, step):
    """Positions far from zero (10^5 .. 2^24, the largest the entry accepts): the phase p f_j is
    reduced exactly, so the error bound is the one small positions get."""
    dm, rows = 256, 70
    w, _ = linear_weights(dm, dm, seed=14, dtype=dtype, device=DEV, bias=False)
    starts = np.array([100003, -524287, 999999, -1000000, 2 ** 24 - rows, -(2 ** 24) + rows])
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    got = pkc.rel_pos_projection(w, rows, pos_start=st, pos_step=step)
    torch.cuda.synchronize()
    w64 = host64(w)
    ref = oracle.rel_pos_projection(w64, starts, step, rows)
    pos = oracle.table_positions(starts, step, rows)
    assert np.abs(pos).max() <= 2 ** 24
    assert_within(host64(got), ref, _pos_bound(w64, pos, dtype, dm, ref), f"large_{step}")


# --------------------------------------------------------------------------------------------
# one whole attention layer: projections, append, attention, output projection
# --------------------------------------------------------------------------------------------

def test_layer_end_to_end_against_the_oracle_chain():
    """x -> Q/K/V projection + append -> linear_pos table -> chunk attention -> linear_out, on the
    GPU, against the same chain in float64. The GPU rounds q, K/V and the table to bf16 between
    steps; the comparison uses the attention tests' bf16 tolerance on unit-scale outputs."""
    B, H, D, C, S, dm = 4, 4, 64, 16, 16, 256
    caches = [0, 20, 64, 100]
    co = make_chunk_cohort(B, H, D, C, S, caches, seed=21, device=DEV)
    k0, v0 = host64(co.k_pool), host64(co.v_pool)
    bt, cs = co.block_tables.cpu().numpy(), co.cache_seqlens.cpu().numpy()
    x = activations((B, C, dm), seed=22, device=DEV)
    w_qkv, b_qkv = linear_weights(3 * H * D, dm, seed=23, device=DEV)
    w_pos, _ = linear_weights(H * D, dm, seed=24, device=DEV, bias=False)
    w_out, b_out = linear_weights(dm, H * D, seed=25, device=DEV)
    center = co.max_cache_seqlen + C - 1
    q = pkc.paged_kv_qkv_append(x, w_qkv, b_qkv, co.k_pool, co.v_pool, co.block_tables,
                                co.cache_seqlens, co.max_cache_seqlen, H)
    pos = pkc.rel_pos_projection(w_pos, 2 * center + 1, pos_first=center, pos_step=-1)[0]
    att = pkc.chunk_paged_relpos_attn(q, co.k_pool, co.v_pool, co.block_tables, co.cache_seqlens,
                                      pos.reshape(-1, H, D), co.pos_bias_u, co.pos_bias_v,
                                      co.max_cache_seqlen)
    out = pkc.linear(att.reshape(B, C, H * D), w_out, b_out)
    torch.cuda.synchronize()
    q_r, k_r, v_r = oracle.qkv_append(host64(x), host64(w_qkv), host64(b_qkv), k0, v0, bt, cs, H, H, D)
    pos_r = oracle.rel_pos_projection(host64(w_pos), [center], -1, 2 * center + 1)[0].reshape(-1, H, D)
    att_r = oracle.chunk_relpos_attn(q_r, k_r, v_r, bt, cs, pos_r, host64(co.pos_bias_u),
                                     host64(co.pos_bias_v))
    out_r = oracle.linear(att_r.reshape(B, C, H * D), host64(w_out), host64(b_out))
    err = np.abs(host64(out) - out_r).max()
    assert err < 2e-2, err
