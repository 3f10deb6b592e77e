"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a flipped distance
sign, an off-by-one table centre, a transposed operand, a wrong page address) fails at least one
of them; ``test_planted_mistakes_are_caught`` plants such slips in the oracle and checks that.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.relpos_attn as orc
from synth import descending_table, embed_distances, make_chunk_cohort, make_varlen_cohort, relpos_projection
from synth import WORKLOADS, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64


def np64(t):
    return t.detach().cpu().to(F64).numpy()


# --------------------------------------------------------------------------------------------
# Append and page addressing
# --------------------------------------------------------------------------------------------

def test_append_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "append_worked_example.json")))
    S, N, Hk, D, C = g["block_size"], g["num_blocks"], g["n_kv_head"], g["head_dim"], g["chunk_size"]
    bt = np.array(g["block_tables"])
    cs = np.array(g["cache_seqlens"])
    B = bt.shape[0]
    k_new = np.zeros((B, C, Hk, D))
    for b in range(B):
        for t in range(C):
            for d in range(D):
                k_new[b, t, :, d] = 100 * b + 10 * t + d
    v_new = -k_new - 1000
    kp = np.full((N, Hk, S, D), np.nan)
    vp = np.full((N, Hk, D, S), np.nan)
    k2, v2 = oracle.paged_kv_append(kp, vp, k_new, v_new, bt, cs)
    expect_k = np.full_like(kp, np.nan)
    expect_v = np.full_like(vp, np.nan)
    for p in g["placements"]:
        expect_k[p["block"], :, p["slot"], :] = k_new[p["stream"], p["t"]]
        expect_v[p["block"], :, :, p["slot"]] = v_new[p["stream"], p["t"]]
    np.testing.assert_array_equal(k2, expect_k)
    np.testing.assert_array_equal(v2, expect_v)


@pytest.mark.parametrize("S", [4, 8, 16])
def test_append_then_gather_round_trip(S):
    """Appending chunks step by step and reading back through the table returns the stream's
    frames in order; no element outside the written slots changes (bit patterns compared)."""
    rng = np.random.default_rng(S)
    B, Hk, D, C, steps = 3, 2, 4, 5, 4
    pages = (C * steps + S - 1) // S
    N = B * pages + 3
    ids = rng.permutation(N)
    bt = np.full((B, pages + 2), -1)
    for b in range(B):
        bt[b, :pages] = ids[b * pages:(b + 1) * pages]
    kp = np.full((N, Hk, S, D), np.nan)
    vp = np.full((N, Hk, D, S), np.nan)
    seq_k = rng.standard_normal((B, C * steps, Hk, D))
    seq_v = rng.standard_normal((B, C * steps, Hk, D))
    for step in range(steps):
        cs = np.full(B, step * C)
        kp, vp = oracle.paged_kv_append(kp, vp, seq_k[:, step * C:(step + 1) * C],
                                        seq_v[:, step * C:(step + 1) * C], bt, cs)
    for b in range(B):
        k, v = oracle.gather_stream(kp, vp, bt[b], C * steps)
        np.testing.assert_array_equal(k, seq_k[b])
        np.testing.assert_array_equal(v, seq_v[b])
    written = B * C * steps * Hk * D
    assert np.count_nonzero(~np.isnan(kp)) == written
    assert np.count_nonzero(~np.isnan(vp)) == written


def test_append_is_bit_exact_on_bf16_patterns():
    """The append is a copy: bf16 bit patterns (as int16) survive untouched, NaN payloads too."""
    rng = np.random.default_rng(1)
    kp = rng.integers(-2**15, 2**15, size=(6, 1, 4, 2)).astype(np.int16)
    vp = rng.integers(-2**15, 2**15, size=(6, 1, 2, 4)).astype(np.int16)
    k_new = rng.integers(-2**15, 2**15, size=(1, 3, 1, 2)).astype(np.int16)
    v_new = rng.integers(-2**15, 2**15, size=(1, 3, 1, 2)).astype(np.int16)
    bt = np.array([[4, 0]])
    k2, v2 = oracle.paged_kv_append(kp, vp, k_new, v_new, bt, np.array([2]))
    assert (k2[4, :, 2] == k_new[0, 0]).all() and (k2[4, :, 3] == k_new[0, 1]).all()
    assert (k2[0, :, 0] == k_new[0, 2]).all()
    assert (v2[4, :, :, 2] == v_new[0, 0]).all() and (v2[0, :, :, 0] == v_new[0, 2]).all()
    changed = (k2 != kp).any(axis=(1, 3)).sum()
    assert changed <= 3


# --------------------------------------------------------------------------------------------
# Attention pins
# --------------------------------------------------------------------------------------------

def _paged_from_sequences(seq_k, seq_v, caches, C, S, rng, pad_blocks=2):
    """Page full logical sequences into a fresh NaN pool through the oracle's append (which the
    tests above pin), frame by frame; returns pools and tables."""
    B = len(seq_k)
    Hk, D = seq_k[0].shape[1], seq_k[0].shape[2]
    pages = [(c + C + S - 1) // S for c in caches]
    N = sum(pages) + pad_blocks
    ids = rng.permutation(N)
    M = max(pages) + 1
    bt = np.full((B, M), -1)
    at = 0
    for b, n in enumerate(pages):
        bt[b, :n] = ids[at:at + n]
        at += n
    kp = np.full((N, Hk, S, D), np.nan)
    vp = np.full((N, Hk, D, S), np.nan)
    for b in range(B):
        for t in range(caches[b] + C):
            kp, vp = oracle.paged_kv_append(kp, vp, seq_k[b][None, t:t + 1], seq_v[b][None, t:t + 1],
                                            bt[b:b + 1], np.array([t]))
    return kp, vp, bt


def _random_streaming_case(seed, caches, C=4, H=2, Hk=2, D=8, S=4, zero_pos=False, margin=0):
    rng = np.random.default_rng(seed)
    B = len(caches)
    seq_k = [rng.standard_normal((c + C, Hk, D)) for c in caches]
    seq_v = [rng.standard_normal((c + C, Hk, D)) for c in caches]
    q = rng.standard_normal((B, C, H, D))
    u = 0.3 * rng.standard_normal((H, D))
    w = 0.3 * rng.standard_normal((H, D))
    proj = relpos_projection(H * D, torch.Generator().manual_seed(seed))
    if zero_pos:
        proj = proj * 0
        u = u * 0
        w = w * 0
    kp, vp, bt = _paged_from_sequences(seq_k, seq_v, caches, C, S, rng)
    center = max(caches) + C - 1 + margin
    table = descending_table(center, proj, H, D).numpy()
    return dict(q=q, u=u, w=w, proj=proj, kp=kp, vp=vp, bt=bt, cs=np.array(caches), table=table,
                seq_k=seq_k, seq_v=seq_v, C=C, H=H, Hk=Hk, D=D)


def _brute_force(case):
    """Scalar loops over logical sequences; the positional term takes the embedding of the
    distance (cache + i) - j straight from the projected sinusoid, with no table at all."""
    q, u, w = case["q"], case["u"], case["w"]
    C, H, Hk, D = case["C"], case["H"], case["Hk"], case["D"]
    out = np.zeros(q.shape)
    for b, c in enumerate(case["cs"]):
        c = int(c)
        T = c + C
        emb = {}
        for i in range(C):
            for j in range(T):
                dist = (c + i) - j
                if dist not in emb:
                    emb[dist] = embed_distances([dist], case["proj"], H, D).numpy()[0]
        for h in range(H):
            g = (h * Hk) // H
            for i in range(C):
                scores = []
                for j in range(T):
                    a = math.fsum((q[b, i, h, d] + u[h, d]) * case["seq_k"][b][j, g, d] for d in range(D))
                    p = math.fsum((q[b, i, h, d] + w[h, d]) * emb[(c + i) - j][h, d] for d in range(D))
                    scores.append((a + p) / math.sqrt(D))
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                z = math.fsum(ex)
                for d in range(D):
                    out[b, i, h, d] = math.fsum(ex[j] / z * case["seq_v"][b][j, g, d] for j in range(T))
    return out


def _oracle(case, **kw):
    return oracle.chunk_relpos_attn(case["q"], case["kp"], case["vp"], case["bt"], case["cs"],
                                    case["table"], case["u"], case["w"], **kw)


@pytest.mark.parametrize("caches,Hk", [([0, 4, 9], 2), ([3, 12], 1)])
def test_oracle_matches_brute_force(caches, Hk):
    case = _random_streaming_case(11, caches, Hk=Hk)
    err = np.abs(_oracle(case) - _brute_force(case)).max()
    assert err < 1e-12, err


def test_reduces_to_textbook_attention_when_no_position_term():
    """u = v = 0 and p = 0: plain softmax(Q K^T / sqrt(D)) V, from torch's float64 CPU routine."""
    case = _random_streaming_case(5, [0, 7, 13], Hk=2, zero_pos=True)
    out = _oracle(case)
    for b, c in enumerate(case["cs"]):
        qq = torch.from_numpy(case["q"][b]).permute(1, 0, 2)                    # [H, C, D]
        kk = torch.from_numpy(case["seq_k"][b]).permute(1, 0, 2).contiguous()  # [Hk, T, D]
        vv = torch.from_numpy(case["seq_v"][b]).permute(1, 0, 2).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)
        err = np.abs(out[b] - ref.permute(1, 0, 2).numpy()).max()
        assert err < 1e-12, err


def test_probabilities_are_a_distribution():
    case = _random_streaming_case(6, [2, 10])
    _, probs = _oracle(case, return_probs=True)
    for b, p in enumerate(probs):
        assert p.shape[-1] == case["cs"][b] + case["C"]
        assert (p >= 0).all()
        assert np.abs(p.sum(-1) - 1).max() < 1e-12


@pytest.mark.parametrize("dstar", [-3, -1, 0, 2, 5, 9, 40])
def test_one_hot_distance_closed_form(dstar):
    """Only distance d* carries an embedding (alpha on dim 0); q = e_0, u = v = k = 0. Then
    query i boosts exactly key j* = cache + i - d* by alpha / sqrt(D), which fixes the
    probabilities in closed form and pins the sign and origin of the distance."""
    C, H, D, S = 4, 1, 8, 4
    caches = [6, 0]
    alpha = 3.0
    rng = np.random.default_rng(0)
    B = len(caches)
    seq_k = [np.zeros((c + C, 1, D)) for c in caches]
    seq_v = [rng.standard_normal((c + C, 1, D)) for c in caches]
    kp, vp, bt = _paged_from_sequences(seq_k, seq_v, caches, C, S, rng)
    center = max(caches) + C - 1
    table = np.zeros((2 * center + 1, H, D))
    for r in range(table.shape[0]):
        if center - r == dstar:                      # row r holds distance center - r
            table[r, 0, 0] = alpha
    q = np.zeros((B, C, H, D))
    q[..., 0] = 1.0
    zero = np.zeros((H, D))
    out, probs = oracle.chunk_relpos_attn(q, kp, vp, bt, np.array(caches), table, zero, zero,
                                          return_probs=True)
    a = alpha / math.sqrt(D)
    for b, c in enumerate(caches):
        T = c + C
        for i in range(C):
            jstar = c + i - dstar
            expect = np.full(T, 1.0 / T)
            if 0 <= jstar < T:
                expect = np.full(T, 1.0 / (math.exp(a) + T - 1))
                expect[jstar] = math.exp(a) / (math.exp(a) + T - 1)
            assert np.abs(probs[b][0, i] - expect).max() < 1e-14
            np.testing.assert_allclose(out[b, i, 0], expect @ seq_v[b][:, 0], atol=1e-13)


def test_block_permutation_invariance():
    """Relabelling physical blocks (pool'[pi(n)] = pool[n], table' = pi(table)) changes nothing."""
    case = _random_streaming_case(8, [5, 0, 11])
    base = _oracle(case)
    rng = np.random.default_rng(3)
    N = case["kp"].shape[0]
    pi = rng.permutation(N)
    kp2 = np.empty_like(case["kp"])
    vp2 = np.empty_like(case["vp"])
    kp2[pi] = case["kp"]
    vp2[pi] = case["vp"]
    bt2 = np.where(case["bt"] >= 0, pi[np.maximum(case["bt"], 0)], -1)
    out2 = oracle.chunk_relpos_attn(case["q"], kp2, vp2, bt2, case["cs"], case["table"],
                                    case["u"], case["w"])
    np.testing.assert_array_equal(base, out2)


def _dense_blockcausal(q_all, k_all, v_all, u, w, proj, C):
    """Whole-utterance attention with a chunk mask (key chunk <= query chunk) and the positional
    bias (q_t + v) . emb(t - j) / sqrt(D), through torch's float64 scaled_dot_product_attention."""
    n, H, D = q_all.shape
    Hk = k_all.shape[1]
    t = np.arange(n)
    dist = t[:, None] - t[None, :]
    emb = embed_distances(dist.reshape(-1), proj, H, D).numpy().reshape(n, n, H, D)
    out = np.zeros((n, H, D))
    for h in range(H):
        g = h * Hk // H
        bias = np.einsum("td,tjd->tj", q_all[:, h] + w[h], emb[:, :, h]) / math.sqrt(D)
        bias = np.where((t[None, :] // C) <= (t[:, None] // C), bias, -np.inf)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q_all[:, h] + u[h])[None], torch.from_numpy(k_all[:, g])[None],
            torch.from_numpy(v_all[:, g])[None], attn_mask=torch.from_numpy(bias)[None])
        out[:, h] = ref[0].numpy()
    return out


def _streaming_vs_dense(seed, steps=5, C=4, H=2, Hk=1, D=8, S=8, margin=0):
    """Run the chunk oracle step by step from an empty cache, each step with its own table of
    2 (cache + C) - 1 rows, and compare with the dense block-causal reference."""
    rng = np.random.default_rng(seed)
    n = steps * C
    q_all = rng.standard_normal((n, H, D))
    k_all = rng.standard_normal((n, Hk, D))
    v_all = rng.standard_normal((n, Hk, D))
    u = 0.5 * rng.standard_normal((H, D))
    w = 0.5 * rng.standard_normal((H, D))
    proj = relpos_projection(H * D, torch.Generator().manual_seed(seed))
    pages = (n + S - 1) // S
    bt = rng.permutation(pages + 2)[None, :pages]
    kp = np.full((pages + 2, Hk, S, D), np.nan)
    vp = np.full((pages + 2, Hk, D, S), np.nan)
    outs = []
    for step in range(steps):
        c = step * C
        sl = slice(c, c + C)
        kp, vp = oracle.paged_kv_append(kp, vp, k_all[None, sl], v_all[None, sl], bt, np.array([c]))
        table = descending_table(c + C - 1 + margin, proj, H, D).numpy()
        outs.append(oracle.chunk_relpos_attn(q_all[None, sl], kp, vp, bt, np.array([c]), table, u, w)[0])
    stream = np.concatenate(outs)
    dense = _dense_blockcausal(q_all, k_all, v_all, u, w, proj, C)
    return np.abs(stream - dense).max()


def test_streaming_steps_equal_dense_block_causal_attention():
    err = _streaming_vs_dense(21)
    assert err < 1e-12, err


def test_shared_and_per_row_tables_agree():
    """With tables that depend only on distance, one shared table (centred for the longest row)
    and per-row tables (each centred at its own T_b - 1) give identical results; for a uniform
    cache they are the same table."""
    for caches in ([8, 8, 8], [0, 5, 12]):
        case = _random_streaming_case(9, caches)
        shared = _oracle(case)
        C = case["C"]
        P = case["table"].shape[0]
        per_row = np.zeros((len(caches), P, case["H"], case["D"]))
        center = (P - 1) // 2
        for b, c in enumerate(caches):
            T = c + C
            per_row[b, :2 * T - 1] = descending_table(T - 1, case["proj"], case["H"], case["D"]).numpy()
            per_row[b, 2 * T - 1:] = np.nan                     # outside row b's table: never read
            if c == max(caches):
                np.testing.assert_array_equal(per_row[b, :2 * T - 1], case["table"][center - T + 1:center + T])
        out = oracle.chunk_relpos_attn(case["q"], case["kp"], case["vp"], case["bt"], case["cs"],
                                       per_row, case["u"], case["w"], per_row_pos=True)
        assert np.abs(out - shared).max() < 1e-13


def test_row_locality():
    """A stream's output depends only on its own inputs: other rows may change or vanish."""
    case = _random_streaming_case(12, [4, 9, 2])
    full = _oracle(case)
    sub = dict(case)
    sub["q"] = case["q"][1:2]
    sub["bt"] = case["bt"][1:2]
    sub["cs"] = case["cs"][1:2]
    np.testing.assert_array_equal(_oracle(sub)[0], full[1])


def test_varlen_segments_equal_chunk_case_and_dense():
    """A packed segment of length L is the chunk case with cache 0 and C = L, and equals dense
    full-context attention with bias (q_t + v) . emb(t - j); segments never mix."""
    lengths = [5, 1, 9, 3]
    H, D = 2, 8
    co = make_varlen_cohort(lengths, H, D, dtype=F64, seed=4)
    q, k, v = np64(co.q), np64(co.k), np64(co.v)
    u, w = np64(co.pos_bias_u), np64(co.pos_bias_v)
    pos = np64(co.pos)
    out = oracle.varlen_relpos_attn(q, k, v, co.cu_seqlens.numpy(), pos, u, w)
    cu = co.cu_seqlens.numpy()
    for s, n in enumerate(lengths):
        lo, hi = cu[s], cu[s + 1]
        dense = _dense_blockcausal(q[lo:hi], k[lo:hi], v[lo:hi], u, w, co.meta["proj"], C=n)
        assert np.abs(out[lo:hi] - dense).max() < 1e-12
        # chunk entry, cache 0, C = L, one page holding the whole segment
        kp = k[lo:hi].transpose(1, 0, 2)[None]                 # [1, Hk, L, D]
        vp = v[lo:hi].transpose(1, 2, 0)[None]                 # [1, Hk, D, L]
        table = pos[2 * lo: 2 * lo + 2 * n - 1]
        chunk = oracle.chunk_relpos_attn(q[None, lo:hi], kp, vp, np.array([[0]]), np.array([0]),
                                         table, u, w)[0]
        assert np.abs(chunk - out[lo:hi]).max() < 1e-13


def test_workload_geometry_matches_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "workload_geometry.json")))
    co = make_config(0)
    assert co.pos.shape[0] == g["tiny_fp32"]["table_rows"]
    assert co.k_pool.shape[0] == 32
    for fw in g["fixed_window"]:
        pages = (fw["window"] + fw["chunk"] + 16 - 1) // 16
        assert pages == fw["pages_per_stream"]
    assert WORKLOADS[1]["block_size"] == g["engine_defaults"]["block_size_frames"]
    assert WORKLOADS[1]["max_blocks_per_seq"] == g["engine_defaults"]["max_blocks_per_seq"]
    co1 = make_chunk_cohort(2, 4, 64, 16, 16, [256, 256], dtype=torch.bfloat16)
    assert co1.meta["pages"] == [17, 17]


# --------------------------------------------------------------------------------------------
# Sensitivity: plant slips in the oracle and check that the pins above notice them.
# --------------------------------------------------------------------------------------------

def _pin_errors(margin=3):
    # tables carry a few spare rows, so a slipped row index stays inside the table and must be
    # caught by value, not by the oracle's own bounds check
    case = _random_streaming_case(11, [0, 4, 9], margin=margin)
    brute = np.abs(_oracle(case) - _brute_force(case)).max()
    dense = _streaming_vs_dense(21, steps=3, margin=margin)
    return brute, dense


def test_pins_hold_with_spare_table_rows():
    brute, dense = _pin_errors()
    assert brute < 1e-12 and dense < 1e-12


@pytest.mark.parametrize("slip", ["sign", "centre", "no_u", "swap_uv", "no_scale_pos"])
def test_planted_mistakes_are_caught(monkeypatch, slip):
    if slip == "sign":
        monkeypatch.setattr(orc, "table_row", lambda center, cache, i, j: center + (cache + i - j))
    elif slip == "centre":
        monkeypatch.setattr(orc, "table_row", lambda center, cache, i, j: center - (cache + i - j) - 1)
    else:
        real = orc._attend

        def slipped(q, k, v, pos_rows, u, w, center, cache, scale, *a, **kw):
            if slip == "no_u":
                u = u * 0
            elif slip == "swap_uv":
                u, w = w, u
            elif slip == "no_scale_pos":
                pos_rows = pos_rows * math.sqrt(q.shape[-1])
            return real(q, k, v, pos_rows, u, w, center, cache, scale, *a, **kw)
        monkeypatch.setattr(orc, "_attend", slipped)
    # the mirrored distance needs a table long enough on both sides to stay in range
    brute, dense = _pin_errors(margin=30 if slip == "sign" else 3)
    assert max(brute, dense) > 1e-6, (brute, dense)


# --------------------------------------------------------------------------------------------
# Per-row chunk lengths (a short final window) and the padding lane
# --------------------------------------------------------------------------------------------

def _short_final_window(seed, lens, C=4, H=2, Hk=1, D=8, S=4, per_row=False):
    """Stream one utterance chunk by chunk; step k carries lens[k] <= C real frames, padded to C
    with NaN (in q, k_new and v_new alike, so any use of a padded frame shows). Returns the real
    frames' outputs, the padded rows' outputs, the final pools and the dense reference."""
    rng = np.random.default_rng(seed)
    n = sum(lens)
    q_all = rng.standard_normal((n, H, D))
    k_all = rng.standard_normal((n, Hk, D))
    v_all = rng.standard_normal((n, Hk, D))
    u = 0.5 * rng.standard_normal((H, D))
    w = 0.5 * rng.standard_normal((H, D))
    proj = relpos_projection(H * D, torch.Generator().manual_seed(seed))
    pages = (len(lens) * C + S - 1) // S
    bt = rng.permutation(pages + 2)[None, :pages]
    kp = np.full((pages + 2, Hk, S, D), np.nan)
    vp = np.full((pages + 2, Hk, D, S), np.nan)
    real, pad = [], []
    c = 0
    for m in lens:
        def padded(x):
            y = np.full((C,) + x.shape[1:], np.nan)
            y[:m] = x[c:c + m]
            return y[None]
        cl = np.array([m])
        kp, vp = oracle.paged_kv_append(kp, vp, padded(k_all), padded(v_all), bt, np.array([c]), cl)
        table = descending_table(c + C - 1, proj, H, D).numpy()       # built for the full width
        pos = table[None] if per_row else table
        o = oracle.chunk_relpos_attn(padded(q_all), kp, vp, bt, np.array([c]), pos, u, w,
                                     per_row_pos=per_row, chunk_lens=cl)[0]
        real.append(o[:m])
        pad.append(o[m:])
        c += m
    # dense reference over the real frames only: chunk k holds frames [k C, k C + lens[k]), so
    # the block-causal mask is by step index, not by frame // C
    step_of = np.concatenate([np.full(m, k) for k, m in enumerate(lens)])
    t = np.arange(n)
    dist = t[:, None] - t[None, :]
    emb = embed_distances(dist.reshape(-1), proj, H, D).numpy().reshape(n, n, H, D)
    dense = np.zeros((n, H, D))
    for h in range(H):
        g = h * Hk // H
        bias = np.einsum("td,tjd->tj", q_all[:, h] + w[h], emb[:, :, h]) / math.sqrt(D)
        bias = np.where(step_of[None, :] <= step_of[:, None], bias, -np.inf)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q_all[:, h] + u[h])[None], torch.from_numpy(k_all[:, g])[None],
            torch.from_numpy(v_all[:, g])[None], attn_mask=torch.from_numpy(bias)[None])
        dense[:, h] = ref[0].numpy()
    return np.concatenate(real), pad, kp, vp, bt, dense


@pytest.mark.parametrize("per_row", [False, True])
def test_short_final_window_equals_dense_attention_over_real_frames(per_row):
    """Full chunks then a short final window (and a short middle one): the real frames' outputs
    equal dense block-causal attention over the frames that exist, padded frames are never read
    (they are NaN), padded output rows are zero, and nothing is written past the real frames."""
    lens = [4, 4, 2, 4, 3]
    real, pad, kp, vp, bt, dense = _short_final_window(31, lens, per_row=per_row)
    assert np.abs(real - dense).max() < 1e-12
    for p in pad:
        assert (p == 0).all()
    # the pool holds exactly the sum(lens) real frames; every other slot is still NaN
    S = kp.shape[2]
    n = sum(lens)
    written = np.zeros(kp.shape[0] * S, dtype=bool)
    for t in range(n):
        written[bt[0, t // S] * S + t % S] = True
    slots_k = ~np.isnan(kp).all(axis=(1, 3)).reshape(-1)
    assert (slots_k == written).all()


def test_padding_lane_is_inert():
    """A row with chunk length 0 (the padding lane, its table pointing only at a scratch block)
    appends nothing, outputs zeros, and leaves every other row's output unchanged."""
    case = _random_streaming_case(41, [4, 9, 2])
    base = _oracle(case)
    B = len(case["cs"])
    scratch = case["kp"].shape[0]
    kp = np.concatenate([case["kp"], np.full((1,) + case["kp"].shape[1:], np.nan)])
    vp = np.concatenate([case["vp"], np.full((1,) + case["vp"].shape[1:], np.nan)])
    bt = np.concatenate([case["bt"], np.full((1, case["bt"].shape[1]), scratch)])
    cs = np.concatenate([case["cs"], [5]])
    q = np.concatenate([case["q"], np.full((1,) + case["q"].shape[1:], np.nan)])
    lens = np.array([case["C"]] * B + [0])
    junk = np.full((B + 1, case["C"], case["Hk"], case["D"]), np.nan)
    kp2, vp2 = oracle.paged_kv_append(kp, vp, junk, junk, bt, cs, np.array([0] * (B + 1)))
    np.testing.assert_array_equal(kp2, kp)
    out = oracle.chunk_relpos_attn(q, kp, vp, bt, cs, case["table"], case["u"], case["w"],
                                   chunk_lens=lens)
    np.testing.assert_array_equal(out[:B], base)
    assert (out[B] == 0).all()


def test_chunk_lens_of_full_width_change_nothing():
    case = _random_streaming_case(43, [0, 5, 11])
    lens = np.full(len(case["cs"]), case["C"])
    np.testing.assert_array_equal(_oracle(case, chunk_lens=lens), _oracle(case))


# --------------------------------------------------------------------------------------------
# Bounded history: a left-context cap with pages recycled through a ring
# --------------------------------------------------------------------------------------------

def _bounded_stream(seed, steps, K, C=4, S=4, M=None, H=2, Hk=1, D=8):
    """Stream one utterance with at most K chunks of cached history: after each step the commit
    drops whole oldest blocks past the cap, and the table row is a ring of M pages, so pages are
    reused (old frames overwritten) many times over the stream's life. Returns the streamed
    outputs, the dense reference with the limited chunk mask, and the pool's final state."""
    rng = np.random.default_rng(seed)
    n = steps * C
    q_all = rng.standard_normal((n, H, D))
    k_all = rng.standard_normal((n, Hk, D))
    v_all = rng.standard_normal((n, Hk, D))
    u = 0.5 * rng.standard_normal((H, D))
    w = 0.5 * rng.standard_normal((H, D))
    proj = relpos_projection(H * D, torch.Generator().manual_seed(seed))
    cap = K * C
    if M is None:
        M = (cap + C + S - 1) // S + 1
    N = M + 3
    bt = rng.permutation(N)[None, :M]
    kp = np.full((N, Hk, S, D), np.nan)
    vp = np.full((N, Hk, D, S), np.nan)
    cache, start = np.array([0]), np.array([0])
    table = descending_table(cap + C - 1, proj, H, D).numpy()
    outs = []
    for step in range(steps):
        sl = slice(step * C, (step + 1) * C)
        assert start[0] + cache[0] == step * C            # the window ends at the stream's end
        kp, vp = oracle.paged_kv_append(kp, vp, k_all[None, sl], v_all[None, sl], bt, cache,
                                        window_start=start)
        outs.append(oracle.chunk_relpos_attn(q_all[None, sl], kp, vp, bt, cache, table, u, w,
                                             window_start=start)[0])
        cache, start = oracle.commit_chunk(cache, C, window_start=start, max_cached_frames=cap,
                                           block_size=S)
        assert cache[0] <= cap and start[0] % S == 0
    stream = np.concatenate(outs)
    # dense: query chunk a sees key chunks [a - K, a], distances i - j
    t = np.arange(n)
    qa, ka = t[:, None] // C, t[None, :] // C
    dist = t[:, None] - t[None, :]
    emb = embed_distances(dist.reshape(-1), proj, H, D).numpy().reshape(n, n, H, D)
    dense = np.zeros((n, H, D))
    for h in range(H):
        g = h * Hk // H
        bias = np.einsum("td,tjd->tj", q_all[:, h] + w[h], emb[:, :, h]) / math.sqrt(D)
        bias = np.where((ka <= qa) & (ka >= qa - K), bias, -np.inf)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q_all[:, h] + u[h])[None], torch.from_numpy(k_all[:, g])[None],
            torch.from_numpy(v_all[:, g])[None], attn_mask=torch.from_numpy(bias)[None])
        dense[:, h] = ref[0].numpy()
    return stream, dense


@pytest.mark.parametrize("K,S", [(2, 4), (3, 2), (0, 4), (1, 4)])
def test_bounded_history_equals_dense_attention_with_limited_left_context(K, S):
    """num_left_chunks = K with ring-recycled pages: streaming over many more chunks than the
    ring holds equals dense attention where a query chunk sees only its own and the K previous
    chunks, with absolute distances (the window-relative distances of the oracle are the same).
    The block size divides the chunk here, so whole-block eviction keeps exactly K chunks."""
    stream, dense = _bounded_stream(61, steps=9, K=K, C=4, S=S)
    assert np.abs(stream - dense).max() < 1e-12


def test_commit_keeps_the_window_at_the_cap_by_whole_blocks():
    cache, start = oracle.commit_chunk(np.array([0, 30, 60]), 16, chunk_lens=np.array([16, 5, 0]),
                                       window_start=np.array([0, 32, 64]), max_cached_frames=40,
                                       block_size=8)
    # stream 2: 60 frames > 40, so three 8-frame blocks go: 36 frames from position 88
    assert cache.tolist() == [16, 35, 36] and start.tolist() == [0, 32, 88]
    cache, start = oracle.commit_chunk(np.array([3]), 16)
    assert cache.tolist() == [19] and start is None


def test_commit_drops_only_filled_blocks():
    """A cap below one block: 0 + 13 frames with 8-frame blocks and cap 0 drops the one filled
    block and keeps the 5 frames of the partly filled one (the next chunk continues it); dropping
    two blocks would have left -3 frames and a window start past the next write position."""
    cache, start = oracle.commit_chunk(np.array([0, 0, 2]), 16, chunk_lens=np.array([13, 16, 5]),
                                       window_start=np.array([0, 8, 16]), max_cached_frames=0,
                                       block_size=8)
    assert cache.tolist() == [5, 0, 7] and start.tolist() == [8, 24, 16]
    assert (cache >= 0).all()


# --------------------------------------------------------------------------------------------
# Other conventions: WeNet's per-key table (no shift) and the chunked_limited mask
# --------------------------------------------------------------------------------------------

def _per_key_tables(case, starts, width):
    """Per-row WeNet tables: row j of stream b is the projected sinusoid of absolute position
    starts[b] + j (positions start at offset - cache_seqlens)."""
    H, D = case["H"], case["D"]
    return np.stack([embed_distances(np.arange(s, s + width), case["proj"], H, D).numpy()
                     for s in starts])


def test_per_key_positions_match_brute_force():
    """(q_i + v) . emb(start_b + j), computed with scalar loops and the projected sinusoid of each
    key's absolute position directly (no table)."""
    case = _random_streaming_case(71, [0, 5, 9])
    starts = [3, 17, 40]
    C, H, Hk, D = case["C"], case["H"], case["Hk"], case["D"]
    width = max(case["cs"]) + C
    tables = _per_key_tables(case, starts, width)
    out = oracle.chunk_relpos_attn(case["q"], case["kp"], case["vp"], case["bt"], case["cs"], tables,
                                   case["u"], case["w"], per_row_pos=True, per_key_pos=True)
    q, u, w = case["q"], case["u"], case["w"]
    brute = np.zeros(q.shape)
    for b, c in enumerate(case["cs"]):
        T = int(c) + C
        emb = embed_distances(np.arange(starts[b], starts[b] + T), case["proj"], H, D).numpy()
        for h in range(H):
            g = h * Hk // H
            for i in range(C):
                sc = [(math.fsum((q[b, i, h, d] + u[h, d]) * case["seq_k"][b][j, g, d] for d in range(D))
                       + math.fsum((q[b, i, h, d] + w[h, d]) * emb[j, h, d] for d in range(D)))
                      / math.sqrt(D) for j in range(T)]
                mx = max(sc)
                ex = [math.exp(x - mx) for x in sc]
                z = math.fsum(ex)
                for d in range(D):
                    brute[b, i, h, d] = math.fsum(ex[j] / z * case["seq_v"][b][j, g, d] for j in range(T))
    assert np.abs(out - brute).max() < 1e-12


def test_per_key_streaming_equals_dense_absolute_position_bias():
    """WeNet streaming from an empty cache: each step's table holds the keys' absolute positions
    [0, c + C); the concatenated chunks equal dense block-causal attention with the bias
    (q_t + v) . emb(j) of the key's absolute position, through float64 SDPA. A shared per-key
    table (every stream at the same offset) gives the same result as a per-row one."""
    rng = np.random.default_rng(73)
    steps, C, H, Hk, D, S = 4, 4, 2, 1, 8, 4
    n = steps * C
    q_all = rng.standard_normal((n, H, D))
    k_all = rng.standard_normal((n, Hk, D))
    v_all = rng.standard_normal((n, Hk, D))
    u = 0.5 * rng.standard_normal((H, D))
    w = 0.5 * rng.standard_normal((H, D))
    proj = relpos_projection(H * D, torch.Generator().manual_seed(73))
    emb_all = embed_distances(np.arange(n), proj, H, D).numpy()
    pages = n // S
    bt = rng.permutation(pages + 2)[None, :pages]
    kp = np.full((pages + 2, Hk, S, D), np.nan)
    vp = np.full((pages + 2, Hk, D, S), np.nan)
    outs = []
    for step in range(steps):
        c = step * C
        sl = slice(c, c + C)
        kp, vp = oracle.paged_kv_append(kp, vp, k_all[None, sl], v_all[None, sl], bt, np.array([c]))
        shared = emb_all[:c + C]
        o1 = oracle.chunk_relpos_attn(q_all[None, sl], kp, vp, bt, np.array([c]), shared, u, w,
                                      per_key_pos=True)[0]
        o2 = oracle.chunk_relpos_attn(q_all[None, sl], kp, vp, bt, np.array([c]), shared[None], u, w,
                                      per_row_pos=True, per_key_pos=True)[0]
        np.testing.assert_array_equal(o1, o2)
        outs.append(o1)
    stream = np.concatenate(outs)
    t = np.arange(n)
    dense = np.zeros((n, H, D))
    for h in range(H):
        bias = np.einsum("td,jd->tj", q_all[:, h] + w[h], emb_all[:, h]) / math.sqrt(D)
        bias = np.where((t[None, :] // C) <= (t[:, None] // C), bias, -np.inf)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q_all[:, h] + u[h])[None], torch.from_numpy(k_all[:, 0])[None],
            torch.from_numpy(v_all[:, 0])[None], attn_mask=torch.from_numpy(bias)[None])
        dense[:, h] = ref[0].numpy()
    assert np.abs(stream - dense).max() < 1e-12


@pytest.mark.parametrize("chunk,left", [(4, 2), (3, 0), (5, 10)])
def test_chunked_limited_offline_equals_streaming_with_the_trained_window(chunk, left):
    """The chunked_limited mask offline equals running each chunk as one streaming step whose
    cache is the chunk's allowed history (cache = min(a, left) chunks), and dense attention with
    the explicit chunk mask and distance bias."""
    lengths = [17, 9, 4]
    H, D = 2, 8
    co = make_varlen_cohort(lengths, H, D, dtype=F64, seed=75)
    q, k, v = np64(co.q), np64(co.k), np64(co.v)
    u, w = np64(co.pos_bias_u), np64(co.pos_bias_v)
    pos = np64(co.pos)
    cu = co.cu_seqlens.numpy()
    out = oracle.varlen_relpos_attn(q, k, v, cu, pos, u, w, chunk=chunk, left_chunks=left)
    for s, n in enumerate(lengths):
        lo = cu[s]
        for a in range(0, (n + chunk - 1) // chunk):
            f0, f1 = a * chunk, min(n, (a + 1) * chunk)
            h0 = max(0, a - left) * chunk                          # first key of the history
            c = f0 - h0
            kp = k[lo + h0: lo + f1].transpose(1, 0, 2)[None]      # one page holds the window
            vp = v[lo + h0: lo + f1].transpose(1, 2, 0)[None]
            table = descending_table(c + (f1 - f0) - 1, co.meta["proj"], H, D).numpy()
            step = oracle.chunk_relpos_attn(q[None, lo + f0: lo + f1], kp, vp, np.array([[0]]),
                                            np.array([c]), table, u, w)[0]
            assert np.abs(step - out[lo + f0: lo + f1]).max() < 1e-12, (s, a)
        t = np.arange(n)
        dist = t[:, None] - t[None, :]
        emb = embed_distances(dist.reshape(-1), co.meta["proj"], H, D).numpy().reshape(n, n, H, D)
        keep = oracle.chunked_limited_keep(chunk, left)
        mask = np.stack([keep(i, t) for i in range(n)])
        for h in range(H):
            bias = np.einsum("td,tjd->tj", q[lo:lo + n, h] + w[h], emb[:, :, h]) / math.sqrt(D)
            bias = np.where(mask, bias, -np.inf)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[lo:lo + n, h] + u[h])[None], torch.from_numpy(k[lo:lo + n, h])[None],
                torch.from_numpy(v[lo:lo + n, h])[None], attn_mask=torch.from_numpy(bias)[None])
            assert np.abs(ref[0].numpy() - out[lo:lo + n, h]).max() < 1e-12


def test_column_blocked_k_pages():
    """The kernels' K page layout keeps each 32-dim block of every slot's row together:
    element (block, g, c, slot, e) holds dim 32 c + e of the frame in that slot. Appending into
    such a pool puts every value where that definition says, and reading back through it
    returns the same frames as the plain [slot][dim] layout."""
    rng = np.random.default_rng(81)
    B, C, Hk, D, S, N = 2, 5, 2, 64, 8, 6
    bt = np.array([[4, 1, 5], [0, 3, 2]])
    cs = np.array([3, 9])
    k_new = rng.standard_normal((B, C, Hk, D))
    v_new = rng.standard_normal((B, C, Hk, D))
    plain = np.full((N, Hk, S, D), np.nan)
    blocked = np.full((N, Hk, D // 32, S, 32), np.nan)
    vp = np.full((N, Hk, D, S), np.nan)
    kp1, vp1 = oracle.paged_kv_append(plain, vp, k_new, v_new, bt, cs)
    kp2, vp2 = oracle.paged_kv_append(blocked, vp, k_new, v_new, bt, cs)
    np.testing.assert_array_equal(vp1, vp2)
    for b in range(B):
        for t in range(C):
            f = cs[b] + t
            blk, slot = bt[b, f // S], f % S
            for c in range(D // 32):
                np.testing.assert_array_equal(kp2[blk, :, c, slot, :], k_new[b, t, :, 32 * c:32 * c + 32])
    assert np.isnan(kp2).sum() == np.isnan(kp1).sum()
    for b in range(B):
        k1, v1 = oracle.gather_stream(kp1, vp1, bt[b], cs[b] + C)
        k2, v2 = oracle.gather_stream(kp2, vp2, bt[b], cs[b] + C)
        np.testing.assert_array_equal(k1, k2)
        np.testing.assert_array_equal(v1, v2)


# --------------------------------------------------------------------------------------------
# The GEMMs either side: linear, the sinusoidal table and its projection, the Q/K/V append
# --------------------------------------------------------------------------------------------

def test_linear_matches_brute_force():
    rng = np.random.default_rng(40)
    x = rng.normal(size=(2, 3, 5))
    w = rng.normal(size=(4, 5))
    b = rng.normal(size=4)
    y = oracle.linear(x, w, b)
    assert y.shape == (2, 3, 4)
    for i in range(2):
        for t in range(3):
            for n in range(4):
                acc = b[n]
                for k in range(5):
                    acc += x[i, t, k] * w[n, k]
                assert abs(y[i, t, n] - acc) < 1e-12
    assert np.allclose(oracle.linear(x, w), y - b, atol=1e-12)


def test_sinusoid_closed_forms():
    d = 8
    e = oracle.sinusoid([0, 1, -1, 2, 3, 5, 37], d)
    # position 0: sin 0 = 0 in even columns, cos 0 = 1 in odd columns
    assert np.array_equal(e[0], np.array([0.0, 1.0] * (d // 2)))
    # position 1, first pair: frequency 1
    assert abs(e[1, 0] - 0.8414709848078965) < 1e-15 and abs(e[1, 1] - 0.5403023058681398) < 1e-15
    # frequencies 10000^(-2i/d), read back from position 1's angles
    for i in range(d // 2):
        assert abs(math.atan2(e[1, 2 * i], e[1, 2 * i + 1]) - math.pow(10000.0, -2.0 * i / d)) < 1e-13
    # every (sin, cos) pair has unit norm
    assert np.allclose(e[:, 0::2] ** 2 + e[:, 1::2] ** 2, 1.0, atol=1e-14)
    # odd sine, even cosine
    assert np.allclose(e[2, 0::2], -e[1, 0::2], atol=1e-15) and np.allclose(e[2, 1::2], e[1, 1::2], atol=1e-15)
    # angle addition: PE(2 + 3) from PE(2) and PE(3)
    s2, c2, s3, c3 = e[3, 0::2], e[3, 1::2], e[4, 0::2], e[4, 1::2]
    assert np.allclose(e[5, 0::2], s2 * c3 + c2 * s3, atol=1e-13)
    assert np.allclose(e[5, 1::2], c2 * c3 - s2 * s3, atol=1e-13)


def test_rel_pos_projection_matches_brute_force():
    rng = np.random.default_rng(41)
    d, n_out, rows = 6, 4, 5
    w = rng.normal(size=(n_out, d))
    starts, step = [3, -2], -1
    got = oracle.rel_pos_projection(w, starts, step, rows)
    assert got.shape == (2, rows, n_out)
    for t, s0 in enumerate(starts):
        for r in range(rows):
            p = s0 + step * r
            emb = []
            for i in range(d // 2):
                ang = p * math.pow(10000.0, -2.0 * i / d)
                emb += [math.sin(ang), math.cos(ang)]
            for n in range(n_out):
                assert abs(got[t, r, n] - sum(emb[k] * w[n, k] for k in range(d))) < 1e-12


def test_rel_pos_projection_orientation_and_shift():
    rng = np.random.default_rng(42)
    d, n_out = 8, 6
    w = rng.normal(size=(n_out, d))
    center = 4
    tab = oracle.rel_pos_projection(w, [center], -1, 2 * center + 1)[0]
    # row `center` holds distance 0: sin terms vanish, cos terms are 1
    assert np.allclose(tab[center], w[:, 1::2].sum(axis=1), atol=1e-13)
    # row r holds distance center - r: row 0 is the largest positive distance
    assert np.allclose(tab[0], oracle.linear(oracle.sinusoid([center], d), w)[0], atol=1e-13)
    # a table centred 2 further is the same rows shifted by 2
    tab2 = oracle.rel_pos_projection(w, [center + 2], -1, 2 * center + 1)[0]
    assert np.allclose(tab2[2:], tab[:-2], atol=1e-13)
    # ascending (WeNet) tables: row j of start s is position s + j
    asc = oracle.rel_pos_projection(w, [-3], 1, 7)[0]
    assert np.allclose(asc[3], w[:, 1::2].sum(axis=1), atol=1e-13)


def test_qkv_append_addresses_and_order():
    rng = np.random.default_rng(43)
    B, C, dm, H, Hk, D, S, N, M = 2, 3, 6, 2, 1, 4, 2, 9, 4
    x = rng.normal(size=(B, C, dm))
    w = rng.normal(size=((H + 2 * Hk) * D, dm))
    bias = rng.normal(size=(H + 2 * Hk) * D)
    k_pool = rng.normal(size=(N, Hk, S, D))
    v_pool = rng.normal(size=(N, Hk, D, S))
    bt = np.array([[5, 2, 7, 0], [1, 8, 3, 6]])
    cs = np.array([1, 4])
    lens = np.array([3, 2])
    q, k_out, v_out = oracle.qkv_append(x, w, bias, k_pool, v_pool, bt, cs, H, Hk, D, chunk_lens=lens)
    k_ref, v_ref = k_pool.copy(), v_pool.copy()
    for b in range(B):
        for t in range(C):
            row = [sum(x[b, t, c] * w[n, c] for c in range(dm)) + bias[n] for n in range(w.shape[0])]
            for h in range(H):
                assert np.allclose(q[b, t, h], row[h * D:(h + 1) * D], atol=1e-12)
            if t >= lens[b]:
                continue
            frame = cs[b] + t
            blk, slot = bt[b][frame // S], frame % S
            for g in range(Hk):
                k_ref[blk, g, slot, :] = row[H * D + g * D:H * D + (g + 1) * D]
                v_ref[blk, g, :, slot] = row[(H + Hk) * D + g * D:(H + Hk) * D + (g + 1) * D]
    assert np.allclose(k_out, k_ref, atol=1e-12) and np.allclose(v_out, v_ref, atol=1e-12)


_PROJ_PINS = [test_linear_matches_brute_force, test_sinusoid_closed_forms,
              test_rel_pos_projection_matches_brute_force, test_rel_pos_projection_orientation_and_shift,
              test_qkv_append_addresses_and_order]


@pytest.mark.parametrize("slip", ["sin_cos_swapped", "frequency_exponent", "no_bias", "step_sign", "kv_order"])
def test_planted_projection_mistakes_are_caught(monkeypatch, slip):
    import oracle.projections as prj
    real_sin, real_lin, real_pos, real_qkv = prj.sinusoid, prj.linear, prj.table_positions, prj.qkv_project
    if slip == "sin_cos_swapped":
        def bad(positions, d_model):
            e = real_sin(positions, d_model)
            return np.ascontiguousarray(e[:, [c ^ 1 for c in range(d_model)]])
        monkeypatch.setattr(prj, "sinusoid", bad)
        monkeypatch.setattr(oracle, "sinusoid", bad)
    elif slip == "frequency_exponent":
        def bad(positions, d_model):
            p = np.asarray(positions, dtype=np.float64)[:, None]
            f = np.power(10000.0, -np.arange(d_model // 2)[None, :] / d_model)
            e = np.empty((p.shape[0], d_model))
            e[:, 0::2], e[:, 1::2] = np.sin(p * f), np.cos(p * f)
            return e
        monkeypatch.setattr(prj, "sinusoid", bad)
        monkeypatch.setattr(oracle, "sinusoid", bad)
    elif slip == "no_bias":
        bad = lambda x, w, bias=None: real_lin(x, w)
        monkeypatch.setattr(prj, "linear", bad)
        monkeypatch.setattr(oracle, "linear", bad)
    elif slip == "step_sign":
        bad = lambda s, step, rows: real_pos(s, -step, rows)
        monkeypatch.setattr(prj, "table_positions", bad)
        monkeypatch.setattr(oracle, "table_positions", bad)
    elif slip == "kv_order":
        def bad(x, w, b, H, Hk, D):
            q, k, v = real_qkv(x, w, b, H, Hk, D)
            return q, v, k
        monkeypatch.setattr(prj, "qkv_project", bad)
        monkeypatch.setattr(oracle, "qkv_project", bad)
    failed = 0
    for pin in _PROJ_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught the planted {slip}"
