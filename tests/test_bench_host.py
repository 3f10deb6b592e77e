"""Host-side logic of bench.py (CPU): the byte and FLOP counts behind the roofline figures, the
kernel hash that guards stored counter readings, and the one-GPU contract."""

import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
from synth import make_config, make_varlen_cohort  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


@pytest.mark.parametrize("L", [1, 5, 16, 17, 100])
@pytest.mark.parametrize("chunk,left", [(0, 0), (4, 0), (4, 1), (16, 2), (13, 1000), (1, 3)])
def test_visible_pairs_count_the_oracle_mask(L, chunk, left):
    # the FLOP count's pairs against the oracle's own mask, pair by pair
    if chunk == 0:
        brute = L * L
    else:
        keep = oracle.chunked_limited_keep(chunk, left)
        brute = sum(int(keep(i, np.arange(L)).sum()) for i in range(L))
    assert bench.visible_pairs(L, chunk, left) == brute


def test_algorithmic_bytes_of_the_small_cohort():
    # d_model 256 streaming cohort: B 64, H = Hk = 4, D 64, C 16, cache 256, block 16, bf16,
    # one shared table. Term by term: q in and out; k_new, v_new read and appended; the cached
    # K/V; the band's cache + 2 C - 1 rows; u and v; 17 table entries and one cache length per
    # stream.
    co = make_config(1, device="cpu")
    B, C, H, Hk, D, c, eb = 64, 16, 4, 4, 64, 256, 2
    expect = (2 * B * C * H * D * eb + 4 * B * C * Hk * D * eb + 2 * B * c * Hk * D * eb
              + (c + 2 * C - 1) * H * D * eb + 2 * H * D * eb + B * (17 + 1) * 4)
    assert expect == 20_075_520 == 256 * 78_420   # per launch; per chunk-head
    assert bench.algorithmic_bytes(co) == expect


def test_varlen_flops_and_bytes_of_a_small_batch():
    co = make_varlen_cohort([3, 0, 5], 2, 64, device="cpu")
    H, D, eb = 2, 64, 2
    assert bench.varlen_flops(co) == 6 * (9 + 25) * D * H
    # chunks of 2, no earlier chunk: a query sees its own chunk's frames, later ones included
    # (L 3: 2 + 2 + 1 pairs; L 5: 2 + 2 + 2 + 2 + 1)
    assert bench.varlen_flops(co, chunk=2, left=0) == 6 * (5 + 9) * D * H
    # q, k, v in and out written; 2 L - 1 table rows per non-empty utterance; u and v
    assert bench.varlen_bytes(co) == (4 * 8 * H * D + (5 + 9) * H * D + 2 * H * D) * eb


def _copy_sources(dst):
    csrc = os.path.join(dst, "paged_kv_chunk_amd", "csrc")
    shutil.copytree(os.path.join(ROOT, "paged_kv_chunk_amd", "csrc"), csrc)
    return csrc


def test_kernel_hash_ignores_comments_and_sees_code(tmp_path, monkeypatch):
    csrc = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    path = os.path.join(csrc, "pkc_step.h")
    text = open(path).read()
    open(path, "w").write(text.replace("namespace pkc {", "namespace pkc {  // a comment\n\n", 1))
    assert {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES} == base
    open(path, "w").write(text.replace("kRescaleLog2 = 8.f", "kRescaleLog2 = 7.f", 1))
    changed = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    assert changed["chunk"] != base["chunk"] and changed["varlen"] != base["varlen"]
    assert changed["gemm"] == base["gemm"]   # the GEMM does not include the step header


def test_host_sample_gives_the_oracle_the_same_streams():
    """The CPU baseline's host copies of a few streams (only their pages, block IDs renumbered)
    give the oracle exactly the result it gives on the whole cohort for those streams."""
    import numpy as np
    import torch
    import bench
    import oracle
    from synth import make_chunk_cohort
    bench.torch = torch
    co = make_chunk_cohort(4, 2, 64, 16, 16, [0, 40, 129, 7], dtype=torch.float32, seed=5)
    h = lambda t: t.detach().double().numpy()
    bt, cs = co.block_tables.numpy(), co.cache_seqlens.numpy()
    kp, vp = oracle.paged_kv_append(h(co.k_pool), h(co.v_pool), h(co.k_new), h(co.v_new), bt, cs)
    full = oracle.chunk_relpos_attn(h(co.q), kp, vp, bt, cs, h(co.pos), h(co.pos_bias_u),
                                    h(co.pos_bias_v))
    x = bench.host_sample(co, [2, 0])
    assert x["k_pool"].shape[0] == (129 + 16 + 15) // 16 + 1
    kp2, vp2 = oracle.paged_kv_append(x["k_pool"], x["v_pool"], x["k_new"], x["v_new"], x["bt"],
                                      x["cs"])
    part = oracle.chunk_relpos_attn(x["q"], kp2, vp2, x["bt"], x["cs"], x["pos"], x["u"], x["w"])
    np.testing.assert_array_equal(part, full[[2, 0]])


def test_cpu_baseline_records_its_sample_and_library():
    import torch
    import bench
    from synth import make_chunk_cohort
    bench.torch = torch
    co = make_chunk_cohort(3, 2, 64, 16, 16, [0, 16, 32], dtype=torch.float32, seed=6)
    r = bench.cpu_baseline(co, 0.05, name="tiny")
    assert r["value"] > 0 and r["cores"] == 1 and r["threads"] == 1 and r["kind"] == "oracle"
    assert "blas" in r and r["sample"].startswith("tiny: 3 of 3 streams")
