"""Host-only checks of the C ABI: the library loads, exports every function include/pkc.h
declares, and every validation error returns its status before anything is launched.

No call here passes validation: the pointers are fake (never dereferenced), so each case is built
to fail a host-side check.
"""

import ctypes
import os
import re

import pytest

import paged_kv_chunk_amd as pkc
from paged_kv_chunk_amd import build as pkc_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkc.h")

OK, NULL, SHAPE, DTYPE, UNSUP, CAP, HIP, ALIGN = range(8)
P = 0x10000          # a fake, 16-byte aligned "device" address
BAD = 0x10008        # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkc.LIB_PATH):
        pkc_build.build()
    return pkc.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:pkc_status|int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["paged_kv_append", "chunk_paged_relpos_attn", "paged_kv_append_relpos_attn",
              "paged_kv_append_relpos_attn_layers", "paged_kv_commit",
              "varlen_packed_relpos_attn", "pkc_linear", "paged_kv_qkv_append",
              "rel_pos_projection", "pkc_version", "pkc_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(pkc.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
        assert name in pkc.SIGNATURES, name


def test_version_and_status_strings(lib):
    assert pkc.version() >= 100
    for s in range(8):
        assert pkc.status_string(s) and pkc.status_string(s) != "unknown status"
    assert pkc.status_string(99) == "unknown status"


def append(lib, dtype=1, k_new=P, v_new=P, k_pool=P, v_pool=P, bt=P, cs=P, B=2, C=16, Hk=4, D=64,
           S=16, N=32, M=8, max_cache=64):
    return lib.paged_kv_append(dtype, k_new, v_new, k_pool, v_pool, bt, cs, None, None, B, C, Hk,
                               D, S, N, M, max_cache, None)


def attn(lib, dtype=1, q=P, k_pool=P, v_pool=P, bt=P, cs=P, pos=P, pos_len=159, per_row=0, u=P,
         w=P, out=P, B=2, C=16, H=4, Hk=4, D=64, S=16, N=32, M=8, max_cache=64, scale=0.0):
    return lib.chunk_paged_relpos_attn(dtype, q, k_pool, v_pool, bt, cs, None, None, pos, pos_len,
                                       per_row, u, w, out, B, C, H, Hk, D, S, N, M, max_cache,
                                       scale, None)


def fused(lib, k_new=P, v_new=P, **kw):
    a = dict(dtype=1, q=P, k_pool=P, v_pool=P, bt=P, cs=P, pos=P, pos_len=159, per_row=0, u=P,
             w=P, out=P, B=2, C=16, H=4, Hk=4, D=64, S=16, N=32, M=8, max_cache=64, scale=0.0)
    a.update(kw)
    return lib.paged_kv_append_relpos_attn(a["dtype"], a["q"], k_new, v_new, a["k_pool"],
                                           a["v_pool"], a["bt"], a["cs"], None, None, a["pos"],
                                           a["pos_len"],
                                           a["per_row"], a["u"], a["w"], a["out"], a["B"], a["C"],
                                           a["H"], a["Hk"], a["D"], a["S"], a["N"], a["M"],
                                           a["max_cache"], a["scale"], None)


def varlen(lib, dtype=1, q=P, k=P, v=P, cu=P, S=4, total=100, max_len=40, pos=P, u=P, w=P, out=P,
           H=8, Hk=8, D=64, chunk=0, left=0):
    return lib.varlen_packed_relpos_attn(dtype, q, k, v, cu, S, total, max_len, pos, u, w, out, H,
                                         Hk, D, chunk, left, 0.0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), DTYPE),
    (dict(k_new=None), NULL), (dict(v_pool=None), NULL), (dict(bt=None), NULL), (dict(cs=None), NULL),
    (dict(B=0), SHAPE), (dict(C=0), SHAPE), (dict(D=60), SHAPE), (dict(S=0), SHAPE),
    (dict(max_cache=-1), SHAPE), (dict(N=0), SHAPE),
    (dict(max_cache=113), CAP),                      # 113 + 16 > 8 * 16
    (dict(M=4, max_cache=64), CAP),
    (dict(k_pool=BAD), ALIGN), (dict(k_new=BAD), ALIGN),
    # one workgroup of 256 threads per stream and kv head: 2^32 work-items or more are refused
    (dict(B=1 << 20, Hk=16), UNSUP), (dict(B=1 << 24, Hk=1), UNSUP),
    # the V staging tile (64 frames x head_dim) must fit the default 64 KiB of LDS
    (dict(D=512), UNSUP), (dict(dtype=0, D=256), UNSUP),
])
def test_append_validation(lib, kw, status):
    assert append(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=-1), DTYPE),
    (dict(q=None), NULL), (dict(pos=None), NULL), (dict(u=None), NULL), (dict(out=None), NULL),
    (dict(H=6, Hk=4), SHAPE), (dict(H=0), SHAPE),
    (dict(pos_len=158), SHAPE),                      # even shared table
    (dict(pos_len=157), SHAPE),                      # (157 - 1) / 2 < 64 + 16 - 1
    (dict(per_row=1, pos_len=158), SHAPE),           # per-row needs 2 * 80 - 1
    (dict(per_row=8), SHAPE), (dict(per_row=12), SHAPE), (dict(per_row=-1), SHAPE),
    (dict(per_row=2, pos_len=79), SHAPE),            # per-key table needs 64 + 16 rows
    (dict(per_row=3, pos_len=79), SHAPE),
    (dict(D=128), UNSUP), (dict(S=12, M=12), UNSUP), (dict(S=24, M=12), UNSUP),
    (dict(S=4, M=40), UNSUP),
    # one 256-thread workgroup per 16 queries of a stream and head: 2^32 work-items are refused
    (dict(B=1 << 24, H=128, Hk=128), UNSUP),
    (dict(B=1 << 23, H=128, Hk=64, C=32, pos_len=2 * (64 + 32) - 1), UNSUP),
    (dict(B=1 << 20, H=16, Hk=16), UNSUP),
    # positional tables of 2^25 rows or more (32-bit strides of column-blocked tables)
    (dict(pos_len=(1 << 25) + 1), UNSUP),
    (dict(max_cache=120), CAP),
    (dict(q=BAD), ALIGN), (dict(pos=BAD), ALIGN), (dict(out=BAD), ALIGN),
])
def test_attention_validation(lib, kw, status):
    assert attn(lib, **kw) == status


def test_fused_validation(lib):
    assert fused(lib, k_new=None) == NULL
    assert fused(lib, v_new=None) == NULL
    assert fused(lib, k_new=BAD) == ALIGN
    assert fused(lib, max_cache=200) == CAP
    assert fused(lib, pos_len=100) == SHAPE
    # the chunk is staged in LDS: chunks past 512 frames (bf16) / 256 (fp32) are refused, not
    # launched
    assert fused(lib, dtype=0, C=257, M=32, pos_len=2 * (64 + 257) - 1) == UNSUP
    assert fused(lib, C=513, M=40, pos_len=2 * (64 + 513) - 1) == UNSUP
    assert attn(lib, C=513, M=40, pos_len=2 * (64 + 513) - 1) == UNSUP


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), DTYPE), (dict(cu=None), NULL), (dict(k=None), NULL),
    (dict(S=0), SHAPE), (dict(H=6, Hk=4), SHAPE), (dict(max_len=101), SHAPE), (dict(D=12), SHAPE),
    (dict(D=128), UNSUP), (dict(v=BAD), ALIGN),
    (dict(chunk=-1), SHAPE), (dict(chunk=4, left=-2), SHAPE),
    # an utterance's rows are addressed by 32-bit byte offsets: 2 max_seqlen rows of H D elements
    # must stay under 2^31 bytes
    (dict(total=2_000_000, max_len=2_000_000), UNSUP),
    (dict(dtype=0, total=1_100_000, max_len=1_100_000, H=4, Hk=4), UNSUP),
    # one 256-thread workgroup per 128 queries (bf16; 64 for fp32) of an utterance and head:
    # 2^32 work-items are refused
    (dict(S=1 << 20, total=100, max_len=64, H=2048, Hk=2048), UNSUP),
    (dict(S=1 << 19, total=300, max_len=256, H=2048, Hk=1024), UNSUP),
    (dict(dtype=0, S=1 << 19, total=200, max_len=128, H=2048, Hk=1024), UNSUP),
    (dict(S=1 << 16, total=300, max_len=256, H=128, Hk=128), UNSUP),
    # with the chunked_limited mask a bf16 workgroup takes 64 queries: 2^16 x 128 x 2 of them
    (dict(S=1 << 16, total=300, max_len=128, H=128, Hk=128, chunk=16, left=2), UNSUP),
])
def test_varlen_validation(lib, kw, status):
    assert varlen(lib, **kw) == status


def test_varlen_empty_batch_is_a_no_op(lib):
    assert varlen(lib, total=0, max_len=0) == OK


def test_binding_refuses_host_tensors(lib):
    import torch
    x = torch.zeros(2, 16, 4, 64)
    with pytest.raises(ValueError):
        pkc.chunk_paged_relpos_attn(x, torch.zeros(4, 4, 16, 64), torch.zeros(4, 4, 64, 16),
                                    torch.zeros(2, 2, dtype=torch.int32),
                                    torch.zeros(2, dtype=torch.int32), torch.zeros(31, 4, 64),
                                    torch.zeros(4, 64), torch.zeros(4, 64), max_cache_seqlen=0,
                                    out=torch.zeros_like(x))


def layers_call(lib, n_layers=3, hole=None, dtype=1, C=16, max_cache=64):
    """The multi-layer entry with fake pointers; ``hole`` = (array name, layer) set to NULL."""
    names = ["q", "k_new", "v_new", "k_pool", "v_pool", "pos", "u", "w", "out"]
    arrs = {}
    for n in names:
        a = (ctypes.c_void_p * max(n_layers, 1))(*([P] * max(n_layers, 1)))
        if hole and hole[0] == n:
            a[hole[1]] = None
        arrs[n] = a
    return lib.paged_kv_append_relpos_attn_layers(
        dtype, n_layers, arrs["q"], arrs["k_new"], arrs["v_new"], arrs["k_pool"], arrs["v_pool"],
        P, P, None, None, arrs["pos"], 159, 0, arrs["u"], arrs["w"], arrs["out"], 2, C, 4, 4, 64, 16, 32,
        8, max_cache, 0.0, None)


def test_layers_validation_launches_nothing_on_error(lib):
    assert layers_call(lib, n_layers=0) == SHAPE
    assert layers_call(lib, dtype=5) == DTYPE
    # a hole in the last layer is reported as such; had layer 0 been launched first (no GPU
    # here), the call would have failed with a HIP error instead
    assert layers_call(lib, hole=("out", 2)) == NULL
    assert layers_call(lib, hole=("k_new", 1)) == NULL
    assert layers_call(lib, max_cache=113) == CAP


def test_commit_validation(lib):
    assert lib.paged_kv_commit(None, None, None, 0, 4, 16, 16, None) == NULL
    assert lib.paged_kv_commit(P, None, None, 0, 0, 16, 16, None) == SHAPE
    assert lib.paged_kv_commit(P, None, None, 0, 4, 0, 16, None) == SHAPE
    assert lib.paged_kv_commit(P, None, P, 64, 4, 16, 0, None) == SHAPE
    assert lib.paged_kv_commit(P, None, P, -1, 4, 16, 16, None) == SHAPE


# --------------------------------------------------------------------------------------------
# The projections either side of the attention
# --------------------------------------------------------------------------------------------

def linear_call(lib, dtype=1, x=P, w=P, bias=None, y=P, M=100, N=64, K=256):
    return lib.pkc_linear(dtype, x, w, bias, y, M, N, K, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), DTYPE), (dict(x=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL),
    (dict(M=0), SHAPE), (dict(N=0), SHAPE), (dict(K=-32), SHAPE),
    (dict(K=48), UNSUP), (dict(N=40), UNSUP),
    (dict(M=1 << 30), SHAPE),
    # 256-thread workgroups over 128 x 128 .. 64 x 64 output tiles: 2^32 work-items are refused
    (dict(M=(1 << 30) - 1, N=1 << 13), UNSUP),
    (dict(x=BAD), ALIGN), (dict(y=BAD), ALIGN), (dict(bias=BAD), ALIGN),
])
def test_linear_validation(lib, kw, status):
    assert linear_call(lib, **kw) == status


def qkv_call(lib, dtype=1, x=P, w=P, b=P, q=P, k_pool=P, v_pool=P, bt=P, cs=P, B=2, C=16, dm=256,
             H=4, Hk=4, D=64, S=16, N=32, M=8, max_cache=64):
    return lib.paged_kv_qkv_append(dtype, x, w, b, q, k_pool, v_pool, bt, cs, None, None, B, C, dm,
                                   H, Hk, D, S, N, M, max_cache, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), DTYPE), (dict(x=None), NULL), (dict(w=None), NULL), (dict(q=None), NULL),
    (dict(k_pool=None), NULL), (dict(bt=None), NULL), (dict(cs=None), NULL),
    (dict(B=0), SHAPE), (dict(H=6, Hk=4), SHAPE), (dict(H=0), SHAPE), (dict(dm=0), SHAPE),
    (dict(dm=100), UNSUP), (dict(D=48), UNSUP),
    (dict(max_cache=113), CAP),
    # (H + 2 Hk) D output features: formed without int32 overflow, then refused by size
    (dict(H=(1 << 31) - 1, Hk=1), SHAPE),
    (dict(H=1 << 30, Hk=1 << 30), SHAPE),
    (dict(x=BAD), ALIGN), (dict(b=BAD), ALIGN), (dict(v_pool=BAD), ALIGN),
])
def test_qkv_append_validation(lib, kw, status):
    assert qkv_call(lib, **kw) == status


def pos_call(lib, dtype=1, w=P, start=None, first=80, step=-1, n_tables=1, rows=161, dm=256,
             n_out=256, out=P):
    return lib.rel_pos_projection(dtype, w, start, first, step, n_tables, rows, dm, n_out, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=9), DTYPE), (dict(w=None), NULL), (dict(out=None), NULL),
    (dict(rows=0), SHAPE), (dict(n_tables=0), SHAPE),
    (dict(first=1 << 25), SHAPE), (dict(first=0, step=1 << 20, rows=100), SHAPE),
    (dict(dm=72), UNSUP), (dict(n_out=100), UNSUP),
    (dict(w=BAD), ALIGN), (dict(out=BAD), ALIGN),
])
def test_rel_pos_projection_validation(lib, kw, status):
    assert pos_call(lib, **kw) == status


# --------------------------------------------------------------------------------------------
# The binding checks every size the kernels index by, before calling into the library
# --------------------------------------------------------------------------------------------

def _chunk_args(B=2, C=16, H=4, Hk=4, D=64, S=16, N=32, M=8, P=159, per_row=False, blocked=False):
    import torch
    z = lambda *s: torch.zeros(*s)
    if blocked:
        pos = z(B, H, D // 32, P, 32) if per_row else z(H, D // 32, P, 32)
    else:
        pos = z(B, P, H, D) if per_row else z(P, H, D)
    return dict(q=z(B, C, H, D), k_new=z(B, C, Hk, D), v_new=z(B, C, Hk, D),
                k_pool=z(N, Hk, D // 32, S, 32), v_pool=z(N, Hk, D, S),
                block_tables=torch.zeros(B, M, dtype=torch.int32),
                cache_seqlens=torch.zeros(B, dtype=torch.int32), pos=pos, pos_bias_u=z(H, D),
                pos_bias_v=z(H, D), out=z(B, C, H, D))


def _fused(a, **kw):
    return pkc.paged_kv_append_relpos_attn(a["q"], a["k_new"], a["v_new"], a["k_pool"],
                                           a["v_pool"], a["block_tables"], a["cache_seqlens"],
                                           a["pos"], a["pos_bias_u"], a["pos_bias_v"], 64,
                                           out=a["out"], **kw)


@pytest.mark.parametrize("bad", [
    dict(out=(2, 16, 4, 32)), dict(out=(1, 16, 4, 64)), dict(pos_bias_u=(4, 32)),
    dict(pos_bias_v=(2, 64)), dict(k_new=(2, 8, 4, 64)), dict(v_new=(2, 16, 2, 64)),
    dict(pos=(159, 2, 64)), dict(pos=(159, 4, 32)), dict(block_tables=(1, 8)),
    dict(cache_seqlens=(1,)), dict(v_pool=(32, 4, 64, 8)),
])
def test_binding_rejects_mis_shaped_tensors(lib, bad):
    """Any size disagreeing with q / the pools raises ValueError in Python (no kernel could be
    launched with it: the C ABI sees only pointers)."""
    import torch
    a = _chunk_args()
    for k, shape in bad.items():
        a[k] = torch.zeros(*shape, dtype=a[k].dtype)
    with pytest.raises(ValueError):
        _fused(a)


def test_binding_checks_lengths_windows_and_table_layouts(lib):
    import torch
    a = _chunk_args()
    with pytest.raises(ValueError, match="chunk_lens"):
        _fused(a, chunk_lens=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="window_start"):
        _fused(a, window_start=torch.zeros(1, dtype=torch.int32))
    # per-row tables need one table per stream, in the layout the flags name
    with pytest.raises(ValueError, match="pos"):
        _fused(_chunk_args(per_row=False), per_row_pos=True)
    pr = _chunk_args(per_row=True)
    pr["pos"] = pr["pos"][:1]
    with pytest.raises(ValueError, match="pos"):
        _fused(pr, per_row_pos=True)
    with pytest.raises(ValueError, match="pos"):
        _fused(_chunk_args(blocked=False), pos_blocked=True)
    with pytest.raises(ValueError, match="pos"):
        _fused(_chunk_args(blocked=True), pos_blocked=False)
    # correctly shaped host tensors pass every shape check and stop at the device check
    for per_row in (False, True):
        for blocked in (False, True):
            with pytest.raises(ValueError, match="GPU"):
                _fused(_chunk_args(per_row=per_row, blocked=blocked), per_row_pos=per_row,
                       pos_blocked=blocked)


def test_binding_checks_varlen_and_commit_shapes(lib):
    import torch
    H, D, total = 2, 64, 40
    q = torch.zeros(total, H, D)
    k = torch.zeros(total, H, D)
    cu = torch.tensor([0, 15, 40], dtype=torch.int32)
    u = torch.zeros(H, D)
    good_pos = torch.zeros(2 * total, H, D)
    with pytest.raises(ValueError, match="pos"):
        pkc.varlen_packed_relpos_attn(q, k, k, cu, torch.zeros(2 * total - 1, H, D), u, u, 25)
    with pytest.raises(ValueError, match="k must"):
        pkc.varlen_packed_relpos_attn(q, k[:-1], k, cu, good_pos, u, u, 25)
    with pytest.raises(ValueError, match="v must"):
        pkc.varlen_packed_relpos_attn(q, k, k[:, :1], cu, good_pos, u, u, 25)
    with pytest.raises(ValueError, match="out"):
        pkc.varlen_packed_relpos_attn(q, k, k, cu, good_pos, u, u, 25, out=q[:-1])
    with pytest.raises(ValueError, match="GPU"):
        pkc.varlen_packed_relpos_attn(q, k, k, cu, good_pos, u, u, 25)
    cs = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="max_cached_frames"):
        pkc.paged_kv_commit(cs, 16, window_start=torch.zeros(4, dtype=torch.int32), block_size=8)
    with pytest.raises(ValueError, match="chunk_lens"):
        pkc.paged_kv_commit(cs, 16, chunk_lens=torch.zeros(3, dtype=torch.int32))
