"""Python binding of libpkc.so (paged chunk attention with a Transformer-XL relative-position term).

Argument marshalling only: every function here turns torch tensors into device pointers and
sizes, calls the C ABI declared in include/pkc.h on torch's current HIP stream, and raises
PkcError on a non-zero status. All computation happens in the HIP kernels. There is no CPU
fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkc.so")

PKC_F32, PKC_BF16 = 0, 1
_DTYPES = {torch.float32: PKC_F32, torch.bfloat16: PKC_BF16}

_i32 = ctypes.c_int32
_ptr = ctypes.c_void_p
_f32 = ctypes.c_float

# Exported entry points and their argument types (mirrors include/pkc.h).
SIGNATURES = {
    "pkc_version": ([], ctypes.c_int),
    "pkc_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "paged_kv_append": ([ctypes.c_int] + [_ptr] * 8 + [_i32] * 8 + [_ptr], ctypes.c_int),
    "chunk_paged_relpos_attn": ([ctypes.c_int] + [_ptr] * 8 + [_i32, _i32] + [_ptr] * 3
                                + [_i32] * 9 + [_f32, _ptr], ctypes.c_int),
    "paged_kv_append_relpos_attn": ([ctypes.c_int] + [_ptr] * 10 + [_i32, _i32] + [_ptr] * 3
                                    + [_i32] * 9 + [_f32, _ptr], ctypes.c_int),
    "paged_kv_append_relpos_attn_layers": ([ctypes.c_int, _i32] + [_ptr] * 10 + [_i32, _i32]
                                           + [_ptr] * 3 + [_i32] * 9 + [_f32, _ptr], ctypes.c_int),
    "paged_kv_commit": ([_ptr, _ptr, _ptr, _i32, _i32, _i32, _i32, _ptr], ctypes.c_int),
    "varlen_packed_relpos_attn": ([ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _i32, _i32, _i32, _ptr,
                                   _ptr, _ptr, _ptr] + [_i32] * 5 + [_f32, _ptr], ctypes.c_int),
    "pkc_linear": ([ctypes.c_int] + [_ptr] * 4 + [_i32] * 3 + [_ptr], ctypes.c_int),
    "paged_kv_qkv_append": ([ctypes.c_int] + [_ptr] * 10 + [_i32] * 10 + [_ptr], ctypes.c_int),
    "rel_pos_projection": ([ctypes.c_int, _ptr, _ptr] + [_i32] * 6 + [_ptr, _ptr], ctypes.c_int),
    "pkc_gather_read": ([ctypes.c_int] + [_ptr] * 8 + [_i32, _i32] + [_ptr] * 3 + [_i32] * 12
                        + [_ptr], ctypes.c_int),
}


class PkcError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: status {status} ({status_string(status)})")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m paged_kv_chunk_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def version():
    return lib().pkc_version()


def status_string(status):
    return lib().pkc_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise PkcError(status, what)


def _dtype(*ts):
    dt = ts[0].dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for t in ts:
        if t.dtype != dt:
            raise TypeError("all floating-point tensors of a call must share one dtype")
    return _DTYPES[dt]


def _p(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    return t.data_ptr()


def _table(t):
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise TypeError("block tables, cache lengths, chunk lengths and offsets are int32")
    return _p(t)


def _shape(t, shape, name):
    """t must have exactly ``shape`` (the sizes the kernels index it by)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _rows(t, n, name, dims=1):
    """A per-stream (or per-utterance) int32 array: ``dims`` dimensions, at least n rows."""
    if t is None:
        return
    if t.dim() != dims or t.shape[0] < n:
        raise ValueError(f"{name} must have {dims} dimension(s) and at least {n} rows, "
                         f"got {list(t.shape)}")


def _layout(per_row, per_key, blocked=False):
    """pos_layout flags: 1 = one table per stream, 2 = rows are keys (WeNet, no shift),
    4 = stored in 32-dim column blocks per head."""
    return (1 if per_row else 0) | (2 if per_key else 0) | (4 if blocked else 0)


def _pos_geom(pos, B, H, D, per_row, blocked):
    """Rows per table of a positional table tensor, after checking its shape: row-major
    [P, H, D] (shared) or [B', P, H, D] (per row, B' >= B); column-blocked [H, D / 32, P, 32] or
    [B', H, D / 32, P, 32]."""
    if blocked:
        want = 5 if per_row else 4
        tail = (H, D // 32)
        ok = (pos.dim() == want and tuple(pos.shape[want - 4:want - 2]) == tail
              and pos.shape[-1] == 32 and D % 32 == 0)
        rows = pos.shape[-2] if pos.dim() == want else 0
        layout = "[B, H, D / 32, P, 32]" if per_row else "[H, D / 32, P, 32]"
    else:
        want = 4 if per_row else 3
        ok = pos.dim() == want and tuple(pos.shape[-2:]) == (H, D)
        rows = pos.shape[-3] if pos.dim() == want else 0
        layout = "[B, P, H, D]" if per_row else "[P, H, D]"
    if not ok or (per_row and pos.shape[0] < B):
        raise ValueError(f"pos must be {layout} (H={H}, D={D}, at least B={B} tables when per "
                         f"row), got {list(pos.shape)}")
    return rows


def _chunk_common(q, k_pool, v_pool, block_tables, cache_seqlens, pos, pos_bias_u, pos_bias_v,
                  out, chunk_lens, window_start, per_row_pos, pos_blocked):
    """Shape checks shared by the chunk attention entries; returns (B, C, H, D, N, Hk, S, P)."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, C, H, D], got {list(q.shape)}")
    B, C, H, D = q.shape
    N, Hk, S = _pool_geom(k_pool, v_pool, D)
    _shape(out, q.shape, "out")
    _shape(pos_bias_u, (H, D), "pos_bias_u")
    _shape(pos_bias_v, (H, D), "pos_bias_v")
    _rows(block_tables, B, "block_tables", dims=2)
    _rows(cache_seqlens, B, "cache_seqlens")
    _rows(chunk_lens, B, "chunk_lens")
    _rows(window_start, B, "window_start")
    P = _pos_geom(pos, B, H, D, per_row_pos, pos_blocked)
    return B, C, H, D, N, Hk, S, P


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def paged_kv_append(k_new, v_new, k_pool, v_pool, block_tables, cache_seqlens, max_cache_seqlen,
                    chunk_lens=None, window_start=None, stream=None):
    """Write k_new / v_new [B, C, Hk, D] into k_pool [N, Hk, D / 32, S, 32] / v_pool [N, Hk, D, S]
    (only the first chunk_lens[b] frames of stream b when chunk_lens is given; window_start
    int32 [B] addresses the table rows as rings)."""
    if k_new.dim() != 4:
        raise ValueError(f"k_new must be [B, C, Hk, D], got {list(k_new.shape)}")
    B, C, Hk, D = k_new.shape
    _shape(v_new, k_new.shape, "v_new")
    N, Hk_pool, S = _pool_geom(k_pool, v_pool, D)
    if Hk_pool != Hk:
        raise ValueError(f"k_new has {Hk} kv heads, the pools {Hk_pool}")
    _rows(block_tables, B, "block_tables", dims=2)
    _rows(cache_seqlens, B, "cache_seqlens")
    _rows(chunk_lens, B, "chunk_lens")
    _rows(window_start, B, "window_start")
    st = lib().paged_kv_append(_dtype(k_new, v_new, k_pool, v_pool), _p(k_new), _p(v_new),
                               _p(k_pool), _p(v_pool), _table(block_tables), _table(cache_seqlens),
                               _table(chunk_lens), _table(window_start), B, C, Hk, D, S, N,
                               block_tables.shape[1], int(max_cache_seqlen), _stream(stream))
    _check(st, "paged_kv_append")


def _pool_geom(k_pool, v_pool, head_dim):
    """(N, Hk, S) of a K pool [N, Hk, D / 32, S, 32] and V pool [N, Hk, D, S]."""
    if k_pool.dim() != 5 or k_pool.shape[2] * k_pool.shape[4] != head_dim or k_pool.shape[4] != 32:
        raise ValueError("k_pool must be [num_blocks, n_kv_head, head_dim / 32, block_size, 32]")
    N, Hk, _, S, _ = k_pool.shape
    if tuple(v_pool.shape) != (N, Hk, head_dim, S):
        raise ValueError("v_pool must be [num_blocks, n_kv_head, head_dim, block_size]")
    return N, Hk, S


def chunk_paged_relpos_attn(q, k_pool, v_pool, block_tables, cache_seqlens, pos, pos_bias_u,
                            pos_bias_v, max_cache_seqlen, per_row_pos=False, per_key_pos=False,
                            out=None, softmax_scale=0.0, chunk_lens=None, window_start=None,
                            pos_blocked=False, stream=None):
    """Chunk attention; q [B, C, H, D]; pos shared [P, H, D] or per-row [B, P, H, D], rows by
    distance (Transformer-XL) or, with per_key_pos, by key (WeNet); with pos_blocked the same
    tables in 32-dim column blocks ([H, D / 32, P, 32] or [B, H, D / 32, P, 32]); chunk_lens
    int32 [B] (optional): real frames per stream; window_start int32 [B] (optional): bounded
    history."""
    if out is None:
        out = torch.empty_like(q)
    B, C, H, D, N, Hk, S, P = _chunk_common(q, k_pool, v_pool, block_tables, cache_seqlens, pos,
                                            pos_bias_u, pos_bias_v, out, chunk_lens, window_start,
                                            per_row_pos, pos_blocked)
    st = lib().chunk_paged_relpos_attn(
        _dtype(q, k_pool, v_pool, pos, pos_bias_u, pos_bias_v, out), _p(q), _p(k_pool), _p(v_pool),
        _table(block_tables), _table(cache_seqlens), _table(chunk_lens), _table(window_start),
        _p(pos), P, _layout(per_row_pos, per_key_pos, pos_blocked), _p(pos_bias_u),
        _p(pos_bias_v), _p(out), B, C, H, Hk, D, S, N, block_tables.shape[1],
        int(max_cache_seqlen), float(softmax_scale), _stream(stream))
    _check(st, "chunk_paged_relpos_attn")
    return out


def _new_kv(k_new, v_new, B, C, Hk, D):
    _shape(k_new, (B, C, Hk, D), "k_new")
    _shape(v_new, (B, C, Hk, D), "v_new")


def paged_kv_append_relpos_attn(q, k_new, v_new, k_pool, v_pool, block_tables, cache_seqlens, pos,
                                pos_bias_u, pos_bias_v, max_cache_seqlen, per_row_pos=False,
                                per_key_pos=False, out=None, softmax_scale=0.0, chunk_lens=None,
                                window_start=None, pos_blocked=False, stream=None):
    """Append and attention of one layer in one launch (pools are written); arguments as
    chunk_paged_relpos_attn plus k_new / v_new [B, C, Hk, D]."""
    if out is None:
        out = torch.empty_like(q)
    B, C, H, D, N, Hk, S, P = _chunk_common(q, k_pool, v_pool, block_tables, cache_seqlens, pos,
                                            pos_bias_u, pos_bias_v, out, chunk_lens, window_start,
                                            per_row_pos, pos_blocked)
    _new_kv(k_new, v_new, B, C, Hk, D)
    st = lib().paged_kv_append_relpos_attn(
        _dtype(q, k_new, v_new, k_pool, v_pool, pos, pos_bias_u, pos_bias_v, out), _p(q),
        _p(k_new), _p(v_new), _p(k_pool), _p(v_pool), _table(block_tables), _table(cache_seqlens),
        _table(chunk_lens), _table(window_start), _p(pos), P,
        _layout(per_row_pos, per_key_pos, pos_blocked), _p(pos_bias_u), _p(pos_bias_v), _p(out),
        B, C, H, Hk, D, S, N, block_tables.shape[1], int(max_cache_seqlen), float(softmax_scale),
        _stream(stream))
    _check(st, "paged_kv_append_relpos_attn")
    return out


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _p(t)
    return arr


def paged_kv_append_relpos_attn_layers(layers, block_tables, cache_seqlens, max_cache_seqlen,
                                       per_row_pos=False, per_key_pos=False, chunk_lens=None,
                                       window_start=None, softmax_scale=0.0, pos_blocked=False,
                                       stream=None):
    """Fused append + attention of several layers in one call. ``layers``: a sequence of objects
    with attributes q, k_new, v_new, k_pool, v_pool, pos, pos_bias_u, pos_bias_v, out (one per
    layer, same shapes); block tables, cache and chunk lengths and window starts are shared."""
    if len(layers) == 0:
        raise ValueError("no layers")
    l0 = layers[0]
    B, C, H, D, N, Hk, S, P = _chunk_common(l0.q, l0.k_pool, l0.v_pool, block_tables,
                                            cache_seqlens, l0.pos, l0.pos_bias_u, l0.pos_bias_v,
                                            l0.out, chunk_lens, window_start, per_row_pos,
                                            pos_blocked)
    _new_kv(l0.k_new, l0.v_new, B, C, Hk, D)
    names = ["q", "k_new", "v_new", "k_pool", "v_pool", "pos", "pos_bias_u", "pos_bias_v", "out"]
    for x in layers:
        for n in names:
            if getattr(l0, n).shape != getattr(x, n).shape:
                raise ValueError(f"layer buffers of {n} differ in shape")
    dt = _dtype(*[getattr(x, n) for x in layers for n in names])
    arrs = {n: _ptr_array([getattr(x, n) for x in layers]) for n in names}
    st = lib().paged_kv_append_relpos_attn_layers(
        dt, len(layers), arrs["q"], arrs["k_new"], arrs["v_new"], arrs["k_pool"], arrs["v_pool"],
        _table(block_tables), _table(cache_seqlens), _table(chunk_lens), _table(window_start),
        arrs["pos"], P, _layout(per_row_pos, per_key_pos, pos_blocked),
        arrs["pos_bias_u"], arrs["pos_bias_v"], arrs["out"], B, C, H, Hk, D, S, N,
        block_tables.shape[1], int(max_cache_seqlen), float(softmax_scale), _stream(stream))
    _check(st, "paged_kv_append_relpos_attn_layers")


def paged_kv_commit(cache_seqlens, chunk, chunk_lens=None, window_start=None,
                    max_cached_frames=None, block_size=0, stream=None):
    """cache_seqlens[b] += chunk_lens[b] (or chunk) on the device; with window_start, whole
    oldest blocks are then dropped while a cache exceeds max_cached_frames (required then, and
    at least one block)."""
    if cache_seqlens.dim() != 1:
        raise ValueError(f"cache_seqlens must be [B], got {list(cache_seqlens.shape)}")
    B = cache_seqlens.shape[0]
    _rows(chunk_lens, B, "chunk_lens")
    _rows(window_start, B, "window_start")
    if window_start is not None and max_cached_frames is None:
        raise ValueError("paged_kv_commit: max_cached_frames is required with window_start")
    st = lib().paged_kv_commit(_table(cache_seqlens), _table(chunk_lens), _table(window_start),
                               int(max_cached_frames or 0), B, int(chunk), int(block_size),
                               _stream(stream))
    _check(st, "paged_kv_commit")


def varlen_packed_relpos_attn(q, k, v, cu_seqlens, pos, pos_bias_u, pos_bias_v, max_seqlen,
                              out=None, softmax_scale=0.0, mask_chunk=0, mask_left_chunks=0,
                              stream=None):
    """Attention inside each packed utterance; q [total, H, D], k/v [total, Hk, D]; pos
    [2 total, H, D] (utterance s's table at row 2 cu_seqlens[s]); mask_chunk > 0 applies the
    chunked_limited mask (own chunk plus mask_left_chunks earlier ones)."""
    if q.dim() != 3:
        raise ValueError(f"q must be [total, H, D], got {list(q.shape)}")
    total, H, D = q.shape
    if k.dim() != 3 or k.shape[0] != total or k.shape[2] != D:
        raise ValueError(f"k must be [total={total}, Hk, D={D}], got {list(k.shape)}")
    Hk = k.shape[1]
    _shape(v, k.shape, "v")
    if out is None:
        out = torch.empty_like(q)
    _shape(out, q.shape, "out")
    _shape(pos_bias_u, (H, D), "pos_bias_u")
    _shape(pos_bias_v, (H, D), "pos_bias_v")
    if pos.dim() != 3 or pos.shape[0] < 2 * total or tuple(pos.shape[1:]) != (H, D):
        raise ValueError(f"pos must be [>= 2 total = {2 * total}, H, D], got {list(pos.shape)}")
    _rows(cu_seqlens, 2, "cu_seqlens")
    st = lib().varlen_packed_relpos_attn(
        _dtype(q, k, v, pos, pos_bias_u, pos_bias_v, out), _p(q), _p(k), _p(v), _table(cu_seqlens),
        cu_seqlens.shape[0] - 1, total, int(max_seqlen), _p(pos), _p(pos_bias_u), _p(pos_bias_v),
        _p(out), H, Hk, D, int(mask_chunk), int(mask_left_chunks), float(softmax_scale),
        _stream(stream))
    _check(st, "varlen_packed_relpos_attn")
    return out


def linear(x, w, bias=None, out=None, stream=None):
    """y = x w^T + bias: x [..., K], w [N, K], bias [N] or None -> y [..., N] (new tensor unless
    ``out`` is given)."""
    K = x.shape[-1]
    M = x.numel() // K
    N = w.shape[0]
    if w.dim() != 2 or w.shape[1] != K or (bias is not None and tuple(bias.shape) != (N,)):
        raise ValueError("linear: w must be [N, K] and bias [N]")
    y = torch.empty(*x.shape[:-1], N, dtype=x.dtype, device=x.device) if out is None else out
    if y.numel() != M * N or y.shape[-1] != N:
        raise ValueError(f"linear: out must hold [{M}, {N}], got {list(y.shape)}")
    dt = _dtype(x, w, y, *([bias] if bias is not None else []))
    st = lib().pkc_linear(dt, _p(x), _p(w), _p(bias), _p(y), M, N, K, _stream(stream))
    _check(st, "pkc_linear")
    return y


def paged_kv_qkv_append(x, w_qkv, b_qkv, k_pool, v_pool, block_tables, cache_seqlens,
                        max_cache_seqlen, n_head, q_out=None, chunk_lens=None, window_start=None,
                        stream=None):
    """The chunk's Q/K/V projection with the append as its epilogue. x [B, C, d_model],
    w_qkv [(H + 2 Hk) D, d_model] (rows of linear_q, linear_k, linear_v), b_qkv or None.
    Returns q [B, C, H, D]; the chunk's K/V rows are written into the pools."""
    if x.dim() != 3:
        raise ValueError(f"x must be [B, C, d_model], got {list(x.shape)}")
    B, C, dm = x.shape
    if k_pool.dim() != 5:
        raise ValueError("k_pool must be [num_blocks, n_kv_head, head_dim / 32, block_size, 32]")
    N, Hk, S = k_pool.shape[0], k_pool.shape[1], k_pool.shape[3]
    D = w_qkv.shape[0] // (n_head + 2 * Hk)
    _pool_geom(k_pool, v_pool, D)
    _shape(w_qkv, (D * (n_head + 2 * Hk), dm), "w_qkv")
    if b_qkv is not None:
        _shape(b_qkv, (D * (n_head + 2 * Hk),), "b_qkv")
    _rows(block_tables, B, "block_tables", dims=2)
    _rows(cache_seqlens, B, "cache_seqlens")
    _rows(chunk_lens, B, "chunk_lens")
    _rows(window_start, B, "window_start")
    q = torch.empty(B, C, n_head, D, dtype=x.dtype, device=x.device) if q_out is None else q_out
    _shape(q, (B, C, n_head, D), "q_out")
    tensors = [x, w_qkv, q, k_pool, v_pool] + ([b_qkv] if b_qkv is not None else [])
    st = lib().paged_kv_qkv_append(_dtype(*tensors), _p(x), _p(w_qkv), _p(b_qkv), _p(q),
                                   _p(k_pool), _p(v_pool), _table(block_tables),
                                   _table(cache_seqlens), _table(chunk_lens), _table(window_start),
                                   B, C, dm, n_head, Hk, D, S, N, block_tables.shape[1],
                                   int(max_cache_seqlen), _stream(stream))
    _check(st, "paged_kv_qkv_append")
    return q


def rel_pos_projection(w_pos, rows, pos_start=None, pos_first=0, pos_step=-1, n_tables=None,
                       out=None, stream=None):
    """linear_pos over sinusoidal tables: [n_tables, rows, out_features]. Row r of table t holds
    position pos_start[t] + pos_step r (pos_start int32 [n_tables] on the GPU), or
    pos_first + pos_step r for every table when pos_start is None."""
    if w_pos.dim() != 2:
        raise ValueError(f"w_pos must be [out_features, d_model], got {list(w_pos.shape)}")
    n_out, dm = w_pos.shape
    if n_tables is None:
        n_tables = 1 if pos_start is None else pos_start.shape[0]
    _rows(pos_start, n_tables, "pos_start")
    y = torch.empty(n_tables, rows, n_out, dtype=w_pos.dtype, device=w_pos.device) if out is None else out
    _shape(y, (n_tables, rows, n_out), "out")
    st = lib().rel_pos_projection(_dtype(w_pos, y), _p(w_pos), _table(pos_start), int(pos_first),
                                  int(pos_step), int(n_tables), int(rows), dm, n_out, _p(y),
                                  _stream(stream))
    _check(st, "rel_pos_projection")
    return y


def gather_read(q, k_new, v_new, k_pool, v_pool, block_tables, cache_seqlens, pos, pos_bias_u,
                pos_bias_v, max_cache_seqlen, out, per_row_pos=False, pos_blocked=False, waves=4,
                split=1, reads=True, stream=None):
    """Measurement only: one launch that moves the bytes of paged_kv_append_relpos_attn with no
    arithmetic (the pools get the chunk's K/V; ``out`` gets unspecified values). reads=False:
    the same grid only writes ``out`` (the launch floor)."""
    B, C, H, D, N, Hk, S, P = _chunk_common(q, k_pool, v_pool, block_tables, cache_seqlens, pos,
                                            pos_bias_u, pos_bias_v, out, None, None, per_row_pos,
                                            pos_blocked)
    _new_kv(k_new, v_new, B, C, Hk, D)
    st = lib().pkc_gather_read(
        _dtype(q, k_new, v_new, k_pool, v_pool, pos, pos_bias_u, pos_bias_v, out), _p(q),
        _p(k_new), _p(v_new), _p(k_pool), _p(v_pool), _table(block_tables), _table(cache_seqlens),
        _p(pos), P, _layout(per_row_pos, False, pos_blocked), _p(pos_bias_u),
        _p(pos_bias_v), _p(out), B, C, H, Hk, D, S, N, block_tables.shape[1],
        int(max_cache_seqlen), int(waves), int(split), int(bool(reads)), _stream(stream))
    _check(st, "pkc_gather_read")
