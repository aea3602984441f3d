"""ctypes binding of libkvarn.so (the C ABI in include/kvarn.h).

Argument marshalling only: every step of the quantize and decode paths runs in the HIP
kernels of the library. PyTorch supplies device memory and the current stream. Importing
this module fails loudly if the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

# KVARN_LIBRARY names another build of the same library (the host-ASan build of the ABI tests)
_LIB_PATH = os.environ.get("KVARN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libkvarn.so")

KIND_K = 0
KIND_V = 1
K_PAGE_BYTES = 9216
V_PAGE_BYTES = 5120

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace too small", 4: "HIP launch failed"}


class KvarnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


FORMAT_SEPARATE = 1     # page records with r, s, scale, zero stored apart
FORMAT_FOLDED = 2       # each group's normalizer folded into its scale and zero


class Params(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("sinkhorn_iters", ctypes.c_int32),
                ("format", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m kv_cache_quantization_tile_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Params)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "kvarn_abi_version": (i32, []),
        "kvarn_format_version": (i32, []),
        "kvarn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "kvarn_params_from_dtype": (ctypes.c_int, [ctypes.c_char_p, i32, P]),
        "kvarn_params_check": (ctypes.c_int, [P]),
        "kvarn_page_bytes": (sz, [P, ctypes.c_int]),
        "kvarn_quantize_tiles": (ctypes.c_int, [P, ctypes.c_int, vp, i64, i64, i64, vp, vp, i32,
                                                i32, vp, i64, vp]),
        "kvarn_quantize_kv_tiles": (ctypes.c_int, [P, vp, vp, i64, i64, i64, vp, vp, i32, i32,
                                                   vp, vp, i64, vp]),
        "kvarn_append_tokens": (ctypes.c_int, [P, vp, vp, i32, i32, vp, vp, vp, vp, i32, vp, vp,
                                               i64, vp]),
        "kvarn_write_tokens": (ctypes.c_int, [P, vp, vp, i32, vp, i32, i32, i32, vp, vp, vp, vp,
                                              i32, vp, vp, i64, vp]),
        "kvarn_dequantize_tiles": (ctypes.c_int, [P, ctypes.c_int, vp, i64, vp, i32, i32, vp, vp]),
        "kvarn_decode_workspace_bytes": (sz, [P, i32, i32, i32, i32]),
        "kvarn_decode_num_splits": (i32, [P, i32, i32, i32]),
        "kvarn_chunk_workspace_bytes": (sz, [P, i32, i32, i32, i32]),
        "kvarn_decode_attention": (ctypes.c_int, [P, vp, i32, i32, i32, vp, vp, i64, vp, i32, vp,
                                                  i32, vp, vp, ctypes.c_float, vp, sz, vp, vp]),
        "kvarn_decode_noalloc_max_workspace_bytes": (sz, []),
        "kvarn_decode_attention_noalloc": (ctypes.c_int, [P, vp, i32, i32, i32, vp, vp, i64, vp,
                                                          i32, vp, i32, vp, vp, ctypes.c_float,
                                                          vp, vp]),
        "kvarn_chunk_attention": (ctypes.c_int, [P, vp, i32, vp, i32, i32, i32, vp, vp, i64, vp,
                                                 i32, vp, i32, vp, vp, ctypes.c_float, vp, sz,
                                                 vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = ("kvarn_abi_version", "kvarn_format_version", "kvarn_status_str",
            "kvarn_params_from_dtype", "kvarn_params_check", "kvarn_page_bytes",
            "kvarn_quantize_tiles", "kvarn_quantize_kv_tiles", "kvarn_append_tokens",
            "kvarn_write_tokens", "kvarn_dequantize_tiles", "kvarn_decode_workspace_bytes",
            "kvarn_decode_num_splits", "kvarn_decode_attention", "kvarn_chunk_attention",
            "kvarn_chunk_workspace_bytes", "kvarn_decode_noalloc_max_workspace_bytes",
            "kvarn_decode_attention_noalloc")


def _check(status: int, what: str):
    if status != 0:
        raise KvarnError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, device=True):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


# ----------------------------------------------------------------------------- params


def params_from_dtype(kv_cache_dtype: str = "kvarn_k4v2_g128", sinkhorn_iters: int = 8,
                      format: int = FORMAT_SEPARATE) -> Params:
    """Params of a preset string; `format` selects the page record layout."""
    p = Params()
    _check(lib.kvarn_params_from_dtype(kv_cache_dtype.encode(), sinkhorn_iters, ctypes.byref(p)),
           f"kv_cache_dtype {kv_cache_dtype!r}")
    p.format = format
    _check(lib.kvarn_params_check(ctypes.byref(p)), f"format {format}")
    return p


def page_bytes(params: Params, kind: int) -> int:
    return int(lib.kvarn_page_bytes(ctypes.byref(params), kind))


def new_pool(num_pages: int, num_kv_heads: int, kind: int, device="cuda",
             params: Params | None = None) -> torch.Tensor:
    """A zeroed page pool [num_pages, num_kv_heads, record bytes] of uint8 (record size of
    the preset in params; kvarn_k4v2_g128 when omitted)."""
    if params is None:
        nb = K_PAGE_BYTES if kind == KIND_K else V_PAGE_BYTES
    else:
        nb = page_bytes(params, kind)
    return torch.zeros((num_pages, num_kv_heads, nb), dtype=torch.uint8, device=device)


def _pool_n(params: Params, pool, kind: int) -> int:
    _pool_ok(params, pool, kind, "pool")
    return pool.shape[0]


def _pools_n(params: Params, k_pool, v_pool) -> int:
    """Checks a key / value pool pair against the preset; returns their page count."""
    _pool_ok(params, k_pool, KIND_K, "k_pool")
    _pool_ok(params, v_pool, KIND_V, "v_pool")
    if k_pool.shape[0] != v_pool.shape[0]:
        raise ValueError("k_pool and v_pool must have the same number of pages")
    if k_pool.shape[1] != v_pool.shape[1]:
        raise ValueError("k_pool and v_pool must have the same number of KV heads")
    return k_pool.shape[0]


def _pool_ok(params: Params, pool, kind: int, name: str):
    """The kernels address records by the preset's record size: the pool must match it."""
    if pool is None:
        return
    if pool.dim() != 3 or pool.dtype != torch.uint8 or pool.shape[2] != page_bytes(params, kind):
        raise ValueError(f"{name} must be uint8 [pages, Hkv, {page_bytes(params, kind)}] for "
                         f"this preset")


def _staging_ok(k_tail, v_tail, B: int, hkv: int):
    """Staging tiles: both or neither, float16 contiguous [B, Hkv, 128, 128] on the GPU."""
    if (k_tail is None) != (v_tail is None):
        raise ValueError("pass both k_tail and v_tail, or neither")
    if k_tail is None:
        return
    for t, nm in ((k_tail, "k_tail"), (v_tail, "v_tail")):
        _need(t, nm, torch.float16)
        if tuple(t.shape) != (B, hkv, 128, 128) or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous [{B}, {hkv}, 128, 128]")


def _decode_shapes(q, k_pool, v_pool, block_table, seq_lens, k_tail, v_tail, rows=None):
    """Shape checks shared by the read calls; returns (rows, Hq, Hkv). The kernels read
    seq_lens[batch], block_table[batch, width], the pools' records and the staging tiles
    at these shapes, so every one is checked here (batch = block_table rows)."""
    _need(q, "q", torch.float16)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(block_table, "block_table", torch.int32)
    if q.dim() != 3 or q.shape[2] != 128 or not q.is_contiguous():
        raise ValueError("q must be contiguous [rows, Hq, 128]")
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _need(t, nm, torch.uint8)
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous [pages, Hkv, record] pool")
    if k_pool.shape[1] != v_pool.shape[1]:
        raise ValueError("k_pool and v_pool must have the same number of KV heads")
    B = block_table.shape[0] if block_table.dim() == 2 else -1
    if block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous [batch, width]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError(f"seq_lens must be [{B}] (one length per block-table row)")
    if rows is None and q.shape[0] != B:
        raise ValueError(f"q must hold one row per sequence ({B})")
    hkv = k_pool.shape[1]
    _staging_ok(k_tail, v_tail, B, hkv)
    return q.shape[0], q.shape[1], hkv


# ----------------------------------------------------------------------------- quantize


def quantize_tiles(params: Params, kind: int, src: torch.Tensor, tile_src_token: torch.Tensor,
                   tile_dst_page: torch.Tensor, pool: torch.Tensor, stream=None) -> torch.Tensor:
    """Quantize tiles of src ([tokens, Hkv, 128] float16, channel stride 1) into pool."""
    _need(src, "src", torch.float16)
    _need(tile_src_token, "tile_src_token", torch.int64)
    _need(tile_dst_page, "tile_dst_page", torch.int32)
    _need(pool, "pool", torch.uint8)
    if src.dim() != 3 or src.shape[2] != 128 or src.stride(2) != 1:
        raise ValueError("src must be [tokens, Hkv, 128] with unit channel stride")
    hkv = src.shape[1]
    nb = page_bytes(params, kind)
    if pool.dim() != 3 or pool.shape[1] != hkv or pool.shape[2] != nb or not pool.is_contiguous():
        raise ValueError(f"pool must be contiguous [pages, {hkv}, {nb}]")
    n = tile_src_token.numel()
    if tile_dst_page.numel() != n:
        raise ValueError("tile_src_token and tile_dst_page differ in length")
    _check(lib.kvarn_quantize_tiles(ctypes.byref(params), kind, _ptr(src), src.stride(0),
                                    src.stride(1), src.shape[0], _ptr(tile_src_token),
                                    _ptr(tile_dst_page), n, hkv, _ptr(pool), _pool_n(params, pool, kind),
                                    _stream(stream)), "kvarn_quantize_tiles")
    return pool


def _kv_quant_args(params, k_src, v_src, tile_src_token, tile_dst_page, k_pool, v_pool, stream):
    for t, nm in ((k_src, "k_src"), (v_src, "v_src")):
        _need(t, nm, torch.float16)
        if t.dim() != 3 or t.shape[2] != 128 or t.stride(2) != 1:
            raise ValueError(f"{nm} must be [tokens, Hkv, 128] with unit channel stride")
    if k_src.shape != v_src.shape or k_src.stride() != v_src.stride():
        raise ValueError("k_src and v_src must have the same shape and strides")
    _need(tile_src_token, "tile_src_token", torch.int64)
    _need(tile_dst_page, "tile_dst_page", torch.int32)
    hkv = k_src.shape[1]
    for t, nm, kind in ((k_pool, "k_pool", KIND_K), (v_pool, "v_pool", KIND_V)):
        _need(t, nm, torch.uint8)
        nb = page_bytes(params, kind)
        if t.dim() != 3 or t.shape[1] != hkv or t.shape[2] != nb or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous [pages, {hkv}, {nb}]")
    _pools_n(params, k_pool, v_pool)
    n = tile_src_token.numel()
    if tile_dst_page.numel() != n:
        raise ValueError("tile_src_token and tile_dst_page differ in length")
    return (ctypes.byref(params), _ptr(k_src), _ptr(v_src), k_src.stride(0), k_src.stride(1),
            k_src.shape[0], _ptr(tile_src_token), _ptr(tile_dst_page), n, hkv, _ptr(k_pool),
            _ptr(v_pool), k_pool.shape[0], _stream(stream))


def quantize_kv_tiles(params: Params, k_src, v_src, tile_src_token, tile_dst_page, k_pool,
                      v_pool, stream=None):
    """Quantize the same tiles of keys and values ([tokens, Hkv, 128] float16) in one launch."""
    _check(lib.kvarn_quantize_kv_tiles(*_kv_quant_args(params, k_src, v_src, tile_src_token,
                                                       tile_dst_page, k_pool, v_pool, stream)),
           "kvarn_quantize_kv_tiles")
    return k_pool, v_pool


def dequantize_tiles(params: Params, kind: int, pool, pages, out=None, stream=None):
    """Records (pages[i], h) of pool back to float16 tiles [n, Hkv, 128 tokens, 128 channels]
    (test and inspection only)."""
    _need(pool, "pool", torch.uint8)
    _need(pages, "pages", torch.int32)
    hkv = pool.shape[1]
    n = pages.numel()
    if pool.dim() != 3 or pool.shape[2] != page_bytes(params, kind) or not pool.is_contiguous():
        raise ValueError("pool must be a contiguous page pool of this kind")
    if out is None:
        out = torch.empty((n, hkv, 128, 128), dtype=torch.float16, device=pool.device)
    _need(out, "out", torch.float16)
    if tuple(out.shape) != (n, hkv, 128, 128) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous [{n}, {hkv}, 128, 128]")
    _check(lib.kvarn_dequantize_tiles(ctypes.byref(params), kind, _ptr(pool), _pool_n(params, pool, kind),
                                      _ptr(pages), n, hkv, _ptr(out), _stream(stream)),
           "kvarn_dequantize_tiles")
    return out


def append_tokens(params: Params, k_new, v_new, seq_lens, k_tail, v_tail, block_table,
                  k_pool, v_pool, stream=None):
    """Write one token per sequence into staging; quantize staging tiles that fill."""
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_tail, "k_tail"), (v_tail, "v_tail")):
        _need(t, nm, torch.float16)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    _need(seq_lens, "seq_lens", torch.int32)
    _need(block_table, "block_table", torch.int32)
    B, hkv = k_new.shape[0], k_new.shape[1]
    if k_new.dim() != 3 or k_new.shape[2] != 128 or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new / v_new must be [B, Hkv, 128]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError(f"seq_lens must be [{B}]")
    if tuple(k_tail.shape) != (B, hkv, 128, 128) or tuple(v_tail.shape) != (B, hkv, 128, 128):
        raise ValueError("staging must be [B, Hkv, 128, 128]")
    if k_pool.shape[1] != hkv:
        raise ValueError(f"pools must have {hkv} KV heads")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous [B, width]")
    _check(lib.kvarn_append_tokens(ctypes.byref(params), _ptr(k_new), _ptr(v_new), B, hkv,
                                   _ptr(seq_lens), _ptr(k_tail), _ptr(v_tail), _ptr(block_table),
                                   block_table.shape[1], _ptr(k_pool), _ptr(v_pool),
                                   _pools_n(params, k_pool, v_pool),
                                   _stream(stream)), "kvarn_append_tokens")


def write_tokens(params: Params, k_new, v_new, cu_new, seq_lens, k_tail, v_tail, block_table,
                 k_pool, v_pool, max_new_tokens: int | None = None, stream=None):
    """Write a chunk of tokens per sequence (rows cu_new[b] .. cu_new[b+1]-1 of the token-major
    k_new / v_new [total, Hkv, 128]) at positions seq_lens[b] ..: completed tiles are quantized
    into their pages, the partial last tile goes to staging. max_new_tokens bounds every
    chunk (computed from cu_new on the host when omitted, which synchronizes)."""
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_tail, "k_tail"), (v_tail, "v_tail")):
        _need(t, nm, torch.float16)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    _need(cu_new, "cu_new", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(block_table, "block_table", torch.int32)
    B = seq_lens.shape[0]
    total, hkv = k_new.shape[0], k_new.shape[1]
    if tuple(v_new.shape) != tuple(k_new.shape) or k_new.dim() != 3 or k_new.shape[2] != 128:
        raise ValueError("k_new / v_new must be [total, Hkv, 128]")
    if cu_new.shape != (B + 1,):
        raise ValueError("cu_new must be [batch + 1]")
    if tuple(k_tail.shape) != (B, hkv, 128, 128) or tuple(v_tail.shape) != (B, hkv, 128, 128):
        raise ValueError("staging must be [B, Hkv, 128, 128]")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous [B, width]")
    if max_new_tokens is None:
        max_new_tokens = int((cu_new[1:] - cu_new[:-1]).max().item()) if B else 0
    _check(lib.kvarn_write_tokens(ctypes.byref(params), _ptr(k_new), _ptr(v_new), total,
                                  _ptr(cu_new), max(int(max_new_tokens), 0), B, hkv,
                                  _ptr(seq_lens), _ptr(k_tail), _ptr(v_tail), _ptr(block_table),
                                  block_table.shape[1], _ptr(k_pool), _ptr(v_pool),
                                  _pools_n(params, k_pool, v_pool),
                                  _stream(stream)), "kvarn_write_tokens")


# ----------------------------------------------------------------------------- decode


def decode_workspace_bytes(params: Params, batch: int, num_q_heads: int, num_kv_heads: int,
                           max_seq_len: int) -> int:
    return int(lib.kvarn_decode_workspace_bytes(ctypes.byref(params), batch, num_q_heads,
                                                num_kv_heads, max_seq_len))


def chunk_workspace_bytes(params: Params, total_q: int, num_q_heads: int, num_kv_heads: int,
                          max_seq_len: int) -> int:
    return int(lib.kvarn_chunk_workspace_bytes(ctypes.byref(params), total_q, num_q_heads,
                                               num_kv_heads, max_seq_len))


def new_chunk_workspace(params: Params, total_q, num_q_heads, num_kv_heads, max_seq_len,
                        device="cuda"):
    nbytes = chunk_workspace_bytes(params, total_q, num_q_heads, num_kv_heads, max_seq_len)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def decode_num_splits(params: Params, batch: int, num_kv_heads: int, max_seq_len: int) -> int:
    return int(lib.kvarn_decode_num_splits(ctypes.byref(params), batch, num_kv_heads, max_seq_len))


def new_workspace(params: Params, batch, num_q_heads, num_kv_heads, max_seq_len, device="cuda"):
    nbytes = decode_workspace_bytes(params, batch, num_q_heads, num_kv_heads, max_seq_len)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def decode_attention(params: Params, q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int,
                     k_tail=None, v_tail=None, softmax_scale: float | None = None,
                     workspace=None, out=None, stream=None) -> torch.Tensor:
    """Paged decode attention; q [B, Hq, 128] float16 -> out [B, Hq, 128] float16."""
    B, hq, hkv = _decode_shapes(q, k_pool, v_pool, block_table, seq_lens, k_tail, v_tail)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128)
    if workspace is None:
        workspace = new_workspace(params, B, hq, hkv, max_seq_len, q.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16)
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be contiguous and shaped like q")
    _check(lib.kvarn_decode_attention(ctypes.byref(params), _ptr(q), B, hq, hkv, _ptr(k_pool),
                                      _ptr(v_pool), _pools_n(params, k_pool, v_pool),
                                      _ptr(block_table),
                                      block_table.shape[1], _ptr(seq_lens), max_seq_len,
                                      _ptr(k_tail), _ptr(v_tail), float(softmax_scale),
                                      _ptr(workspace), workspace.numel(), _ptr(out),
                                      _stream(stream)), "kvarn_decode_attention")
    return out


def decode_noalloc_max_workspace_bytes() -> int:
    return int(lib.kvarn_decode_noalloc_max_workspace_bytes())


def decode_attention_noalloc(params: Params, q, k_pool, v_pool, block_table, seq_lens,
                             max_seq_len: int, k_tail=None, v_tail=None,
                             softmax_scale: float | None = None, out=None,
                             stream=None) -> torch.Tensor:
    """decode_attention with the library's fixed device scratch as its workspace (the entry
    point that allocates nothing; calls that overlap on one GPU race). out is allocated here
    when omitted, so a caller that must not allocate passes it."""
    B, hq, hkv = _decode_shapes(q, k_pool, v_pool, block_table, seq_lens, k_tail, v_tail)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16)
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be contiguous and shaped like q")
    _check(lib.kvarn_decode_attention_noalloc(ctypes.byref(params), _ptr(q), B, hq, hkv,
                                              _ptr(k_pool), _ptr(v_pool),
                                              _pools_n(params, k_pool, v_pool),
                                              _ptr(block_table), block_table.shape[1],
                                              _ptr(seq_lens), max_seq_len, _ptr(k_tail),
                                              _ptr(v_tail), float(softmax_scale), _ptr(out),
                                              _stream(stream)), "kvarn_decode_attention_noalloc")
    return out


def chunk_attention(params: Params, q, cu_q, k_pool, v_pool, block_table, seq_lens,
                    max_seq_len: int, k_tail=None, v_tail=None, softmax_scale: float | None = None,
                    workspace=None, out=None, stream=None) -> torch.Tensor:
    """Causal attention of the last cu_q[b+1] - cu_q[b] positions of every sequence (query rows
    of q [total_q, Hq, 128] float16) over the quantized cache -> out [total_q, Hq, 128]."""
    _need(cu_q, "cu_q", torch.int32)
    total_q, hq, hkv = _decode_shapes(q, k_pool, v_pool, block_table, seq_lens, k_tail, v_tail,
                                      rows=True)
    B = seq_lens.shape[0]
    if cu_q.shape != (B + 1,):
        raise ValueError("cu_q must be [batch + 1]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128)
    if workspace is None:
        workspace = new_chunk_workspace(params, max(total_q, 1), hq, hkv, max_seq_len, q.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16)
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be contiguous and shaped like q")
    _check(lib.kvarn_chunk_attention(ctypes.byref(params), _ptr(q), total_q, _ptr(cu_q), B, hq,
                                     hkv, _ptr(k_pool), _ptr(v_pool),
                                     _pools_n(params, k_pool, v_pool),
                                     _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                     max_seq_len, _ptr(k_tail), _ptr(v_tail), float(softmax_scale),
                                     _ptr(workspace), workspace.numel(), _ptr(out),
                                     _stream(stream)), "kvarn_chunk_attention")
    return out


# ----------------------------------------------------------------------------- prepared calls


class Prepared:
    """A C-ABI call with every argument marshalled once; calling it re-issues the same launch
    (same buffers, same stream) with no per-call Python checks. For benchmark loops and graph
    capture, where a few microseconds of host work per launch would dominate."""

    def __init__(self, fn, args, what, keep=()):
        # keep: the tensors whose addresses are in args, held so that they outlive the call
        self._fn, self._args, self._what, self._keep = fn, args, what, tuple(keep)

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise KvarnError(st, self._what)


def prepare_quantize(params: Params, kind: int, src, tile_src_token, tile_dst_page, pool,
                     stream=None) -> Prepared:
    _need(src, "src", torch.float16)
    _need(tile_src_token, "tile_src_token", torch.int64)
    _need(tile_dst_page, "tile_dst_page", torch.int32)
    _need(pool, "pool", torch.uint8)
    hkv = src.shape[1]
    args = (ctypes.byref(params), kind, _ptr(src), src.stride(0), src.stride(1), src.shape[0],
            _ptr(tile_src_token), _ptr(tile_dst_page), tile_src_token.numel(), hkv, _ptr(pool),
            _pool_n(params, pool, kind), _stream(stream))
    return Prepared(lib.kvarn_quantize_tiles, args, "kvarn_quantize_tiles",
                    (src, tile_src_token, tile_dst_page, pool))


def prepare_quantize_kv(params: Params, k_src, v_src, tile_src_token, tile_dst_page, k_pool,
                        v_pool, stream=None) -> Prepared:
    args = _kv_quant_args(params, k_src, v_src, tile_src_token, tile_dst_page, k_pool, v_pool,
                          stream)
    return Prepared(lib.kvarn_quantize_kv_tiles, args, "kvarn_quantize_kv_tiles",
                    (k_src, v_src, tile_src_token, tile_dst_page, k_pool, v_pool))


def prepare_append(params: Params, k_new, v_new, seq_lens, k_tail, v_tail, block_table,
                   k_pool, v_pool, stream=None) -> Prepared:
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_tail, "k_tail"), (v_tail, "v_tail")):
        _need(t, nm, torch.float16)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    _need(seq_lens, "seq_lens", torch.int32)
    _need(block_table, "block_table", torch.int32)
    B, hkv = k_new.shape[0], k_new.shape[1]
    if k_new.dim() != 3 or k_new.shape[2] != 128 or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new / v_new must be [B, Hkv, 128]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError(f"seq_lens must be [{B}]")
    if tuple(k_tail.shape) != (B, hkv, 128, 128) or tuple(v_tail.shape) != (B, hkv, 128, 128):
        raise ValueError("staging must be [B, Hkv, 128, 128]")
    if k_pool.shape[1] != hkv:
        raise ValueError(f"pools must have {hkv} KV heads")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous [B, width]")
    args = (ctypes.byref(params), _ptr(k_new), _ptr(v_new), B, hkv, _ptr(seq_lens),
            _ptr(k_tail), _ptr(v_tail), _ptr(block_table), block_table.shape[1], _ptr(k_pool),
            _ptr(v_pool), _pools_n(params, k_pool, v_pool), _stream(stream))
    return Prepared(lib.kvarn_append_tokens, args, "kvarn_append_tokens",
                    (k_new, v_new, seq_lens, k_tail, v_tail, block_table, k_pool, v_pool))


def prepare_decode(params: Params, q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int,
                   workspace, out, k_tail=None, v_tail=None, softmax_scale=None,
                   stream=None) -> Prepared:
    B, hq, hkv = _decode_shapes(q, k_pool, v_pool, block_table, seq_lens, k_tail, v_tail)
    _need(workspace, "workspace", torch.uint8)
    _need(out, "out", torch.float16)
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be contiguous and shaped like q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128)
    args = (ctypes.byref(params), _ptr(q), B, hq, hkv, _ptr(k_pool), _ptr(v_pool),
            _pools_n(params, k_pool, v_pool),
            _ptr(block_table), block_table.shape[1], _ptr(seq_lens), max_seq_len, _ptr(k_tail),
            _ptr(v_tail), float(softmax_scale), _ptr(workspace), workspace.numel(), _ptr(out),
            _stream(stream))
    return Prepared(lib.kvarn_decode_attention, args, "kvarn_decode_attention",
                    (q, k_pool, v_pool, block_table, seq_lens, workspace, out, k_tail, v_tail))
