"""Thin ctypes binding of libpa.so (include/pa.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream, every computation runs in the library's HIP kernels.  The library is
required: importing this module raises if libpa.so is missing.  Each function
has the name of the C entry point it calls and raises ``PaError`` (a
RuntimeError) with the library's status text when the call is rejected.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2
PA_DECODE_SHARED_PAGES = 1
PA_MULTI_QUERY_TILES_ONLY = 1
PA_MULTI_QUERY_ONE_STREAM = 2
PA_PARTITION_FIXED = 0
PA_PARTITION_FILL = 1
STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_DTYPE",
          -4: "PA_ERR_UNSUPPORTED", -5: "PA_ERR_ALIGN", -6: "PA_ERR_WORKSPACE",
          -7: "PA_ERR_LAUNCH", -8: "PA_ERR_VALUE", -9: "PA_ERR_SCRATCH"}
PA_DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20
EXPORTS = ("pa_reshape_and_cache", "pa_copy_blocks", "pa_decode_partition_tokens",
           "pa_decode_workspace_size",
           "pa_decode", "pa_decode_noalloc", "pa_decode_shared_prefix_workspace_size",
           "pa_decode_shared_prefix",
           "pa_multi_query_workspace_size", "pa_multi_query", "pa_side_stream_create",
           "pa_side_stream_destroy", "pa_swap_blocks", "pa_status_string")

_c_int, _c_size, _c_float, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p


class SideStream(ctypes.Structure):
    """pa_side_stream: a second HIP stream and its fork / join events, owned by
    whoever created it (``create`` / ``destroy`` call the library's helpers)."""

    _fields_ = [("stream", ctypes.c_void_p), ("fork_event", ctypes.c_void_p),
                ("join_event", ctypes.c_void_p)]

    @classmethod
    def create(cls) -> "SideStream":
        side = cls()
        _check(LIB.pa_side_stream_create(ctypes.byref(side)), "pa_side_stream_create")
        return side

    def destroy(self) -> None:
        _check(LIB.pa_side_stream_destroy(ctypes.byref(self)), "pa_side_stream_destroy")


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {pa_status_string(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m paged_kv_cache_321_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.pa_reshape_and_cache.argtypes = ([_vp, _vp, _vp, _vp, _vp] + [_c_int] * 7 +
                                         [_c_float, _c_float, _vp])
    lib.pa_reshape_and_cache.restype = _c_int
    lib.pa_copy_blocks.argtypes = [_vp, _vp, _vp] + [_c_int] * 6 + [_vp]
    lib.pa_copy_blocks.restype = _c_int
    lib.pa_decode_partition_tokens.argtypes = [_c_int] * 9
    lib.pa_decode_partition_tokens.restype = _c_int
    lib.pa_decode_workspace_size.argtypes = [_c_int] * 9
    lib.pa_decode_workspace_size.restype = _c_size
    lib.pa_decode.argtypes = ([_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp] + [_c_int] * 7 +
                              [_c_float, _c_int, _c_int, _c_float, _c_float, _c_int, _c_int, _vp,
                               _c_size, _vp])
    lib.pa_decode.restype = _c_int
    lib.pa_decode_noalloc.argtypes = ([_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp] + [_c_int] * 7 +
                                      [_c_float, _c_int, _c_int, _c_float, _c_float, _c_int, _c_int,
                                       _vp])
    lib.pa_decode_noalloc.restype = _c_int
    lib.pa_decode_shared_prefix_workspace_size.argtypes = [_c_int] * 11
    lib.pa_decode_shared_prefix_workspace_size.restype = _c_size
    lib.pa_decode_shared_prefix.argtypes = ([_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp] +
                                            [_c_int] * 9 +
                                            [_c_float, _c_int, _c_int, _c_float, _c_float, _c_int,
                                             _c_int, _vp, _c_size, _vp])
    lib.pa_decode_shared_prefix.restype = _c_int
    lib.pa_multi_query_workspace_size.argtypes = [_c_int] * 10
    lib.pa_multi_query_workspace_size.restype = _c_size
    lib.pa_multi_query.argtypes = ([_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp] + [_c_int] * 9 +
                                   [_c_float, _c_int, _c_int, _c_float, _c_float, _c_int, _c_int,
                                    _vp, _c_size, _vp, _vp])
    lib.pa_multi_query.restype = _c_int
    lib.pa_side_stream_create.argtypes = [_vp]
    lib.pa_side_stream_create.restype = _c_int
    lib.pa_side_stream_destroy.argtypes = [_vp]
    lib.pa_side_stream_destroy.restype = _c_int
    lib.pa_swap_blocks.argtypes = [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 7 + [_vp]
    lib.pa_swap_blocks.restype = _c_int
    lib.pa_status_string.argtypes = [_c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    return lib


LIB = load_library()


def pa_status_string(status: int) -> str:
    return LIB.pa_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise PaError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    """Element type code; caches of E4M3 codes may be float8_e4m3fn or uint8."""
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return PA_FP8_E4M3
    raise TypeError(f"unsupported element type {t.dtype} (float32, bfloat16, or fp8 codes)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _device_contig(name: str, t: torch.Tensor) -> None:
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def pa_reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                         v_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None,
                         k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Store key/value [T, Hkv, D] into caches [NB, Hkv, BS, D] at slot_mapping [T].

    fp8 caches (float8_e4m3fn or uint8 code tensors) receive the E4M3 codes of
    key / k_scale and value / v_scale.
    """
    for n, t in (("key", key), ("value", value), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("slot_mapping", slot_mapping)):
        _device_contig(n, t)
    _need(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
    _need(key.dtype == value.dtype and k_cache.dtype == v_cache.dtype, "element types differ")
    nb, hkv, bs, d = k_cache.shape
    _need(v_cache.shape == k_cache.shape, "k_cache and v_cache shapes differ")
    t = key.shape[0]
    _need(key.shape == (t, hkv, d) and value.shape == key.shape, "key/value must be [T, Hkv, D]")
    _need(slot_mapping.shape == (t,), "slot_mapping must be [T]")
    st = LIB.pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(slot_mapping), t, nb, hkv, bs, d, _dtype_code(key),
                                  _dtype_code(k_cache), float(k_scale), float(v_scale),
                                  _stream(stream))
    _check(st, "pa_reshape_and_cache")


def pa_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_pairs: torch.Tensor,
                   stream=None) -> None:
    """Copy whole blocks src -> dst for block_pairs [P, 2] (int64)."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("block_pairs", block_pairs)):
        _device_contig(n, t)
    _need(block_pairs.dtype == torch.int64, "block_pairs must be int64")
    _need(block_pairs.dim() == 2 and block_pairs.shape[1] == 2, "block_pairs must be [P, 2]")
    _need(k_cache.dtype == v_cache.dtype and k_cache.shape == v_cache.shape, "cache mismatch")
    nb, hkv, bs, d = k_cache.shape
    st = LIB.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), block_pairs.shape[0],
                            nb, hkv, bs, d, _dtype_code(k_cache), _stream(stream))
    _check(st, "pa_copy_blocks")


def pa_decode_partition_tokens(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                               block_size: int, max_context_len: int, dtype: int,
                               cache_dtype: Optional[int] = None,
                               policy: int = PA_PARTITION_FIXED) -> int:
    """Partition length ``policy`` picks for a pa_decode call of these sizes."""
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    t = LIB.pa_decode_partition_tokens(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                       max_context_len, dtype, cache_dtype, policy)
    _check(t if t < 0 else 0, "pa_decode_partition_tokens")
    return t


def pa_decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                             block_size: int, max_context_len: int, dtype: int,
                             partition_tokens: int = 0, cache_dtype: Optional[int] = None) -> int:
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    n = LIB.pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, dtype, cache_dtype, partition_tokens)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("pa_decode_workspace_size: arguments rejected by the library")
    return n


def longest_first(context_lens, device="cuda") -> torch.Tensor:
    """Dispatch order with the longest contexts first, from host-side lengths.

    Ties keep their index order, so the order is a function of the lengths only.
    """
    lens = torch.as_tensor(context_lens, dtype=torch.int64).cpu()
    order = sorted(range(len(lens)), key=lambda i: (-int(lens[i]), i))
    return torch.tensor(order, dtype=torch.int32, device=device)


def pa_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
              max_context_len: int, partition_tokens: int = 0,
              workspace: Optional[torch.Tensor] = None, stream=None,
              shared_pages: bool = False, seq_order: Optional[torch.Tensor] = None,
              k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Decode attention of q [S, H, D] over the paged caches into out [S, H, D].

    ``workspace`` (uint8 device tensor) is allocated here when not given and
    the shape needs one.  ``shared_pages`` sets PA_DECODE_SHARED_PAGES (pages
    may be shared between sequences: read them with the default cache policy).
    ``seq_order`` (int32 device tensor [S], a permutation) sets the dispatch
    order of the sequences; see ``longest_first``.  fp8 caches (float8_e4m3fn
    or uint8 codes) stand for code * k_scale / code * v_scale.
    """
    for n, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _device_contig(n, t)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    _need(q.dtype == out.dtype and k_cache.dtype == v_cache.dtype, "element types differ")
    s, h, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    _need(d2 == d and out.shape == q.shape and v_cache.shape == k_cache.shape, "shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == s, "block_tables must be [S, MB]")
    _need(context_lens.shape == (s,), "context_lens must be [S]")
    if seq_order is not None:
        _device_contig("seq_order", seq_order)
        _need(seq_order.dtype == torch.int32 and seq_order.shape == (s,),
              "seq_order must be int32 [S]")
    code = _dtype_code(q)
    ccode = _dtype_code(k_cache)
    need = pa_decode_workspace_size(s, h, hkv, d, bs, max_context_len, code, partition_tokens,
                                    ccode) if h > 0 and hkv > 0 and h % hkv == 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = LIB.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                       block_tables.shape[1], _ptr(context_lens), _ptr(seq_order), s, h, hkv, d, bs, nb,
                       int(max_context_len), float(scale), code, ccode, float(k_scale),
                       float(v_scale), int(partition_tokens),
                       PA_DECODE_SHARED_PAGES if shared_pages else 0,
                       _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "pa_decode")


def pa_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                      scale: float, max_context_len: int, partition_tokens: int = 0, stream=None,
                      shared_pages: bool = False, seq_order: Optional[torch.Tensor] = None,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """pa_decode without a workspace: the library's static scratch buffer
    holds the partition results, and nothing is allocated here or in the
    library.  Arguments as for ``pa_decode``."""
    for n, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _device_contig(n, t)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    _need(q.dtype == out.dtype and k_cache.dtype == v_cache.dtype, "element types differ")
    s, h, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    _need(d2 == d and out.shape == q.shape and v_cache.shape == k_cache.shape, "shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == s, "block_tables must be [S, MB]")
    _need(context_lens.shape == (s,), "context_lens must be [S]")
    if seq_order is not None:
        _device_contig("seq_order", seq_order)
        _need(seq_order.dtype == torch.int32 and seq_order.shape == (s,),
              "seq_order must be int32 [S]")
    st = LIB.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                               block_tables.shape[1], _ptr(context_lens), _ptr(seq_order), s, h, hkv,
                               d, bs, nb, int(max_context_len), float(scale), _dtype_code(q),
                               _dtype_code(k_cache), float(k_scale), float(v_scale),
                               int(partition_tokens), PA_DECODE_SHARED_PAGES if shared_pages else 0,
                               _stream(stream))
    _check(st, "pa_decode_noalloc")


def pa_decode_shared_prefix_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int,
                                           head_dim: int, block_size: int, max_context_len: int,
                                           max_prefix_blocks: int, max_tail_len: int, dtype: int,
                                           partition_tokens: int = 0,
                                           cache_dtype: Optional[int] = None) -> int:
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    n = LIB.pa_decode_shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                   block_size, max_context_len, max_prefix_blocks,
                                                   max_tail_len, dtype, cache_dtype,
                                                   partition_tokens)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("pa_decode_shared_prefix_workspace_size: arguments rejected by the library")
    return n


def pa_decode_shared_prefix(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, prefix_leader: torch.Tensor,
                            prefix_blocks: torch.Tensor, scale: float, max_context_len: int,
                            max_prefix_blocks: int, max_tail_len: int, partition_tokens: int = 0,
                            workspace: Optional[torch.Tensor] = None, stream=None,
                            k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Decode attention where groups of sequences share leading cache blocks.

    ``prefix_leader`` and ``prefix_blocks`` (int32 device tensors [S]) name
    each sequence's group leader and, at leaders, the number of shared leading
    blocks; ``max_prefix_blocks`` and ``max_tail_len`` bound them on the host
    (see ``block_pool.prefix_groups`` and ``block_pool.prefix_bounds``).  Same
    result as ``pa_decode``.
    """
    for n, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("prefix_leader", prefix_leader), ("prefix_blocks", prefix_blocks)):
        _device_contig(n, t)
    _need(all(t.dtype == torch.int32 for t in (block_tables, context_lens, prefix_leader,
                                                prefix_blocks)),
          "block_tables, context_lens, prefix_leader and prefix_blocks must be int32")
    _need(q.dtype == out.dtype and k_cache.dtype == v_cache.dtype, "element types differ")
    s, h, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    _need(d2 == d and out.shape == q.shape and v_cache.shape == k_cache.shape, "shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == s, "block_tables must be [S, MB]")
    _need(context_lens.shape == (s,) and prefix_leader.shape == (s,) and prefix_blocks.shape == (s,),
          "context_lens, prefix_leader and prefix_blocks must be [S]")
    code = _dtype_code(q)
    ccode = _dtype_code(k_cache)
    need = pa_decode_shared_prefix_workspace_size(s, h, hkv, d, bs, max_context_len,
                                                  max_prefix_blocks, max_tail_len, code,
                                                  partition_tokens, ccode) \
        if h > 0 and hkv > 0 and h % hkv == 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = LIB.pa_decode_shared_prefix(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                     _ptr(prefix_leader), _ptr(prefix_blocks), s, h, hkv, d, bs, nb,
                                     int(max_context_len), int(max_prefix_blocks),
                                     int(max_tail_len), float(scale), code, ccode, float(k_scale),
                                     float(v_scale), int(partition_tokens), 0, _ptr(workspace),
                                     ws_bytes, _stream(stream))
    _check(st, "pa_decode_shared_prefix")


def pa_multi_query_workspace_size(num_seqs: int, num_query_tokens: int, num_heads: int,
                                  num_kv_heads: int, head_dim: int, block_size: int,
                                  max_context_len: int, dtype: int, partition_tokens: int = 0,
                                  cache_dtype: Optional[int] = None) -> int:
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    n = LIB.pa_multi_query_workspace_size(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                          head_dim, block_size, max_context_len, dtype, cache_dtype,
                                          partition_tokens)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("pa_multi_query_workspace_size: arguments rejected by the library")
    return n


# Side streams this binding made, one per device, for the calls that do not
# pass their own; a lock keeps them to one call at a time.
_SIDE = {}
_SIDE_LOCK = threading.Lock()


def _default_side(device: torch.device) -> SideStream:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _SIDE:
        with torch.cuda.device(idx):
            _SIDE[idx] = SideStream.create()
    return _SIDE[idx]


def pa_multi_query(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                   query_start: torch.Tensor, scale: float, max_context_len: int,
                   max_query_len: int, partition_tokens: int = 0,
                   workspace: Optional[torch.Tensor] = None, stream=None, k_scale: float = 1.0,
                   v_scale: float = 1.0, tiles_only: bool = False,
                   one_stream: bool = False, side: Optional[SideStream] = None) -> None:
    """Causal attention of each sequence's new query tokens over the paged caches.

    q, out [T, H, D] (bf16) hold sequence s's queries in rows
    query_start[s] .. query_start[s + 1] - 1 (int32 device tensor [S + 1]); they
    are the last positions of its context_lens[s] cached tokens.  ``tiles_only``
    sets PA_MULTI_QUERY_TILES_ONLY (no decode launch for single-query sequences),
    ``one_stream`` PA_MULTI_QUERY_ONE_STREAM (no side stream for the decode rows).
    ``side``: the side stream for the decode rows (a ``SideStream``); by default
    one this binding creates per device and keeps.
    """
    for n, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start", query_start)):
        _device_contig(n, t)
    _need(all(t.dtype == torch.int32 for t in (block_tables, context_lens, query_start)),
          "block_tables, context_lens and query_start must be int32")
    _need(q.dtype == out.dtype and k_cache.dtype == v_cache.dtype, "element types differ")
    t, h, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    s = context_lens.shape[0]
    _need(d2 == d and out.shape == q.shape and v_cache.shape == k_cache.shape, "shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == s, "block_tables must be [S, MB]")
    _need(query_start.shape == (s + 1,), "query_start must be [S + 1]")
    code = _dtype_code(q)
    ccode = _dtype_code(k_cache)
    need = pa_multi_query_workspace_size(s, t, h, hkv, d, bs, max_context_len, code,
                                         partition_tokens, ccode) \
        if h > 0 and hkv > 0 and h % hkv == 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    shared_side = side is None and not one_stream
    if shared_side:
        side = _default_side(q.device)

    def call():
        return LIB.pa_multi_query(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                  block_tables.shape[1], _ptr(context_lens), _ptr(query_start), s, t,
                                  int(max_query_len), h, hkv, d, bs, nb, int(max_context_len),
                                  float(scale), code, ccode, float(k_scale), float(v_scale),
                                  int(partition_tokens),
                                  (PA_MULTI_QUERY_TILES_ONLY if tiles_only else 0)
                                  | (PA_MULTI_QUERY_ONE_STREAM if one_stream else 0),
                                  _ptr(workspace), ws_bytes,
                                  None if side is None else ctypes.byref(side), _stream(stream))

    if shared_side:
        with _SIDE_LOCK:
            st = call()
    else:
        st = call()
    _check(st, "pa_multi_query")


def pa_swap_blocks(dst_k_cache: torch.Tensor, dst_v_cache: torch.Tensor, src_k_cache: torch.Tensor,
                   src_v_cache: torch.Tensor, block_pairs: torch.Tensor, stream=None) -> None:
    """Copy whole blocks src_pool[src] -> dst_pool[dst] for block_pairs [P, 2] (int64).

    Each pool is a device tensor or a pinned host tensor (``pin_memory=True``),
    as is ``block_pairs``.
    """
    for n, t in (("dst_k_cache", dst_k_cache), ("dst_v_cache", dst_v_cache),
                 ("src_k_cache", src_k_cache), ("src_v_cache", src_v_cache),
                 ("block_pairs", block_pairs)):
        _need(t.is_cuda or t.is_pinned(), f"{n} must be a device tensor or pinned host memory")
        _need(t.is_contiguous(), f"{n} must be contiguous")
    _need(block_pairs.dtype == torch.int64, "block_pairs must be int64")
    _need(block_pairs.dim() == 2 and block_pairs.shape[1] == 2, "block_pairs must be [P, 2]")
    _need(dst_k_cache.dtype == dst_v_cache.dtype == src_k_cache.dtype == src_v_cache.dtype,
          "element types differ")
    _need(dst_k_cache.shape == dst_v_cache.shape and src_k_cache.shape == src_v_cache.shape and
          dst_k_cache.shape[1:] == src_k_cache.shape[1:], "pool shapes differ")
    nbd, hkv, bs, d = dst_k_cache.shape
    st = LIB.pa_swap_blocks(_ptr(dst_k_cache), _ptr(dst_v_cache), _ptr(src_k_cache), _ptr(src_v_cache),
                            _ptr(block_pairs), block_pairs.shape[0], src_k_cache.shape[0], nbd, hkv,
                            bs, d, _dtype_code(dst_k_cache), _stream(stream))
    _check(st, "pa_swap_blocks")
