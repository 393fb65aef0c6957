"""Plain CPU oracle for decode attention over a paged KV cache.

THIS MODULE IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
It shares no code with the HIP library (``paged_kv_cache_321_amd``) and never
imports it; the product path never imports this module.

Everything here is deliberately slow and direct: NumPy in float64, one
sequence and one head at a time, with no blocking, fusion or reordering beyond
what the definitions below state.  Sources (the web pages this project is
built from):

* [tbr8] "详解vLLM推理引擎架构：PagedAttention原理与LLM高效部署实践"
  (tbr8.org/?p=10846): section "KV Cache 的传统管理方式" (the KV-size formula
  and its LLaMA-13B example), section "PagedAttention 的核心思想" (logical
  blocks mapped to physical pages through a block table), section
  "Copy-on-Write 与内存共享" (block copy before writing a shared block).
* [xdnf] "vLLM高性能大语言模型推理与服务引擎的技术架构与深度解析"
  (xdnf.cn/news/213146): section 3.2 (the Block0/1/2 -> Page3/1/5 diagram).
* [luoboask] "vLLM 深度解读" (luoboask.github.io/fde-learning/opensource/vllm/):
  section 2 "BlockManager" (block counts, ceil(tokens / block_size)),
  section 3 "PagedAttention CUDA Kernel" (what the decode kernel computes:
  per (sequence, head) a scaled q.k score for every context token reached
  through the block table, softmax over them, weighted sum of V),
  section 7 "模型实现 — 以 Llama 为例" (store the new token's K/V into the
  cache, then run paged attention).
* [tbr8] sections "Chunked Prefill（分块预填充）" and "结合 Speculative
  Decoding 加速" (several new tokens per sequence in one pass), see
  ``multi_query``.

Readings taken where the pages are silent or inconsistent (each is listed in
the design notes of the repository as well):

* Cache layout is [num_blocks, num_kv_heads, block_size, head_dim]; a
  (block, kv_head) page is a contiguous block_size x head_dim tile.
* Grouped-query attention: query head h reads kv head h // (H / Hkv).
* A sequence with context length 0 yields an all-zero output row.
* The new-token write addresses slots as slot = physical_block * block_size +
  offset; a negative slot means "no write".
* Block copy copies the whole block (K and V, all slots); the sources are read
  as they were before any copy of the same call.
* The KV-size formula's "h" and "d" are the head count and the per-head
  dimension (so h * d is the hidden size), see ``kv_cache_bytes``.

Floating point: bf16 inputs arrive as uint16 bit patterns, fp32 inputs as
float32 arrays and E4M3 cache entries as uint8 codes; all are widened exactly
to float64 here.  The attention
result is the exact softmax attention in float64 (the plain definition that
the paged kernel reaches up to rounding order).

Parity status: every function below is pinned by the CPU tests in
``tests/test_oracle.py`` (brute force, a library routine, printed worked
examples and invariants).  No function is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "BF16",
    "F32",
    "FP8",
    "widen",
    "e4m3_values",
    "e4m3_encode",
    "e4m3_inverse_scale",
    "kv_cache_bytes",
    "num_required_blocks",
    "kv_head_for",
    "reshape_and_cache",
    "copy_blocks",
    "gather_context",
    "softmax",
    "attend_one",
    "decode",
    "decode_rows",
    "swap_blocks",
    "query_rows",
    "query_position",
    "multi_query",
]

BF16 = "bf16"
F32 = "f32"
FP8 = "fp8"   # OCP 8-bit floating point E4M3 codes, stored as uint8


# --------------------------------------------------------------------------
# FP8 (E4M3) KV cache.  [tbr8] section "量化集成与部署" offers an fp8 KV
# cache option without fixing a format; the reading taken here is the OCP
# E4M3 format (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
# infinities, S.1111.111 = NaN, largest finite 448) with one float32 scale
# per cache: the stored code of x is the finite E4M3 value nearest to
# x * fl32(1 / scale) (ties to the even code, magnitudes beyond 448 become
# 448), and a code c stands for value(c) * scale.
# --------------------------------------------------------------------------

def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes (NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


def e4m3_inverse_scale(scale: float) -> np.float32:
    """fl32(1 / scale): the factor new tokens are multiplied by before encoding."""
    return np.float32(1.0) / np.float32(scale)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 code of each float32 value (ties to even codes).

    Written from the definition: compare |x| against every non-negative finite
    E4M3 magnitude (codes 0x00..0x7E, increasing), take the closest, break a
    tie towards the code with a zero lowest bit, saturate beyond 448, keep the
    sign bit (so -0.0 -> 0x80), and map NaN to 0x7F with the sign bit of x.
    """
    x = np.asarray(x, dtype=np.float32)
    mags = e4m3_values()[:0x7F]                      # 0x00 .. 0x7E, increasing
    flat = x.reshape(-1).astype(np.float64)
    out = np.empty(flat.shape, dtype=np.uint8)
    signs = np.signbit(x.reshape(-1))
    for i, v in enumerate(flat):
        sign = 0x80 if signs[i] else 0x00
        if np.isnan(v):
            out[i] = sign | 0x7F
            continue
        a = abs(v)
        if a >= mags[-1]:
            out[i] = sign | 0x7E
            continue
        hi = int(np.searchsorted(mags, a, side="left"))  # mags[hi-1] < a <= mags[hi]
        if mags[hi] == a:
            code = hi
        else:
            lo = hi - 1
            dlo, dhi = a - mags[lo], mags[hi] - a
            if dlo < dhi:
                code = lo
            elif dhi < dlo:
                code = hi
            else:
                code = lo if lo % 2 == 0 else hi
        out[i] = sign | code
    return out.reshape(x.shape)


# --------------------------------------------------------------------------
# Element types
# --------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of cache/query elements to float64.

    bf16 values are the upper 16 bits of an IEEE binary32 number, so the
    widening puts the 16 stored bits on top of 16 zero bits and reads the
    result as binary32 (exact), then as binary64 (exact).
    """
    if dtype == BF16:
        if x.dtype != np.uint16:
            raise TypeError("bf16 data must be given as uint16 bit patterns")
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        if x.dtype != np.float32:
            raise TypeError("f32 data must be given as float32")
        return x.astype(np.float64)
    if dtype == FP8:
        if x.dtype != np.uint8:
            raise TypeError("fp8 data must be given as uint8 E4M3 codes")
        return e4m3_values()[x]
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# Sizes ([tbr8] "KV Cache 的传统管理方式"; [luoboask] section 2)
# --------------------------------------------------------------------------

def kv_cache_bytes(num_layers: int, num_heads: int, num_tokens: int,
                   head_dim: int, itemsize: int) -> int:
    """KV-cache bytes: 2 (K and V) x layers x heads x tokens x head_dim x size.

    [tbr8] "KV Cache 的传统管理方式" writes the product with l layers, h heads,
    L tokens and a dimension d.  Its LLaMA-13B example plugs in d = 5120 (the
    hidden size), which would count the hidden size h times over; the
    consistent reading is d = per-head dimension (5120 / 40 = 128).
    """
    return 2 * num_layers * num_heads * num_tokens * head_dim * itemsize


def num_required_blocks(num_tokens: int, block_size: int) -> int:
    """Blocks needed for ``num_tokens`` tokens: ceil(num_tokens / block_size).

    [luoboask] section 2, ``get_num_required_blocks``.
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    return math.ceil(num_tokens / block_size)


def kv_head_for(head: int, num_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``head``: contiguous groups of H / Hkv heads.

    The kernel sketch of [luoboask] section 3 takes ``num_kv_heads`` but only
    shows H == Hkv; grouping consecutive query heads onto one KV head is the
    reading used here.
    """
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return head // (num_heads // num_kv_heads)


# --------------------------------------------------------------------------
# Cache writes ([luoboask] section 7; [tbr8] "Copy-on-Write 与内存共享")
# --------------------------------------------------------------------------

def reshape_and_cache(key: np.ndarray, value: np.ndarray,
                      k_cache: np.ndarray, v_cache: np.ndarray,
                      slot_mapping: np.ndarray, src_dtype: str = None,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Store each new token's K and V rows into its cache slot, in place.

    key, value: [T, Hkv, D]; k_cache, v_cache: [NB, Hkv, BS, D];
    slot_mapping: [T] integers.  Token i goes to block slot // BS, offset
    slot % BS, for every kv head; a negative slot is skipped.  When the caches
    hold the same element type as key/value the elements are copied as they
    are (raw bits for bf16), so the result is exact.  When the caches hold
    E4M3 codes (uint8) and key/value are ``src_dtype`` values, each row is
    encoded as e4m3_encode(fl32(x) * fl32(1 / scale)) in float32 arithmetic.
    """
    block_size = k_cache.shape[2]
    if k_cache.dtype == np.uint8 and key.dtype != np.uint8:
        if src_dtype is None:
            raise ValueError("src_dtype is needed to encode into an fp8 cache")
        kf = widen(key, src_dtype).astype(np.float32) * e4m3_inverse_scale(k_scale)
        vf = widen(value, src_dtype).astype(np.float32) * e4m3_inverse_scale(v_scale)
        key, value = e4m3_encode(kf), e4m3_encode(vf)
    for i in range(key.shape[0]):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        k_cache[block, :, offset, :] = key[i]
        v_cache[block, :, offset, :] = value[i]


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray,
                block_pairs: np.ndarray) -> None:
    """Copy whole blocks src -> dst in both caches, in place.

    block_pairs: [P, 2] (src, dst).  All sources are read as they stood before
    the call, then written to their destinations.
    """
    pairs = np.asarray(block_pairs).reshape(-1, 2)
    k_src = {int(s): k_cache[int(s)].copy() for s, _ in pairs}
    v_src = {int(s): v_cache[int(s)].copy() for s, _ in pairs}
    for src, dst in pairs:
        k_cache[int(dst)] = k_src[int(src)]
        v_cache[int(dst)] = v_src[int(src)]


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray,
                dst_v: np.ndarray, block_pairs: np.ndarray) -> None:
    """Copy whole blocks from one pool to another, in place on the destination.

    [tbr8] (the scheduler section) swaps a preempted request's KV cache out
    to CPU memory and back in later; [luoboask] section 4 keeps such requests
    in a SWAPPED queue.  For each (src, dst) pair, block dst of the destination
    pool (K and V, every kv head and slot) becomes block src of the source pool.
    """
    for src, dst in np.asarray(block_pairs).reshape(-1, 2):
        dst_k[int(dst)] = src_k[int(src)]
        dst_v[int(dst)] = src_v[int(src)]


# --------------------------------------------------------------------------
# Attention ([luoboask] section 3; [tbr8] "PagedAttention 的核心思想")
# --------------------------------------------------------------------------

def gather_context(cache: np.ndarray, block_table_row: np.ndarray,
                   context_len: int) -> np.ndarray:
    """Contiguous [Hkv, context_len, D] view of one sequence's cached tokens.

    Logical block j of the sequence lives in physical block
    ``block_table_row[j]``; logical token t is slot t % BS of logical block
    t // BS.  The blocks are concatenated in logical order and the result is
    cut at context_len (slots past the end of the last block are never read).
    """
    block_size = cache.shape[2]
    nblocks = num_required_blocks(context_len, block_size)
    if nblocks == 0:
        return cache[:0].reshape(cache.shape[1], 0, cache.shape[3])
    pages = [cache[int(block_table_row[j])] for j in range(nblocks)]
    return np.concatenate(pages, axis=1)[:, :context_len, :]


def softmax(z: np.ndarray) -> np.ndarray:
    """Softmax of a 1-D float64 vector, with the maximum subtracted first."""
    w = np.exp(z - z.max())
    return w / w.sum()


def attend_one(q: np.ndarray, k: np.ndarray, v: np.ndarray,
               scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one query over L keys/values (float64).

    q: [D]; k, v: [L, D].  Returns (out [D], weights [L]) with
    weights = softmax(scale * k @ q) and out = weights @ v.
    """
    z = scale * (k @ q)
    w = softmax(z)
    return w @ v, w


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray,
           scale: float, dtype: str, return_weights: bool = False,
           cache_dtype: str = None, k_scale: float = 1.0, v_scale: float = 1.0):
    """Single-query decode attention over a paged cache, float64 result.

    q: [S, H, D]; caches [NB, Hkv, BS, D]; block_tables [S, MB];
    context_lens [S].  ``scale`` is taken as the float32 value the GPU path
    receives, promoted exactly.  Sequences with context length 0 give zeros.
    ``cache_dtype`` (default: ``dtype``) is the cache element type; for E4M3
    caches a code c stands for value(c) * k_scale (keys) or * v_scale (values).
    Returns out [S, H, D] (and, if asked, a list of per-(s, h) weights).
    """
    num_seqs, num_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    scale64 = float(np.float32(scale))
    out = np.zeros((num_seqs, num_heads, head_dim), dtype=np.float64)
    weights = {}
    for s in range(num_seqs):
        out[s], w = decode_rows(q[s], k_cache, v_cache, block_tables[s],
                                int(context_lens[s]), scale64, dtype,
                                num_heads, num_kv_heads, cache_dtype=cache_dtype,
                                k_scale=k_scale, v_scale=v_scale)
        if return_weights:
            for h, wh in enumerate(w):
                weights[(s, h)] = wh
    if return_weights:
        return out, weights
    return out


def decode_rows(q_s: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                block_table_row: np.ndarray, context_len: int, scale: float,
                dtype: str, num_heads: int, num_kv_heads: int,
                heads=None, cache_dtype: str = None, k_scale: float = 1.0,
                v_scale: float = 1.0):
    """Decode output for one sequence (all heads, or the listed ``heads``).

    q_s: [H, D].  Returns (out [len(heads), D] float64, list of weights).
    """
    heads = list(range(num_heads)) if heads is None else list(heads)
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    head_dim = q_s.shape[-1]
    out = np.zeros((len(heads), head_dim), dtype=np.float64)
    weights = []
    if context_len == 0:
        return out, [np.zeros(0) for _ in heads]
    k_ctx = widen(gather_context(k_cache, block_table_row, context_len), cache_dtype)
    v_ctx = widen(gather_context(v_cache, block_table_row, context_len), cache_dtype)
    if cache_dtype == FP8:
        k_ctx = k_ctx * float(np.float32(k_scale))
        v_ctx = v_ctx * float(np.float32(v_scale))
    q64 = widen(np.ascontiguousarray(q_s), dtype)
    for i, h in enumerate(heads):
        kvh = kv_head_for(h, num_heads, num_kv_heads)
        out[i], w = attend_one(q64[h], k_ctx[kvh], v_ctx[kvh], float(np.float32(scale)))
        weights.append(w)
    return out, weights


# --------------------------------------------------------------------------
# Several new query tokens per sequence.  [tbr8] section "Chunked Prefill（分块
# 预填充）": a long prompt is processed in chunks that are interleaved with
# decoding requests; section "结合 Speculative Decoding 加速": a small draft
# model proposes N tokens and the large model checks them all in one pass.
# Reading (the pages give no formula): the K/V of a sequence's q_len new
# tokens are already in the cache (stored by reshape_and_cache, as for
# decode); the new tokens are the last q_len positions of its context; each
# attends to every cached token at or before its own position (causal
# attention, the rule that makes the chunked result equal the unchunked one).
# --------------------------------------------------------------------------

def query_rows(query_start: np.ndarray, s: int) -> tuple[int, int]:
    """Rows [t0, t1) of q / out holding sequence s's queries (CSR offsets)."""
    return int(query_start[s]), int(query_start[s + 1])


def query_position(context_len: int, query_len: int, i: int) -> int:
    """Position in its sequence of query i of a chunk of ``query_len`` new
    tokens that end the sequence's ``context_len`` tokens."""
    return context_len - query_len + i


def multi_query(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                block_tables: np.ndarray, context_lens: np.ndarray,
                query_start: np.ndarray, scale: float, dtype: str,
                cache_dtype: str = None, k_scale: float = 1.0, v_scale: float = 1.0):
    """Causal attention of each sequence's new query tokens over its paged cache.

    q: [T, H, D] with sequence s's queries in rows query_rows(query_start, s);
    caches [NB, Hkv, BS, D]; block_tables [S, MB]; context_lens [S] (cached
    tokens, the new ones included); query_start [S + 1].  The query at
    position p (``query_position``) gets softmax over tokens 0..p of
    scale * q.k, applied to V.  A sequence with more queries than context
    tokens is an error.  Returns out [T, H, D] float64 (rows of no sequence
    stay zero).
    """
    num_rows, num_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    scale64 = float(np.float32(scale))
    q64 = widen(np.ascontiguousarray(q), dtype)
    out = np.zeros((num_rows, num_heads, head_dim), dtype=np.float64)
    for s in range(len(context_lens)):
        t0, t1 = query_rows(query_start, s)
        query_len = t1 - t0
        context_len = int(context_lens[s])
        if query_len == 0:
            continue
        if query_len > context_len:
            raise ValueError(f"sequence {s}: {query_len} queries but {context_len} tokens")
        k_ctx = widen(gather_context(k_cache, block_tables[s], context_len), cache_dtype)
        v_ctx = widen(gather_context(v_cache, block_tables[s], context_len), cache_dtype)
        if cache_dtype == FP8:
            k_ctx = k_ctx * float(np.float32(k_scale))
            v_ctx = v_ctx * float(np.float32(v_scale))
        for i in range(query_len):
            visible = query_position(context_len, query_len, i) + 1
            for h in range(num_heads):
                kvh = kv_head_for(h, num_heads, num_kv_heads)
                out[t0 + i, h], _ = attend_one(q64[t0 + i, h], k_ctx[kvh, :visible],
                                               v_ctx[kvh, :visible], scale64)
    return out

