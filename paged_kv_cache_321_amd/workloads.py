"""Seeded synthetic inputs for paged-KV decode.

This module only makes inputs: shapes, context lengths, shuffled physical
block assignments, block tables, new-token slots, copy-on-write pairs and
random K/V/Q values.  It contains none of the attention arithmetic, and both
the GPU path's tests and the CPU oracle's tests draw their inputs from it.

Workloads (all bf16 except the tiny one; values N(0, 1) cast to the element
type with round-to-nearest-even):

``tiny``      4 sequences, context lengths 1, 17, 33, 100; 4 heads (no
              grouping), head_dim 64, block_size 16, fp32, a 64-block pool;
              every sequence's newest token is stored before attention.
``llama7b``   64 sequences, context lengths uniform in [128, 2048]; 32 heads,
              head_dim 128, block_size 16 (LLaMA-7B attention shape).
``llama13b``  128 sequences at context 2048; 40 heads, head_dim 128,
              block_size 16 (LLaMA-13B shape); 128 new tokens are stored at
              their sequences' newest slots, in a shuffled token order.
``gqa70b``    16 sequences at context 32768; 64 query heads over 8 KV heads,
              head_dim 128, block_size 32; Q is N(0, 1) / 2.
``beam``      32 groups x 4 beams sharing a 1024-token prefix (the same
              physical blocks, reference count 4) plus per-beam tails of 1 to
              256 tokens (the tail includes the new token); 32 query heads over
              8 KV heads, head_dim 128, block_size 16.  A seeded 10% of the
              beams whose last block already holds tokens find that block
              shared (reference count 2) and must copy it before the write.

``specdec70b``  speculative verification: 32 sequences with contexts uniform
              in [1024, 8192], each ending with 6 new tokens (the accepted
              token and 5 drafts) whose K/V the step stores; 64 query heads
              over 8 KV heads, head_dim 128, block_size 16.
``chunked13b``  a chunked-prefill batch of 3136 query tokens: a 2048-token
              chunk after 2048 cached tokens, a first chunk of 1024 tokens, and
              64 decoding sequences (contexts uniform in [128, 4096]); 40
              heads, head_dim 128, block_size 16 (LLaMA-13B shape).

``<name>_fp8``  the same workload with an fp8 (OCP E4M3) KV cache and two
              different scales, k_scale = 0.02 and v_scale = 0.03 (neither a
              power of two, so a swapped pair or a division in place of the
              multiplication by fl32(1 / scale) shows in the results):
              history entries are N(0, 1) draws divided by their cache's
              scale and cast to float8_e4m3fn (torch's cast, clamped to
              +-448), new tokens stay bf16 and are encoded by
              reshape_and_cache.

Physical pools hold ceil(1.1 x blocks needed) blocks unless a size is given;
blocks are handed out in the order of a seeded permutation, sequence by
sequence, so logically adjacent blocks are physically scattered.  Slots that
hold no token (unused blocks, slots past the end of a sequence, slots about to
be written) are NaN when ``poison`` is set and zero otherwise.  Block-table
rows are padded with -1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from .block_pool import BlockPool, BlockTable, padded_rows

__all__ = ["Spec", "FP8_K_SCALE", "FP8_V_SCALE", "fp8_scales", "Plan", "Inputs", "SPECS",
           "uniform_plan", "beam_plan", "prefix_plan", "multi_query_plan",
           "make_plan", "build_inputs", "make_inputs", "to_host_numpy",
           "TORCH_DTYPE"]

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}

# Scales of the fp8 caches: distinct, and not powers of two.
FP8_K_SCALE = 0.02
FP8_V_SCALE = 0.03


def fp8_scales(cache_dtype: Optional[str]) -> dict:
    """Spec keyword arguments for the cache scales of ``cache_dtype``."""
    if cache_dtype == "fp8":
        return dict(k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    return dict(k_scale=1.0, v_scale=1.0)


@dataclass(frozen=True)
class Spec:
    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                  # query / output / new-token element type
    seed: int
    q_std: float = 1.0
    kv_dtype: Optional[str] = None   # cache element type (None: same as dtype)
    k_scale: float = 1.0             # fp8 caches: a K code stands for value * k_scale,
    v_scale: float = 1.0             # a V code for value * v_scale
    recipe: Optional[str] = None     # plan recipe (None: the name)

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype


SPECS: Dict[str, Spec] = {
    "tiny": Spec("tiny", 4, 4, 64, 16, "f32", seed=101),
    "llama7b": Spec("llama7b", 32, 32, 128, 16, "bf16", seed=102),
    "llama13b": Spec("llama13b", 40, 40, 128, 16, "bf16", seed=103),
    "gqa70b": Spec("gqa70b", 64, 8, 128, 32, "bf16", seed=104, q_std=0.5),
    "beam": Spec("beam", 32, 8, 128, 16, "bf16", seed=105),
    "specdec70b": Spec("specdec70b", 64, 8, 128, 16, "bf16", seed=106),
    "chunked13b": Spec("chunked13b", 40, 40, 128, 16, "bf16", seed=107),
}
for _base in ("llama7b", "llama13b", "gqa70b", "beam", "specdec70b", "chunked13b"):
    _b = SPECS[_base]
    SPECS[_base + "_fp8"] = Spec(_base + "_fp8", _b.num_heads, _b.num_kv_heads, _b.head_dim,
                                 _b.block_size, _b.dtype, seed=_b.seed + 1000, q_std=_b.q_std,
                                 kv_dtype="fp8", recipe=_base, **fp8_scales("fp8"))


@dataclass
class Plan:
    """Integer structure of one decode step (host side)."""

    block_size: int
    num_blocks: int
    context_lens: np.ndarray            # int32 [S]
    block_tables: np.ndarray            # int32 [S, MB], tables used by decode
    history_tables: np.ndarray          # int32 [S, MB], tables before copy-on-write
    new_token_seqs: np.ndarray          # int64 [T], sequence of each new token
    slot_mapping: np.ndarray            # int64 [T]
    block_pairs: np.ndarray             # int64 [P, 2] (src, dst)
    shared_prefix_blocks: List[int] = field(default_factory=list)
    query_lens: Optional[np.ndarray] = None  # int32 [S] new queries per sequence (None: decode)

    @property
    def query_start(self) -> Optional[np.ndarray]:
        """int32 [S + 1] CSR offsets of each sequence's query rows (multi-query plans)."""
        if self.query_lens is None:
            return None
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


def _pool_size(needed: int, pool_factor: float, num_blocks: Optional[int]) -> int:
    if num_blocks is not None:
        if num_blocks < needed:
            raise ValueError("pool smaller than the blocks needed")
        return num_blocks
    return max(1, math.ceil(pool_factor * needed))


def uniform_plan(context_lens: Sequence[int], block_size: int, gen: torch.Generator,
                 new_tokens: bool, pool_factor: float = 1.1,
                 num_blocks: Optional[int] = None, shuffle_tokens: bool = False,
                 table_width: Optional[int] = None) -> Plan:
    """Independent sequences with the given context lengths.

    With ``new_tokens`` every sequence with a non-empty context gets its newest
    token (position ctx - 1) stored by the step; ``shuffle_tokens`` puts the
    new tokens in a seeded random order.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    per_seq = [BlockTable.blocks_for(int(c), block_size) for c in ctx]
    nb = _pool_size(sum(per_seq), pool_factor, num_blocks)
    order = torch.randperm(nb, generator=gen).tolist()
    pool = BlockPool(nb, order)
    tables = []
    for c in ctx:
        t = BlockTable(pool, block_size)
        t.ensure_tokens(int(c))
        tables.append(t)
    width = max(1, max(per_seq, default=1)) if table_width is None else table_width
    rows = np.asarray(padded_rows([t.blocks for t in tables], width), dtype=np.int32)
    seqs = [s for s in range(len(ctx)) if ctx[s] > 0] if new_tokens else []
    if shuffle_tokens and seqs:
        perm = torch.randperm(len(seqs), generator=gen).tolist()
        seqs = [seqs[i] for i in perm]
    slots = [tables[s].slot_of(int(ctx[s]) - 1) for s in seqs]
    return Plan(block_size, nb, ctx.astype(np.int32), rows, rows.copy(),
                np.asarray(seqs, dtype=np.int64), np.asarray(slots, dtype=np.int64),
                np.zeros((0, 2), dtype=np.int64))


def beam_plan(groups: int, beams: int, prefix_len: int, tail_lo: int, tail_hi: int,
              block_size: int, cow_fraction: float, gen: torch.Generator,
              pool_factor: float = 1.1) -> Plan:
    """Beam groups sharing a prefix, with copy-on-write of shared last blocks."""
    n = groups * beams
    tails = torch.randint(tail_lo, tail_hi + 1, (n,), generator=gen).tolist()
    ctx = [prefix_len + t for t in tails]
    # The new token sits at position ctx - 1; its block already holds tokens
    # unless the token opens a new block.
    partial = [i for i in range(n) if (ctx[i] - 1) % block_size != 0
               and (ctx[i] - 1) >= prefix_len]
    n_cow = int(round(cow_fraction * len(partial)))
    pick = torch.randperm(len(partial), generator=gen)[:n_cow].tolist()
    cow_seqs = sorted(partial[i] for i in pick)

    prefix_blocks = BlockTable.blocks_for(prefix_len, block_size)
    tail_blocks = sum(BlockTable.blocks_for(c, block_size) - prefix_blocks for c in ctx)
    needed = groups * prefix_blocks + tail_blocks + n_cow
    nb = _pool_size(needed, pool_factor, None)
    pool = BlockPool(nb, torch.randperm(nb, generator=gen).tolist())

    tables: List[BlockTable] = []
    shared = []
    for g in range(groups):
        first = BlockTable(pool, block_size)
        first.ensure_tokens(prefix_len)
        shared.extend(first.blocks)
        members = [first] + [first.fork() for _ in range(beams - 1)]
        for b, t in enumerate(members):
            t.ensure_tokens(ctx[g * beams + b])
        tables.extend(members)
    # A sibling forked earlier still holds the last block of the chosen beams.
    for s in cow_seqs:
        pool.incref(tables[s].blocks[-1])
    width = max(len(t.blocks) for t in tables)
    history = np.asarray(padded_rows([t.blocks for t in tables], width), dtype=np.int32)
    pairs = []
    for s in range(n):
        cp = tables[s].prepare_write((ctx[s] - 1) // block_size)
        if cp is not None:
            pairs.append(cp)
    rows = np.asarray(padded_rows([t.blocks for t in tables], width), dtype=np.int32)
    slots = [tables[s].slot_of(ctx[s] - 1) for s in range(n)]
    return Plan(block_size, nb, np.asarray(ctx, dtype=np.int32), rows, history,
                np.arange(n, dtype=np.int64), np.asarray(slots, dtype=np.int64),
                np.asarray(pairs, dtype=np.int64).reshape(-1, 2), shared)


def prefix_plan(groups: Sequence[Tuple[int, Sequence[int]]], block_size: int,
                gen: torch.Generator, pool_factor: float = 1.1) -> Plan:
    """Groups of sequences forked from one prompt, consecutive in the batch.

    ``groups`` lists ``(prefix_len, [context_len of each member])``; the first
    member's ``prefix_len`` tokens (a multiple of ``block_size``) are shared by
    the forks, each member then grows its own tail.  Every member whose context
    extends past the prefix stores its newest token in a block of its own.
    """
    counts = []
    for prefix_len, ctxs in groups:
        if prefix_len % block_size or any(c < prefix_len for c in ctxs) or not ctxs:
            raise ValueError("prefix must be whole blocks and no longer than any member")
        pb = prefix_len // block_size
        counts.append(pb + sum(BlockTable.blocks_for(int(c), block_size) - pb for c in ctxs))
    nb = _pool_size(sum(counts), pool_factor, None)
    pool = BlockPool(nb, torch.randperm(nb, generator=gen).tolist())
    tables: List[BlockTable] = []
    shared: List[int] = []
    ctx: List[int] = []
    for prefix_len, ctxs in groups:
        first = BlockTable(pool, block_size)
        first.ensure_tokens(prefix_len)
        if len(ctxs) > 1:
            shared.extend(first.blocks)
        members = [first] + [first.fork() for _ in ctxs[1:]]
        for t, c in zip(members, ctxs):
            t.ensure_tokens(int(c))
        tables.extend(members)
        ctx.extend(int(c) for c in ctxs)
    width = max(1, max(len(t.blocks) for t in tables))
    rows = np.asarray(padded_rows([t.blocks for t in tables], width), dtype=np.int32)
    prefix_of = [p for p, ctxs in groups for _ in ctxs]
    seqs = [s for s in range(len(ctx)) if ctx[s] > prefix_of[s]]
    slots = [tables[s].slot_of(ctx[s] - 1) for s in seqs]
    return Plan(block_size, nb, np.asarray(ctx, dtype=np.int32), rows, rows.copy(),
                np.asarray(seqs, dtype=np.int64), np.asarray(slots, dtype=np.int64),
                np.zeros((0, 2), dtype=np.int64), shared)


def multi_query_plan(context_lens: Sequence[int], query_lens: Sequence[int], block_size: int,
                     gen: torch.Generator, pool_factor: float = 1.1) -> Plan:
    """Independent sequences each ending with ``query_lens[s]`` new tokens.

    The new tokens (positions ctx - q_len .. ctx - 1 of each sequence) are
    stored by the step, sequence by sequence in position order, which is also
    the order of the query rows.
    """
    ctx = [int(c) for c in context_lens]
    qlens = [int(n) for n in query_lens]
    if len(ctx) != len(qlens) or any(n > c or n < 0 for c, n in zip(ctx, qlens)):
        raise ValueError("every sequence needs 0 <= query_len <= context_len")
    per_seq = [BlockTable.blocks_for(c, block_size) for c in ctx]
    nb = _pool_size(sum(per_seq), pool_factor, None)
    pool = BlockPool(nb, torch.randperm(nb, generator=gen).tolist())
    tables = []
    for c in ctx:
        t = BlockTable(pool, block_size)
        t.ensure_tokens(c)
        tables.append(t)
    rows = np.asarray(padded_rows([t.blocks for t in tables], max(1, max(per_seq, default=1))),
                      dtype=np.int32)
    seqs = [s for s in range(len(ctx)) for _ in range(qlens[s])]
    slots = [tables[s].slot_of(pos) for s in range(len(ctx)) for pos in range(ctx[s] - qlens[s], ctx[s])]
    return Plan(block_size, nb, np.asarray(ctx, dtype=np.int32), rows, rows.copy(),
                np.asarray(seqs, dtype=np.int64), np.asarray(slots, dtype=np.int64),
                np.zeros((0, 2), dtype=np.int64), query_lens=np.asarray(qlens, dtype=np.int32))


def make_plan(name: str, gen: torch.Generator, **kw) -> Plan:
    """The integer plan of a named workload (keyword overrides shrink it)."""
    spec = SPECS[name]
    bs = kw.pop("block_size", spec.block_size)
    name = spec.recipe or name
    if name == "tiny":
        plan = uniform_plan(kw.pop("context_lens", [1, 17, 33, 100]), bs, gen,
                            new_tokens=True, num_blocks=kw.pop("num_blocks", 64))
    elif name == "llama7b":
        s = kw.pop("num_seqs", 64)
        lo, hi = kw.pop("ctx_range", (128, 2048))
        ctx = torch.randint(lo, hi + 1, (s,), generator=gen).tolist()
        plan = uniform_plan(ctx, bs, gen, new_tokens=kw.pop("new_tokens", False))
    elif name == "llama13b":
        s = kw.pop("num_seqs", 128)
        c = kw.pop("context_len", 2048)
        plan = uniform_plan([c] * s, bs, gen, new_tokens=True, shuffle_tokens=True)
    elif name == "gqa70b":
        s = kw.pop("num_seqs", 16)
        c = kw.pop("context_len", 32768)
        plan = uniform_plan([c] * s, bs, gen, new_tokens=kw.pop("new_tokens", False))
    elif name == "specdec70b":
        s = kw.pop("num_seqs", 32)
        lo, hi = kw.pop("ctx_range", (1024, 8192))
        ctx = torch.randint(lo, hi + 1, (s,), generator=gen).tolist()
        plan = multi_query_plan(ctx, [kw.pop("query_len", 6)] * s, bs, gen)
    elif name == "chunked13b":
        chunks = kw.pop("chunks", [(2048, 2048), (0, 1024)])  # (history, new tokens)
        s = kw.pop("num_decodes", 64)
        lo, hi = kw.pop("ctx_range", (128, 4096))
        dec = torch.randint(lo, hi + 1, (s,), generator=gen).tolist()
        plan = multi_query_plan([h + n for h, n in chunks] + dec, [n for _, n in chunks] + [1] * s,
                                bs, gen)
    elif name == "beam":
        plan = beam_plan(kw.pop("groups", 32), kw.pop("beams", 4),
                         kw.pop("prefix_len", 1024), kw.pop("tail_lo", 1),
                         kw.pop("tail_hi", 256), bs, kw.pop("cow_fraction", 0.1), gen)
    else:
        raise KeyError(name)
    if kw:
        raise TypeError(f"unknown overrides for {name}: {sorted(kw)}")
    return plan


@dataclass
class Inputs:
    spec: Spec
    plan: Plan
    q: torch.Tensor              # [S, H, D]
    k_cache: torch.Tensor        # [NB, Hkv, BS, D]
    v_cache: torch.Tensor
    key: torch.Tensor            # [T, Hkv, D]
    value: torch.Tensor
    slot_mapping: torch.Tensor   # int64 [T]
    block_tables: torch.Tensor   # int32 [S, MB]
    context_lens: torch.Tensor   # int32 [S]
    block_pairs: torch.Tensor    # int64 [P, 2]
    scale: float
    k_scale: float = 1.0         # fp8 caches only
    v_scale: float = 1.0
    query_start: Optional[torch.Tensor] = None  # int32 [S + 1] (multi-query plans)

    @property
    def max_context_len(self) -> int:
        return self.plan.max_context_len


def _randn(shape, gen, device, std, dtype, chunk_rows: int = 1024):
    """N(0, std^2) values drawn in float32 and rounded to ``dtype``."""
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1] = x.to(out.dtype)
    return out


def _fp8_codes(shape, gen, device, scale, chunk_rows: int = 256):
    """E4M3 codes of N(0, 1) / scale draws (torch's float8_e4m3fn cast)."""
    out = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device, dtype=torch.float32)
        flat[r0:r1] = x.mul_(1.0 / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return out


def _history_mask(plan: Plan) -> np.ndarray:
    """[NB, BS] True where a slot holds a token before the step's writes."""
    mask = np.zeros((plan.num_blocks, plan.block_size), dtype=bool)
    written = {}
    for s in plan.new_token_seqs.tolist():
        written[s] = written.get(s, 0) + 1
    bs = plan.block_size
    for s in range(plan.num_seqs):
        n = int(plan.context_lens[s]) - written.get(s, 0)
        row = plan.history_tables[s]
        full, rest = divmod(n, bs)
        for j in range(full):
            mask[row[j], :] = True
        if rest:
            mask[row[full], :rest] = True
    return mask


def build_inputs(spec: Spec, plan: Plan, device="cpu", poison: bool = True) -> Inputs:
    """Random tensors for ``plan`` on ``device`` (seeded by the spec).

    q has one row per sequence, or one per new query token for a multi-query
    plan.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed * 7919 + 17)
    s = plan.num_seqs if plan.query_lens is None else int(plan.query_lens.sum())
    nb, bs = plan.num_blocks, plan.block_size
    hkv, d = spec.num_kv_heads, spec.head_dim
    q = _randn((s, spec.num_heads, d), gen, device, spec.q_std, spec.dtype)
    if spec.cache_dtype == "fp8":
        k_cache = _fp8_codes((nb, hkv, bs, d), gen, device, spec.k_scale)
        v_cache = _fp8_codes((nb, hkv, bs, d), gen, device, spec.v_scale)
    else:
        k_cache = _randn((nb, hkv, bs, d), gen, device, 1.0, spec.dtype, chunk_rows=256)
        v_cache = _randn((nb, hkv, bs, d), gen, device, 1.0, spec.dtype, chunk_rows=256)
    t = int(plan.slot_mapping.shape[0])
    key = _randn((max(t, 1), hkv, d), gen, device, 1.0, spec.dtype)[:t]
    value = _randn((max(t, 1), hkv, d), gen, device, 1.0, spec.dtype)[:t]
    empty = torch.from_numpy(~_history_mask(plan)).to(device)
    if spec.cache_dtype == "fp8":  # 0x7F is the E4M3 NaN code
        for c in (k_cache, v_cache):
            c.view(torch.uint8).masked_fill_(empty[:, None, :, None], 0x7F if poison else 0)
    else:
        fill = float("nan") if poison else 0.0
        k_cache.masked_fill_(empty[:, None, :, None], fill)
        v_cache.masked_fill_(empty[:, None, :, None], fill)
    return Inputs(
        spec=spec, plan=plan, q=q, k_cache=k_cache, v_cache=v_cache,
        key=key.contiguous(), value=value.contiguous(),
        slot_mapping=torch.from_numpy(plan.slot_mapping.copy()).to(device),
        block_tables=torch.from_numpy(plan.block_tables.copy()).to(device),
        context_lens=torch.from_numpy(plan.context_lens.copy()).to(device),
        block_pairs=torch.from_numpy(plan.block_pairs.copy()).to(device),
        scale=float(np.float32(1.0 / math.sqrt(d))),
        k_scale=spec.k_scale if spec.cache_dtype == "fp8" else 1.0,
        v_scale=spec.v_scale if spec.cache_dtype == "fp8" else 1.0,
        query_start=None if plan.query_lens is None
        else torch.from_numpy(plan.query_start).to(device),
    )


def make_inputs(name: str, device="cpu", poison: bool = True, **overrides) -> Inputs:
    """Plan and tensors of a named workload; ``overrides`` shrink the plan."""
    spec = SPECS[name]
    if "block_size" in overrides:
        spec = Spec(**{**spec.__dict__, "block_size": overrides["block_size"]})
    gen = torch.Generator()
    gen.manual_seed(spec.seed)
    plan = make_plan(name, gen, **overrides)
    return build_inputs(spec, plan, device=device, poison=poison)


def to_host_numpy(t: torch.Tensor) -> np.ndarray:
    """Host NumPy view of a tensor: bf16 as uint16 bit patterns, fp8 as uint8 codes."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
