#!/usr/bin/env python3
"""Benchmark of one decode step over a paged KV cache on one MI355X.

A step is one pass of the whole path over one batch: copy_blocks (when the
workload has copy-on-write pairs), reshape_and_cache of the new tokens (when
it has any), then pa_decode.  Inputs are generated on the device before the
timed region.  The headline workload is the LLaMA-13B-shaped layer: 128
sequences at context 2048, 40 heads, head_dim 128, block size 16, bf16, with
128 new tokens stored through a shuffled slot mapping.

Printed: one JSON line with tokens/s per layer (value), the decode kernel's
roofline (algorithmic HBM bytes / measured launch time against 8 TB/s), the
oracle timed on the host cores on a bounded sample (cpu_baseline), and the
other workloads' figures under "workloads".
"""

from __future__ import annotations

import argparse
import hashlib
from concurrent.futures import ThreadPoolExecutor
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "paged-attn decode tokens/s per layer + achieved HBM GB/s (% of peak), 1 GPU"
PEAK_GBPS = 8000.0  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(HERE, "profiles", "decode_traffic.json")
# Sources that determine the attention kernels; a workload's counter record
# is valid only for the exact text of the sources its kernels are built from.
DECODE_SRCS = ("pa_device.h", "pa_mfma.h", "pa_decode.hip", "pa_decode_valu.hip", "pa_decode_mfma.hip")
MULTI_QUERY_SRCS = DECODE_SRCS + ("pa_lds_dma.h", "pa_multi_query.hip")

DESCRIPTION = {
    "llama13b": "LLaMA-13B-shaped layer decode: 128 seqs x ctx 2048, H=Hkv=40, D=128, BS=16, bf16, "
                "reshape_and_cache of 128 new tokens + pa_decode",
    "llama7b": "LLaMA-7B-shaped layer decode: 64 seqs, ctx U[128,2048], H=Hkv=32, D=128, BS=16, bf16",
    "gqa70b": "GQA 70B-shaped long-context decode: 16 seqs x ctx 32768, H=64, Hkv=8, D=128, BS=32, bf16",
    "beam": "beam decode with copy-on-write: 32 groups x 4 beams, shared 1024-token prefix + tails "
            "U[1,256], H=32, Hkv=8, D=128, BS=16, bf16; copy_blocks + reshape_and_cache + pa_decode",
    "tiny": "tiny paged decode: 4 seqs ctx {1,17,33,100}, H=Hkv=4, D=64, BS=16, fp32",
}
DESCRIPTION.update({
    "specdec70b": "speculative verification, 70B GQA shape: 32 seqs, ctx U[1024,8192] ending with 6 new "
                  "tokens each, H=64, Hkv=8, D=128, BS=16, bf16; reshape_and_cache + pa_multi_query",
    "chunked13b": "chunked-prefill batch, LLaMA-13B shape: a 2048-token chunk after 2048 cached tokens, "
                  "a first 1024-token chunk and 64 decodes (ctx U[128,4096]), 3136 query tokens, "
                  "H=Hkv=40, D=128, BS=16, bf16; reshape_and_cache + pa_multi_query",
})
for _n in ("llama7b", "llama13b", "gqa70b", "beam", "specdec70b", "chunked13b"):
    DESCRIPTION[_n + "_fp8"] = DESCRIPTION[_n].replace(", bf16", ", bf16 query / fp8 E4M3 KV cache")
# Variants of a workload's plan: (base workload, plan overrides).
# Two long sequences of the GQA 70B shape have too few (sequence, kv head,
# partition) workgroups to fill the chip at the fixed partition length;
# "+fill" runs the same step at the batch-shaped length (PA_PARTITION_FILL).
# Verification of 4 drafted tokens over an E4M3 cache (32 rows per sequence):
# the shortest verification rows of the 70B shape.
# "chunked13b_chunks" keeps only the two prefill chunks of the chunked-prefill
# batch (no decode rows, so no side-stream launch): the multi-query tile
# kernel alone, compute-bound.
VARIANTS = {"gqa70b_x2": ("gqa70b", {"num_seqs": 2}), "gqa70b_fp8_x2": ("gqa70b_fp8", {"num_seqs": 2}),
            "specdec70b_fp8_q4": ("specdec70b_fp8", {"query_len": 4}),
            "chunked13b_chunks": ("chunked13b", {"num_decodes": 0}),
            "chunked13b_fp8_chunks": ("chunked13b_fp8", {"num_decodes": 0})}
for _n in ("gqa70b_x2", "gqa70b_fp8_x2"):
    DESCRIPTION[_n] = DESCRIPTION[VARIANTS[_n][0]].replace("16 seqs", "2 seqs") + ", fixed partitions"
    DESCRIPTION[_n + "+fill"] = DESCRIPTION[_n].replace("fixed partitions", "batch-shaped partitions")
DESCRIPTION["specdec70b_fp8_q4"] = DESCRIPTION["specdec70b_fp8"].replace("6 new tokens", "4 new tokens")
for _n in ("chunked13b", "chunked13b_fp8"):
    DESCRIPTION[_n + "_chunks"] = DESCRIPTION[_n].replace(
        " and 64 decodes (ctx U[128,4096]), 3136 query tokens", ", 3072 query tokens, no decodes")
DESCRIPTION["swap13b"] = ("swap_blocks of 1024 random blocks of the LLaMA-13B-shaped pool (Hkv=40, BS=16, "
                          "D=128, bf16: 320 KiB of K+V per block) to pinned host memory and back")
# "+prefix": the same step with pa_decode_shared_prefix (each shared page read
# once per chunk of sequences) in place of pa_decode.
for _n in ("beam", "beam_fp8"):
    DESCRIPTION[_n + "+prefix"] = DESCRIPTION[_n].replace("+ pa_decode", "+ pa_decode_shared_prefix")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama13b",
                    choices=sorted(n for n in DESCRIPTION if n != "swap13b"))
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--cold", action="store_true",
                    help="flush the MALL between the timed steps of --workload (as for the beam cold rows)")
    ap.add_argument("--others", default="tiny,llama7b,gqa70b,beam,beam+prefix,llama13b_fp8,gqa70b_fp8,"
                                        "beam_fp8+prefix,specdec70b,specdec70b_fp8,specdec70b_fp8_q4,"
                                        "chunked13b,chunked13b_chunks,gqa70b_x2,gqa70b_x2+fill,swap13b",
                    help="comma list of extra workloads to report ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cache-ops", dest="cache_ops", action="store_false",
                    help="skip the separate timing of reshape_and_cache and copy_blocks")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter scaling)")
    return ap.parse_args()


def algorithmic_bytes(plan, spec) -> int:
    """K and V read once + q read + out written + block-table entries + context lengths
    (+ query offsets for a multi-query plan, whose q/out have one row per query token)."""
    e = 4 if spec.dtype == "f32" else 2
    ekv = {"f32": 4, "bf16": 2, "fp8": 1}[spec.cache_dtype]
    ctx = [int(c) for c in plan.context_lens]
    kv = sum(2 * spec.num_kv_heads * c * spec.head_dim * ekv for c in ctx)
    rows = len(ctx) if plan.query_lens is None else int(plan.query_lens.sum())
    qo = 2 * rows * spec.num_heads * spec.head_dim * e
    if plan.query_lens is not None:
        qo += 4 * (len(ctx) + 1)
    table = 4 * sum(-(-c // plan.block_size) for c in ctx)
    return kv + qo + table + 4 * len(ctx)


def attention_flops(plan, spec) -> int:
    """Multiply-adds x 2 of the causal attention: each query row at position p
    and each query head does 2*D for q.k and 2*D for p*V over p + 1 tokens."""
    total = 0
    qlens = plan.query_lens if plan.query_lens is not None else [1] * plan.num_seqs
    for c, n in zip(plan.context_lens.tolist(), list(qlens)):
        c, n = int(c), int(n)
        seen = sum(c - n + i + 1 for i in range(n))
        total += 4 * spec.head_dim * spec.num_heads * seen
    return total


def decode_kernel_name(label, spec) -> str:
    """The partition kernel a workload's decode launches (the dominant kernel)."""
    group = spec.num_heads // spec.num_kv_heads
    cache = {"f32": "f32", "bf16": "bf16", "fp8": "fp8 E4M3"}[spec.cache_dtype]
    shape = f"D={spec.head_dim}, BS={spec.block_size}, G={group}"
    if spec.recipe in ("specdec70b", "chunked13b") or label.startswith(("specdec70b", "chunked13b")):
        return f"pa_multi_query: multi_query_kernel<{cache} cache, {shape}>"
    if label.endswith("+prefix"):
        return f"pa_decode_shared_prefix: decode_partition_mfma_kernel<{cache} cache, {shape}, shared>"
    if spec.dtype == "bf16" and group >= 2:
        return f"pa_decode: decode_partition_mfma_kernel<{cache} cache, {shape}>"
    return f"pa_decode: decode_partition_valu_kernel<{spec.dtype} q, {cache} cache, {shape}>"


def unique_bytes(plan, spec) -> int:
    """Like algorithmic_bytes, but a physical block shared by several sequences
    counts once (with the most tokens any of them uses from it): the K/V bytes
    HBM has to deliver when each page is fetched once per call."""
    ekv = {"f32": 4, "bf16": 2, "fp8": 1}[spec.cache_dtype]
    bs = plan.block_size
    used = {}
    ctx = [int(c) for c in plan.context_lens]
    for s, c in enumerate(ctx):
        for j in range(-(-c // bs)):
            b = int(plan.block_tables[s][j])
            used[b] = max(used.get(b, 0), min(bs, c - j * bs))
    kv_unique = 2 * spec.num_kv_heads * spec.head_dim * ekv * sum(used.values())
    kv_logical = sum(2 * spec.num_kv_heads * c * spec.head_dim * ekv for c in ctx)
    return algorithmic_bytes(plan, spec) - kv_logical + kv_unique


def kernel_sources(workload: str):
    """Source files of the kernels a workload's attention call runs."""
    names = MULTI_QUERY_SRCS if workload.split("_")[0].split("+")[0] in ("specdec70b", "chunked13b") \
        else DECODE_SRCS
    return [os.path.join(HERE, "paged_kv_cache_321_amd", "csrc", n) for n in names]


def kernel_hash(workload: str) -> str:
    h = hashlib.sha256()
    for path in kernel_sources(workload):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode launch from rocprofv3 counters, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_sha256_16") != kernel_hash(workload):
        return None
    return entry.get("bytes_per_launch")


def run_workload(label, steps, warmup, partition_tokens, flush=False, settle_s=0.0):
    import torch
    from paged_kv_cache_321_amd import binding
    from paged_kv_cache_321_amd import workloads as wl
    from paged_kv_cache_321_amd.block_pool import prefix_bounds, prefix_groups

    name, _, variant = label.partition("+")
    shared_prefix = variant == "prefix"
    if name in VARIANTS:
        x = wl.make_inputs(VARIANTS[name][0], device="cuda", poison=False, **VARIANTS[name][1])
    else:
        x = wl.make_inputs(name, device="cuda", poison=False)
    spec, plan = x.spec, x.plan
    out = torch.empty_like(x.q)
    code = binding.PA_F32 if spec.dtype == "f32" else binding.PA_BF16
    ccode = {"f32": binding.PA_F32, "bf16": binding.PA_BF16,
             "fp8": binding.PA_FP8_E4M3}[spec.cache_dtype]
    if shared_prefix:  # grouping and bounds from the host-side tables, before the timed region
        lead, nblk = prefix_groups(plan.block_tables, plan.context_lens, plan.block_size)
        bounds = prefix_bounds(lead, nblk, plan.context_lens, plan.block_size)
        lead = torch.tensor(lead, dtype=torch.int32, device="cuda")
        nblk = torch.tensor(nblk, dtype=torch.int32, device="cuda")
        ws_bytes = binding.pa_decode_shared_prefix_workspace_size(
            plan.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim, plan.block_size,
            plan.max_context_len, bounds[0], bounds[1], code, partition_tokens, ccode)
    else:
        if variant == "fill":
            partition_tokens = binding.pa_decode_partition_tokens(
                plan.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim, plan.block_size,
                plan.max_context_len, code, ccode, policy=binding.PA_PARTITION_FILL)
        ws_bytes = binding.pa_decode_workspace_size(
            plan.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim, plan.block_size,
            plan.max_context_len, code, partition_tokens, ccode)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if flush else None
    stream = torch.cuda.current_stream()
    multi_query = plan.query_lens is not None
    if multi_query:
        ws_bytes = binding.pa_multi_query_workspace_size(
            plan.num_seqs, int(plan.query_lens.sum()), spec.num_heads, spec.num_kv_heads, spec.head_dim,
            plan.block_size, plan.max_context_len, code, partition_tokens, ccode)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        max_q = int(plan.query_lens.max())
        # No single-query sequence in the batch: no decode launch.
        tiles_only = int(plan.query_lens.min()) > 1
    has_pairs = plan.block_pairs.shape[0] > 0
    has_tokens = plan.slot_mapping.shape[0] > 0
    # Workloads whose sequences share physical blocks (beam prefixes) ask for
    # the default cache policy so later readers of a shared page hit in cache.
    shared = bool(plan.shared_prefix_blocks)
    # Dispatch order from the host-side lengths: longest contexts first, except
    # when sequences share pages (beams of a group stay adjacent, so a shared
    # page is still cached when the next beam reads it).
    order = None if shared else binding.longest_first(plan.context_lens)

    def step(ev=None):
        if has_pairs:
            binding.pa_copy_blocks(x.k_cache, x.v_cache, x.block_pairs, stream=stream)
        if has_tokens:
            binding.pa_reshape_and_cache(x.key, x.value, x.k_cache, x.v_cache, x.slot_mapping,
                                         stream=stream, k_scale=x.k_scale, v_scale=x.v_scale)
        if ev is not None:
            ev[0].record(stream)
        if multi_query:
            binding.pa_multi_query(out, x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens,
                                   x.query_start, x.scale, plan.max_context_len, max_q,
                                   partition_tokens=partition_tokens, workspace=ws, stream=stream,
                                   k_scale=x.k_scale, v_scale=x.v_scale, tiles_only=tiles_only)
        elif shared_prefix:
            binding.pa_decode_shared_prefix(out, x.q, x.k_cache, x.v_cache, x.block_tables,
                                            x.context_lens, lead, nblk, x.scale,
                                            plan.max_context_len, bounds[0], bounds[1],
                                            partition_tokens=partition_tokens,
                                            workspace=ws, stream=stream, k_scale=x.k_scale,
                                            v_scale=x.v_scale)
        else:
            binding.pa_decode(out, x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens,
                              x.scale, plan.max_context_len, partition_tokens=partition_tokens,
                              workspace=ws, stream=stream, shared_pages=shared, seq_order=order,
                              k_scale=x.k_scale, v_scale=x.v_scale)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Further untimed steps until settle_s seconds have passed (0 for the
    # headline workload, which takes exactly the requested warmup): a freshly
    # built pool and a GPU that idled while it was built run their first tens
    # of milliseconds slower.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle_s:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    wall = 0.0
    if flush:
        # Cold cache: the scratch write between steps evicts the 256 MiB MALL;
        # only the step itself (between the events) is timed.
        for i in range(steps):
            scratch.fill_(i & 0xFF)
            events[i][2].record(stream)
            step((events[i][0], events[i][1]))
            events[i][3].record(stream)
        torch.cuda.synchronize()
        step_ms = [a[2].elapsed_time(a[3]) for a in events]
        ms_per_step = sum(step_ms) / steps
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        events[0][2].record(stream)
        for i in range(steps):
            step((events[i][0], events[i][1]))
        events[-1][3].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = events[0][2].elapsed_time(events[-1][3]) / steps
    decode_ms = [a[0].elapsed_time(a[1]) for a in events]
    decode_ms.sort()
    avg_decode_ms = sum(decode_ms) / len(decode_ms)
    med_decode_ms = decode_ms[len(decode_ms) // 2]
    p10_decode_ms = decode_ms[(len(decode_ms) - 1) // 10]
    p90_decode_ms = decode_ms[(len(decode_ms) - 1) * 9 // 10]
    nbytes = algorithmic_bytes(plan, spec)
    ubytes = unique_bytes(plan, spec)
    flops = attention_flops(plan, spec)
    ntok = int(plan.query_lens.sum()) if multi_query else plan.num_seqs
    res = {
        "workload": label,
        "description": DESCRIPTION[label],
        "num_seqs": plan.num_seqs,
        "partition_tokens": partition_tokens,
        "total_context_tokens": int(sum(int(c) for c in plan.context_lens)),
        "ms_per_step": ms_per_step,
        "wall_ms_per_step": wall * 1e3 / steps if wall else None,
        "tokens_per_s": ntok / (ms_per_step / 1e3),
        "decode_avg_us": avg_decode_ms * 1e3,
        "decode_median_us": med_decode_ms * 1e3,
        "decode_p10_us": p10_decode_ms * 1e3,
        "decode_p90_us": p90_decode_ms * 1e3,
        "decode_tokens_per_s": ntok / (avg_decode_ms / 1e3),
        "attention_flops": flops,
        "attention_TFLOPs": flops / (avg_decode_ms / 1e3) / 1e12,
        "decode_algorithmic_bytes": nbytes,
        # The HBM rate counts each physical page once per call (unique bytes:
        # a page that several sequences share is fetched from HBM once); the
        # logical rate counts it once per sequence that reads it.  They are
        # equal unless sequences share pages.
        "decode_GBps": ubytes / (avg_decode_ms / 1e3) / 1e9,
        "decode_frac_of_peak": ubytes / (avg_decode_ms / 1e3) / 1e9 / PEAK_GBPS,
        "decode_unique_bytes": ubytes,
        "decode_logical_GBps": nbytes / (avg_decode_ms / 1e3) / 1e9,
        "copy_pairs": int(plan.block_pairs.shape[0]),
        "new_tokens": int(plan.slot_mapping.shape[0]),
        "partition_tokens": partition_tokens,
        "shared_pages_flag": shared and not shared_prefix,
        "decode_entry_point": ("pa_multi_query" if multi_query else
                               "pa_decode_shared_prefix" if shared_prefix else "pa_decode"),
        "query_tokens": ntok,
        "cache": "cold (MALL flushed between steps)" if flush else "warm",
        "kv_cache_dtype": spec.cache_dtype,
    }
    del x, out, ws, scratch
    torch.cuda.empty_cache()
    return res, spec, plan


PCIE_GBPS = 64.0  # PCIe 5.0 x16, one direction, published


def run_swap(label, steps, warmup, blocks=1024):
    """Swap-out (device -> pinned host) and swap-in of scattered blocks."""
    import torch
    from paged_kv_cache_321_amd import binding
    from paged_kv_cache_321_amd import workloads as wl

    x = wl.make_inputs("llama13b", device="cuda", poison=False)
    nb = x.plan.num_blocks
    shape = (blocks,) + tuple(x.k_cache.shape[1:])
    host_k = torch.empty(shape, dtype=x.k_cache.dtype).pin_memory()
    host_v = torch.empty(shape, dtype=x.k_cache.dtype).pin_memory()
    g = torch.Generator().manual_seed(11)
    dev_ids = torch.randperm(nb, generator=g)[:blocks]
    host_ids = torch.randperm(blocks, generator=g)
    out_pairs = torch.stack([dev_ids, host_ids], 1).to(torch.int64).to("cuda")
    in_pairs = torch.stack([host_ids, dev_ids], 1).to(torch.int64).to("cuda")
    stream = torch.cuda.current_stream()
    res = {"workload": label, "description": DESCRIPTION[label], "blocks": blocks}
    nbytes = 2 * blocks * x.k_cache[0].numel() * x.k_cache.element_size()
    for what, args in (("out", (host_k, host_v, x.k_cache, x.v_cache, out_pairs)),
                       ("in", (x.k_cache, x.v_cache, host_k, host_v, in_pairs))):
        for _ in range(warmup):
            binding.pa_swap_blocks(*args, stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            binding.pa_swap_blocks(*args, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        res[f"swap_{what}_us"] = us
        res[f"swap_{what}_GBps"] = nbytes / (us / 1e6) / 1e9
        res[f"swap_{what}_frac_of_pcie"] = res[f"swap_{what}_GBps"] / PCIE_GBPS
    res["bytes_per_direction"] = nbytes
    del x, host_k, host_v
    torch.cuda.empty_cache()
    return res


def run_cache_ops(steps, warmup):
    """The two cache writes alone, each call between its own pair of events.

    reshape_and_cache of the LLaMA-13B-shaped step's 128 new tokens (bf16, and
    encoded into an E4M3 cache), copy_blocks of the beam workload's
    copy-on-write pairs, and copy_blocks of 1024 scattered LLaMA-13B-shaped
    blocks.  Bytes are the data the op moves: every row or block read once and
    written once (plus the slot or pair indices).
    """
    import torch
    from paged_kv_cache_321_amd import binding
    from paged_kv_cache_321_amd import workloads as wl

    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        # A few milliseconds of GPU spin first, so every call below is queued
        # before the GPU reaches it: the events then time the GPU, not the
        # host's launch latency (these kernels take microseconds).
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(5_000_000)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps * 1e3

    res = []
    for name in ("llama13b", "llama13b_fp8"):
        x = wl.make_inputs(name, device="cuda", poison=False)
        t = x.key.shape[0]
        row = x.key[0].numel()
        nbytes = t * row * 2 * (x.key.element_size() + x.k_cache.element_size()) + 8 * t
        us = timed(lambda: binding.pa_reshape_and_cache(x.key, x.value, x.k_cache, x.v_cache,
                                                        x.slot_mapping, stream=stream,
                                                        k_scale=x.k_scale, v_scale=x.v_scale))
        res.append({"op": "pa_reshape_and_cache", "workload": name, "new_tokens": t,
                    "kv_cache_dtype": x.spec.cache_dtype, "avg_us": us, "bytes": nbytes,
                    "GBps": nbytes / (us / 1e6) / 1e9})
        del x
    x = wl.make_inputs("beam", device="cuda", poison=False)
    pairs = x.block_pairs
    blk = x.k_cache[0].numel() * x.k_cache.element_size()
    nbytes = pairs.shape[0] * 2 * 2 * blk + 16 * pairs.shape[0]
    us = timed(lambda: binding.pa_copy_blocks(x.k_cache, x.v_cache, pairs, stream=stream))
    res.append({"op": "pa_copy_blocks", "workload": "beam", "pairs": int(pairs.shape[0]),
                "avg_us": us, "bytes": nbytes, "GBps": nbytes / (us / 1e6) / 1e9})
    del x
    x = wl.make_inputs("llama13b", device="cuda", poison=False)
    g = torch.Generator().manual_seed(12)
    ids = torch.randperm(x.plan.num_blocks, generator=g)[:2048]
    pairs = torch.stack([ids[:1024], ids[1024:]], 1).to(torch.int64).to("cuda")
    blk = x.k_cache[0].numel() * x.k_cache.element_size()
    nbytes = 1024 * 2 * 2 * blk + 16 * 1024
    us = timed(lambda: binding.pa_copy_blocks(x.k_cache, x.v_cache, pairs, stream=stream))
    res.append({"op": "pa_copy_blocks", "workload": "1024 scattered LLaMA-13B-shaped blocks",
                "pairs": 1024, "avg_us": us, "bytes": nbytes, "GBps": nbytes / (us / 1e6) / 1e9,
                "frac_of_peak": nbytes / (us / 1e6) / 1e9 / PEAK_GBPS})
    # The same bytes as one contiguous device-to-device copy: the rate a copy
    # reaches on this GPU when nothing is scattered.
    src = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    us = timed(lambda: dst.copy_(src))
    res.append({"op": "contiguous device copy (torch copy_)", "bytes": 2 * src.numel(), "avg_us": us,
                "GBps": 2 * src.numel() / (us / 1e6) / 1e9,
                "frac_of_peak": 2 * src.numel() / (us / 1e6) / 1e9 / PEAK_GBPS})
    del x, src, dst
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, target_s):
    """The oracle on a bounded sample of the workload: single-threaded, then
    the same sequence-steps spread over a thread per available core."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    import oracle.paged_attention as op
    from paged_kv_cache_321_amd import workloads as wl
    from paged_kv_cache_321_amd.workloads import to_host_numpy

    x = wl.make_inputs(name, device="cuda", poison=False)
    plan, spec = x.plan, x.spec
    bs = plan.block_size
    # Host copies of each sequence's pages, made once (not timed).
    host = []
    for s in range(plan.num_seqs):
        nb = -(-int(plan.context_lens[s]) // bs)
        idx = torch.tensor([int(b) for b in plan.block_tables[s][:nb]], dtype=torch.long, device="cuda")
        tok = np.nonzero(plan.new_token_seqs == s)[0]
        host.append((to_host_numpy(x.k_cache.index_select(0, idx)).copy(),
                     to_host_numpy(x.v_cache.index_select(0, idx)).copy(),
                     to_host_numpy(x.q[s:s + 1]), nb, plan.context_lens[s:s + 1],
                     (to_host_numpy(x.key[tok[0]:tok[0] + 1]), to_host_numpy(x.value[tok[0]:tok[0] + 1]))
                     if len(tok) else None))
        if s >= 15:  # a bounded sample of sequences, cycled below
            break

    def one(i):
        """The oracle's step for sample item i: store the new token (if any), decode."""
        kc0, vc0, q, nb, ctx, new = host[i % len(host)]
        kc, vc = kc0.copy(), vc0.copy()
        table = np.arange(nb, dtype=np.int32)[None]
        t0 = time.perf_counter()
        if new is not None:
            pos = int(ctx[0]) - 1
            op.reshape_and_cache(new[0], new[1], kc, vc, np.array([pos], dtype=np.int64))
        op.decode(q, kc, vc, table, ctx, x.scale, spec.dtype)
        return time.perf_counter() - t0, int(ctx[0])

    done = 0
    tokens = 0
    t_total = 0.0
    with threadpool_limits(limits=1):
        while t_total < target_s and done < 64 * len(host):
            dt, c = one(done)
            t_total += dt
            tokens += c
            done += 1
    # The same items over a pool of threads, one per available core (BLAS
    # single-threaded inside each), timed by the wall clock around the pool.
    cores = len(os.sched_getaffinity(0))
    n_par = max(cores, min(64 * len(host), int(done * cores * 0.5)))
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        list(ex.map(one, range(n_par)))
        t_par = time.perf_counter() - t0
    n_host = len(host)
    # K and V bytes each sequence-step reads, as counted for the GPU.
    ekv = {"f32": 4, "bf16": 2, "fp8": 1}[spec.cache_dtype]

    def kv_bytes(ctx_tokens):
        return 2 * spec.num_kv_heads * spec.head_dim * ekv * ctx_tokens

    par_tokens = sum(int(host[i % n_host][4][0]) for i in range(n_par))
    del x, host
    torch.cuda.empty_cache()
    return {
        "value": done / t_total,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} sequence-steps cycling over the first {n_host} of the "
                  f"{plan.num_seqs} sequences of the {name} workload ({tokens} context tokens "
                  f"in total): reshape_and_cache of the new token + decode, fp64 NumPy oracle, "
                  f"one BLAS thread, {t_total:.1f} s",
        "seconds": t_total,
        "GBps": kv_bytes(tokens) / t_total / 1e9,
        "threaded": {"value": n_par / t_par, "unit": "tokens/s", "cores": cores,
                     "GBps": kv_bytes(par_tokens) / t_par / 1e9,
                     "sample": f"{n_par} sequence-steps of the same sample over {cores} threads "
                               f"(one BLAS thread each), {t_par:.1f} s wall"},
        "host_cpus_available": cores,
        "cpu_model": _cpu_model(),
    }


def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: the full "model name" field,
    with the vendor and the family / model / stepping numbers beside it."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = ", ".join(f"{k} {fields[k]}" for k in ("vendor_id", "cpu family", "model", "stepping")
                    if k in fields)
    return f"{name} ({ids})" if ids else name


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, for scaling the HBM counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}))


# The five configurations the metric is quoted on, by workload label.
BASELINE_CONFIGS = {"tiny": 1, "llama7b": 2, "llama13b": 3, "gqa70b": 4, "beam": 5, "beam+prefix": 5}


def baseline_summary(head, others):
    """One short entry per run of a configuration of the metric: decode call
    time, decode tokens/s, HBM GB/s (each page once) and its fraction of peak,
    and the whole step's time."""
    rows = []
    for r in [head] + others:
        cfg = BASELINE_CONFIGS.get(r.get("workload"))
        if cfg is None:
            continue
        rows.append({"cfg": cfg, "w": r["workload"] + (" cold" if r["cache"].startswith("cold") else ""),
                     "us": round(r["decode_avg_us"], 1), "tok_s": round(r["decode_tokens_per_s"]),
                     "GBps": round(r["decode_GBps"]), "frac": round(r["decode_frac_of_peak"], 3),
                     "step_us": round(r["ms_per_step"] * 1e3, 1)})
    return sorted(rows, key=lambda e: e["cfg"])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measured on one GPU only (asked for --gpus {args.gpus}); "
              "the decode path needs no collective and is measured at N=1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return

    head, spec, plan = run_workload(args.workload, args.steps, args.warmup, args.partition_tokens,
                                    flush=args.cold)
    others = []
    for name in [n for n in args.others.split(",") if n and n != args.workload]:
        if name == "swap13b":
            others.append(run_swap(name, min(args.steps, 10), min(args.warmup, 2)))
            continue
        r, _, _ = run_workload(name, args.steps, args.warmup, args.partition_tokens, settle_s=0.1)
        r["decode_traffic_bytes"] = measured_traffic(name)
        others.append(r)
        if name.startswith("beam"):
            r2, _, _ = run_workload(name, args.steps, args.warmup, args.partition_tokens, flush=True,
                                    settle_s=0.1)
            others.append(r2)

    cache_ops = run_cache_ops(args.steps, args.warmup) if args.cache_ops else None
    traffic = measured_traffic(args.workload)
    roof = {
        "bound": "hbm",
        "kernel": decode_kernel_name(args.workload, spec),
        "achieved": head["decode_GBps"],
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": head["decode_GBps"] / PEAK_GBPS,
        "traffic": traffic,
        "algorithmic_bytes_per_launch": head["decode_algorithmic_bytes"],
        "avg_launch_us": head["decode_avg_us"],
    }
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload.split("+")[0],
                                                             args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) K/V/Q, shuffled physical blocks; no weights)",
        "config": {
            "workload": DESCRIPTION[args.workload],
            "num_seqs": plan.num_seqs,
            "context_len": plan.max_context_len,
            "num_heads": spec.num_heads,
            "num_kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim,
            "block_size": plan.block_size,
            "num_blocks": plan.num_blocks,
            "new_tokens": head["new_tokens"],
            "parallelism": "single GPU",
        },
        "decode": {k: head[k] for k in ("decode_avg_us", "decode_median_us", "decode_p10_us",
                                        "decode_p90_us", "decode_tokens_per_s", "decode_GBps",
                                        "decode_frac_of_peak")},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cache_ops": cache_ops,
        "workloads": others,
        # Last, so that the tail of the output holds it: the five configurations
        # of the metric, one compact entry per run.
        "configs": baseline_summary(head, others),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
