"""GPU parity of multi-query paged attention (pa_multi_query) against the oracle.

Each case stores the new tokens' K/V with pa_reshape_and_cache (bit-exact
against the oracle's store) and compares the attention output element by
element with oracle.multi_query: atol 5e-3 + rtol 1e-2 (bf16 output).
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_321_amd import binding
from paged_kv_cache_321_amd import workloads as wl

from gpu_helpers import (as_f64, assert_close, bits, gpu_mq_step, gpu_step, on_device,
                         oracle_mq_step, oracle_step, sampled_mq_reference, to_top_of_pool)

pytestmark = pytest.mark.gpu


def check_mq(x, partition_tokens=0, **kw):
    out, t = gpu_mq_step(x, partition_tokens=partition_tokens, **kw)
    ref, kc, vc = oracle_mq_step(x)
    assert np.array_equal(bits(t["k_cache"]), bits(kc))
    assert np.array_equal(bits(t["v_cache"]), bits(vc))
    return assert_close(as_f64(out), ref, "bf16", x.spec.name), out


SMALL = {
    "specdec70b": dict(num_seqs=5, ctx_range=(6, 900)),
    "chunked13b": dict(chunks=[(300, 200), (0, 97)], num_decodes=5, ctx_range=(1, 700)),
}
for _n in list(SMALL):
    SMALL[_n + "_fp8"] = SMALL[_n]


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("pt", [0, 64, 256])
def test_workload_small(name, pt):
    x = wl.make_inputs(name, **SMALL[name])
    check_mq(x, partition_tokens=pt)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("pt", [0, 64])
@pytest.mark.parametrize("chunks", [[(300, 200), (0, 180), (64, 150)], [(0, 97), (10, 90)]])
def test_chunks_only(kv, pt, chunks):
    """Batches of long chunks alone (every sequence more than one 64-row
    block; the shortest provably so from the batch's query count and longest
    query, so no merge is launched): 128-row blocks on the two-tile ring, and
    two 64-row blocks per sequence on the one-tile ring."""
    name = "chunked13b" if kv == "bf16" else "chunked13b_fp8"
    x = wl.make_inputs(name, chunks=chunks, num_decodes=0)
    check_mq(x, partition_tokens=pt, tiles_only=True)


def shape_case(h, hkv, d, bs, kv="bf16", seed=0):
    """Query lengths 1, 6, 17, 64/G+1 (two row blocks), 100 and 0, over
    contexts with and without history, ragged last pages."""
    spec = wl.Spec(f"mq{h}x{hkv}x{d}x{bs}{kv}", h, hkv, d, bs, "bf16", seed=13 * h + d + bs + seed,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    g = h // hkv
    qlens = [1, 6, 17, 64 // g + 1, 100, 0, 3, 6]
    ctx = [1, 700, 17, 64 // g + 40, 333, 50, 3, 6 + 2 * bs + 1]
    plan = wl.multi_query_plan(ctx, qlens, bs, torch.Generator().manual_seed(spec.seed))
    return wl.build_inputs(spec, plan)


SHAPES = [  # (H, Hkv, D, BS): G = 1, 2, 4, 8 on both block sizes and head dims
    (8, 8, 128, 16), (4, 4, 64, 32), (16, 8, 64, 16), (16, 8, 128, 32),
    (32, 8, 128, 16), (16, 4, 64, 32), (64, 8, 128, 32), (16, 2, 64, 16),
]


@pytest.mark.parametrize("h,hkv,d,bs", SHAPES)
def test_shapes(h, hkv, d, bs):
    x = shape_case(h, hkv, d, bs)
    check_mq(x)
    check_mq(x, partition_tokens=2 * bs)
    check_mq(x, tiles_only=True)   # single-query sequences in the tiles as well


@pytest.mark.parametrize("h,hkv,d,bs", SHAPES)
def test_shapes_single_block(h, hkv, d, bs):
    """Every sequence's rows fit one 64-row block: query lengths up to 64 / G
    over ragged contexts, with and without partitions.  Sequences of more rows
    than the streaming kernel takes run on the two-stage ring beside it."""
    g = h // hkv
    spec = wl.Spec(f"mq1b{h}x{hkv}x{d}x{bs}", h, hkv, d, bs, "bf16", seed=7 * h + d + bs)
    qmax = 64 // g
    qlens = [1, min(6, qmax), qmax, 2, 0, 3, qmax]
    ctx = [1, 700, qmax + 40, 333, 50, 6 + 2 * bs + 1, qmax]
    plan = wl.multi_query_plan(ctx, qlens, bs, torch.Generator().manual_seed(spec.seed))
    x = wl.build_inputs(spec, plan)
    check_mq(x)
    check_mq(x, partition_tokens=2 * bs)
    check_mq(x, tiles_only=True)


def stream_case(h, hkv, d, bs, cap, kv="bf16", seed=0):
    """Sequences of at most `cap` rows (query lengths up to cap / G) over ragged
    contexts, one of them a single query, one empty."""
    g = h // hkv
    spec = wl.Spec(f"mqs{h}x{hkv}x{d}x{bs}{kv}{cap}", h, hkv, d, bs, "bf16", seed=11 * h + d + bs + cap + seed,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    qmax = max(1, cap // g)
    qlens = [qmax, 1, min(2, qmax), 0, qmax, max(1, qmax // 2)]
    ctx = [qmax + 700, 333, 6 + 2 * bs + 1, 50, qmax, 2 * bs + qmax + 3]
    plan = wl.multi_query_plan(ctx, qlens, bs, torch.Generator().manual_seed(spec.seed))
    return wl.build_inputs(spec, plan)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("h,hkv,d,bs", SHAPES)
def test_shapes_stream(h, hkv, d, bs, kv):
    """Verification-shaped batches: at most 16, 32 and 48 rows per sequence,
    with and without partitions, single queries in the tiles too.  Over an
    E4M3 cache at head_dim 64 or G = 1 the first two run on the streaming
    kernel at one and two 16-row tiles, the third beside the ring kernel;
    E4M3 at head_dim 128 with G >= 2, and bf16, run on the ring."""
    for cap in (16, 32, 48):
        if cap < h // hkv:
            continue
        x = stream_case(h, hkv, d, bs, cap, kv=kv)
        check_mq(x)
        check_mq(x, partition_tokens=2 * bs)
        check_mq(x, tiles_only=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_stream_partition_of_256_pages(kv):
    """A partition of exactly 256 pages (64 per wave, the streaming kernel's
    bound) and one page more, cut in two, at G = 1 (E4M3: streamed); the
    40-row sequence beside them runs on the ring."""
    bs = 16
    spec = wl.Spec(f"mqs256{kv}", 8, 8, 128, bs, "bf16", seed=77,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    plan = wl.multi_query_plan([256 * bs, 256 * bs + 5, 90], [4, 2, 40], bs,
                               torch.Generator().manual_seed(8))
    check_mq(wl.build_inputs(spec, plan), partition_tokens=256 * bs)


@pytest.mark.parametrize("h,hkv,d,bs", [(8, 8, 128, 16), (64, 8, 128, 32), (16, 8, 64, 16),
                                        (32, 4, 128, 32)])
def test_shapes_fp8(h, hkv, d, bs):
    x = shape_case(h, hkv, d, bs, kv="fp8")
    check_mq(x)
    check_mq(x, partition_tokens=3 * bs)


def test_single_queries_match_decode():
    """q_len = 1 everywhere is a decode step: both kernels against the oracle."""
    spec = wl.SPECS["gqa70b"]
    ctx = [1, 40, 513, 2000, 4100]
    plan = wl.multi_query_plan(ctx, [1] * len(ctx), spec.block_size, torch.Generator().manual_seed(3))
    x = wl.build_inputs(spec, plan)
    _, out_mq = check_mq(x)
    dec, _ = gpu_step(x, copy=False)
    ref, _, _ = oracle_step(x, copy=False)
    assert_close(as_f64(dec), ref, "bf16", "decode")
    assert_close(as_f64(out_mq), ref, "bf16", "multi-query vs decode oracle")


def test_chunking_matches_one_pass():
    """A chunk cut in two (the first half at the shorter context) gives the
    rows of the single pass, within tolerance of the same oracle values."""
    spec = wl.Spec("mqchunk", 32, 8, 128, 16, "bf16", seed=77)
    plan = wl.multi_query_plan([600], [300], 16, torch.Generator().manual_seed(5))
    x = wl.build_inputs(spec, plan)
    whole, t = gpu_mq_step(x)
    ref, _, _ = oracle_mq_step(x)
    first = torch.empty_like(t["q"][:120])
    binding.pa_multi_query(first, t["q"][:120].contiguous(), t["k_cache"], t["v_cache"],
                           t["block_tables"], torch.tensor([420], dtype=torch.int32, device="cuda"),
                           torch.tensor([0, 120], dtype=torch.int32, device="cuda"), x.scale, 600, 120)
    torch.cuda.synchronize()
    assert_close(as_f64(first), ref[:120], "bf16", "first half")
    assert_close(as_f64(whole), ref, "bf16", "whole")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_bad_device_values(kv):
    """Page ids past the pool and negative ones (ring kernel; for E4M3 the
    24-row sequence runs on the streaming kernel), too few tokens, invalid
    query ranges."""
    x = shape_case(32, 8, 128, 16, kv=kv)
    t = on_device(x)
    t["query_start"] = x.query_start.to("cuda").clone()
    qs = x.query_start.tolist()
    t["block_tables"][1, 3] = x.plan.num_blocks + 7   # page id past the pool: sequence 1's rows NaN
    t["block_tables"][2, 0] = -5                      # negative id of a page every row reads: NaN
    t["context_lens"][4] = 99                         # 100 queries > 99 tokens: rows NaN
    sentinel = torch.full_like(t["q"], 7.0)
    t["query_start"][7] = qs[7] + 1000                # sequences 6 and 7: invalid ranges, unwritten
    out, _ = gpu_mq_step(x, t=t, out=sentinel)
    o = out.float()
    ref, _, _ = oracle_mq_step(x)
    rows = lambda s: list(range(qs[s], qs[s + 1]))
    for s in (1, 2, 4):
        assert torch.isnan(o[rows(s)]).all(), s
    for s in (6, 7):
        assert (o[rows(s)] == 7.0).all(), s
    keep = rows(0) + rows(3)
    assert_close(as_f64(out)[keep], ref[keep], "bf16", "rows keeping the preconditions")


def test_repeat_is_deterministic():
    x = wl.make_inputs("specdec70b", **SMALL["specdec70b"])
    a, _ = gpu_mq_step(x)
    b, _ = gpu_mq_step(x)
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("h,hkv,d,bs", [(16, 8, 128, 16), (8, 8, 64, 32), (32, 4, 128, 32)])
def test_long_context_page_window(h, hkv, d, bs, kv):
    """A workgroup that walks more than 256 pages reloads its page-id window:
    a chunk of two row blocks over a context of 256 pages and more (the
    three-stage ring for bf16), and single-block sequences whose one partition
    spans more than 256 pages (the two-stage ring)."""
    g = h // hkv
    spec = wl.Spec(f"mqlong{h}x{hkv}x{d}x{bs}{kv}", h, hkv, d, bs, "bf16", seed=5 * h + d + bs,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    long_ctx = 256 * bs + 700
    plan = wl.multi_query_plan([long_ctx, 300], [64 // g + 1, 3], bs,
                               torch.Generator().manual_seed(spec.seed))
    check_mq(wl.build_inputs(spec, plan))
    plan = wl.multi_query_plan([long_ctx, 2 * long_ctx, 40], [6, 64 // g, 1], bs,
                               torch.Generator().manual_seed(spec.seed + 1))
    check_mq(wl.build_inputs(spec, plan), partition_tokens=512 * bs)


@pytest.mark.parametrize("name,kw", [("specdec70b", {}), ("chunked13b", {}), ("specdec70b_fp8", {}),
                                     ("specdec70b_fp8", dict(query_len=4))])
def test_full_size_sampled(name, kw):
    """Full-size workloads in the benchmark's configuration; the oracle checks
    every row of a few sampled sequences (both chunks of the prefill batch).
    Four drafted tokens over the E4M3 cache (32 rows) stream."""
    torch.cuda.empty_cache()
    x = wl.make_inputs(name, device="cuda", poison=True, **kw)
    qs = x.query_start.tolist()
    seqs = [0, 1, len(qs) - 2] if name.startswith("chunked") else [0, 7, 31]
    refs = sampled_mq_reference(x, seqs)  # host copies taken before the GPU step
    out, t = gpu_mq_step(x, t={n: getattr(x, n) for n in ("q", "k_cache", "v_cache", "key",
                                                            "value", "slot_mapping", "block_tables",
                                                            "context_lens", "block_pairs")})
    assert torch.isfinite(out.float()).all()
    for s in seqs:
        assert_close(as_f64(out[qs[s]:qs[s + 1]]), refs[s], "bf16", f"{name} seq {s}")
    del x, t, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("own_handle", [False, True])
def test_side_stream_same_bits_and_ordered(own_handle):
    """Decode rows on a side stream (the binding's per-device one, or a
    handle the caller creates and destroys) give the bits of the one-stream
    launch, on a caller stream other than the default one, and work queued on
    that stream after the call sees the whole output (the join)."""
    x = wl.make_inputs("chunked13b", **SMALL["chunked13b"])
    one, t = gpu_mq_step(x, one_stream=True)
    ref, _, _ = oracle_mq_step(x)
    assert_close(as_f64(one), ref, "bf16", "one stream")
    side = binding.SideStream.create() if own_handle else None
    caller = torch.cuda.Stream()
    out = torch.full_like(t["q"], float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(caller):
        binding.pa_multi_query(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                               t["context_lens"], t["query_start"], x.scale, x.max_context_len,
                               int(x.plan.query_lens.max()), stream=caller, side=side)
        seen = out.clone()
    torch.cuda.synchronize()
    if side is not None:
        side.destroy()
        assert side.stream is None and side.fork_event is None
    assert np.array_equal(bits(out), bits(one))
    assert np.array_equal(bits(seen), bits(one))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("pt", [256, 160])
def test_fixed_partitions_batch_invariant(kv, pt):
    """With partition_tokens fixed, a sequence's rows are the same bits alone as
    in a batch (the default partition size follows the batch shape, so this is
    the caller's way to batch-invariant rows).  Over an E4M3 cache the 24-,
    20- and 12-row sequences stream (two tiles in the batch, the 12-row one
    one tile alone) beside the 120-row one on the ring.  In the batch the
    other sequences run on the three-stage ring, alone on the two-stage one,
    which split a partition of 8 (or 5) steps differently between unmasked and
    masked steps.  Head_dim 64, where E4M3 verification rows stream."""
    spec = wl.Spec(f"mqinv{kv}", 32, 8, 64, 16, "bf16", seed=91,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    plan = wl.multi_query_plan([900, 2500, 40, 1300, 700], [6, 5, 1, 30, 3], 16,
                               torch.Generator().manual_seed(4))
    x = wl.build_inputs(spec, plan)
    whole, t = gpu_mq_step(x, partition_tokens=pt)
    ref, _, _ = oracle_mq_step(x)
    assert_close(as_f64(whole), ref, "bf16", spec.name)
    qs = x.query_start.tolist()
    for s in (0, 1, 3, 4):
        rows = slice(qs[s], qs[s + 1])
        q = t["q"][rows].contiguous()
        alone = torch.empty_like(q)
        binding.pa_multi_query(alone, q, t["k_cache"], t["v_cache"], t["block_tables"][s:s + 1].contiguous(),
                               t["context_lens"][s:s + 1].contiguous(),
                               torch.tensor([0, qs[s + 1] - qs[s]], dtype=torch.int32, device="cuda"),
                               x.scale, x.max_context_len, qs[s + 1] - qs[s], partition_tokens=pt,
                               k_scale=x.k_scale, v_scale=x.v_scale)
        torch.cuda.synchronize()
        assert np.array_equal(bits(alone), bits(whole[rows])), s


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_work_list_and_in_kernel_lookup_agree(kv):
    """A verification batch of 80 sequences takes its work list from the
    schedule kernel, a batch of at most 64 finds the items in the kernel: the
    oracle checks the large batch, and 40 of its sequences run as a batch of
    their own give the same bits (fixed partitions)."""
    spec = wl.Spec(f"mqlist{kv}", 64, 8, 128, 16, "bf16", seed=93,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    g = torch.Generator().manual_seed(8)
    n = 80
    ctx = torch.randint(8, 600, (n,), generator=g).tolist()
    qlen = torch.randint(2, 7, (n,), generator=g).tolist()
    plan = wl.multi_query_plan(ctx, qlen, 16, g)
    x = wl.build_inputs(spec, plan)
    whole, t = gpu_mq_step(x, partition_tokens=128)
    ref, _, _ = oracle_mq_step(x)
    assert_close(as_f64(whole), ref, "bf16", spec.name)
    qs = x.query_start.tolist()
    sub = list(range(20, 60))
    rows = torch.cat([torch.arange(qs[s], qs[s + 1]) for s in sub]).cuda()
    starts = [0]
    for s in sub:
        starts.append(starts[-1] + qs[s + 1] - qs[s])
    q = t["q"].index_select(0, rows).contiguous()
    part = torch.empty_like(q)
    binding.pa_multi_query(part, q, t["k_cache"], t["v_cache"], t["block_tables"][sub].contiguous(),
                           t["context_lens"][sub].contiguous(),
                           torch.tensor(starts, dtype=torch.int32, device="cuda"), x.scale,
                           x.max_context_len, max(qlen), partition_tokens=128,
                           k_scale=x.k_scale, v_scale=x.v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(part), bits(whole.index_select(0, rows)))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("n", [40, 80])
def test_every_work_item_runs(kv, n):
    """Work items are listed in two classes (full partitions and row blocks
    first, then each cut sequence's last partition): with the workspace filled
    with NaN before the call, every partition result the merge reads must have
    been written by this call.  40 sequences find their items in the kernel,
    80 take them from the schedule kernel; contexts of 8-1200 tokens in
    partitions of 128 (1-10 per sequence) and some long chunks."""
    spec = wl.Spec(f"mqitems{kv}", 32, 8, 128, 16, "bf16", seed=95,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    g = torch.Generator().manual_seed(12)
    ctx = torch.randint(8, 1200, (n,), generator=g).tolist()
    qlen = [min(c, q) for c, q in zip(ctx, torch.randint(1, 7, (n,), generator=g).tolist())]
    qlen[3] = min(ctx[3], 40)  # 320 rows: three 128-row blocks
    x = wl.build_inputs(spec, wl.multi_query_plan(ctx, qlen, 16, g))
    t = on_device(x)
    t["query_start"] = x.query_start.to("cuda").clone()
    binding.pa_reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], t["slot_mapping"],
                                 k_scale=x.k_scale, v_scale=x.v_scale)
    ccode = binding.PA_FP8_E4M3 if kv == "fp8" else binding.PA_BF16
    nbytes = binding.pa_multi_query_workspace_size(n, int(x.query_start[-1]), spec.num_heads, spec.num_kv_heads,
                                                   spec.head_dim, 16, x.max_context_len, binding.PA_BF16, 128,
                                                   ccode)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")  # float NaN everywhere
    out = torch.empty_like(t["q"])
    binding.pa_multi_query(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                           t["query_start"], x.scale, x.max_context_len, max(qlen), partition_tokens=128,
                           workspace=ws, k_scale=x.k_scale, v_scale=x.v_scale)
    torch.cuda.synchronize()
    ref, _, _ = oracle_mq_step(x)
    assert_close(as_f64(out), ref, "bf16", spec.name)


@pytest.mark.parametrize("kv,hkv,group,d", [("bf16", 4, 1, 128), ("fp8", 2, 8, 64)])
def test_rows_of_no_sequence(kv, hkv, group, d):
    """query_start may leave rows of q to no sequence.  The host's bound on
    the shortest sequence (num_query_tokens - (num_seqs - 1) * max_query_len
    queries) then does not hold, and a short sequence must still be computed:
    3 queries over 3000 tokens beside a 100-query chunk, with 97 rows of no
    sequence after them, at partitions of 256 tokens (bf16: one-tile ring;
    E4M3 at G = 8 and head_dim 64: the short rows would otherwise stream)."""
    spec = wl.Spec(f"mqgap{kv}", hkv * group, hkv, d, 16, "bf16", seed=99,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    gen = torch.Generator().manual_seed(14)
    x = wl.build_inputs(spec, wl.multi_query_plan([2000, 3000], [100, 3], 16, gen))
    t = on_device(x)
    binding.pa_reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], t["slot_mapping"],
                                 k_scale=x.k_scale, v_scale=x.v_scale)
    extra = torch.randn(97, spec.num_heads, d, generator=gen).to(torch.bfloat16).cuda()
    q = torch.cat([t["q"], extra]).contiguous()
    out = torch.full_like(q, float("nan"))
    binding.pa_multi_query(out, q, t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                           x.query_start.to("cuda").clone(), x.scale, x.max_context_len, 100,
                           partition_tokens=256, k_scale=x.k_scale, v_scale=x.v_scale)
    torch.cuda.synchronize()
    ref, _, _ = oracle_mq_step(x)
    assert_close(as_f64(out[: x.q.shape[0]]), ref, "bf16", spec.name)


@pytest.mark.parametrize("h,hkv,bs,kv", [(40, 40, 16, "bf16"), (64, 8, 32, "bf16"), (64, 8, 32, "fp8")])
def test_pool_past_2g_elements(h, hkv, bs, kv):
    """Every page of the batch lies past 2^31 elements of a 2.29e9-element
    cache: the ring's buffer descriptors, the streaming kernel and the decode
    rows all address it with 64-bit offsets."""
    torch.cuda.empty_cache()
    d = 128
    per_block = hkv * bs * d
    nb = (2_290_000_000 + per_block - 1) // per_block
    spec = wl.Spec(f"mqbig{h}x{hkv}x{bs}{kv}", h, hkv, d, bs, "bf16", seed=h + bs + 5,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    plan = wl.multi_query_plan([700, 2049, 5000, 3000], [1, 6, 4, 100], bs,
                               torch.Generator().manual_seed(spec.seed))
    plan = to_top_of_pool(plan, nb)
    assert int(plan.block_tables[plan.block_tables >= 0].min()) * per_block > 2 ** 31
    x = wl.build_inputs(spec, plan, device="cuda", poison=True)
    qs = x.query_start.tolist()
    seqs = [0, 1, 2, 3]
    refs = sampled_mq_reference(x, seqs)
    out, t = gpu_mq_step(x, t={n: getattr(x, n) for n in ("q", "k_cache", "v_cache", "key",
                                                            "value", "slot_mapping", "block_tables",
                                                            "context_lens", "block_pairs")})
    for s in seqs:
        assert_close(as_f64(out[qs[s]:qs[s + 1]]), refs[s], "bf16", f"{spec.name} seq {s}")
    del x, t, out
    torch.cuda.empty_cache()
